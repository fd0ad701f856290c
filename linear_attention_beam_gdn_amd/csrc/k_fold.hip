// Fold a chain of transition records onto a dense state:
//   S <- alpha_j S + k_j delta_j^T       (channel decay: diag(a_j) S + ...)
// in chain order.  This is the eager GDN update written with the stored
// record r_j = (alpha_j, delta_j, k_j) (OneLA §3.2, GTR equation), so the
// result is the dense state the chain stands for.  It serves the bounded-log
// merge of DeltaLog (Figure 4: at a full log the logical state is written
// back into the dense base; Figure 5: the merge writes back base tiles) and
// the materialisation of any beam's state.
//
// One workgroup per (item, head, row slice): each thread owns RPG rows x 4
// columns of the [d_k][d_v] state in registers, streams them in and out with
// 16-byte accesses, and applies every record to them; the key entries and
// decays of a record are the same for a whole row, the update vector for a
// column.  States up to 128 x 128 take one slice; wider ones (d_v = 512 or
// d_k = 256) are cut into NSL slices of d_k rows.
//
// Update vectors are FP32, or bf16 for the plain rule (the RWKV6 row of
// DeltaLog Table 1, whose log keeps U in BF16 per Table 3).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

struct FoldArgs {
  const float* src;
  float* dst;
  const float* rec_delta;  // FP32 update vectors (bf16 bit patterns when UB16)
  const uint16_t* rec_k;
  const float* rec_alpha;
  const int32_t* anc;
  const int32_t* rb;
  int R, Wm, H, L, t, beam;
  int Hk, gq;  // key heads; value head h uses key head h / gq
  int dst_per_item;
};

template <int DK, int DV>
struct FoldGeom {
  static constexpr int C4 = DV / 4;
  static_assert(C4 <= 256, "d_v of at most 1024");
  static constexpr int NRG0 = 256 / C4;
  static constexpr int NRG = NRG0 < DK ? NRG0 : DK;
  static_assert(DK % NRG == 0, "d_k must split evenly over row groups");
  static constexpr int RPG0 = DK / NRG;
  static constexpr int RPG = RPG0 < 16 ? RPG0 : 16;  // rows per thread
  static constexpr int NSL = DK / (NRG * RPG);       // row slices
  static_assert(NSL * NRG * RPG == DK, "d_k must split evenly over row slices");
  static constexpr int NT = C4 * NRG;
  // 16-byte pieces of a record row staged in LDS (bf16 key, FP32 update
  // vector, FP32 per-channel decays) and the pieces a thread loads at most
  static_assert(DK % 8 == 0 && DV % 4 == 0, "record rows must be whole 16-byte pieces");
  static constexpr int KCH = DK / 8, DCH = DV / 4, ACH = DK / 4;
  static constexpr int NKL = (GDN_MAX_STEPS * KCH + NT - 1) / NT;
  static constexpr int NDL = (GDN_MAX_STEPS * DCH + NT - 1) / NT;
  static constexpr int VCH = DV / 8;  // 16-byte pieces of a bf16 update vector
  static constexpr int NDL16 = (GDN_MAX_STEPS * VCH + NT - 1) / NT;
  static constexpr int NAL = (GDN_MAX_STEPS * ACH + NT - 1) / NT;
};

// Dynamic LDS of a chain of n records (floats): keys [n][d_k], update vectors
// [n][d_v], decays [n][A] padded to a multiple of four.
__host__ __device__ constexpr int fold_lds_floats(int dk, int dv, int a, int n) {
  return n * dk + n * dv + ((n * a + 3) & ~3);
}

// Built for four waves per SIMD (at most 128 registers) where that needs no
// spills: d_v up to 256, and d_v = 128 with per-channel decay.
template <int DK, int DV, bool CH, bool UB16>
__global__ __launch_bounds__((FoldGeom<DK, DV>::NT), ((DV <= 256 && !(CH && DV > 128)) ? 4 : 1))
void k_fold(FoldArgs a) {
  using G = FoldGeom<DK, DV>;
  constexpr int A = CH ? DK : 1;
  const int tid = threadIdx.x;
  const int h = blockIdx.x % a.H;
  const int sl = (blockIdx.x / a.H) % G::NSL;
  const int item = blockIdx.x / (a.H * G::NSL);
  const int c4 = tid % G::C4;
  const int rg = tid / G::C4;
  const int row0 = (sl * G::NRG + rg) * G::RPG;  // this thread's first row
  int r = item, b = a.beam;
  if (a.rb) {
    r = a.rb[2 * item];
    b = a.rb[2 * item + 1];
  }
  r = clampi(r, 0, a.R - 1);
  b = clampi(b, 0, a.Wm - 1);
  const int t = a.t;
  const int n = t + 1;  // records in the chain: the ancestors' and the beam's own

  const float* src = a.src + ((size_t)r * a.H + h) * DK * DV;
  float* dst = a.dst_per_item ? a.dst + ((size_t)item * a.H + h) * DK * DV
                              : a.dst + ((size_t)r * a.H + h) * DK * DV;

  // The chain's records in one batch of 16-byte loads (each piece looks up
  // its record's slot in the beam's ancestry row), issued before the state's
  // rows and put in LDS while those are in flight, so the fold below reads
  // LDS only.
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  float* lk = dyn;              // [n][DK] keys
  float* ld = lk + n * DK;      // [n][DV] update vectors
  float* la = ld + n * DV;      // [n][A] decays
  const int32_t* arow = a.anc + (((size_t)t * a.R + r) * a.Wm + b) * a.L;
  // the beam's own record: at its order key (the last entry of its ancestry
  // row) for scalar decay with beams after step 0, else at its index
  const int own = (!CH && a.Wm > 1 && t > 0) ? clampi(arow[a.L - 1], 0, a.Wm - 1) : b;
  auto rec_at = [&](int j) -> size_t {
    const int slot = j < t ? clampi(arow[j], 0, a.Wm - 1) : own;
    return (((size_t)j * a.R + r) * a.Wm + slot) * a.H + h;
  };
  auto rec_at_k = [&](int j) -> size_t {
    const int slot = j < t ? clampi(arow[j], 0, a.Wm - 1) : own;
    return (((size_t)j * a.R + r) * a.Wm + slot) * a.Hk + h / a.gq;
  };
  const int nk = n * G::KCH, nd = UB16 ? n * G::VCH : n * G::DCH;
  constexpr int NDLX = UB16 ? G::NDL16 : G::NDL;
  u32x4 kb[G::NKL];
  f32x4 db[UB16 ? 1 : G::NDL], ab[CH ? G::NAL : 1];
  u32x4 db16[UB16 ? G::NDL16 : 1];
  const uint16_t* rec_u16 = reinterpret_cast<const uint16_t*>(a.rec_delta);
  float as = 0.f;
#pragma unroll
  for (int m = 0; m < G::NKL; ++m) {
    const int c = min(tid + m * G::NT, nk - 1);
    kb[m] = *reinterpret_cast<const u32x4*>(a.rec_k + rec_at_k(c / G::KCH) * DK + (c % G::KCH) * 8);
  }
#pragma unroll
  for (int m = 0; m < NDLX; ++m) {
    const int c = min(tid + m * G::NT, nd - 1);
    if constexpr (UB16)
      db16[m] = *reinterpret_cast<const u32x4*>(rec_u16 + rec_at(c / G::VCH) * DV + (c % G::VCH) * 8);
    else
      db[m] = *reinterpret_cast<const f32x4*>(a.rec_delta + rec_at(c / G::DCH) * DV + (c % G::DCH) * 4);
  }
  if constexpr (CH) {
#pragma unroll
    for (int m = 0; m < G::NAL; ++m) {
      const int c = min(tid + m * G::NT, n * G::ACH - 1);
      ab[m] = *reinterpret_cast<const f32x4*>(a.rec_alpha + rec_at(c / G::ACH) * A + (c % G::ACH) * 4);
    }
  } else {
    if (tid < n) as = a.rec_alpha[rec_at(tid)];
  }

  f32x4 st[G::RPG];
#pragma unroll
  for (int i = 0; i < G::RPG; ++i)
    st[i] = *reinterpret_cast<const f32x4*>(src + (size_t)(row0 + i) * DV + c4 * 4);

#pragma unroll
  for (int m = 0; m < G::NKL; ++m) {
    const int c = tid + m * G::NT;
    if (c < nk) {
      const u32x4 w = kb[m];
      *reinterpret_cast<f32x4*>(lk + c * 8) = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      *reinterpret_cast<f32x4*>(lk + c * 8 + 4) = f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
    }
  }
#pragma unroll
  for (int m = 0; m < NDLX; ++m) {
    const int c = tid + m * G::NT;
    if constexpr (UB16) {
      if (c < nd) {
        const u32x4 w = db16[m];
        *reinterpret_cast<f32x4*>(ld + c * 8) = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
        *reinterpret_cast<f32x4*>(ld + c * 8 + 4) = f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
      }
    } else {
      if (c < nd) *reinterpret_cast<f32x4*>(ld + c * 4) = db[m];
    }
  }
  if constexpr (CH) {
#pragma unroll
    for (int m = 0; m < G::NAL; ++m)
      if (tid + m * G::NT < n * G::ACH) *reinterpret_cast<f32x4*>(la + (tid + m * G::NT) * 4) = ab[m];
  } else {
    if (tid < n) la[tid] = as;
  }
  __syncthreads();

  // the records in chain order (a do-while: every chain has at least the
  // beam's own record, and this loop shape keeps the state in one set of
  // registers across the loop instead of a copy per entry)
  int j = 0;
  do {
    const f32x4 dj = *reinterpret_cast<const f32x4*>(ld + j * DV + c4 * 4);
    const float aj0 = CH ? 0.f : la[j];
#pragma unroll
    for (int i = 0; i < G::RPG; ++i) {
      const int row = row0 + i;
      const float kj = lk[j * DK + row];
      const float aj = CH ? la[j * A + row] : aj0;
      st[i] = apply_record(st[i], aj, kj, dj);
    }
  } while (++j <= t);
#pragma unroll
  for (int i = 0; i < G::RPG; ++i)
    *reinterpret_cast<f32x4*>(dst + (size_t)(row0 + i) * DV + c4 * 4) = st[i];
}

template <int DK, int DV, bool CH, bool UB16 = false>
int launch(const gdn_shape& sh, const gdn_store& st, int t, const int32_t* rb, int beam, int n,
           const float* src, float* dst, bool dst_per_item, hipStream_t stream) {
  FoldArgs a;
  a.src = src;
  a.dst = dst;
  a.rec_delta = st.rec_delta;
  a.rec_k = st.rec_k;
  a.rec_alpha = st.rec_alpha;
  a.anc = st.anc;
  a.rb = rb;
  a.R = sh.R;
  a.Wm = sh.W_max;
  a.H = sh.H;
  a.L = sh.L_max;
  a.t = t;
  a.beam = beam;
  a.Hk = key_heads(sh);
  a.gq = sh.H / a.Hk;
  a.dst_per_item = dst_per_item ? 1 : 0;
  const long grid = (long)n * sh.H * FoldGeom<DK, DV>::NSL;
  if (grid > 0x7FFFFFFFL) return GDN_EINVAL;
  const size_t lds = (size_t)fold_lds_floats(DK, DV, CH ? DK : 1, t + 1) * sizeof(float);
  hipLaunchKernelGGL((k_fold<DK, DV, CH, UB16>), dim3((unsigned)grid), dim3(FoldGeom<DK, DV>::NT), lds,
                     stream, a);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // namespace

int launch_fold(const gdn_shape& sh, const gdn_store& st, int t, const int32_t* rb, int beam, int n,
                const float* src, float* dst, bool dst_per_item, hipStream_t stream) {
  // the fold is the same for both channel rules; the plain rule keeps its
  // update vectors (v_t itself) in bf16
  const bool ch = sh.decay_kind != GDN_DECAY_SCALAR;
  const bool plain = sh.decay_kind == GDN_DECAY_CHANNEL_PLAIN;
#define GDN_CASE(DK_, DV_)                                                                          \
  if (sh.dk == DK_ && sh.dv == DV_) {                                                               \
    if (plain) return launch<DK_, DV_, true, true>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream); \
    return ch ? launch<DK_, DV_, true>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream)      \
              : launch<DK_, DV_, false>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream);    \
  }
  GDN_CASE(16, 16)
  GDN_CASE(32, 32)
  GDN_CASE(64, 64)
  GDN_CASE(128, 128)
#undef GDN_CASE
#define GDN_CASE(DK_, DV_)                                                           \
  if (sh.dk == DK_ && sh.dv == DV_ && !plain)                                        \
    return ch ? launch<DK_, DV_, true>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream) \
              : launch<DK_, DV_, false>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream);
  GDN_CASE(128, 256)
  GDN_CASE(128, 512)
#undef GDN_CASE
  if (!ch && sh.dk == 256) {
    if (sh.dv == 128) return launch<256, 128, false>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream);
    if (sh.dv == 256) return launch<256, 256, false>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream);
    if (sh.dv == 512) return launch<256, 512, false>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream);
  }
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn
