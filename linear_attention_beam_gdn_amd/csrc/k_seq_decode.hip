// Decode step for independent sequences (one beam per request): the
// bounded-log scheme of DeltaLog (Figure 4: dense base plus a log of compact
// records, append while the log is not full).  With a single beam there is
// no cross-beam reuse of the base, so the step is a matrix-vector product
// bound by reading the base: one workgroup per (sequence, head) streams the
// [d_k][d_v] FP32 base once with 16-byte loads, forms the two projections
// base^T x_q and base^T x_k with FP32 FMAs, reduces them across row groups in
// LDS, replays the log on them, and appends the new record.
//
// The merge path (DeltaLog Figure 5 caption: the same structure, writing back
// dense-base tiles; Figure 4: the log is folded into the base when it is
// full) is the same kernel with MRG set: after the token's append, each
// thread folds records 0..t (the new one included) into the base rows it
// already holds, S <- alpha_j S + k_j delta_j^T in log order, and writes them
// back, so a merge costs no second read of the base.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

struct SeqArgs {
  const float* S;
  float* S_out;  // the base written back by the merge path
  float* rec_delta;
  uint16_t* rec_k;
  float* rec_alpha;
  int32_t* anc;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  float* o;
  int R, H, L, t;
  int Hk, gq;  // key heads; value head h uses key head h / gq
};

template <int DK, int DV>
struct SeqGeom {
  static_assert(DV % 8 == 0 && DK % 8 == 0, "d_k and d_v must be multiples of 8");
  static constexpr int C4 = DV / 4;                      // float4 column groups
  static constexpr int NRG0 = 256 / C4;
  static constexpr int NRG = NRG0 < DK ? NRG0 : DK;      // row groups
  static_assert(DK % NRG == 0, "d_k must split evenly over row groups");
  static constexpr int RPG = DK / NRG;                   // rows per thread
  static constexpr int NT = C4 * NRG;                    // threads
  static constexpr int NWV = (NT + 63) / 64;             // waves
  // 16-byte pieces of the rows staged in LDS: a bf16 row of d_k (keys, q),
  // a bf16 row of d_v (v), an FP32 row of d_v (update vectors), an FP32 row
  // of d_k (per-channel decays); and the pieces each thread loads at most
  static constexpr int KCH = DK / 8, VCH = DV / 8, DCH = DV / 4, ACH = DK / 4;
  static constexpr int NKL = ((GDN_MAX_STEPS + 1) * KCH + NT - 1) / NT;
  static constexpr int NVL = (VCH + NT - 1) / NT;
  static constexpr int NDL = ((GDN_MAX_STEPS - 1) * DCH + NT - 1) / NT;
  static constexpr int NAL = (GDN_MAX_STEPS * ACH + NT - 1) / NT;
};

// Dynamic LDS of a step with log length t (floats): the keys of log entries
// 0..t-1, k_t and q_t as rows 0..t+1 of [d_k]; v_t; the update vectors of
// entries 0..t (row t: this token's) as [d_v] rows; the decays of entries
// 0..t (one each, or a [d_k] row each), padded to a multiple of four.
__host__ __device__ constexpr int seq_lds_floats(int dk, int dv, int a, int t) {
  return (t + 2) * dk + dv + (t + 1) * dv + (((t + 1) * a + 3) & ~3);
}

__device__ __forceinline__ void put_bf16x8(float* dst, const u32x4& w) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
}

// PLAIN: the RWKV6 update pair (k_t, v_t) (channel decay, no delta
// correction): delta_t = v_t, and no projection of k_t is formed.
// The merge path holds the base rows in registers to the end; it is built
// for four waves per SIMD (at most 128 registers), so that four workgroups
// per compute unit overlap their read, fold and write phases.
template <int DK, int DV, bool CH, bool MRG, bool PLAIN>
__global__ __launch_bounds__((SeqGeom<DK, DV>::NT), (MRG ? 4 : 1)) void k_seq_decode(SeqArgs a) {
  static_assert(CH || !PLAIN, "the plain update rule comes with channel decay");
  using G = SeqGeom<DK, DV>;
  constexpr int A = CH ? DK : 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int h = blockIdx.x % a.H;
  const int r = blockIdx.x / a.H;
  const int c4 = tid % G::C4;
  const int rg = tid / G::C4;
  const int t = a.t;
  const size_t tok = (size_t)r * a.H + h;                 // (r, beam 0, h)
  auto rec_at = [&](int j) -> size_t { return ((size_t)j * a.R + r) * a.H + h; };
  // the key head's q, k and record keys (one value head writes the record key)
  const size_t tk = (size_t)r * a.Hk + h / a.gq;
  auto rec_at_k = [&](int j) -> size_t { return ((size_t)j * a.R + r) * a.Hk + h / a.gq; };
  const bool key_writer = h % a.gq == 0;

  __shared__ float probe_q[DK], probe_k[DK];
  __shared__ float red_q[G::NRG][DV], red_k[G::NRG][DV];
  __shared__ float dots_q[GDN_MAX_STEPS], dots_k[GDN_MAX_STEPS], dot_qk;
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  float* lk = dyn;                     // [t + 2][DK]: keys 0..t-1, k_t, q_t
  float* sq = lk + (t + 1) * DK;
  float* sk = lk + t * DK;
  float* sv = lk + (t + 2) * DK;       // [DV]
  float* ld = sv + DV;                 // [t + 1][DV]
  float* la = ld + (t + 1) * DV;       // [t + 1][A]

  // One batch of loads: the token's q, k, v, the log's keys, update vectors
  // and decays (16-byte pieces into registers), then this thread's rows of
  // the base; the pieces go to LDS while the base is still in flight, so no
  // later phase waits on memory but the one that needs the base.
  const float bt = a.beta[tok];
  const int nk = (t + 2) * G::KCH, nd = t * G::DCH;
  u32x4 kb[G::NKL], vb[G::NVL];
  f32x4 db[G::NDL], ab[CH ? G::NAL : 1];
  float as = 0.f;
#pragma unroll
  for (int m = 0; m < G::NKL; ++m) {
    const int c = min(tid + m * G::NT, nk - 1);
    const int j = c / G::KCH, part = c % G::KCH;
    const uint16_t* src = j < t ? a.rec_k + rec_at_k(j) * DK : (j == t ? a.k : a.q) + tk * DK;
    kb[m] = *reinterpret_cast<const u32x4*>(src + part * 8);
  }
#pragma unroll
  for (int m = 0; m < G::NVL; ++m) {
    const int c = min(tid + m * G::NT, G::VCH - 1);
    vb[m] = *reinterpret_cast<const u32x4*>(a.v + tok * DV + c * 8);
  }
#pragma unroll
  for (int m = 0; m < G::NDL; ++m) {
    const int c = tid + m * G::NT;
    if (c < nd) db[m] = *reinterpret_cast<const f32x4*>(a.rec_delta + rec_at(c / G::DCH) * DV + (c % G::DCH) * 4);
  }
  if constexpr (CH) {
#pragma unroll
    for (int m = 0; m < G::NAL; ++m) {
      const int c = min(tid + m * G::NT, (t + 1) * G::ACH - 1);
      const int j = c / G::ACH, part = c % G::ACH;
      const float* src = j < t ? a.rec_alpha + rec_at(j) * DK : a.alpha + tok * DK;
      ab[m] = *reinterpret_cast<const f32x4*>(src + part * 4);
    }
  } else {
    if (tid <= t) as = tid < t ? a.rec_alpha[rec_at(tid)] : a.alpha[tok];
  }

  const float* S = a.S + tok * DK * DV;
  f32x4 st[G::RPG];
#pragma unroll
  for (int i = 0; i < G::RPG; ++i)
    st[i] = *reinterpret_cast<const f32x4*>(S + (size_t)(rg * G::RPG + i) * DV + c4 * 4);

#pragma unroll
  for (int m = 0; m < G::NKL; ++m)
    if (tid + m * G::NT < nk) put_bf16x8(lk + (tid + m * G::NT) * 8, kb[m]);
#pragma unroll
  for (int m = 0; m < G::NVL; ++m)
    if (tid + m * G::NT < G::VCH) put_bf16x8(sv + (tid + m * G::NT) * 8, vb[m]);
#pragma unroll
  for (int m = 0; m < G::NDL; ++m)
    if (tid + m * G::NT < nd) *reinterpret_cast<f32x4*>(ld + (tid + m * G::NT) * 4) = db[m];
  if constexpr (CH) {
#pragma unroll
    for (int m = 0; m < G::NAL; ++m)
      if (tid + m * G::NT < (t + 1) * G::ACH) *reinterpret_cast<f32x4*>(la + (tid + m * G::NT) * 4) = ab[m];
  } else {
    if (tid <= t) la[tid] = as;
  }
  __syncthreads();

  // probes x_q = c * q, x_k = c * k with c = prod_{i<=t} a_i (channel decay)
  for (int kk = tid; kk < DK; kk += G::NT) {
    float cq = 1.f;
    if constexpr (CH) {
      cq = la[t * DK + kk];
      for (int j = 0; j < t; ++j) cq *= la[j * DK + kk];
    }
    probe_q[kk] = cq * sq[kk];
    if constexpr (!PLAIN) probe_k[kk] = cq * sk[kk];
  }
  // dot products of the replay: wave wv takes log entries j = wv, wv + NWV, ..
  // (entry t is k_t . q_t); channel decay weights them by prod_{i=j+1..t} a_i
  for (int j = wv; j <= t; j += G::NWV) {
    float pq = 0.f, pk = 0.f;
    for (int kk = lane; kk < DK; kk += 64) {
      const float qv = sq[kk];
      if (j == t) {
        pq += sk[kk] * qv;
      } else {
        float y = lk[j * DK + kk];
        if constexpr (CH) {
          y *= la[t * DK + kk];
          for (int i = j + 1; i < t; ++i) y *= la[i * DK + kk];
        }
        pq += y * qv;
        if constexpr (!PLAIN) pk += y * sk[kk];
      }
    }
    pq = wave_sum(pq);
    pk = wave_sum(pk);
    if (lane == 0) {
      if (j == t) dot_qk = pq;
      else {
        dots_q[j] = pq;
        dots_k[j] = pk;
      }
    }
  }
  __syncthreads();

  // partial projections over this thread's rows
  f32x4 pq = {0.f, 0.f, 0.f, 0.f}, pk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < G::RPG; ++i) {
    const int row = rg * G::RPG + i;
    pq += st[i] * probe_q[row];
    if constexpr (!PLAIN) pk += st[i] * probe_k[row];
  }
  *reinterpret_cast<f32x4*>(&red_q[rg][c4 * 4]) = pq;
  if constexpr (!PLAIN) *reinterpret_cast<f32x4*>(&red_k[rg][c4 * 4]) = pk;
  __syncthreads();

  const float at = CH ? 1.f : la[t];
  const size_t rec_t = rec_at(t);
  for (int col = tid; col < DV; col += G::NT) {
    float uq = 0.f, uk = 0.f;
#pragma unroll 8
    for (int g = 0; g < G::NRG; ++g) {
      uq += red_q[g][col];
      if constexpr (!PLAIN) uk += red_k[g][col];
    }
    for (int j = 0; j < t; ++j) {
      const float dj = ld[j * DV + col];
      if constexpr (!CH) {
        const float aj = la[j];
        uq = aj * uq + dj * dots_q[j];
        uk = aj * uk + dj * dots_k[j];
      } else {
        uq += dj * dots_q[j];
        if constexpr (!PLAIN) uk += dj * dots_k[j];
      }
    }
    const float vv = sv[col];
    const float d = PLAIN ? vv : bt * (vv - at * uk);
    a.o[tok * DV + col] = at * uq + d * dot_qk;
    a.rec_delta[rec_t * DV + col] = d;
    if constexpr (MRG) ld[t * DV + col] = d;
  }
  // the appended key and decay are bit copies of the token's inputs (a bf16
  // value widened to FP32 and cut back is the same value)
  for (int kk = tid; kk < DK; kk += G::NT) {
    if (key_writer) a.rec_k[rec_at_k(t) * DK + kk] = (uint16_t)(__float_as_uint(sk[kk]) >> 16);
    if constexpr (CH) a.rec_alpha[rec_t * A + kk] = la[t * DK + kk];
  }
  if constexpr (!CH)
    if (tid == 0) a.rec_alpha[rec_t] = at;
  if (h == 0 && tid < t) a.anc[(((size_t)t * a.R + r) * 1 + 0) * a.L + tid] = 0;

  if constexpr (MRG) {
    // fold the full log into this thread's rows of the base, records 0..t in
    // log order (the same update, in the same order, as the stand-alone
    // merge), from the staged log and this token's update vector (a do-while,
    // which keeps the base in one set of registers across the loop)
    __syncthreads();
    int j = 0;
    do {
      const f32x4 dj = *reinterpret_cast<const f32x4*>(&ld[j * DV + c4 * 4]);
      const float aj0 = CH ? 0.f : la[j];
#pragma unroll
      for (int i = 0; i < G::RPG; ++i) {
        const int row = rg * G::RPG + i;
        const float kj = lk[j * DK + row];
        const float aj = CH ? la[j * DK + row] : aj0;
        st[i] = apply_record(st[i], aj, kj, dj);
      }
    } while (++j <= t);
    float* Sw = a.S_out + tok * DK * DV;
#pragma unroll
    for (int i = 0; i < G::RPG; ++i)
      *reinterpret_cast<f32x4*>(Sw + (size_t)(rg * G::RPG + i) * DV + c4 * 4) = st[i];
  }
}

template <int DK, int DV, bool CH, bool MRG, bool PLAIN = false>
int launch(const gdn_shape& sh, const gdn_store& st, int t, const StepIO& io, hipStream_t stream) {
  SeqArgs a;
  a.S = st.S;
  a.S_out = st.S;
  a.rec_delta = st.rec_delta;
  a.rec_k = st.rec_k;
  a.rec_alpha = st.rec_alpha;
  a.anc = st.anc;
  a.q = io.q;
  a.k = io.k;
  a.v = io.v;
  a.alpha = io.alpha;
  a.beta = io.beta;
  a.o = io.o;
  a.R = sh.R;
  a.H = sh.H;
  a.L = sh.L_max;
  a.t = t;
  a.Hk = key_heads(sh);
  a.gq = sh.H / a.Hk;
  const long grid = (long)sh.R * sh.H;
  if (grid > 0x7FFFFFFFL) return GDN_EINVAL;
  const size_t lds = (size_t)seq_lds_floats(DK, DV, CH ? DK : 1, t) * sizeof(float);
  hipLaunchKernelGGL((k_seq_decode<DK, DV, CH, MRG, PLAIN>), dim3((unsigned)grid), dim3(SeqGeom<DK, DV>::NT),
                     lds, stream, a);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // namespace

int launch_seq_decode(const gdn_shape& sh, const gdn_store& st, int t, bool merge, const StepIO& io,
                      hipStream_t stream) {
  const bool ch = sh.decay_kind == GDN_DECAY_CHANNEL;
  const bool plain = sh.decay_kind == GDN_DECAY_CHANNEL_PLAIN;
#define GDN_CASE(DK_, DV_)                                                                         \
  if (sh.dk == DK_ && sh.dv == DV_) {                                                              \
    if (plain)                                                                                     \
      return merge ? launch<DK_, DV_, true, true, true>(sh, st, t, io, stream)                     \
                   : launch<DK_, DV_, true, false, true>(sh, st, t, io, stream);                   \
    if (merge)                                                                                     \
      return ch ? launch<DK_, DV_, true, true>(sh, st, t, io, stream)                              \
                : launch<DK_, DV_, false, true>(sh, st, t, io, stream);                            \
    return ch ? launch<DK_, DV_, true, false>(sh, st, t, io, stream)                               \
              : launch<DK_, DV_, false, false>(sh, st, t, io, stream);                             \
  }
  GDN_CASE(16, 16)
  GDN_CASE(32, 32)
  GDN_CASE(64, 64)
  GDN_CASE(128, 128)
#undef GDN_CASE
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn
