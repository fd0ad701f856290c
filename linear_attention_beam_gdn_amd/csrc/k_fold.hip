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
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

struct FoldArgs {
  const float* src;
  float* dst;
  const float* rec_delta;
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
};

template <int DK, int DV, bool CH>
__global__ __launch_bounds__((FoldGeom<DK, DV>::NT)) void k_fold(FoldArgs a) {
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

  const float* src = a.src + ((size_t)r * a.H + h) * DK * DV;
  float* dst = a.dst_per_item ? a.dst + ((size_t)item * a.H + h) * DK * DV
                              : a.dst + ((size_t)r * a.H + h) * DK * DV;
  f32x4 st[G::RPG];
#pragma unroll
  for (int i = 0; i < G::RPG; ++i)
    st[i] = *reinterpret_cast<const f32x4*>(src + (size_t)(row0 + i) * DV + c4 * 4);

  const int32_t* arow = a.anc + (((size_t)t * a.R + r) * a.Wm + b) * a.L;
  // (a do-while: t >= 0, and this loop shape keeps the state in one set of
  // registers across the loop instead of a copy per entry)
  int j = 0;
  do {
    const int slot = j < t ? clampi(arow[j], 0, a.Wm - 1) : b;
    const size_t rj = (((size_t)j * a.R + r) * a.Wm + slot) * a.H + h;
    const size_t rjk = (((size_t)j * a.R + r) * a.Wm + slot) * a.Hk + h / a.gq;
    const f32x4 dj = *reinterpret_cast<const f32x4*>(a.rec_delta + rj * DV + c4 * 4);
    const float aj0 = CH ? 0.f : a.rec_alpha[rj];
#pragma unroll
    for (int i = 0; i < G::RPG; ++i) {
      const int row = row0 + i;
      const float kj = bf16_at(a.rec_k[rjk * DK + row]);
      const float aj = CH ? a.rec_alpha[rj * A + row] : aj0;
      st[i] = apply_record(st[i], aj, kj, dj);
    }
  } while (++j <= t);
#pragma unroll
  for (int i = 0; i < G::RPG; ++i)
    *reinterpret_cast<f32x4*>(dst + (size_t)(row0 + i) * DV + c4 * 4) = st[i];
}

template <int DK, int DV, bool CH>
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
  hipLaunchKernelGGL((k_fold<DK, DV, CH>), dim3((unsigned)grid), dim3(FoldGeom<DK, DV>::NT), 0,
                     stream, a);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // namespace

int launch_fold(const gdn_shape& sh, const gdn_store& st, int t, const int32_t* rb, int beam, int n,
                const float* src, float* dst, bool dst_per_item, hipStream_t stream) {
  const bool ch = sh.decay_kind != GDN_DECAY_SCALAR;  // the fold is the same for both channel rules
#define GDN_CASE(DK_, DV_)                                                           \
  if (sh.dk == DK_ && sh.dv == DV_)                                                  \
    return ch ? launch<DK_, DV_, true>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream) \
              : launch<DK_, DV_, false>(sh, st, t, rb, beam, n, src, dst, dst_per_item, stream);
  GDN_CASE(16, 16)
  GDN_CASE(32, 32)
  GDN_CASE(64, 64)
  GDN_CASE(128, 128)
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
