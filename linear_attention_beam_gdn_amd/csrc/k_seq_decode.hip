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
  static_assert(DV % 4 == 0, "d_v must be a multiple of 4");
  static constexpr int C4 = DV / 4;                      // float4 column groups
  static constexpr int NRG0 = 256 / C4;
  static constexpr int NRG = NRG0 < DK ? NRG0 : DK;      // row groups
  static_assert(DK % NRG == 0, "d_k must split evenly over row groups");
  static constexpr int RPG = DK / NRG;                   // rows per thread
  static constexpr int NT = C4 * NRG;                    // threads
  static constexpr int NWV = (NT + 63) / 64;             // waves
};

// PLAIN: the RWKV6 update pair (k_t, v_t) (channel decay, no delta
// correction): delta_t = v_t, and no projection of k_t is formed.
template <int DK, int DV, bool CH, bool MRG, bool PLAIN>
__global__ __launch_bounds__((SeqGeom<DK, DV>::NT)) void k_seq_decode(SeqArgs a) {
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
  __shared__ float d_new[MRG ? DV : 1];

  // stream this thread's rows of the base first
  const float* S = a.S + tok * DK * DV;
  f32x4 st[G::RPG];
#pragma unroll
  for (int i = 0; i < G::RPG; ++i)
    st[i] = *reinterpret_cast<const f32x4*>(S + (size_t)(rg * G::RPG + i) * DV + c4 * 4);

  // probes x_q = c * q, x_k = c * k with c = prod_{i<=t} a_i (channel decay)
  for (int kk = tid; kk < DK; kk += G::NT) {
    float cq = 1.f;
    if constexpr (CH) {
      cq = a.alpha[tok * DK + kk];
      for (int j = 0; j < t; ++j) cq *= a.rec_alpha[rec_at(j) * A + kk];
    }
    probe_q[kk] = cq * bf16_at(a.q[tk * DK + kk]);
    if constexpr (!PLAIN) probe_k[kk] = cq * bf16_at(a.k[tk * DK + kk]);
  }
  // dot products of the replay: wave wv takes log entries j = wv, wv + NWV, ..
  // (entry t is k_t . q_t); channel decay weights them by prod_{i=j+1..t} a_i
  for (int j = wv; j <= t; j += G::NWV) {
    float pq = 0.f, pk = 0.f;
    for (int kk = lane; kk < DK; kk += 64) {
      const float qv = bf16_at(a.q[tk * DK + kk]);
      if (j == t) {
        pq += bf16_at(a.k[tk * DK + kk]) * qv;
      } else {
        float y = bf16_at(a.rec_k[rec_at_k(j) * DK + kk]);
        if constexpr (CH) {
          y *= a.alpha[tok * DK + kk];
          for (int i = j + 1; i < t; ++i) y *= a.rec_alpha[rec_at(i) * A + kk];
        }
        pq += y * qv;
        if constexpr (!PLAIN) pk += y * bf16_at(a.k[tk * DK + kk]);
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

  const float at = CH ? 1.f : a.alpha[tok];
  const float bt = a.beta[tok];
  const size_t rec_t = rec_at(t);
  for (int col = tid; col < DV; col += G::NT) {
    float uq = 0.f, uk = 0.f;
#pragma unroll 8
    for (int g = 0; g < G::NRG; ++g) {
      uq += red_q[g][col];
      if constexpr (!PLAIN) uk += red_k[g][col];
    }
    for (int j = 0; j < t; ++j) {
      const float dj = a.rec_delta[rec_at(j) * DV + col];
      if constexpr (!CH) {
        const float aj = a.rec_alpha[rec_at(j)];
        uq = aj * uq + dj * dots_q[j];
        uk = aj * uk + dj * dots_k[j];
      } else {
        uq += dj * dots_q[j];
        if constexpr (!PLAIN) uk += dj * dots_k[j];
      }
    }
    const float vv = bf16_at(a.v[tok * DV + col]);
    const float d = PLAIN ? vv : bt * (vv - at * uk);
    a.o[tok * DV + col] = at * uq + d * dot_qk;
    a.rec_delta[rec_t * DV + col] = d;
    if constexpr (MRG) d_new[col] = d;
  }
  for (int kk = tid; kk < DK; kk += G::NT) {
    if (key_writer) a.rec_k[rec_at_k(t) * DK + kk] = a.k[tk * DK + kk];
    if constexpr (CH) a.rec_alpha[rec_t * A + kk] = a.alpha[tok * DK + kk];
  }
  if constexpr (!CH)
    if (tid == 0) a.rec_alpha[rec_t] = at;
  if (h == 0 && tid < t) a.anc[(((size_t)t * a.R + r) * 1 + 0) * a.L + tid] = 0;

  if constexpr (MRG) {
    // fold the full log into this thread's rows of the base: records 0..t-1
    // from the store, record t (this token's) from its inputs and d_new; the
    // same update, in the same order, as the stand-alone merge
    __syncthreads();
    for (int j = 0; j <= t; ++j) {
      const size_t rj = rec_at(j);
      const f32x4 dj = j < t ? *reinterpret_cast<const f32x4*>(a.rec_delta + rj * DV + c4 * 4)
                             : *reinterpret_cast<const f32x4*>(&d_new[c4 * 4]);
      const float aj0 = CH ? 0.f : (j < t ? a.rec_alpha[rj] : at);
#pragma unroll
      for (int i = 0; i < G::RPG; ++i) {
        const int row = rg * G::RPG + i;
        const float kj = bf16_at(j < t ? a.rec_k[rec_at_k(j) * DK + row] : a.k[tk * DK + row]);
        const float aj = CH ? (j < t ? a.rec_alpha[rj * A + row] : a.alpha[tok * DK + row]) : aj0;
        st[i] = apply_record(st[i], aj, kj, dj);
      }
    }
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
  hipLaunchKernelGGL((k_seq_decode<DK, DV, CH, MRG, PLAIN>), dim3((unsigned)grid), dim3(SeqGeom<DK, DV>::NT),
                     0, stream, a);
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
