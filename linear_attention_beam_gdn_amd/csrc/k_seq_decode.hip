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
//
// With the plain rule (the RWKV6 row of DeltaLog Table 1) the update vector
// is v_t itself, and the log keeps it as bf16 (Table 3: BF16/BF16 log): the
// kernel reads the log's update vectors as bf16 rows and appends v_t's bits.
//
// Value tiles (the split-replay ablation of DeltaLog Figure 9; the three
// stages of the Figure 5 caption).  With NS > 1 the d_v columns of a
// (sequence, head) are cut into NS tiles of VT = d_v / NS columns, one
// workgroup each, which read only their columns of the base, of v and of the
// log's update vectors, and write only their columns of o, delta_t and (merge
// path) the base.  Every column's replay needs the same preparation: the
// probes x_q = c * q_t, x_k = c * k_t (c = prod_{i<=t} a_i with channel
// decay, 1 otherwise) and the dot products k_j . x of the log's records.
// PREP = 0: every tile forms that preparation itself from q, k and the log's
// keys and decays (the preparation is repeated NS times), and tile 0 commits
// the record's key, decay and ancestry row.  PREP = 1: k_seq_prep has formed
// it once per (sequence, head) into a workspace and committed the record's
// key, decay and ancestry row (the single writer); the tiles read it there.
// Both arms run the same arithmetic in the same order, so they give the same
// bits.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

struct SeqArgs {
  const float* S;
  float* S_out;  // the base written back by the merge path
  float* rec_delta;  // FP32 update vectors (bf16 bit patterns for the plain rule)
  uint16_t* rec_k;
  float* rec_alpha;
  int32_t* anc;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  float* o;
  float* prep;  // split path: per (sequence, head) replay preparation, prep_floats(d_k) floats
  int R, H, L, t;
  int Hk, gq;  // key heads; value head h uses key head h / gq
};

// The replay preparation of one (sequence, head) as the workspace holds it:
// probe_q [d_k], probe_k [d_k], dots_q [GDN_MAX_STEPS], dots_k
// [GDN_MAX_STEPS], k_t . q_t, then padding to a 16-byte multiple.
__host__ __device__ constexpr int prep_floats(int dk) { return 2 * dk + 2 * GDN_MAX_STEPS + 4; }

template <int DK, int VT>
struct SeqGeom {
  static_assert(VT % 8 == 0 && DK % 8 == 0, "d_k and the tile's d_v columns must be multiples of 8");
  static constexpr int C4 = VT / 4;                      // float4 column groups
  static constexpr int NRG0 = 256 / C4;
  static constexpr int NRG = NRG0 < DK ? NRG0 : DK;      // row groups
  static_assert(DK % NRG == 0, "d_k must split evenly over row groups");
  static constexpr int RPG = DK / NRG;                   // rows per thread
  static constexpr int NT = C4 * NRG;                    // threads
  static constexpr int NWV = (NT + 63) / 64;             // waves
  // 16-byte pieces of the rows staged in LDS: a bf16 row of d_k (keys, q),
  // the tile's bf16 columns of v, the tile's columns of an update vector
  // (FP32, or bf16 with the plain rule), an FP32 row of d_k (per-channel
  // decays); and the pieces each thread loads at most
  static constexpr int KCH = DK / 8, VCH = VT / 8, DCH = VT / 4, ACH = DK / 4;
  static constexpr int NKL = ((GDN_MAX_STEPS + 1) * KCH + NT - 1) / NT;
  static constexpr int NVL = (VCH + NT - 1) / NT;
  static constexpr int NDL = ((GDN_MAX_STEPS - 1) * DCH + NT - 1) / NT;
  static constexpr int NDL16 = ((GDN_MAX_STEPS - 1) * VCH + NT - 1) / NT;  // bf16 update vectors
  static constexpr int NAL = (GDN_MAX_STEPS * ACH + NT - 1) / NT;
};

// Dynamic LDS of a step with log length t (floats): the keys of log entries
// 0..t-1, k_t and q_t as rows 0..t+1 of [d_k]; the tile's columns of v_t;
// the tile's columns of the update vectors of entries 0..t (row t: this
// token's); the decays of entries 0..t (one each, or a [d_k] row each),
// padded to a multiple of four.
__host__ __device__ constexpr int seq_lds_floats(int dk, int vt, int a, int t) {
  return (t + 2) * dk + vt + (t + 1) * vt + (((t + 1) * a + 3) & ~3);
}

__device__ __forceinline__ void put_bf16x8(float* dst, const u32x4& w) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])};
}

// Load (16-byte pieces, into registers) and stage in LDS the rows the
// preparation and the fold read: the log's keys, k_t and q_t as rows 0..t+1
// of lk, and the decays of entries 0..t (scalars, or [d_k] rows) in la.
// `stage` runs between the loads and the LDS writes (the caller issues its
// own loads there, so that they are in flight together).
template <int DK, int NT, bool CH, class Stage>
__device__ __forceinline__ void load_rows(const SeqArgs& a, int r, int h, int tid, float* lk, float* la,
                                          Stage stage) {
  constexpr int A = CH ? DK : 1;
  constexpr int KCH = DK / 8, ACH = DK / 4;
  constexpr int NKL = ((GDN_MAX_STEPS + 1) * KCH + NT - 1) / NT;
  constexpr int NAL = (GDN_MAX_STEPS * ACH + NT - 1) / NT;
  const int t = a.t;
  const size_t tok = (size_t)r * a.H + h;
  const size_t tk = (size_t)r * a.Hk + h / a.gq;
  const int nk = (t + 2) * KCH;
  u32x4 kb[NKL];
  f32x4 ab[CH ? NAL : 1];
  float as = 0.f;
#pragma unroll
  for (int m = 0; m < NKL; ++m) {
    const int c = min(tid + m * NT, nk - 1);
    const int j = c / KCH, part = c % KCH;
    const uint16_t* src = j < t ? a.rec_k + (((size_t)j * a.R + r) * a.Hk + h / a.gq) * DK : (j == t ? a.k : a.q) + tk * DK;
    kb[m] = *reinterpret_cast<const u32x4*>(src + part * 8);
  }
  if constexpr (CH) {
#pragma unroll
    for (int m = 0; m < NAL; ++m) {
      const int c = min(tid + m * NT, (t + 1) * ACH - 1);
      const int j = c / ACH, part = c % ACH;
      const float* src = j < t ? a.rec_alpha + (((size_t)j * a.R + r) * a.H + h) * A : a.alpha + tok * DK;
      ab[m] = *reinterpret_cast<const f32x4*>(src + part * 4);
    }
  } else {
    if (tid <= t) as = tid < t ? a.rec_alpha[((size_t)tid * a.R + r) * a.H + h] : a.alpha[tok];
  }
  stage();
#pragma unroll
  for (int m = 0; m < NKL; ++m)
    if (tid + m * NT < nk) put_bf16x8(lk + (tid + m * NT) * 8, kb[m]);
  if constexpr (CH) {
#pragma unroll
    for (int m = 0; m < NAL; ++m)
      if (tid + m * NT < (t + 1) * ACH) *reinterpret_cast<f32x4*>(la + (tid + m * NT) * 4) = ab[m];
  } else {
    if (tid <= t) la[tid] = as;
  }
}

// The replay preparation from the staged rows (after a barrier): probes
// x_q = c * q, x_k = c * k with c = prod_{i<=t} a_i (channel decay), and the
// dot products of the replay, wave wv taking log entries j = wv, wv + NWV,
// .. (entry t is k_t . q_t; channel decay weights entry j by
// prod_{i=j+1..t} a_i).  Each dot product is formed by one wave, lanes
// striding d_k by 64, whatever the wave count, so every kernel that prepares
// gets the same bits.
template <int DK, int NT, bool CH, bool PLAIN>
__device__ __forceinline__ void prepare(int t, int tid, const float* lk, const float* la, float* probe_q,
                                        float* probe_k, float* dots_q, float* dots_k, float* dot_qk) {
  constexpr int NWV = (NT + 63) / 64;
  const int lane = tid & 63, wv = tid >> 6;
  const float* sq = lk + (t + 1) * DK;
  const float* sk = lk + t * DK;
  for (int kk = tid; kk < DK; kk += NT) {
    float cq = 1.f;
    if constexpr (CH) {
      cq = la[t * DK + kk];
      for (int j = 0; j < t; ++j) cq *= la[j * DK + kk];
    }
    probe_q[kk] = cq * sq[kk];
    if constexpr (!PLAIN) probe_k[kk] = cq * sk[kk];
  }
  for (int j = wv; j <= t; j += NWV) {
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
      if (j == t) *dot_qk = pq;
      else {
        dots_q[j] = pq;
        dots_k[j] = pk;
      }
    }
  }
}

// The record's key and decay (bit copies of the token's inputs: a bf16 value
// widened to FP32 and cut back is the same value) and the ancestry row of
// sequence r at step t; one writer per (sequence, head).
template <int DK, int NT, bool CH>
__device__ __forceinline__ void commit_record(const SeqArgs& a, int r, int h, int tid, const float* lk,
                                              const float* la) {
  const int t = a.t;
  const size_t rec_t = ((size_t)t * a.R + r) * a.H + h;
  const float* sk = lk + t * DK;
  const bool key_writer = h % a.gq == 0;
  for (int kk = tid; kk < DK; kk += NT) {
    if (key_writer) a.rec_k[(((size_t)t * a.R + r) * a.Hk + h / a.gq) * DK + kk] = (uint16_t)(__float_as_uint(sk[kk]) >> 16);
    if constexpr (CH) a.rec_alpha[rec_t * DK + kk] = la[t * DK + kk];
  }
  if constexpr (!CH)
    if (tid == 0) a.rec_alpha[rec_t] = la[t];
  if (h == 0 && tid < t) a.anc[(((size_t)t * a.R + r) * 1 + 0) * a.L + tid] = 0;
}

// PLAIN: the RWKV6 update pair (k_t, v_t) (channel decay, no delta
// correction): delta_t = v_t, and no projection of k_t is formed.
// The merge path holds the base rows in registers to the end; it is built
// for four waves per SIMD (at most 128 registers), so that four workgroups
// per compute unit overlap their read, fold and write phases.
template <int DK, int DV, int NS, bool CH, bool MRG, bool PLAIN, int PREP>
__global__ __launch_bounds__((SeqGeom<DK, DV / NS>::NT), (MRG ? 4 : 1)) void k_seq_decode(SeqArgs a) {
  static_assert(CH || !PLAIN, "the plain update rule comes with channel decay");
  constexpr int VT = DV / NS;  // the tile's value columns
  static_assert(VT * NS == DV, "d_v must split evenly over the tiles");
  using G = SeqGeom<DK, VT>;
  constexpr bool ROWS = PREP == 0 || MRG;  // keys (and decays) staged: preparation or fold
  const int tid = threadIdx.x;
  const int tile = blockIdx.x % NS;
  const int h = (blockIdx.x / NS) % a.H;
  const int r = blockIdx.x / (NS * a.H);
  const int col0 = tile * VT;
  const int c4 = tid % G::C4;
  const int rg = tid / G::C4;
  const int t = a.t;
  const size_t tok = (size_t)r * a.H + h;                 // (r, beam 0, h)
  auto rec_at = [&](int j) -> size_t { return ((size_t)j * a.R + r) * a.H + h; };

  __shared__ float probe_q[DK], probe_k[DK];
  __shared__ float red_q[G::NRG][VT], red_k[G::NRG][VT];
  __shared__ float dots_q[GDN_MAX_STEPS], dots_k[GDN_MAX_STEPS], dot_qk;
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  float* lk = dyn;                     // [t + 2][DK]: keys 0..t-1, k_t, q_t
  float* sv = lk + (t + 2) * DK;       // [VT]
  float* ld = sv + VT;                 // [t + 1][VT]
  float* la = ld + (t + 1) * VT;       // [t + 1][A]

  // One batch of loads: the token's q, k, the log's keys and decays (when
  // this workgroup prepares or folds), the tile's columns of v and of the
  // log's update vectors (16-byte pieces into registers), then this thread's
  // rows of the base; the pieces go to LDS while the base is still in
  // flight, so no later phase waits on memory but the one that needs the base.
  const float bt = PLAIN ? 0.f : a.beta[tok];  // the plain rule has no beta
  const int nd = PLAIN ? t * G::VCH : t * G::DCH;
  constexpr int NDLX = PLAIN ? G::NDL16 : G::NDL;
  u32x4 vb[G::NVL];
  f32x4 db[PLAIN ? 1 : G::NDL];
  u32x4 db16[PLAIN ? G::NDL16 : 1];
  const uint16_t* rec_u16 = reinterpret_cast<const uint16_t*>(a.rec_delta);
  f32x4 st[G::RPG];
  const float* S = a.S + tok * DK * DV + col0;
  auto own_loads = [&] {
#pragma unroll
    for (int m = 0; m < G::NVL; ++m) {
      const int c = min(tid + m * G::NT, G::VCH - 1);
      vb[m] = *reinterpret_cast<const u32x4*>(a.v + tok * DV + col0 + c * 8);
    }
#pragma unroll
    for (int m = 0; m < NDLX; ++m) {
      const int c = tid + m * G::NT;
      if constexpr (PLAIN) {
        if (c < nd)
          db16[m] = *reinterpret_cast<const u32x4*>(rec_u16 + rec_at(c / G::VCH) * DV + col0 + (c % G::VCH) * 8);
      } else {
        if (c < nd)
          db[m] = *reinterpret_cast<const f32x4*>(a.rec_delta + rec_at(c / G::DCH) * DV + col0 + (c % G::DCH) * 4);
      }
    }
#pragma unroll
    for (int i = 0; i < G::RPG; ++i)
      st[i] = *reinterpret_cast<const f32x4*>(S + (size_t)(rg * G::RPG + i) * DV + c4 * 4);
  };
  if constexpr (ROWS) {
    load_rows<DK, G::NT, CH>(a, r, h, tid, lk, la, own_loads);
  } else {
    own_loads();
    if constexpr (!CH) {  // the scalar decays of the replay
      if (tid <= t) la[tid] = tid < t ? a.rec_alpha[rec_at(tid)] : a.alpha[tok];
    }
  }
  if constexpr (PREP == 1) {  // the shared preparation of this (sequence, head)
    const float* pw = a.prep + tok * prep_floats(DK);
    for (int kk = tid; kk < DK; kk += G::NT) {
      probe_q[kk] = pw[kk];
      if constexpr (!PLAIN) probe_k[kk] = pw[DK + kk];
    }
    if (tid < t) {
      dots_q[tid] = pw[2 * DK + tid];
      if constexpr (!PLAIN) dots_k[tid] = pw[2 * DK + GDN_MAX_STEPS + tid];
    }
    if (tid == 0) dot_qk = pw[2 * DK + 2 * GDN_MAX_STEPS];
  }
#pragma unroll
  for (int m = 0; m < G::NVL; ++m)
    if (tid + m * G::NT < G::VCH) put_bf16x8(sv + (tid + m * G::NT) * 8, vb[m]);
#pragma unroll
  for (int m = 0; m < NDLX; ++m) {
    if constexpr (PLAIN) {
      if (tid + m * G::NT < nd) put_bf16x8(ld + (tid + m * G::NT) * 8, db16[m]);
    } else {
      if (tid + m * G::NT < nd) *reinterpret_cast<f32x4*>(ld + (tid + m * G::NT) * 4) = db[m];
    }
  }
  __syncthreads();

  if constexpr (PREP == 0) {
    prepare<DK, G::NT, CH, PLAIN>(t, tid, lk, la, probe_q, probe_k, dots_q, dots_k, &dot_qk);
    __syncthreads();
  }

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
  for (int col = tid; col < VT; col += G::NT) {
    float uq = 0.f, uk = 0.f;
#pragma unroll 8
    for (int g = 0; g < G::NRG; ++g) {
      uq += red_q[g][col];
      if constexpr (!PLAIN) uk += red_k[g][col];
    }
    for (int j = 0; j < t; ++j) {
      const float dj = ld[j * VT + col];
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
    a.o[tok * DV + col0 + col] = at * uq + d * dot_qk;
    if constexpr (PLAIN)  // v_t's own bits (a bf16 widened to FP32 and cut back)
      reinterpret_cast<uint16_t*>(a.rec_delta)[rec_t * DV + col0 + col] = (uint16_t)(__float_as_uint(vv) >> 16);
    else
      a.rec_delta[rec_t * DV + col0 + col] = d;
    if constexpr (MRG) ld[t * VT + col] = d;
  }
  if constexpr (PREP == 0)
    if (tile == 0) commit_record<DK, G::NT, CH>(a, r, h, tid, lk, la);

  if constexpr (MRG) {
    // fold the full log into this thread's rows of the base, records 0..t in
    // log order (the same update, in the same order, as the stand-alone
    // merge), from the staged log and this token's update vector (a do-while,
    // which keeps the base in one set of registers across the loop)
    __syncthreads();
    int j = 0;
    do {
      const f32x4 dj = *reinterpret_cast<const f32x4*>(&ld[j * VT + c4 * 4]);
      const float aj0 = CH ? 0.f : la[j];
#pragma unroll
      for (int i = 0; i < G::RPG; ++i) {
        const int row = rg * G::RPG + i;
        const float kj = lk[j * DK + row];
        const float aj = CH ? la[j * DK + row] : aj0;
        st[i] = apply_record(st[i], aj, kj, dj);
      }
    } while (++j <= t);
    float* Sw = a.S_out + tok * DK * DV + col0;
#pragma unroll
    for (int i = 0; i < G::RPG; ++i)
      *reinterpret_cast<f32x4*>(Sw + (size_t)(rg * G::RPG + i) * DV + c4 * 4) = st[i];
  }
}

// The shared preparation (first stage of the split path): one workgroup per
// (sequence, head) forms the probes and dot products once, writes them to
// the workspace, and commits the record's key, decay and ancestry row.
template <int DK, bool CH, bool PLAIN>
__global__ __launch_bounds__(256) void k_seq_prep(SeqArgs a) {
  constexpr int NT = 256;
  constexpr int A = CH ? DK : 1;
  const int tid = threadIdx.x;
  const int h = blockIdx.x % a.H;
  const int r = blockIdx.x / a.H;
  const int t = a.t;
  __shared__ float probe_q[DK], probe_k[DK];
  __shared__ float dots_q[GDN_MAX_STEPS], dots_k[GDN_MAX_STEPS], dot_qk;
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  float* lk = dyn;                     // [t + 2][DK]
  float* la = lk + (t + 2) * DK;       // [t + 1][A]
  load_rows<DK, NT, CH>(a, r, h, tid, lk, la, [] {});
  __syncthreads();
  prepare<DK, NT, CH, PLAIN>(t, tid, lk, la, probe_q, probe_k, dots_q, dots_k, &dot_qk);
  __syncthreads();
  float* pw = a.prep + ((size_t)r * a.H + h) * prep_floats(DK);
  for (int kk = tid; kk < DK; kk += NT) {
    pw[kk] = probe_q[kk];
    pw[DK + kk] = PLAIN ? 0.f : probe_k[kk];
  }
  if (tid < GDN_MAX_STEPS) {
    pw[2 * DK + tid] = tid < t ? dots_q[tid] : 0.f;
    pw[2 * DK + GDN_MAX_STEPS + tid] = (tid < t && !PLAIN) ? dots_k[tid] : 0.f;
  }
  if (tid < 4) pw[2 * DK + 2 * GDN_MAX_STEPS + tid] = tid == 0 ? dot_qk : 0.f;
  commit_record<DK, NT, CH>(a, r, h, tid, lk, la);
  (void)A;
}

SeqArgs make_args(const gdn_shape& sh, const gdn_store& st, int t, const StepIO& io, float* prep) {
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
  a.prep = prep;
  a.R = sh.R;
  a.H = sh.H;
  a.L = sh.L_max;
  a.t = t;
  a.Hk = key_heads(sh);
  a.gq = sh.H / a.Hk;
  return a;
}

template <int DK, int DV, int NS, bool CH, bool MRG, bool PLAIN, int PREP>
int launch(const gdn_shape& sh, const gdn_store& st, int t, const StepIO& io, float* prep, hipStream_t stream) {
  const SeqArgs a = make_args(sh, st, t, io, prep);
  const long grid = (long)sh.R * sh.H * NS;
  if (grid > 0x7FFFFFFFL) return GDN_EINVAL;
  if constexpr (PREP == 1) {
    const size_t lds = (size_t)((t + 2) * DK + (((t + 1) * (CH ? DK : 1) + 3) & ~3)) * sizeof(float);
    GDN_DISPATCH(io.ev_start, (hipEvent_t) nullptr, (k_seq_prep<DK, CH, PLAIN>), dim3((unsigned)(sh.R * sh.H)),
                 dim3(256), lds, stream, a);
    if (hipGetLastError() != hipSuccess) return GDN_EHIP;
  }
  const size_t lds = (size_t)seq_lds_floats(DK, DV / NS, CH ? DK : 1, t) * sizeof(float);
  GDN_DISPATCH(PREP == 1 ? (hipEvent_t) nullptr : io.ev_start, io.ev_stop, (k_seq_decode<DK, DV, NS, CH, MRG, PLAIN, PREP>),
               dim3((unsigned)grid), dim3(SeqGeom<DK, DV / NS>::NT), lds, stream, a);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

template <int DK, int DV, int NS, int PREP>
int launch_kind(const gdn_shape& sh, const gdn_store& st, int t, bool merge, const StepIO& io, float* prep,
                hipStream_t stream) {
  const bool ch = sh.decay_kind == GDN_DECAY_CHANNEL;
  if (sh.decay_kind == GDN_DECAY_CHANNEL_PLAIN)
    return merge ? launch<DK, DV, NS, true, true, true, PREP>(sh, st, t, io, prep, stream)
                 : launch<DK, DV, NS, true, false, true, PREP>(sh, st, t, io, prep, stream);
  if (merge)
    return ch ? launch<DK, DV, NS, true, true, false, PREP>(sh, st, t, io, prep, stream)
              : launch<DK, DV, NS, false, true, false, PREP>(sh, st, t, io, prep, stream);
  return ch ? launch<DK, DV, NS, true, false, false, PREP>(sh, st, t, io, prep, stream)
            : launch<DK, DV, NS, false, false, false, PREP>(sh, st, t, io, prep, stream);
}

}  // namespace

size_t seq_split_workspace_bytes(const gdn_shape& sh) {
  return (size_t)sh.R * sh.H * prep_floats(sh.dk) * sizeof(float);
}

bool seq_split_supported(const gdn_shape& sh, int n_split) {
  return sh.dk == 128 && sh.dv == 128 && (n_split == 1 || n_split == 2 || n_split == 4);
}

int launch_seq_decode(const gdn_shape& sh, const gdn_store& st, int t, bool merge, const StepIO& io,
                      hipStream_t stream) {
#define GDN_CASE(DK_, DV_) \
  if (sh.dk == DK_ && sh.dv == DV_) return launch_kind<DK_, DV_, 1, 0>(sh, st, t, merge, io, nullptr, stream);
  GDN_CASE(16, 16)
  GDN_CASE(32, 32)
  GDN_CASE(64, 64)
  GDN_CASE(128, 128)
#undef GDN_CASE
  return GDN_EUNSUPPORTED;
}

int launch_seq_split(const gdn_shape& sh, const gdn_store& st, int t, bool merge, int n_split, bool shared_prep,
                     float* prep, const StepIO& io, hipStream_t stream) {
  if (!seq_split_supported(sh, n_split)) return GDN_EUNSUPPORTED;
  if (shared_prep) {
    switch (n_split) {
      case 1: return launch_kind<128, 128, 1, 1>(sh, st, t, merge, io, prep, stream);
      case 2: return launch_kind<128, 128, 2, 1>(sh, st, t, merge, io, prep, stream);
      case 4: return launch_kind<128, 128, 4, 1>(sh, st, t, merge, io, prep, stream);
      default: break;
    }
  } else {
    switch (n_split) {
      case 1: return launch_kind<128, 128, 1, 0>(sh, st, t, merge, io, nullptr, stream);
      case 2: return launch_kind<128, 128, 2, 0>(sh, st, t, merge, io, nullptr, stream);
      case 4: return launch_kind<128, 128, 4, 0>(sh, st, t, merge, io, nullptr, stream);
      default: break;
    }
  }
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn
