// Shared-context decode step for scalar-decay GDN beams, with the per-beam
// inputs staged through LDS (OneLA §3.4, Figure 5; replay equations of §3.2;
// ancestry of §3.3).
//
// One workgroup takes one (request r, head h) and a chunk of beams; its NW
// waves split d_v into 32-row slices (the B_V tile of §3.4).  Each wave holds
// its slice of S0[r,h] in registers for the whole chunk, split into NPL bf16
// planes in the A layout of the gfx950 16x16x32 bf16 MFMA, so S0 is read once
// per workgroup and reused by every beam.
//
// Per 16-beam tile:
//  * the tile's q, k and v rows are copied by all waves together straight
//    from HBM into LDS (global_load_lds, no register round trip) into one of
//    two buffers while the previous tile computes; rows are XOR-swizzled in
//    16-byte units so the per-lane fragment reads are bank-conflict free;
//  * each wave reads its B fragments (q, k) and value rows from LDS, runs
//    the MFMA contraction S0^T [q | k], then replays the ancestral records
//    (alpha_j, delta_j, k_j) with bf16 dot2 products reduced over the four
//    lane groups of a beam, keeping two records in flight;
//  * delta_t and o_t are formed in registers and stored after the tile
//    barrier, so the store traffic of one tile overlaps the next tile.
// The chunk's ancestry slots h_t(b, j) are resolved once per workgroup into
// LDS (parent pointer, then the parent's row of step t-1), and the h == 0
// workgroups write the step's ancestry rows.
#include "beam_common.h"

namespace gdn {
namespace {

constexpr int kMaxChunk = 256;

template <int DK, int DV>
struct StagedGeom {
  static_assert(DK % 32 == 0 && DV % 32 == 0, "the staged kernel needs d_k, d_v multiples of 32");
  static constexpr int NW = DV / 32;  // waves: 32 value rows each
  static constexpr int NT = NW * 64;
  static constexpr int MT = 2;        // 16-row MFMA tiles per wave
  static constexpr int KS = DK / 32;  // MFMA steps over d_k
  static constexpr int QCH = DK / 8;  // 16-byte chunks per q/k row
  static constexpr int VCH = DV / 8;  // 16-byte chunks per v row
};

// LDS slot (in 16-byte units) of chunk ch of tile row b.
template <int NCH>
__device__ __forceinline__ int swz(int b, int ch) {
  return b * NCH + (ch ^ (b % NCH));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

// Copy rows [b0, b0 + nvalid) (16 at most) of a [beam][NCH x 16 B] operand
// into a swizzled LDS tile.  Lane i of an instruction lands at slot base + i,
// so each thread loads the global chunk that belongs in its slot.
template <int NCH, int NT>
__device__ __forceinline__ void stage_tile(const uint16_t* rows, size_t row_stride, int nvalid,
                                           uint16_t* lds) {
  const int lane = threadIdx.x & 63;
  for (int idx = threadIdx.x; idx < 16 * NCH; idx += NT) {
    const int b = idx / NCH;
    const int ch = (idx % NCH) ^ (b % NCH);
    if (b < nvalid) {
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(rows + (size_t)b * row_stride + ch * 8),
          (__attribute__((address_space(3))) void*)(lds + (size_t)(idx - lane) * 8), 16, 0, 0);
    }
  }
}

// s_waitcnt with vmcnt = 0 and the other counters left alone (gfx9 encoding)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int KS>
struct RecRegs {
  u32x4 k[KS];
  f32x4 d[2];
  float a;
};

template <int DK, int DV, int NPL>
__global__ __launch_bounds__((StagedGeom<DK, DV>::NT)) void k_beam_staged(BeamArgs a) {
  using G = StagedGeom<DK, DV>;
  constexpr int KS = G::KS;
  __shared__ __attribute__((aligned(16))) uint16_t s_q[2][16 * DK];
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][16 * DK];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[2][16 * DV];
  __shared__ int s_slot[kMaxChunk * GDN_MAX_STEPS];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int c = lane & 15;

  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);  // chunks of one (r,h) share an XCD
  const int chunk_id = bid % a.nchunk;
  const int rh = bid / a.nchunk;
  const int h = rh % a.H;
  const int r = rh / a.H;
  const int b_begin = chunk_id * a.chunk;
  const int b_end = min(b_begin + a.chunk, a.Wt);
  const int nb = b_end - b_begin;
  const int t = a.t;
  const int ntiles = (nb + 15) / 16;
  const size_t row_stride_k = (size_t)a.H * DK;
  const size_t row_stride_v = (size_t)a.H * DV;
  const uint16_t* q_rows = a.q + ((size_t)r * a.Wt * a.H + h) * DK;
  const uint16_t* k_rows = a.k + ((size_t)r * a.Wt * a.H + h) * DK;
  const uint16_t* v_rows = a.v + ((size_t)r * a.Wt * a.H + h) * DV;

  // ---- first tile's inputs start streaming into LDS buffer 0
  stage_tile<G::QCH, G::NT>(q_rows + b_begin * row_stride_k, row_stride_k, min(16, nb), s_q[0]);
  stage_tile<G::QCH, G::NT>(k_rows + b_begin * row_stride_k, row_stride_k, min(16, nb), s_k[0]);
  stage_tile<G::VCH, G::NT>(v_rows + b_begin * row_stride_v, row_stride_v, min(16, nb), s_v[0]);

  // ---- ancestry of the chunk's beams: h_t(b, t-1) = parent, h_t(b, j) =
  // h_{t-1}(parent, j); the h == 0 workgroups also write the step's rows
  if (t > 0) {
    for (int idx = threadIdx.x; idx < nb * t; idx += G::NT) {
      const int i = idx / t;
      const int j = idx - i * t;
      const int b = b_begin + i;
      const int par = clampi(a.parent[(size_t)r * a.Wt + b], 0, a.Wm - 1);
      int slot = par;
      if (j < t - 1) slot = clampi(a.anc[(((size_t)(t - 1) * a.R + r) * a.Wm + par) * a.L + j], 0, a.Wm - 1);
      s_slot[i * GDN_MAX_STEPS + j] = slot;
      if (h == 0) a.anc[(((size_t)t * a.R + r) * a.Wm + b) * a.L + j] = slot;
    }
  }

  // ---- this wave's slice of S0[r,h] as bf16 planes (MFMA A layout); A row m
  // of tile mt is value row w*32 + (m/4)*8 + mt*4 + m%4, so C row 4g+i of tile
  // mt is value row dv0 + mt*4 + i with dv0 = w*32 + g*8
  u32x4 As[G::MT][KS][NPL];
  {
    const float* S = a.S + ((size_t)r * a.H + h) * DK * DV;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) {
      const int col = w * 32 + (c >> 2) * 8 + mt * 4 + (c & 3);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int k0 = kchunk<DK>(g, s);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = S[(size_t)(k0 + e) * DV + col];
        split_planes<NPL>(x, As[mt][s]);
      }
    }
  }
  const int dv0 = w * 32 + g * 8;

  wait_vmem();
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int t0 = b_begin + it * 16;
    if (it + 1 < ntiles) {  // prefetch the next tile into the other buffer
      const int n1 = min(16, b_end - (t0 + 16));
      stage_tile<G::QCH, G::NT>(q_rows + (t0 + 16) * row_stride_k, row_stride_k, n1, s_q[buf ^ 1]);
      stage_tile<G::QCH, G::NT>(k_rows + (t0 + 16) * row_stride_k, row_stride_k, n1, s_k[buf ^ 1]);
      stage_tile<G::VCH, G::NT>(v_rows + (t0 + 16) * row_stride_v, row_stride_v, n1, s_v[buf ^ 1]);
    }
    const int b = t0 + c;
    const bool valid = b < b_end;
    const int bi = valid ? b : b_begin;
    const size_t tok = ((size_t)r * a.Wt + bi) * a.H + h;
    const float at = a.alpha[tok];
    const float bt = a.beta[tok];

    // ancestral records: the slot of a dead lane is 0 (loads stay in bounds)
    auto load_rec = [&](RecRegs<KS>& R, int j) {
      const int slot = valid ? s_slot[(b - b_begin) * GDN_MAX_STEPS + j] : 0;
      const size_t rj = (((size_t)j * a.R + r) * a.Wm + slot) * a.H + h;
#pragma unroll
      for (int s = 0; s < KS; ++s) R.k[s] = *reinterpret_cast<const u32x4*>(a.rec_k + rj * DK + kchunk<DK>(g, s));
      R.d[0] = *reinterpret_cast<const f32x4*>(a.rec_delta + rj * DV + dv0);
      R.d[1] = *reinterpret_cast<const f32x4*>(a.rec_delta + rj * DV + dv0 + 4);
      R.a = a.rec_alpha[rj];
    };
    RecRegs<KS> ra, rb;
    if (t > 0) load_rec(ra, 0);

    // B fragments and value rows from LDS
    u32x4 qf[KS], kf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int ch = kchunk<DK>(g, s) >> 3;
      qf[s] = *reinterpret_cast<const u32x4*>(&s_q[buf][swz<G::QCH>(c, ch) * 8]);
      kf[s] = *reinterpret_cast<const u32x4*>(&s_k[buf][swz<G::QCH>(c, ch) * 8]);
    }
    const u32x4 vw = *reinterpret_cast<const u32x4*>(&s_v[buf][swz<G::VCH>(c, dv0 >> 3) * 8]);

    // S0^T [q | k] on the matrix cores (smallest plane first)
    f32x4 uq[G::MT], uk[G::MT];
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt) {
      uq[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      uk[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int p = NPL - 1; p >= 0; --p) {
          uq[mt] = mfma16x16x32(As[mt][s][p], qf[s], uq[mt]);
          uk[mt] = mfma16x16x32(As[mt][s][p], kf[s], uk[mt]);
        }

    float sqq = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) sqq = dot2(kf[s][e], qf[s][e], sqq);
    sqq = sum_lane_groups(sqq);

    auto apply_rec = [&](const RecRegs<KS>& R) {
      float pq = 0.f, pk = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pq = dot2(R.k[s][e], qf[s][e], pq);
          pk = dot2(R.k[s][e], kf[s][e], pk);
        }
      pq = sum_lane_groups(pq);
      pk = sum_lane_groups(pk);
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uq[mt][i] = R.a * uq[mt][i] + R.d[mt][i] * pq;
          uk[mt][i] = R.a * uk[mt][i] + R.d[mt][i] * pk;
        }
    };
    // replay j = 0..t-1 in order with the next record already in flight
    for (int j = 0; j < t; j += 2) {
      if (j + 1 < t) load_rec(rb, j + 1);
      apply_rec(ra);
      if (j + 1 < t) {
        if (j + 2 < t) load_rec(ra, j + 2);
        apply_rec(rb);
      }
    }

    // current transition
    f32x4 dt[G::MT], ot[G::MT];
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float vv = bf16x8_elem(vw, mt * 4 + i);
        dt[mt][i] = bt * (vv - at * uk[mt][i]);
        ot[mt][i] = at * uq[mt][i] + dt[mt][i] * sqq;
      }

    // next tile staged and every wave done with this buffer
    wait_vmem();
    __syncthreads();

    if (valid) {
      const size_t rec_t = (((size_t)t * a.R + r) * a.Wm + b) * a.H + h;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) {
        *reinterpret_cast<f32x4*>(a.o + tok * DV + dv0 + mt * 4) = ot[mt];
        *reinterpret_cast<f32x4*>(a.rec_delta + rec_t * DV + dv0 + mt * 4) = dt[mt];
      }
      if (w == 0) {
#pragma unroll
        for (int s = 0; s < KS; ++s) *reinterpret_cast<u32x4*>(a.rec_k + rec_t * DK + kchunk<DK>(g, s)) = kf[s];
        if (g == 0) a.rec_alpha[rec_t] = at;
      }
    }
  }
}

template <int DK, int DV>
int launch(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io, hipStream_t stream) {
  constexpr int NPL = 3;
  BeamArgs a;
  a.S = st.S;
  a.rec_delta = st.rec_delta;
  a.rec_k = st.rec_k;
  a.rec_alpha = st.rec_alpha;
  a.anc = st.anc;
  a.parent = io.parent;
  a.q = io.q;
  a.k = io.k;
  a.v = io.v;
  a.alpha = io.alpha;
  a.beta = io.beta;
  a.o = io.o;
  a.R = sh.R;
  a.Wm = sh.W_max;
  a.H = sh.H;
  a.L = sh.L_max;
  a.t = t;
  a.Wt = Wt;
  a.chunk = pick_chunk(sh.R * sh.H, Wt, kMaxChunk, 1024);
  a.nchunk = (Wt + a.chunk - 1) / a.chunk;
  const long grid = (long)sh.R * sh.H * a.nchunk;
  if (grid > 0x7FFFFFFFL) return GDN_EINVAL;
  hipLaunchKernelGGL((k_beam_staged<DK, DV, NPL>), dim3((unsigned)grid), dim3(StagedGeom<DK, DV>::NT), 0,
                     stream, a);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // namespace

bool beam_staged_supported(const gdn_shape& sh) {
  return sh.decay_kind == GDN_DECAY_SCALAR &&
         ((sh.dk == 32 && sh.dv == 32) || (sh.dk == 64 && sh.dv == 64) || (sh.dk == 128 && sh.dv == 128));
}

int launch_beam_staged(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io,
                       hipStream_t stream) {
  if (sh.dk == 32 && sh.dv == 32) return launch<32, 32>(sh, st, t, Wt, io, stream);
  if (sh.dk == 64 && sh.dv == 64) return launch<64, 64>(sh, st, t, Wt, io, stream);
  if (sh.dk == 128 && sh.dv == 128) return launch<128, 128>(sh, st, t, Wt, io, stream);
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn
