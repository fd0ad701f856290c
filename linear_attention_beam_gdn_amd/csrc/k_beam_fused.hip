// Fused shared-context decode step for scalar-decay GDN beams (OneLA §3.4,
// Figure 5; replay equations of §3.2; ancestry index of §3.3), built as a
// producer/consumer pipeline for gfx950.
//
// Work split.  A workgroup takes one (request r, head h) and a chunk of its
// beams, 16 beams (one MFMA N block) per tile.  It has NW consumer waves,
// each owning 32 value rows (the B_V tile of §3.4), and one loader wave.
//
// Loader wave.  Streams every per-tile operand from HBM straight into a ring
// of NBUF LDS buffers with LDS-DMA loads (global_load_lds, no register round
// trip): the tile's q, k and v rows, its alpha and beta, and for each beam
// the T ancestral records (alpha_j, delta_j, k_j) found through the ancestry
// index.  It keeps up to NBUF - 1 tiles in flight and, before each barrier,
// waits only for the tile the consumers take next.
//
// Consumer waves.  Hold their slice of the shared state S0[r, h] in registers
// for the whole chunk as three bf16 planes (hi + mid + lo, each the RNE of
// the FP32 residual) in the MFMA A layout, so S0 is read once per workgroup
// and reused by every beam.  Per tile: S0^T [q | k] on the matrix cores (q
// and k are bf16, so every plane product is exact; FP32 accumulation), the
// replay of the T records (bf16 dot2 products reduced over the four lane
// groups of a beam), then delta_t and o_t, stored with 64-byte contiguous
// writes per beam, plus the appended record.  They issue no vector loads in
// the tile loop, so they never stall on memory, and they never wait for
// their own stores.
//
// LDS tile layout ("beam fastest"): a 16-row array with NCH 16-byte chunks
// per row keeps chunk ch of row b at 16-byte slot (ch/4)*64 + (ch%4)*16 + b.
// DMA instruction m then fills slots m*64 .. m*64+63 with lane l loading
// chunk 4m + l/16 of row l%16 (so every loader lane serves one beam), and a
// consumer read of chunk 4s + g for beam c by lane 16g + c is one contiguous
// 1 KiB access, free of bank conflicts.
#include "beam_common.h"

namespace gdn {
namespace {

constexpr int kMaxChunkF = 512;         // beams per workgroup at most
constexpr int kLdsBytes = 160 * 1024;   // LDS of one gfx950 compute unit

template <int DK, int DV, int T>
struct FusedGeom {
  static_assert(DK % 32 == 0 && DV % 32 == 0, "the fused kernel needs d_k, d_v multiples of 32");
  static constexpr int NW = DV / 32;       // consumer waves
  static constexpr int NT = (NW + 1) * 64; // plus the loader wave
  static constexpr int KS = DK / 32;       // 32-deep MFMA steps over d_k
  static constexpr int QB = 16 * DK * 2;   // bytes of a q (or k) tile
  static constexpr int VB = 16 * DV * 2;   // bytes of a v tile
  static constexpr int NSM = (2 + T) * 16 > 64 ? 2 : 1;  // dword DMAs for alpha, beta, alpha_j
  static constexpr int SMB = NSM * 256;
  static constexpr int RKB = 16 * DK * 2;  // keys of one record depth
  static constexpr int RDB = 16 * DV * 4;  // update vectors of one record depth
  static constexpr int RECB = RKB + RDB;
  static constexpr int OQ = 0, OKK = QB, OV = 2 * QB, OS = 2 * QB + VB, OR = OS + SMB;
  static constexpr int BUF = OR + T * RECB;
  static constexpr int SLOTB = T * kMaxChunkF * 4;
  static constexpr int NBUF0 = (kLdsBytes - SLOTB) / BUF;
  static constexpr int NBUF = NBUF0 > 6 ? 6 : NBUF0;
  static_assert(NBUF >= 2, "tile buffers do not fit in LDS");
  static constexpr int LDS = NBUF * BUF + SLOTB;
  // LDS-DMA instructions the loader issues per tile
  static constexpr int OPT = 2 * (QB / 1024) + VB / 1024 + NSM + T * (RECB / 1024);
  static_assert(QB % 1024 == 0 && VB % 1024 == 0 && RDB % 1024 == 0, "tile arrays must be whole DMA blocks");
  static_assert((2 + T) * 16 <= 128, "too many record depths for the small-value block");
};

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

// 64 lanes x 16 (or 4) bytes from per-lane global addresses into the LDS
// block at `blk` (wave-uniform), lane l at blk + l * size.
__device__ __forceinline__ void dma16(const void* src, uint8_t* blk) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)blk, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* blk) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)blk, 4, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N < 63 ? N : 63) : "memory");
}

// Wait until at most k tiles of OPT loads each (k <= KMAX) are in flight.
template <int OPT, int KMAX>
__device__ __forceinline__ void wait_tiles(int k) {
  if constexpr (KMAX >= 4)
    if (k >= 4) return wait_vm<4 * OPT>();
  if constexpr (KMAX >= 3)
    if (k == 3) return wait_vm<3 * OPT>();
  if constexpr (KMAX >= 2)
    if (k == 2) return wait_vm<2 * OPT>();
  if constexpr (KMAX >= 1)
    if (k == 1) return wait_vm<OPT>();
  wait_vm<0>();
}

// Workgroup barrier after this wave's LDS accesses have completed; also a
// compiler barrier for memory accesses.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS read issued as opaque assembly: the compiler does not order it behind
// this wave's outstanding LDS-DMA loads (which target other LDS bytes).
__device__ __forceinline__ int lds_read_opaque(const void* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int DK, int DV, int T>
__global__ __launch_bounds__((FusedGeom<DK, DV, T>::NT)) void k_beam_fused(BeamArgs a) {
  using G = FusedGeom<DK, DV, T>;
  constexpr int KS = G::KS;
  constexpr int NPL = 3;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS];
  int* s_slot = reinterpret_cast<int*>(smem + G::NBUF * G::BUF);  // [T][kMaxChunkF]

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // Workgroups are handed to the 8 XCDs round-robin; renumber them so that
  // the chunks of one (r, h) run on one XCD and share its L2.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int chunk_id = bid % a.nchunk;
  const int rh = bid / a.nchunk;
  const int h = rh % a.H;
  const int r = rh / a.H;
  const int b_begin = chunk_id * a.chunk;
  const int b_end = min(b_begin + a.chunk, a.Wt);
  const int nb = b_end - b_begin;
  const int ntiles = (nb + 15) >> 4;

  if (w == G::NW) {
    // ================================================================ loader
    const int cg = lane >> 4;
    if constexpr (T > 0) {
      // Ancestry (§3.3): h_t(b, T-1) = parent, h_t(b, j) = h_{T-1}(parent, j).
      // All parent pointers first, then all parent rows, with every load
      // unconditional (indices past the chunk repeat its last beam) so that
      // each batch is one round trip.
      constexpr int QMAX = kMaxChunkF / 64;
      int slot[QMAX][T];
#pragma unroll
      for (int qi = 0; qi < QMAX; ++qi) {
        const int i = min(lane + 64 * qi, nb - 1);
        slot[qi][T - 1] = clampi(a.parent[(size_t)r * a.Wt + b_begin + i], 0, a.Wm - 1);
      }
#pragma unroll
      for (int qi = 0; qi < QMAX; ++qi) {
        const int32_t* prow = a.anc + (((size_t)(T - 1) * a.R + r) * a.Wm + slot[qi][T - 1]) * a.L;
#pragma unroll
        for (int j = 0; j < T - 1; ++j) slot[qi][j] = clampi(prow[j], 0, a.Wm - 1);
      }
      // (table rows past the chunk hold copies and are never read)
#pragma unroll
      for (int qi = 0; qi < QMAX; ++qi) {
        const int i = lane + 64 * qi;
#pragma unroll
        for (int j = 0; j < T; ++j) s_slot[j * kMaxChunkF + i] = slot[qi][j];
        if (h == 0 && i < nb) {
          int32_t* crow = a.anc + (((size_t)T * a.R + r) * a.Wm + b_begin + i) * a.L;
#pragma unroll
          for (int j = 0; j < T; ++j) crow[j] = slot[qi][j];
        }
      }
    }

    auto dma_tile = [&](int p) {
      uint8_t* buf = smem + (p % G::NBUF) * G::BUF;
      const int ib = min(p * 16 + (lane & 15), nb - 1);  // rows past the chunk repeat its last beam
      const size_t tok = ((size_t)r * a.Wt + b_begin + ib) * a.H + h;
      const uint16_t* qrow = a.q + tok * DK;
      const uint16_t* krow = a.k + tok * DK;
      const uint16_t* vrow = a.v + tok * DV;
#pragma unroll
      for (int m = 0; m < G::QB / 1024; ++m) dma16(qrow + (m * 4 + cg) * 8, buf + G::OQ + m * 1024);
#pragma unroll
      for (int m = 0; m < G::QB / 1024; ++m) dma16(krow + (m * 4 + cg) * 8, buf + G::OKK + m * 1024);
#pragma unroll
      for (int m = 0; m < G::VB / 1024; ++m) dma16(vrow + (m * 4 + cg) * 8, buf + G::OV + m * 1024);
      size_t rj[T > 0 ? T : 1];
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const int slot = lds_read_opaque(&s_slot[j * kMaxChunkF + ib]);
        rj[j] = (((size_t)j * a.R + r) * a.Wm + slot) * a.H + h;
      }
#pragma unroll
      for (int j = 0; j < T; ++j) {
        uint8_t* rec = buf + G::OR + j * G::RECB;
#pragma unroll
        for (int m = 0; m < G::RKB / 1024; ++m) dma16(a.rec_k + rj[j] * DK + (m * 4 + cg) * 8, rec + m * 1024);
#pragma unroll
        for (int m = 0; m < G::RDB / 1024; ++m)
          dma16(a.rec_delta + rj[j] * DV + (m * 4 + cg) * 4, rec + G::RKB + m * 1024);
      }
      // dword block: group 0 alpha_t, 1 beta_t, 2 + j alpha_j (16 beams each)
#pragma unroll
      for (int n = 0; n < G::NSM; ++n) {
        const int grp = n * 4 + cg;
        const float* src = grp == 1 ? a.beta + tok : a.alpha + tok;
#pragma unroll
        for (int j = 0; j < T; ++j)
          if (grp == 2 + j) src = a.rec_alpha + rj[j];
        dma4(src, buf + G::OS + n * 256);
      }
    };

    const int npro = min(G::NBUF - 1, ntiles);
    for (int p = 0; p < npro; ++p) dma_tile(p);
    wait_tiles<G::OPT, G::NBUF - 2>(npro - 1);  // tile 0 resident
    lds_barrier();
    for (int i = 0; i < ntiles; ++i) {
      // the consumers released buffer (i - 1) % NBUF at the last barrier
      if (i + G::NBUF - 1 < ntiles) dma_tile(i + G::NBUF - 1);
      const int last = min(i + G::NBUF - 1, ntiles - 1);
      wait_tiles<G::OPT, G::NBUF - 2>(max(0, last - (i + 1)));  // tile i + 1 resident
      lds_barrier();
    }
    return;
  }

  // ================================================================ consumers
  const int g = lane >> 4;
  const int c = lane & 15;

  // This wave's slice of S0[r, h] as bf16 planes in the MFMA A layout: lane
  // (g, c) of tile mt holds key channels 32s + 8g .. +7 of value row
  // 32w + 16mt + c, so C row 4g + i of tile mt is value row 32w + 16mt + 4g + i.
  u32x4 As[2][KS][NPL];
  {
    const float* S = a.S + ((size_t)r * a.H + h) * DK * DV;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int col = w * 32 + mt * 16 + c;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = S[(size_t)(s * 32 + g * 8 + e) * DV + col];
        split_planes<NPL>(x, As[mt][s]);
      }
    }
  }
  lds_barrier();

  for (int it = 0; it < ntiles; ++it) {
    const uint8_t* buf = smem + (it % G::NBUF) * G::BUF;
    const float* sm = reinterpret_cast<const float*>(buf + G::OS);

    u32x4 qf[KS], kf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = *reinterpret_cast<const u32x4*>(buf + G::OQ + (s * 64 + lane) * 16);
      kf[s] = *reinterpret_cast<const u32x4*>(buf + G::OKK + (s * 64 + lane) * 16);
    }
    u32x2 vw[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int ch = w * 4 + mt * 2 + (g >> 1);
      vw[mt] = *reinterpret_cast<const u32x2*>(buf + G::OV + ((ch >> 2) * 64 + (ch & 3) * 16 + c) * 16 + (g & 1) * 8);
    }
    const float at = sm[c];
    const float bt = sm[16 + c];

    // S0^T [q | k] on the matrix cores, smallest plane first
    f32x4 uq[2], uk[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      uq[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      uk[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
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

    // Replay of the ancestral records j = 0 .. T-1 (§3.2) with the decays
    // gathered into per-beam scalars: alpha_t u^(T-1) = c_0 u^(-1) +
    // sum_j c_{j+1} (k_j . x) delta_j, where c_j = alpha_t prod_{i >= j} alpha_i
    // over the chain (c_T = alpha_t), so every record costs one FMA per
    // value row and projection.
    float wq[T > 0 ? T : 1], wk[T > 0 ? T : 1];
    float cdec = at;
#pragma unroll
    for (int j = T - 1; j >= 0; --j) {
      const uint8_t* rec = buf + G::OR + j * G::RECB;
      float pq = 0.f, pk = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4 kj = *reinterpret_cast<const u32x4*>(rec + (s * 64 + lane) * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pq = dot2(kj[e], qf[s][e], pq);
          pk = dot2(kj[e], kf[s][e], pk);
        }
      }
      wq[j] = cdec * sum_lane_groups(pq);
      wk[j] = cdec * sum_lane_groups(pk);
      cdec *= sm[(2 + j) * 16 + c];
    }
    f32x4 xq[2], xk[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      xq[mt] = cdec * uq[mt];
      xk[mt] = cdec * uk[mt];
    }
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const uint8_t* rec = buf + G::OR + j * G::RECB;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f32x4 dj = *reinterpret_cast<const f32x4*>(rec + G::RKB + ((w * 2 + mt) * 64 + lane) * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xq[mt][i] += wq[j] * dj[i];
          xk[mt][i] += wk[j] * dj[i];
        }
      }
    }

    // current transition and append (§3.2, §3.4)
    f32x4 dt[2], ot[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t word = vw[mt][i >> 1];
        const float vv = (i & 1) ? bf16_hi(word) : bf16_lo(word);
        dt[mt][i] = bt * (vv - xk[mt][i]);
        ot[mt][i] = xq[mt][i] + dt[mt][i] * sqq;
      }
    const int b = b_begin + it * 16 + c;
    if (b < b_end) {
      const size_t tok = ((size_t)r * a.Wt + b) * a.H + h;
      const size_t rec_t = (((size_t)T * a.R + r) * a.Wm + b) * a.H + h;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        *reinterpret_cast<f32x4*>(a.o + tok * DV + w * 32 + mt * 16 + 4 * g) = ot[mt];
        *reinterpret_cast<f32x4*>(a.rec_delta + rec_t * DV + w * 32 + mt * 16 + 4 * g) = dt[mt];
      }
#pragma unroll
      for (int s = 0; s < KS; ++s)
        if (s % G::NW == w) *reinterpret_cast<u32x4*>(a.rec_k + rec_t * DK + s * 32 + g * 8) = kf[s];
      if (w == 0 && g == 0) a.rec_alpha[rec_t] = at;
    }
    lds_barrier();
  }
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int DK, int DV, int T>
int launch(const gdn_shape& sh, const gdn_store& st, int Wt, const StepIO& io, hipStream_t stream) {
  using G = FusedGeom<DK, DV, T>;
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
  a.t = T;
  a.Wt = Wt;
  // as many workgroups as can be resident at once
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_beam_fused<DK, DV, T>, G::NT, 0) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  a.chunk = pick_chunk(sh.R * sh.H, Wt, kMaxChunkF, cu_count() * per_cu);
  a.nchunk = (Wt + a.chunk - 1) / a.chunk;
  const long grid = (long)sh.R * sh.H * a.nchunk;
  if (grid > 0x7FFFFFFFL) return GDN_EINVAL;
  hipLaunchKernelGGL((k_beam_fused<DK, DV, T>), dim3((unsigned)grid), dim3(G::NT), 0, stream, a);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

template <int DK, int DV>
int launch_dims(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io, hipStream_t stream) {
  switch (t) {
    case 0: return launch<DK, DV, 0>(sh, st, Wt, io, stream);
    case 1: return launch<DK, DV, 1>(sh, st, Wt, io, stream);
    case 2: return launch<DK, DV, 2>(sh, st, Wt, io, stream);
    case 3: return launch<DK, DV, 3>(sh, st, Wt, io, stream);
    case 4: return launch<DK, DV, 4>(sh, st, Wt, io, stream);
    default: return GDN_EUNSUPPORTED;
  }
}

}  // namespace

bool beam_fused_supported(const gdn_shape& sh, int t) {
  return sh.decay_kind == GDN_DECAY_SCALAR && t >= 0 && t <= kFusedMaxSteps &&
         ((sh.dk == 32 && sh.dv == 32) || (sh.dk == 64 && sh.dv == 64) || (sh.dk == 128 && sh.dv == 128));
}

int launch_beam_fused(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io,
                      hipStream_t stream) {
  if (sh.dk == 32 && sh.dv == 32) return launch_dims<32, 32>(sh, st, t, Wt, io, stream);
  if (sh.dk == 64 && sh.dv == 64) return launch_dims<64, 64>(sh, st, t, Wt, io, stream);
  if (sh.dk == 128 && sh.dv == 128) return launch_dims<128, 128>(sh, st, t, Wt, io, stream);
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn
