// Fused shared-context decode step for beams with per-channel decay: the KDA
// row of DeltaLog Table 1 (transform D(a_t) S_{t-1}, update pair
// (k_t, beta_t (v_t - (D(a_t) S_{t-1})^T k_t)), diagonal decay), decoded with
// OneLA's shared context state, transition records and ancestry index (§3.2,
// §3.3, §3.4) on LDS-DMA staged tiles like the scalar-decay kernel.
//
// Replay with channel decay.  With Q_j = a_j * a_{j+1} * ... * a_t taken
// channel by channel (Q_{t+1} = 1), the two projections a step needs are
//   u_x = S0^T (Q_0 * x) + sum_{j<t} delta_j (k_j . (Q_{j+1} * x)),  x in {q_t, k_t},
// then delta_t = beta_t (v_t - u_k) and o_t = u_q + delta_t (k_t . q_t).  The
// decay acts on the d_k side, so it lives in the probes: the S0 contraction
// takes the FP32 probes Q_0 * q and Q_0 * k, split into two bf16 planes.
//
// Work split.  A workgroup takes one (request r, head h), a slice of at most
// 128 value rows (d_v = 256 and 512 take two and four slices, each preparing
// the probes and weights itself; with chains of at most three records the
// slices hold 256 rows, two 16-row blocks per consumer wave) and a chunk of its
// beams, 8 beams per tile.  The 16 columns of the gfx950 16x16x32 bf16 MFMA
// carry the q-probes (columns 0-7) and the k-probes (columns 8-15) of the
// same 8 beams, so one MFMA forms both projections.
// * Two DMA waves (alternate tiles) build the ancestry-ordered schedule and
//   stream each tile's q|k rows, v, alpha_t, beta_t and, per beam, the keys
//   and decay vectors of its T ancestral records into a ring of LDS buffers
//   with LDS-DMA loads and counted waits.
// * The consumer waves (one per 16 value rows of the slice, or per 32 in
//   the 256-row slices) each hold their value rows of S0[r, h] as two
//   bf16 planes in registers.  Between two barriers a consumer wave
//   - prepares its share of the next tile (8 / (d_v / 16) beams): each half
//     wave takes the q or the k row of a beam, walks the chain from the
//     current step down (y = a_t * x; weight_j = k_j . y; y = a_j * y), and
//     writes the probe Q_0 * x as hi and lo bf16 planes over the raw row, the
//     record weights and k_t . q_t (chains of up to six records; the T + 1
//     sums of a half wave reduced together, halving the set at each lane
//     exchange); in the first value slice it also appends the beam's key row
//     and decay vector to the record store;
//   - then finishes the current tile: hi*hi + hi*lo + lo*hi plane products
//     on the matrix cores; each lane replays its own column's projection
//     (u_q in the q columns, u_k in the k columns) with its side's record
//     weights and the ancestral update vectors (loaded into registers one
//     tile ahead, addressed by 32-bit offsets from per-depth bases);
//     delta_t is formed in the k columns and handed to the q columns of the
//     same beam by a DPP row rotation, which form o_t; the q columns give
//     o_t and the k columns delta_t to an LDS staging buffer, from which the
//     tile leaves after the next barrier as whole 128-byte lines (where LDS
//     allows; else each lane stores its 16 bytes).
//
// Two heads per workgroup (NI = 2).  When the grid would hold two rounds of
// workgroups or more, a workgroup takes two heads h, h + 1 of one request in
// turn instead (one value slice of up to 128 rows, one chunk): their beams
// and parents are the same, so they share one schedule, and one tile loop
// runs over both heads' tiles, the DMA waves streaming the second head's
// first tiles while the consumers finish the first's.  The consumers load the
// second head's part of S0 from memory and form its planes when they reach
// its first tile.  This
// spares the second head the prologue a second round of workgroups would pay
// (the schedule's loads and sort, S0 and the first tiles in flight); every
// beam's arithmetic is unchanged.
//
// LDS layouts: the 16-row q|k arrays use the beam-fastest layout of the
// scalar kernel (chunk ch of row b at slot (ch/4)*64 + (ch%4)*16 + b); the
// 8-row arrays keep chunk ch of beam b at slot (ch/8)*64 + (ch%8)*8 + b, so
// DMA instruction m fills slots m*64 .. m*64+63 with lane l loading chunk
// 8m + l/8 of beam l%8.  Both put beam b's data in the slots congruent to b
// mod 8, which lets a wave write a beam's probe planes over that beam's raw
// q|k rows and decay vector.
#include "fused_common.h"

#include "stamps.h"

// Clock stamps (GDN_STAMPS builds): consumer wave 0 stamps kernel entry,
// each prologue barrier and its last tile, and where it ran; consumer waves
// 0 and NC - 1 add up their preparation, their finishing work and their
// waits at the loop's barriers, the DMA waves their waits for tiles.

namespace gdn {
namespace {

using namespace fused;

template <int DK, int DV, int T>
struct KdaGeom {
  static_assert(DK % 64 == 0 && DV % 64 == 0, "the channel-decay kernel needs d_k, d_v multiples of 64");
  static constexpr int TB = 8;             // beams per tile
  // 16-row blocks of S0 a consumer wave holds: two for d_v of 256 and more
  // with chains of at most three records, so that a slice has 256 value rows
  // (half the slices, each preparing the probes and weights itself) with
  // eight consumer waves; one for longer chains, whose update vectors would
  // not fit the registers beside two blocks of S0 planes
  static constexpr int NRB = (DV >= 256 && T <= 3) ? 2 : 1;
  // the next tile's update vectors loaded in one batch at the top of a tile
  // (two sets held) where the registers allow it, else block by block right
  // after use (one set)
  static constexpr bool DBUF = NRB == 1 || T <= 1;
  static constexpr int VS = DV < 128 ? DV : 128 * NRB;  // value rows per workgroup
  static_assert(DV % VS == 0, "d_v must split evenly over value slices");
  static constexpr int NVS = DV / VS;      // value slices
  // 32-bit offsets from per-depth bases (24-bit products) for the update
  // vectors, the outputs and the appends: faster with one row block per
  // consumer wave (seven steps at 16 x 256 beams: 10 % faster), slower with
  // two (the 256-row slices: 18 % slower at t = 1), which keep 64-bit
  // addresses and plain products
  static constexpr bool LEAN = NRB == 1;
  static constexpr int NC = VS / (16 * NRB);  // consumer waves, 16 NRB value rows each
  static_assert(TB % NC == 0, "each consumer wave prepares whole beams");
  static constexpr int BPW = TB / NC;      // beams a consumer wave prepares per tile
  static constexpr int EPL = DK / 32;      // channels per lane in the preparation
  static constexpr int WDMA = NC;          // first DMA wave
  static constexpr int NDMA = 2;
  static constexpr int NT = (NC + NDMA) * 64;
  static constexpr int KS = DK / 32;
  static constexpr int QKB = 16 * DK * 2;  // q|k rows; then the probes' hi plane
  // alpha_t of the 8 beams; then the probes' lo plane.  The 8-row slots of
  // beam b are exactly the 16-row slots of rows b and b + 8, so the wave that
  // prepares beam b overwrites only what it has already read.
  static constexpr int VB = TB * VS * 2;
  static constexpr int AB = TB * DK * 4;
  static constexpr int SMB = 256;          // beta_t
  // weights per beam: beta_t and k_t . q_t in the first 16 bytes, then the T
  // q-side and the T k-side record weights, each side padded to 16 bytes, so
  // that a lane reads its own side's weights in whole 16-byte words
  static constexpr int P4 = (T + 3) / 4 * 4;
  static constexpr int NWT = 4 + 2 * P4;
  static constexpr int WTB = TB * NWT * 4;
  static constexpr int RKB = TB * DK * 2;  // keys of one record depth
  static_assert(AB == QKB, "the lo plane of a tile takes the place of its decay vectors");
  static constexpr int OQK = 0, OV = QKB, OA = OV + VB, OLO = OA, OS = OA + AB, OW = OS + SMB, ORK = OW + WTB,
                       ORA = ORK + T * RKB;
  static constexpr int BUF = ORA + T * AB;
  static_assert(T <= 6, "the channel-decay kernel takes at most six record depths");
  // schedule table: per position {beam, slot_0, slot_1, slot_2}, plus slots 3 .. T-1
  static constexpr int SLOTB = T > 0 ? kMaxChunkF * 16 + (T > 3 ? (T - 3) * kMaxChunkF * 4 : 0) : 0;
  // Output staging, as in the scalar-decay kernel: a consumer wave holds 16
  // value rows (64 bytes) of each beam's o or delta, so the tile's o and
  // delta wait in LDS and leave after the next barrier as whole 128-byte
  // lines (8 beams x 32 value rows per store instruction).  Two buffers
  // (tiles alternate), beam rows padded by 16 bytes; used where the ring
  // keeps three buffers beside them (at d_v = 512, t = 3 the staging with
  // three buffers measured 6 % faster than half-line stores with four, and
  // chains of five to seven records 1-3 % faster; the scalar-decay kernel
  // keeps four: with three its wide state ran t = 2 and 3 slower).
  static constexpr int PITCH = VS * 4 + 16;
  static constexpr int STGB = 2 * 2 * TB * PITCH;  // [tile parity][o | delta][beam][value row]
  static constexpr bool STAGE = (kLdsBytes - SLOTB - STGB) / BUF >= 3;
  static constexpr int NBUF0 = (kLdsBytes - SLOTB - (STAGE ? STGB : 0)) / BUF;
  static constexpr int NBUF = NBUF0 > 6 ? 6 : NBUF0;
  static_assert(NBUF >= 3, "tile buffers do not fit in LDS");
  // The slice of S0[r, h] ([d_k][VS]) is staged in LDS past the first two
  // tile buffers until the consumers have split it into planes, when it fits
  // (chains of up to five records); otherwise the consumers load it from HBM
  // themselves.  The schedule's scratch is the first two buffers.
  static constexpr int S0B = DK * VS * 4, OS0 = 2 * BUF;
  static constexpr bool S0_LDS = OS0 + S0B + SLOTB <= kLdsBytes;
  // the output staging follows the ring (S0 may extend over it: S0 has left
  // LDS before the first tile's outputs arrive), then the schedule table
  static constexpr int OSTG = NBUF * BUF;
  static constexpr int RINGB = (S0_LDS && OS0 + S0B > OSTG + (STAGE ? STGB : 0)) ? OS0 + S0B
                                                                                : OSTG + (STAGE ? STGB : 0);
  static constexpr int LDS = RINGB + SLOTB;
  static_assert(LDS <= kLdsBytes, "LDS layout does not fit");
  static_assert(!S0_LDS || S0B % 1024 == 0, "S0 is staged in whole DMA blocks");
  // LDS-DMA instructions per tile (q|k, v, alpha_t, beta_t, then per record k_j, a_j)
  static constexpr int OPT = QKB / 1024 + VB / 1024 + AB / 1024 + 1 + T * (RKB / 1024 + AB / 1024);
  static_assert(QKB % 1024 == 0 && VB % 1024 == 0 && AB % 1024 == 0 && RKB % 1024 == 0,
                "tile arrays must be whole DMA blocks");
};

// 16-byte slot of chunk ch of row b in the 16-row and the 8-row layouts
__device__ __forceinline__ int slot16(int b, int ch) { return (ch >> 2) * 64 + (ch & 3) * 16 + b; }
__device__ __forceinline__ int slot8(int b, int ch) { return (ch >> 3) * 64 + (ch & 7) * 8 + b; }

// value of lane l^8 within each 16-lane row (DPP row_ror:8)
__device__ __forceinline__ float swap8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, true));
}

// Sum over each 32-lane half of a wave64: quad swaps and row rotations by
// DPP within the 16-lane rows, then the row pair (0, 1) or (2, 3) with the
// gfx950 row-swap instruction.  Lane 0 of a half always forms the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum_half(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp<0x124>(x);  // row_ror:4
  x += dpp<0x128>(x);  // row_ror:8
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// NV sums (NV = 1, 2, 4 or 8) over each 32-lane half at once.  Exchanges
// that halve the set come first: a lane keeps half of its values and adds
// its partner's copy of them, sending the other half, which its partner
// keeps (partners l and 7 - l choosing on bit 2, then l ^ 1 on bit 0, then
// l ^ 2 on bit 1); plain sums over the remaining lane bits follow.  Lane l
// ends with the sum of value 4 b2 + 2 b0 + b1 (NV = 8), 2 b0 + b1 (NV = 4),
// b0 (NV = 2) or 0 (NV = 1), b_i being bit i of l.  v is overwritten.
template <int NV>
__device__ __forceinline__ float sum_half_many(float* v, int lane) {
  static_assert(NV == 1 || NV == 2 || NV == 4 || NV == 8, "NV must be 1, 2, 4 or 8");
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4;
  if constexpr (NV == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float keep = b2 ? v[4 + i] : v[i], send = b2 ? v[i] : v[4 + i];
      v[i] = keep + dpp<0x141>(send);  // row_half_mirror: l <-> 7 - l
    }
  }
  if constexpr (NV >= 2) {
    constexpr int HV = NV >= 4 ? 2 : 1;
#pragma unroll
    for (int i = 0; i < HV; ++i) {
      const float keep = b0 ? v[HV + i] : v[i], send = b0 ? v[i] : v[HV + i];
      v[i] = keep + dpp<0xB1>(send);  // l ^ 1
    }
  }
  if constexpr (NV >= 4) {
    const float keep = b1 ? v[1] : v[0], send = b1 ? v[0] : v[1];
    v[0] = keep + dpp<0x4E>(send);  // l ^ 2
  }
  float x = v[0];
  if constexpr (NV < 2) x += dpp<0xB1>(x);
  if constexpr (NV < 4) x += dpp<0x4E>(x);
  if constexpr (NV < 8) x += dpp<0x124>(x);  // row_ror:4
  x += dpp<0x128>(x);                        // row_ror:8
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
// the value whose sum lane l (bits 0 .. 4 of its index) holds after sum_half_many<NV>
template <int NV>
__device__ __forceinline__ int sum_half_many_index(int l) {
  const int b0 = l & 1, b1 = (l >> 1) & 1, b2 = (l >> 2) & 1;
  return NV == 8 ? 4 * b2 + 2 * b0 + b1 : NV == 4 ? 2 * b0 + b1 : NV == 2 ? b0 : 0;
}

// EPL consecutive bf16 (EPL = 2 or 4) as packed words, and EPL floats
template <int EPL>
__device__ __forceinline__ void lds_bf16(const uint8_t* p, uint32_t* w) {
  if constexpr (EPL == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v[0];
    w[1] = v[1];
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}
template <int EPL>
__device__ __forceinline__ void lds_f32(const uint8_t* p, float* x) {
  if constexpr (EPL == 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v[e];
  } else {
    const float2 v = *reinterpret_cast<const float2*>(p);
    x[0] = v.x;
    x[1] = v.y;
  }
}
template <int EPL>
__device__ __forceinline__ void lds_put(uint8_t* p, const uint32_t* w) {
  if constexpr (EPL == 4)
    *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
  else
    *reinterpret_cast<uint32_t*>(p) = w[0];
}

template <int DK, int DV, int T, int NI>
__global__ __launch_bounds__((KdaGeom<DK, DV, T>::NT)) void k_beam_fused_kda(BeamArgs a) {
  using G = KdaGeom<DK, DV, T>;
  constexpr int KS = G::KS;
  constexpr int EPL = G::EPL;
  constexpr int TT = T > 0 ? T : 1;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS];
  u32x4* s_tab = reinterpret_cast<u32x4*>(smem + G::RINGB);
  int* s_slot_hi = reinterpret_cast<int*>(smem + G::RINGB + kMaxChunkF * 16);  // depths 3 .. T-1

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  static_assert(NI == 1 || (NI == 2 && G::NVS == 1), "two heads per workgroup take one value slice each");
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  // (with NI = 2 the launch has one chunk and one value slice, and bid runs
  // over (request, head pair))
  const int chunk_id = bid % a.nchunk;
  const int vsl = (bid / a.nchunk) % G::NVS;  // value slice
  const int rh = bid / (a.nchunk * G::NVS);
  const int hpr = a.H / NI;                    // head groups per request
  const int h = (rh % hpr) * NI;               // first head of the workgroup
  const int r = rh / hpr;
  const int vs0 = vsl * G::VS;  // first value row of the slice
  const bool slice0 = vsl == 0;  // writes ancestry, record keys and decays
  const int b_begin = chunk_id * a.chunk;
  const int b_end = min(b_begin + a.chunk, a.Wt);
  const int nb = b_end - b_begin;
  const int ntiles = (nb + G::TB - 1) / G::TB;  // per head
  const int ntot = NI * ntiles;                 // tiles of the loop over the heads
  // head item (0 or 1) of loop tile p, and p's tile within that head (tiles
  // past the end count as the last head's)
  auto item_of = [&](int p) { return NI > 1 && p >= ntiles ? 1 : 0; };
  auto local = [&](int p) { return NI > 1 && p >= ntiles ? p - ntiles : p; };

  // Barriers: Q (t > 0: the schedule's loads have arrived), P (schedule
  // table written), S (S0 staged in LDS), A (tile 0 resident), then
  // 0 .. ntot.  Between barrier i and i + 1 the consumers finish tile i and
  // prepare tile i + 1, and a DMA wave refills the buffer of tile i - 1.

  if (w >= G::WDMA) {
    // ============================================================ DMA waves
    const int dw = w - G::WDMA;
    // the slice of S0[r, h] into LDS as [d_k][VS] (wave 1), after the
    // schedule's loads have gone out; 256 floats per DMA instruction
    auto stage_s0 = [&] {
      if constexpr (G::S0_LDS) {
        const float* S = a.S + ((size_t)r * a.H + h) * DK * DV + vs0;
#pragma unroll
        for (int m = 0; m < G::S0B / 1024; ++m) {
          const int e0 = m * 256 + lane * 4;
          dma16(S + (size_t)(e0 / G::VS) * DV + e0 % G::VS, smem + G::OS0 + m * 1024);
        }
      }
    };
    if (T > 0) {
      if (dw == 0) {
        build_schedule<T, false>(a, r, h == 0 && slice0, b_begin, nb, lane, G::OS0, smem, s_tab, s_slot_hi,
                          [] { lds_barrier(); });  // Q inside, once its loads have arrived
      } else {
        lds_barrier();  // Q
        stage_s0();
      }
    } else if (dw == 1) {
      stage_s0();
    }

    auto dma_tile = [&](int p) {
      uint8_t* buf = smem + (p % G::NBUF) * G::BUF;
      const int hp = h + item_of(p);
      const int posi = min(local(p) * G::TB + (lane & 7), nb - 1);  // positions past the chunk repeat its last
      int ib = posi, sl[TT > 3 ? TT : 3] = {};
      if constexpr (T > 0) {
        const u32x4 e = lds_read128_opaque(&s_tab[posi]);
        ib = (int)e[0];
        sl[0] = (int)e[1];
        sl[1] = (int)e[2];
        sl[2] = (int)e[3];
#pragma unroll
        for (int j = 3; j < T; ++j) sl[j] = lds_read_opaque(&s_slot_hi[(j - 3) * kMaxChunkF + posi]);
      }
      const size_t tok = ((size_t)r * a.Wt + b_begin + ib) * a.H + hp;
      // q|k: rows 0-7 the q rows, rows 8-15 the k rows of the tile's beams
      const size_t tok_k = ((size_t)r * a.Wt + b_begin + ib) * a.Hk + hp / a.gq;  // its key head
      const uint16_t* qkrow = ((lane & 8) ? a.k : a.q) + tok_k * DK;
#pragma unroll
      for (int m = 0; m < G::QKB / 1024; ++m) dma16(qkrow + (m * 4 + (lane >> 4)) * 8, buf + G::OQK + m * 1024);
#pragma unroll
      for (int m = 0; m < G::VB / 1024; ++m) dma16(a.v + tok * DV + vs0 + (m * 8 + (lane >> 3)) * 8, buf + G::OV + m * 1024);
#pragma unroll
      for (int m = 0; m < G::AB / 1024; ++m)
        dma16(a.alpha + tok * DK + (m * 8 + (lane >> 3)) * 4, buf + G::OA + m * 1024);
      dma4(a.beta + tok, buf + G::OS);
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const size_t rj = (((size_t)j * a.R + r) * a.Wm + sl[j]) * a.H + hp;
        const size_t rjk = (((size_t)j * a.R + r) * a.Wm + sl[j]) * a.Hk + hp / a.gq;
#pragma unroll
        for (int m = 0; m < G::RKB / 1024; ++m)
          dma16(a.rec_k + rjk * DK + (m * 8 + (lane >> 3)) * 8, buf + G::ORK + j * G::RKB + m * 1024);
#pragma unroll
        for (int m = 0; m < G::AB / 1024; ++m)
          dma16(a.rec_alpha + rj * DK + (m * 8 + (lane >> 3)) * 4, buf + G::ORA + j * G::AB + m * 1024);
      }
    };

    auto later = [&](int q, int last) { return last > q ? (last - q) / 2 : 0; };
    lds_barrier();  // P
    // tiles 0 and 1 first, on their own; the other prologue tiles follow A,
    // once S0 has left LDS
    const int npro = min(G::NBUF - 1, ntot);
    if (dw < npro) dma_tile(dw);
    if (dw == 1) {
      if (npro > 1) wait_vm<G::OPT>();  // S0 staged; tile 1 may still be in flight
      else wait_vm<0>();
    }
    lds_barrier();              // S
    if (dw == 0) wait_vm<0>();  // tile 0 resident
    lds_barrier();              // A
    for (int p = 2 + dw; p < npro; p += 2) dma_tile(p);
    if (dw == 1) wait_tiles<G::OPT, 2>(later(1, npro - 1));  // tile 1 resident
    lds_barrier();                                          // 0
    unsigned long long waited = 0;
    for (int i = 0; i < ntot; ++i) {
      const int p = i + G::NBUF - 1;  // into the buffer released at the last barrier
      if (p < ntot && (p & 1) == dw) dma_tile(p);
      const int last = min(p, ntot - 1);
      const unsigned long long w0 = stamp_now();
      if (i + 2 < ntot && ((i + 2) & 1) == dw) wait_tiles<G::OPT, 2>(later(i + 2, last));  // tile i + 2 resident
      waited += stamp_now() - w0;
      lds_barrier();                                                                     // i + 1
    }
    GDN_STAMP_AT(11 + dw, G::WDMA + dw, waited);
    return;
  }

  // ============================================================ consumers
  GDN_STAMP(0);
  GDN_STAMP_WHERE();
  // record-store windows over the chunk's beams (appends at step T) of the
  // head prep() works on (with NI = 2 they move to the second head before
  // its first tile is prepared)
  const int sk = a.Hk * DK * 2, sa = a.H * DK * 4;  // bytes between beams
  __amdgpu_buffer_rsrc_t w_k, w_a;
  bool key_writer;
  auto prep_head = [&](int hh) {
    const size_t rec0 = (((size_t)T * a.R + r) * a.Wm + b_begin) * a.H + hh;
    // the record key lives per key head: one of its value heads writes it
    const size_t rec0k = (((size_t)T * a.R + r) * a.Wm + b_begin) * a.Hk + hh / a.gq;
    key_writer = hh % a.gq == 0 && slice0;
    w_k = store_window(a.rec_k + rec0k * DK, (nb - 1) * sk + DK * 2);
    w_a = store_window(a.rec_alpha + rec0 * DK, (nb - 1) * sa + DK * 4);
  };
  prep_head(h);

  // Preparation of beams w * BPW .. w * BPW + BPW - 1 of tile p.  Lane
  // (side, el): channels EPL * el .. EPL * el + EPL - 1 of the q row
  // (side 0) or the k row (side 1).
  const int ps = lane >> 5;
  const int el = lane & 31;
  const int e0 = el * EPL;
  const int oqk = slot16(0, e0 >> 3) * 16 + (e0 & 7) * 2;  // row 0; row b adds 16 b
  const int o8h = slot8(0, e0 >> 3) * 16 + (e0 & 7) * 2;   // bf16 8-row arrays; beam b adds 16 b
  const int o8f = slot8(0, e0 >> 2) * 16 + (e0 & 3) * 4;   // f32 8-row arrays
  auto prep = [&](int p) {
    uint8_t* buf = smem + (p % G::NBUF) * G::BUF;
#pragma unroll
    for (int u = 0; u < G::BPW; ++u) {
      const int pb = w * G::BPW + u;
      uint32_t xw[EPL / 2], kw[EPL / 2];
      float at[EPL], y[EPL];
      lds_bf16<EPL>(buf + G::OQK + oqk + (pb + 8 * ps) * 16, xw);
      lds_bf16<EPL>(buf + G::OQK + oqk + (pb + 8) * 16, kw);
      lds_f32<EPL>(buf + G::OA + o8f + pb * 16, at);
      const float beta = reinterpret_cast<const float*>(buf + G::OS)[pb];
      float sqq = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float xe = (e & 1) ? bf16_hi(xw[e >> 1]) : bf16_lo(xw[e >> 1]);
        const float ke = (e & 1) ? bf16_hi(kw[e >> 1]) : bf16_lo(kw[e >> 1]);
        y[e] = at[e] * xe;
        sqq += ke * xe;
      }
      // walk the chain from the current step down: weight_j = k_j . (Q_{j+1} x)
      float wj[TT];
#pragma unroll
      for (int j = T - 1; j >= 0; --j) {
        uint32_t kj[EPL / 2];
        float aj[EPL];
        lds_bf16<EPL>(buf + G::ORK + j * G::RKB + o8h + pb * 16, kj);
        lds_f32<EPL>(buf + G::ORA + j * G::AB + o8f + pb * 16, aj);
        float pj = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          pj += ((e & 1) ? bf16_hi(kj[e >> 1]) : bf16_lo(kj[e >> 1])) * y[e];
          y[e] *= aj[e];
        }
        wj[j] = pj;
      }
      // appends of step T: the key row (side 1) and the decay vector (side 0)
      const int posi = local(p) * G::TB + pb;
      const bool live = posi < nb;
      const int ib = T > 0 ? (int)s_tab[min(posi, nb - 1)][0] : posi;  // read unconditionally: no branch
      // byte offsets of the beam's appends (24-bit products where a consumer
      // wave holds one row block: beams and strides are far below 2^24; the
      // 256-row slices measured faster with plain products)
      const int ib_k = G::LEAN ? (int)__umul24((uint32_t)ib, (uint32_t)sk) : ib * sk;
      const int ib_a = G::LEAN ? (int)__umul24((uint32_t)ib, (uint32_t)sa) : ib * sa;
      if constexpr (EPL == 4) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{kw[0], kw[1]}, w_k,
                                              live && ps && key_writer ? ib_k + e0 * 2 : kOutside, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{at[0], at[1], at[2], at[3]}), w_a,
                                               live && !ps && slice0 ? ib_a + e0 * 4 : kOutside, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(kw[0], w_k, live && ps && key_writer ? ib_k + e0 * 2 : kOutside,
                                              0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(at[0]), __float_as_uint(at[1])}, w_a,
                                              live && !ps && slice0 ? ib_a + e0 * 4 : kOutside, 0, 0);
      }
      // probe Q_0 x as hi + lo bf16 planes, over the raw row and this beam's alpha_t
      uint32_t hw[EPL / 2], lw[EPL / 2];
#pragma unroll
      for (int e = 0; e < EPL; e += 2) {
        hw[e >> 1] = bf16x2_rne(y[e], y[e + 1]);
        lw[e >> 1] = bf16x2_rne(y[e] - bf16_lo(hw[e >> 1]), y[e + 1] - bf16_hi(hw[e >> 1]));
      }
      lds_put<EPL>(buf + G::OQK + oqk + (pb + 8 * ps) * 16, hw);
      lds_put<EPL>(buf + G::OLO + oqk + (pb + 8 * ps) * 16, lw);
      // weights: k.q (side 0), the q-weights (side 0 sums) and the
      // k-weights (side 1 sums), all summed over the half-waves at once
      constexpr int NV = T == 0 ? 1 : T == 1 ? 2 : T <= 3 ? 4 : 8;
      float sv[NV];
      sv[0] = sqq;
#pragma unroll
      for (int i = 1; i < NV; ++i) sv[i] = i <= T ? wj[i <= T ? i - 1 : 0] : 0.f;
      const float red = sum_half_many<NV>(sv, lane);
      // one store for the wave, no branch: the lanes holding value i of
      // their side write it (side 0: k.q to entry 1, q-weight j to 4 + j;
      // side 1: k-weight j to 4 + P4 + j); every other lane writes beta to
      // entry 0
      const int l5 = lane & 31, qi = sum_half_many_index<NV>(l5);
      const bool has = l5 < NV && qi <= T && (qi > 0 || ps == 0);
      const int wi = !has ? 0 : qi == 0 ? 1 : 3 + qi + ps * G::P4;
      reinterpret_cast<float*>(buf + G::OW)[pb * G::NWT + wi] = has ? red : beta;
    }
  };

  // Part of S0[r, h] as hi + lo bf16 planes in the MFMA A layout: lane
  // (g, c) holds, in row block rb, key channels 32s + 8g .. +7 of value row
  // vs0 + 16 (NRB w + rb) + c, so C row 4g + i of that block is value row
  // vs0 + 16 (NRB w + rb) + 4g + i.
  const int g = lane >> 4;
  const int c = lane & 15;
  const int bb = c & 7;     // beam of this lane within the tile
  const int side = c >> 3;  // 0: q column, 1: k column
  // A DMA wave stages S0 in LDS, or (chains of six records) each lane loads
  // its entries from HBM here; the planes are formed between barriers S and A.
  constexpr int NRB = G::NRB;
  float s0x[G::S0_LDS ? 1 : NRB][G::S0_LDS ? 1 : KS][8];
  if constexpr (!G::S0_LDS) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float* Sg = a.S + ((size_t)r * a.H + h) * DK * DV + vs0 + (w * NRB + rb) * 16 + c;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) s0x[rb][s][e] = Sg[(size_t)(s * 32 + g * 8 + e) * DV];
    }
  }
  if (T > 0) lds_barrier();  // Q
  GDN_STAMP(1);
  // this lane's first value row in row block rb: row0 + 16 rb
  const int row0 = vs0 + w * NRB * 16 + 4 * g;
  const int so = a.H * DV * 4;
  // windows of o and the appended update vectors of the head being finished
  __amdgpu_buffer_rsrc_t w_o, w_d;
  auto out_head = [&](int hh) {
    const size_t tok0 = ((size_t)r * a.Wt + b_begin) * a.H + hh;
    const size_t rec0 = (((size_t)T * a.R + r) * a.Wm + b_begin) * a.H + hh;
    w_o = store_window(a.o + tok0 * DV, (nb - 1) * so + DV * 4);
    w_d = store_window(a.rec_delta + rec0 * DV, (nb - 1) * so + DV * 4);
  };
  out_head(h);

  // ancestral update vectors of tile p, this lane's 4 rows of beam bb in row
  // blocks rb0 .. rb1 - 1.  LEAN: slot s of depth j sits s * so bytes past
  // the depth's first slot of the head (a 32-bit offset: the store holds
  // less than 2 GiB of update vectors per depth and request); the depths'
  // bases move to the second head (NI = 2) before its first tile's vectors
  // load.
  const uint8_t* dbase[TT];
  auto delta_head = [&](int hh) {
#pragma unroll
    for (int j = 0; j < T; ++j)
      dbase[j] = reinterpret_cast<const uint8_t*>(a.rec_delta + ((((size_t)j * a.R + r) * a.Wm) * a.H + hh) * DV);
  };
  delta_head(h);
  auto load_deltas = [&](int p, f32x4 (*d)[NRB], int rb0 = 0, int rb1 = G::NRB) {
    if constexpr (T > 0) {
      const int posi = min(local(p) * G::TB + bb, nb - 1);
      const u32x4 e = s_tab[posi];
      int sl[TT > 3 ? TT : 3] = {(int)e[1], (int)e[2], (int)e[3]};
#pragma unroll
      for (int j = 3; j < T; ++j) sl[j] = s_slot_hi[(j - 3) * kMaxChunkF + posi];
#pragma unroll
      for (int j = 0; j < T; ++j) {
        if constexpr (G::LEAN) {
          const uint32_t off = __umul24((uint32_t)sl[j], (uint32_t)so) + (uint32_t)row0 * 4;
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            if (rb >= rb0 && rb < rb1) d[j][rb] = *reinterpret_cast<const f32x4*>(dbase[j] + off + 64 * rb);
        } else {
          const size_t rj = (((size_t)j * a.R + r) * a.Wm + sl[j]) * a.H + h + item_of(p);
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
            if (rb >= rb0 && rb < rb1)
              d[j][rb] = *reinterpret_cast<const f32x4*>(a.rec_delta + rj * DV + row0 + 16 * rb);
        }
      }
    }
  };

  lds_barrier();  // P
  GDN_STAMP(2);
  f32x4 dnext[TT][NRB];
  load_deltas(0, dnext);
  lds_barrier();  // S: S0 staged
  GDN_STAMP(3);
  u32x4 As[NRB][KS][2];
  if constexpr (G::S0_LDS) {
    const float* S = reinterpret_cast<const float*>(smem + G::OS0);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = S[(s * 32 + g * 8 + e) * G::VS + (w * NRB + rb) * 16 + c];
        split_planes<2>(x, As[rb][s]);
      }
  } else {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int s = 0; s < KS; ++s) split_planes<2>(s0x[rb][s], As[rb][s]);
  }
  lds_barrier();  // A: tile 0 resident
  GDN_STAMP(4);
  prep(0);
  lds_barrier();  // 0
  GDN_STAMP(5);

  unsigned long long c_prep = 0, c_fin = 0, c_bar = 0;
  // Staged outputs of tile p (written by every consumer wave before the
  // barrier that ends tile p, the head's windows still current): this wave
  // stores line blocks NRB w .. NRB w + NRB - 1 of the tile's o (blocks
  // 0 .. VS/32 - 1) and delta (the next VS/32), each value rows 32m .. 32m + 31
  // of the 8 beams, lane (beam l / 8, rows 32m + 4 (l % 8) .. + 3).
  constexpr int PF = G::PITCH / 4;  // floats per staged beam row
  float* const stg = reinterpret_cast<float*>(smem + G::OSTG);
  auto store_staged = [&](int p) {
    constexpr int NM = G::VS / 32;
    const int bl = lane >> 3;
    const int pos = local(p) * G::TB + bl;
    const bool lv = pos < nb;
    const int ibb = lv ? (T > 0 ? (int)s_tab[pos][0] : pos) : 0;
#pragma unroll
    for (int k = 0; k < NRB; ++k) {
      const int idx = w * NRB + k;
      const int arr = idx / NM;  // 0: o, 1: delta
      const int rrow = (idx % NM) * 32 + (lane & 7) * 4;
      const u32x4 v =
          *reinterpret_cast<const u32x4*>(stg + (p & 1) * (2 * G::TB * PF) + (arr * G::TB + bl) * PF + rrow);
      __builtin_amdgcn_raw_buffer_store_b128(v, arr ? w_d : w_o, lv ? ibb * so + (vs0 + rrow) * 4 : kOutside, 0,
                                             kStreamStore);
    }
  };
  // one tile of the loop (the loop runs once per head, so that the planes of
  // S0 stay fixed inside it)
  auto step = [&](int it) {
    const unsigned long long c0 = stamp_now();
    if constexpr (NI > 1) {
      if (it + 1 == ntiles) delta_head(h + 1);  // the next tile's update vectors are the second head's
    }
    // Double-buffered: this tile's update vectors move to dcur and the next
    // tile's are loaded at once.  Otherwise each row block's next update
    // vectors are loaded into dnext right after the block has used them
    // (below), which holds one set instead of two.
    constexpr bool DBUF = G::DBUF;
    f32x4 dcur[DBUF ? TT : 1][DBUF ? NRB : 1];
    if constexpr (DBUF) {
#pragma unroll
      for (int j = 0; j < T; ++j)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) dcur[j][rb] = dnext[j][rb];
      load_deltas(it + 1, dnext);
    }
    // the previous tile of this head's outputs (issued after the next tile's
    // update vectors where those load in one batch).  With three records and
    // two row blocks per wave, the register-bound case, they leave after the
    // next tile's preparation instead: two registers spilled instead of four,
    // and t = 3 at d_v = 512 8 % faster (at t = 2, or with one row block, that
    // placement was 2-4 % slower).  At one record with one 256-row slice
    // (d_v = 256) they leave at the end of the tile: no register spilled
    // instead of three, t = 1 at 16 x 256 beams 9 % faster (at d_v = 512 that
    // placement was not faster).
    constexpr bool LATE_STORE = T == 3 && G::NRB == 2;
    constexpr bool END_STORE = T == 1 && G::NRB == 2 && G::NVS == 1;
    if constexpr (G::STAGE && !LATE_STORE && !END_STORE)
      if (local(it) > 0) store_staged(it - 1);
    // Next tile, unconditionally so that it shares a basic block with this
    // tile's work.  Past the last tile it reads a free buffer (no load of
    // this launch targets it any more), writes only there, and its appends
    // fall outside the store windows.
    if constexpr (NI > 1) {
      if (it + 1 == ntiles) prep_head(h + 1);
    }
    prep(it + 1);
    if constexpr (G::STAGE && LATE_STORE)
      if (local(it) > 0) store_staged(it - 1);
    const unsigned long long c1 = stamp_now();

    const uint8_t* buf = smem + (it % G::NBUF) * G::BUF;
    u32x4 bh[KS], bl[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bh[s] = *reinterpret_cast<const u32x4*>(buf + G::OQK + slot16(c, s * 4 + g) * 16);
      bl[s] = *reinterpret_cast<const u32x4*>(buf + G::OLO + slot16(c, s * 4 + g) * 16);
    }
    // beta_t and k_t . q_t, then this lane's side's record weights
    const f32x4 w01 = *reinterpret_cast<const f32x4*>(buf + G::OW + bb * G::NWT * 4);
    float ws[G::P4 > 0 ? G::P4 : 1];
#pragma unroll
    for (int v = 0; v < G::P4; v += 4) {
      const f32x4 q4 = *reinterpret_cast<const f32x4*>(buf + G::OW + (bb * G::NWT + 4 + side * G::P4 + v) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) ws[v + e] = q4[e];
    }
    const int posi = local(it) * G::TB + bb;
    const bool live = posi < nb;
    const int ib = T > 0 ? (int)s_tab[min(posi, nb - 1)][0] : posi;

#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      // 16-byte v chunk holding this lane's rows row0 + 16 rb .. + 3
      const int vch = (w * NRB + rb) * 2 + (g >> 1);
      const u32x2 vw = *reinterpret_cast<const u32x2*>(buf + G::OV + slot8(bb, vch) * 16 + (g & 1) * 8);

      // S0^T [Q_0 q | Q_0 k] for the tile's 8 beams: hi*hi + hi*lo + lo*hi
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u = mfma16x16x32(As[rb][s][1], bh[s], u);
        u = mfma16x16x32(As[rb][s][0], bl[s], u);
        u = mfma16x16x32(As[rb][s][0], bh[s], u);
      }
      // Replay of this lane's own projection (u_q in the q columns, u_k in
      // the k columns), delta_t formed in the k columns and handed to the q
      // columns of the same beam (lane c ^ 8), o_t formed there.
      f32x4 x = u;
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const f32x4 dj = DBUF ? dcur[DBUF ? j : 0][DBUF ? rb : 0] : dnext[j][rb];
        x += ws[j] * dj;
      }
      f32x4 dt, ot;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t word = vw[i >> 1];
        const float vv = (i & 1) ? bf16_hi(word) : bf16_lo(word);
        dt[i] = w01[0] * (vv - x[i]);
        ot[i] = x[i] + swap8(dt[i]) * w01[1];
      }

      // output (q-column lanes) and the appended update vector (k-column lanes)
      if constexpr (G::STAGE) {
        *reinterpret_cast<f32x4*>(stg + (it & 1) * (2 * G::TB * PF) + (side * G::TB + bb) * PF +
                                  (w * NRB + rb) * 16 + 4 * g) = side ? dt : ot;
      } else {
        const int off = live ? (G::LEAN ? (int)__umul24((uint32_t)ib, (uint32_t)so) : ib * so) + (row0 + 16 * rb) * 4
                             : kOutside;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ot), w_o, side ? kOutside : off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dt), w_d, side ? off : kOutside, 0, 0);
      }
      if constexpr (!DBUF) load_deltas(it + 1, dnext, rb, rb + 1);
    }
    if constexpr (G::STAGE && END_STORE)
      if (local(it) > 0) store_staged(it - 1);
    const unsigned long long c2 = stamp_now();
    lds_barrier();  // it + 1
    c_prep += c1 - c0;
    c_fin += c2 - c1;
    c_bar += stamp_now() - c2;
  };
  for (int it = 0; it < ntiles; ++it) step(it);
  // the head's last tile (its barrier has passed) before the windows move on
  if constexpr (G::STAGE)
    if (ntiles > 0) store_staged(ntiles - 1);
  if constexpr (NI > 1) {
    // the second head: its part of S0 from memory into the planes, its
    // output windows, then its tiles
    out_head(h + 1);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float* Sg = a.S + ((size_t)r * a.H + h + 1) * DK * DV + vs0 + (w * NRB + rb) * 16 + c;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = Sg[(size_t)(s * 32 + g * 8 + e) * DV];
        split_planes<2>(x, As[rb][s]);
      }
    }
    for (int it = ntiles; it < ntot; ++it) step(it);
    if constexpr (G::STAGE)
      if (ntot > ntiles) store_staged(ntot - 1);
  }
  GDN_STAMP(6);
  GDN_STAMP_AT(8, 0, c_prep);
  GDN_STAMP_AT(9, 0, c_fin);
  GDN_STAMP_AT(10, 0, c_bar);
  GDN_STAMP_AT(13, G::NC - 1, c_prep + c_fin);
  GDN_STAMP_AT(14, G::NC - 1, c_bar);
}

template <int DK, int DV, int T>
int launch(const gdn_shape& sh, const gdn_store& st, int Wt, const StepIO& io, hipStream_t stream) {
  using G = KdaGeom<DK, DV, T>;
  BeamArgs a;
  a.S = st.S;
  a.rec_delta = st.rec_delta;
  a.rec_k = st.rec_k;
  a.rec_alpha = st.rec_alpha;
  a.anc = st.anc;
  a.parent = io.parent;
  a.bad_parents = io.bad_parents;
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
  a.Hk = key_heads(sh);
  a.gq = sh.H / a.Hk;
  // one workgroup per compute unit: the tile ring takes most of its LDS
  const int cus = cu_count(stream);
  a.chunk = pick_chunk(sh.R * sh.H * G::NVS, Wt, kMaxChunkF, cus);
  a.nchunk = (Wt + a.chunk - 1) / a.chunk;
  const long grid = (long)sh.R * sh.H * G::NVS * a.nchunk;
  if (grid > 0x7FFFFFFFL) return GDN_EINVAL;
  // Two heads per workgroup where a grid of one per head would run two
  // rounds or more (one chunk, one value slice, chains of up to three records,
  // whose registers leave room for the second head's S0).  Not with two row
  // blocks per consumer wave (d_v = 256 in one slice): there the pair spills
  // registers and 16 x 32 heads of 256 beams ran no faster (four steps 746
  // against 740 us).  GDN_BEAM_PAIR=0 turns it off, for comparisons.
  if constexpr (G::NVS == 1 && G::NRB == 1 && T <= 3) {
    const char* pair = getenv("GDN_BEAM_PAIR");
    const bool off = pair != nullptr && pair[0] == '0';
    if (!off && a.nchunk == 1 && sh.H % 2 == 0 && grid >= 2L * cus) {
      GDN_DISPATCH(io.ev_start, io.ev_stop, (k_beam_fused_kda<DK, DV, T, 2>), dim3((unsigned)(grid / 2)), dim3(G::NT),
                   0, stream, a);
      return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
    }
  }
  GDN_DISPATCH(io.ev_start, io.ev_stop, (k_beam_fused_kda<DK, DV, T, 1>), dim3((unsigned)grid), dim3(G::NT), 0, stream,
               a);
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
    case 5: return launch<DK, DV, 5>(sh, st, Wt, io, stream);
    case 6: return launch<DK, DV, 6>(sh, st, Wt, io, stream);
    default: return GDN_EUNSUPPORTED;
  }
}

}  // namespace

bool beam_fused_kda_supported(const gdn_shape& sh, int t) {
  // the consumers address a depth's update vectors with 32-bit offsets
  const bool offsets_fit = (long long)sh.W_max * sh.H * sh.dv * 4 < (1LL << 31);
  return sh.decay_kind == GDN_DECAY_CHANNEL && t >= 0 && t <= 6 &&
         ((sh.dk == 64 && sh.dv == 64) || (sh.dk == 128 && (sh.dv == 128 || sh.dv == 256 || sh.dv == 512))) &&
         windows_fit(sh) && offsets_fit;
}

int launch_beam_fused_kda(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io,
                          hipStream_t stream) {
  if (sh.dk == 64 && sh.dv == 64) return launch_dims<64, 64>(sh, st, t, Wt, io, stream);
  if (sh.dk == 128 && sh.dv == 128) return launch_dims<128, 128>(sh, st, t, Wt, io, stream);
  if (sh.dk == 128 && sh.dv == 256) return launch_dims<128, 256>(sh, st, t, Wt, io, stream);
  if (sh.dk == 128 && sh.dv == 512) return launch_dims<128, 512>(sh, st, t, Wt, io, stream);
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn

#ifdef GDN_STAMPS
// Measurement builds only: rows of 16 stamps per workgroup (entry, barriers
// Q, P, S, A, 0, after the last tile, (XCD << 32 | hardware id), then clock
// ticks over the tile loop: consumer wave 0's preparation, finishing work and
// time at the barriers, the two DMA waves' waits, consumer wave NC - 1's work
// and time at the barriers, and one spare).
GDN_STAMPS_READER(gdn_kda_stamps_read)
#endif
