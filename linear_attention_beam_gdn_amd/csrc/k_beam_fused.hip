// Fused shared-context decode step for scalar-decay GDN beams (OneLA §3.4,
// Figure 5; replay equations of §3.2; ancestry index of §3.3), built as a
// three-role pipeline for gfx950.
//
// Work split.  A workgroup takes one (request r, head h), a slice of at most
// 128 value rows (d_v = 256 and 512 take two and four slices, each forming
// the per-beam dot products itself) and a chunk of its beams, 16 beams (one
// MFMA N block) per tile, and runs three kinds of wave:
//
// * Two DMA waves, taking alternate tiles.  Wave 0 builds the chunk's
//   ancestry slot table in LDS (its inputs in one batch of loads, barrier Q,
//   then the sort, barrier P); wave 1 meanwhile stages S0[r, h] into LDS,
//   which the consumers split into planes between barriers S and A (with
//   d_k = 256 the slice does not fit beside the tile ring, and the consumers
//   load their part of it from HBM at the start instead).  Both
//   then stream every tile's q, k, v, alpha, beta and, for each beam, the
//   decays of its T ancestral records and the keys of the first TL of them
//   (all T unless that would leave fewer than four buffers) straight from
//   HBM into a ring
//   of NBUF LDS buffers with LDS-DMA loads (global_load_lds, no register
//   round trip): tiles 0 and 1 first, the rest of the prologue after A.  They
//   keep tiles in flight (a wave holds at most 63 memory operations, so two
//   waves double the depth) and, before each barrier, the owner of the tile
//   the dot wave takes next waits for it alone (counted vmcnt waits).
// * Dot wave.  One tile ahead of the consumers, forms for every beam the
//   replay's dot products k_j . q_t, k_j . k_t and k_t . q_t (bf16 dot2
//   products reduced over four lane groups) and folds the scalar decays of
//   the chain into per-beam weights:
//       alpha_t u^(T-1) = c_0 u^(-1) + sum_j c_{j+1} (k_j . x) delta_j,
//       c_j = alpha_t prod_{i >= j} alpha_i,  c_T = alpha_t,
//   so the consumers' replay is one FMA per record and value row.  It
//   publishes c_0, beta_t, k_t . q_t and the 2T record weights in the tile's
//   LDS buffer.  The keys of depths TL .. T-1, which the tile buffers do
//   not stage, it loads from the record store itself, one depth at a time.
// * Consumer waves (one per 16 value rows of the slice, two per SIMD for
//   128 rows).  Each holds its 16-row part of the shared state S0[r, h] in
//   registers for the whole chunk as three bf16 planes (hi + mid + lo, each
//   the RNE of the FP32 residual; two for d_k = 256) in the MFMA A layout,
//   so S0 is read once per workgroup and reused by every beam.  Per tile:
//   S0^T [q | k] on the matrix cores (q and k are bf16, so every plane
//   product is exact; FP32 accumulation), the replay on its value rows with
//   the ancestral update vectors delta_j (loaded into registers one tile
//   ahead, each wave its own rows), then delta_t and o_t (o at the beam's
//   index, delta_t at its slot), plus the appended record (by the first
//   value slice).  A wave holds 64 bytes of each beam's o and delta_t rows,
//   so where LDS allows, the tile's o and delta_t pass through an LDS staging
//   buffer and go out one tile later as whole 128-byte lines (8 beams x 32
//   value rows per store instruction, non-temporal); the key rows go out as
//   whole lines too, read from the tile buffer.  Measured at 8 x 512 beams,
//   H = 32, d = 128: writes of half lines, and of 8-byte key pieces, kept the
//   second consumer wave on each SIMD blocked on store issue for half of
//   every tile, and the four launches took 13 % longer.  Two waves per SIMD
//   hide each other's latencies.
//
// Schedule.  With one chunk per (r, h), the beams are taken in the depth-
// first order of the beam tree (lexicographic in their ancestry rows), so that
// beams sharing ancestors share tiles and every ancestral record is gathered
// from memory about once.  That order is a stable sort of the beams by their
// parent's position in the previous step's order, which each step keeps in
// the otherwise unused last entry of its ancestry rows; one wave sorts with a
// counting sort in LDS.  The order only decides which tile and lane computes
// a beam: every beam's arithmetic, and so its result, is the same in any
// order.  A step stores its records at the beams' positions in that order
// (their keys), and the ancestry rows hold those slots, so the next steps'
// tiles gather each depth's records in increasing slot order.
//
// LDS tile layout ("beam fastest"): a 16-row array with NCH 16-byte chunks
// per row keeps chunk ch of row b at 16-byte slot (ch/4)*64 + (ch%4)*16 + b.
// DMA instruction m then fills slots m*64 .. m*64+63 with lane l loading
// chunk 4m + l/16 of row l%16 (so every DMA lane serves one beam), and a
// fragment read of chunk 4s + g for beam c by lane 16g + c is one contiguous
// 1 KiB access, free of bank conflicts.
#include "fused_common.h"

#include "stamps.h"

// Clock stamps (GDN_STAMPS builds): consumer wave 0 stamps kernel entry,
// each prologue barrier and its last tile, and where it ran; the dot wave,
// consumer wave 0 and the DMA waves add up the time they spend working and
// waiting in the tile loop.

namespace gdn {
namespace {

using namespace fused;

template <int DK, int DV, int T>
struct FusedGeom {
  static_assert(DK % 32 == 0 && DV % 32 == 0, "the fused kernel needs d_k, d_v multiples of 32");
  // value rows per workgroup: d_v up to 128 in one slice, wider d_v in NVS
  // slices of 128 (every value row's replay is independent once the per-beam
  // dot products are known; each slice's dot wave forms them itself)
  static constexpr int VS = DV < 128 ? DV : 128;
  static_assert(DV % VS == 0, "d_v must split evenly over value slices");
  static constexpr int NVS = DV / VS;
  static constexpr int NC = VS / 16;       // consumer waves, 16 value rows each
  static constexpr int WDMA = NC;          // wave index of the first DMA wave
  static constexpr int NDMA = 2;           // DMA waves (tile p belongs to DMA wave p % 2)
  static constexpr int WDOT = NC + NDMA;   // wave index of the dot wave
  static constexpr int NT = (NC + NDMA + 1) * 64;
  static constexpr int KS = DK / 32;       // 32-deep MFMA steps over d_k
  static constexpr int QB = 16 * DK * 2;   // bytes of a q (or k) tile
  static constexpr int VB = 16 * VS * 2;   // bytes of a v tile (the slice's value rows)
  static constexpr int NSM = (2 + T) * 16 > 64 ? 2 : 1;  // dword DMAs: alpha_t, beta_t, alpha_j
  static constexpr int SMB = NSM * 256;
  static constexpr int RKB = 16 * DK * 2;  // keys of one record depth
  static constexpr int NWT = (3 + 2 * T + 3) / 4 * 4;  // weights per beam, padded to 16 B
  static constexpr int WTB = 16 * NWT * 4;
  static constexpr int OQ = 0, OKK = QB, OV = 2 * QB, OS = 2 * QB + VB, OW = OS + SMB, ORK = OW + WTB;
  // schedule table: per position {beam, slot_0, slot_1, slot_2}, plus slot_3
  static constexpr int SLOTB = T > 0 ? kMaxChunkF * 16 + (T > 3 ? (T - 3) * kMaxChunkF * 4 : 0) : 0;
  // Record-key depths staged in the tile buffer (the dot wave gathers the
  // keys of the others, depths TL .. T-1, from memory).  Staged are the most
  // depths (every one up to d_k = 128, at most three at d_k = 256, where a
  // depth takes 8 KiB of every buffer) that leave room for four ring
  // buffers (a DMA wave's next tile in flight while the consumers and the
  // dot wave hold two) with the dot wave gathering at most two depths (more
  // and its gathers pace the pipeline); if none does, all that fit.
  // Measured at 8 x 512 beams, H = 16, d_k = 256, d_v = 512: t = 3 and 4 take
  // 204 and 222 us with two staged depths, against 231 and 240 us with
  // three; at d_k = d_v = 128, H = 32, t = 6 stages five.
  static constexpr int staged_depths() {
    const int most = DK > 128 ? (T < 3 ? T : 3) : T;
    for (int tl = most; tl >= 1 && T - tl <= 2; --tl)
      if ((kLdsBytes - SLOTB) / (ORK + tl * RKB) >= 4) return tl;
    return most;
  }
  static constexpr int TL = staged_depths();
  static constexpr int BUF = ORK + TL * RKB;
  // Output staging.  A consumer wave holds 16 value rows (64 bytes) of each
  // beam's o and delta, so its own stores would write half lines; instead
  // the consumers leave a tile's o and delta in LDS and, after the next
  // barrier, each wave stores a block of 8 beams x 32 value rows of each
  // (every store instruction writes whole 128-byte lines).  Two staging
  // buffers (tiles alternate), beam rows padded by 16 bytes so that the
  // consumers' writes are free of bank conflicts; used where the tile ring
  // keeps four buffers beside it.
  static constexpr int PITCH = VS * 4 + 16;
  static constexpr int STGB = 2 * 2 * 16 * PITCH;  // [tile parity][o | delta][beam][value row]
  static constexpr bool STAGE = (kLdsBytes - SLOTB - STGB) / BUF >= 4;
  static constexpr int NBUF0 = (kLdsBytes - SLOTB - (STAGE ? STGB : 0)) / BUF;
  static constexpr int NBUF = NBUF0 > 6 ? 6 : NBUF0;
  static_assert(NBUF >= 3, "tile buffers do not fit in LDS");
  // The slice of S0[r, h] is staged in LDS past the first two tile buffers
  // (which the prologue fills first) until the consumers have split it into
  // planes, when it fits (d_k <= 128); with d_k = 256 the consumers load it
  // from HBM themselves.  The schedule's scratch (bucket counts, staged
  // ancestry rows) is the first two buffers.  The output staging follows the
  // ring (S0 may extend over it: S0 has left LDS before the first tile's
  // outputs arrive), then the schedule table.
  static constexpr int S0B = DK * VS * 4, OS0 = 2 * BUF;
  static constexpr bool S0_LDS = OS0 + S0B + SLOTB <= kLdsBytes;
  static constexpr int OSTG = NBUF * BUF;
  static constexpr int RINGB = (S0_LDS && OS0 + S0B > OSTG + (STAGE ? STGB : 0)) ? OS0 + S0B
                                                                                : OSTG + (STAGE ? STGB : 0);
  static constexpr int LDS = RINGB + SLOTB;
  static_assert(LDS <= kLdsBytes, "LDS layout does not fit");
  static_assert(!S0_LDS || S0B % 1024 == 0, "S0 is staged in whole DMA blocks");
  static_assert(NC >= KS, "every 32-channel step of the appended key row needs a consumer wave");
  // LDS-DMA instructions the DMA wave issues per tile
  static constexpr int OPT = 2 * (QB / 1024) + VB / 1024 + NSM + TL * (RKB / 1024);
  static_assert(QB % 1024 == 0 && VB % 1024 == 0, "tile arrays must be whole DMA blocks");
  static_assert((2 + T) * 16 <= 128, "too many record depths for the small-value block");
  static_assert(T <= 6, "at most six record depths (the small-value block holds 2 + T groups of 16)");
};

template <int DK, int DV, int T>
__global__ __launch_bounds__((FusedGeom<DK, DV, T>::NT)) void k_beam_fused(BeamArgs a) {
  using G = FusedGeom<DK, DV, T>;
  constexpr int KS = G::KS;
  // bf16 planes of S0: three (to about 2^-27 relative), two for d_k = 256
  // (to about 2^-18: the registers of a 16-row slice of 256 key channels, and
  // a third less matrix-core work where it is close to the HBM time)
  constexpr int NPL = DK > 128 ? 2 : 3;
  constexpr int TT = T > 0 ? T : 1;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS];
  u32x4* s_tab = reinterpret_cast<u32x4*>(smem + G::RINGB);                    // [position]
  int* s_slot_hi = reinterpret_cast<int*>(smem + G::RINGB + kMaxChunkF * 16);  // depths 3 .. T-1

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // Workgroups are handed to the 8 XCDs round-robin; renumber them so that
  // the chunks of one (r, h), and the heads of one request, share an XCD.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int chunk_id = bid % a.nchunk;
  const int vsl = (bid / a.nchunk) % G::NVS;  // value slice
  const int rh = bid / (a.nchunk * G::NVS);
  const int h = rh % a.H;
  const int r = rh / a.H;
  const int vs0 = vsl * G::VS;  // first value row of the slice
  // the first slice writes what is not per value row: ancestry, record keys
  // and decays
  const bool slice0 = vsl == 0;
  const int b_begin = chunk_id * a.chunk;
  const int b_end = min(b_begin + a.chunk, a.Wt);
  const int nb = b_end - b_begin;
  const int ntiles = (nb + 15) >> 4;
  const int g = lane >> 4;
  const int c = lane & 15;

  // Barriers: Q (t > 0: the schedule's loads have arrived), P (schedule
  // table written), S (S0 staged in LDS), A (tile 0 resident), then
  // 0 .. ntiles.
  // Between barrier i and i + 1 the consumers take tile i, the dot wave
  // tile i + 1, and a DMA wave refills the buffer of tile i - 1.

  if (w >= G::WDMA && w < G::WDMA + G::NDMA) {
    // ============================================================ DMA waves
    const int dw = w - G::WDMA;  // this wave owns tiles p with p % 2 == dw
    const int cg = lane >> 4;
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
        build_schedule<T, true>(a, r, h == 0 && slice0, b_begin, nb, lane, G::OS0, smem, s_tab, s_slot_hi,
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
      const int posi = min(p * 16 + (lane & 15), nb - 1);  // positions past the chunk repeat its last
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
      const size_t tok = ((size_t)r * a.Wt + b_begin + ib) * a.H + h;
      const size_t tok_k = ((size_t)r * a.Wt + b_begin + ib) * a.Hk + h / a.gq;  // its key head
      const uint16_t* qrow = a.q + tok_k * DK;
      const uint16_t* krow = a.k + tok_k * DK;
      const uint16_t* vrow = a.v + tok * DV + vs0;
#pragma unroll
      for (int m = 0; m < G::QB / 1024; ++m) dma16(qrow + (m * 4 + cg) * 8, buf + G::OQ + m * 1024);
#pragma unroll
      for (int m = 0; m < G::QB / 1024; ++m) dma16(krow + (m * 4 + cg) * 8, buf + G::OKK + m * 1024);
#pragma unroll
      for (int m = 0; m < G::VB / 1024; ++m) dma16(vrow + (m * 4 + cg) * 8, buf + G::OV + m * 1024);
      size_t rj[TT];
#pragma unroll
      for (int j = 0; j < T; ++j) rj[j] = (((size_t)j * a.R + r) * a.Wm + sl[j]) * a.H + h;
#pragma unroll
      for (int j = 0; j < G::TL; ++j)
#pragma unroll
        for (int m = 0; m < G::RKB / 1024; ++m)
          dma16(a.rec_k + ((((size_t)j * a.R + r) * a.Wm + sl[j]) * a.Hk + h / a.gq) * DK + (m * 4 + cg) * 8,
                buf + G::ORK + j * G::RKB + m * 1024);
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

    // tiles this wave issued after tile q, up to tile `last`
    auto later = [&](int q, int last) { return last > q ? (last - q) / 2 : 0; };
    lds_barrier();  // P
    // Tiles 0 and 1 first, on their own, so that they are not queued behind
    // the rest of the prologue (every workgroup of the grid starts at once);
    // the other prologue tiles follow barrier A, once S0 has left LDS.
    const int npro = min(G::NBUF - 1, ntiles);
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
    for (int i = 0; i < ntiles; ++i) {
      // buffer (i - 1) % NBUF was released at the last barrier
      const int p = i + G::NBUF - 1;
      if (p < ntiles && (p & 1) == dw) dma_tile(p);
      const int last = min(p, ntiles - 1);
      const unsigned long long w0 = stamp_now();
      if (i + 2 < ntiles && ((i + 2) & 1) == dw) wait_tiles<G::OPT, 2>(later(i + 2, last));  // tile i + 2 resident
      waited += stamp_now() - w0;
      lds_barrier();                                                                     // i + 1
    }
    GDN_STAMP_AT(11 + dw, G::WDMA + dw, waited);
    return;
  }

  if (w == G::WDOT) {
    // ============================================================ dot wave
    // With d_k = 256 the dot wave's work paces the tile loop from t = 2 on,
    // and it shares its SIMD with two consumer waves: it issues first
    // (measured at 8 x 512 beams, H = 16, d_v = 512: t = 3 4 % faster; at
    // d_k = 128, where it does not pace the loop, no gain).
    if constexpr (DK > 128) __builtin_amdgcn_s_setprio(3);
    // keys of record depth j of tile p's beams from the record store
    auto load_key = [&](int p, int j, u32x4* kj) {
      const int posi = min(p * 16 + c, nb - 1);
      const int slot = j < 3 ? (int)s_tab[posi][1 + j] : s_slot_hi[(j - 3) * kMaxChunkF + posi];
      const uint16_t* key = a.rec_k + ((((size_t)j * a.R + r) * a.Wm + slot) * a.Hk + h / a.gq) * DK;
#pragma unroll
      for (int s = 0; s < KS; ++s) kj[s] = *reinterpret_cast<const u32x4*>(key + s * 32 + g * 8);
    };
    auto dots = [&](int p) {
      uint8_t* buf = smem + (p % G::NBUF) * G::BUF;
      const float* sm = reinterpret_cast<const float*>(buf + G::OS);
      u32x4 qf[KS], kf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qf[s] = *reinterpret_cast<const u32x4*>(buf + G::OQ + (s * 64 + lane) * 16);
        kf[s] = *reinterpret_cast<const u32x4*>(buf + G::OKK + (s * 64 + lane) * 16);
      }
      float wt[3 + 2 * T];
      float sqq = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) sqq = dot2(kf[s][e], qf[s][e], sqq);
      // Depths past the staged ones: their keys straight from the record
      // store, one depth at a time with the next depth's loads in flight
      // (lane (g, c) takes channels 32s + 8g .. +7 of beam c's key, the
      // fragment the staged layout would give it).
      constexpr int TG = T > G::TL ? T - G::TL : 1;
      float pqg[TG], pkg[TG];
      if constexpr (T > G::TL) {
        u32x4 cur[KS], nxt[KS];
        load_key(p, G::TL, cur);
#pragma unroll
        for (int j = G::TL; j < T; ++j) {
          if (j + 1 < T) load_key(p, j + 1, nxt);
          float pq = 0.f, pk = 0.f;
#pragma unroll
          for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pq = dot2(cur[s][e], qf[s][e], pq);
              pk = dot2(cur[s][e], kf[s][e], pk);
            }
          pqg[j - G::TL] = sum_lane_groups(pq);
          pkg[j - G::TL] = sum_lane_groups(pk);
#pragma unroll
          for (int s = 0; s < KS; ++s) cur[s] = nxt[s];
        }
      }
      float cdec = sm[c];  // alpha_t
#pragma unroll
      for (int j = T - 1; j >= 0; --j) {
        float pq = 0.f, pk = 0.f;
        if (j < G::TL) {
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const u32x4 kj = *reinterpret_cast<const u32x4*>(buf + G::ORK + j * G::RKB + (s * 64 + lane) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pq = dot2(kj[e], qf[s][e], pq);
              pk = dot2(kj[e], kf[s][e], pk);
            }
          }
          pq = sum_lane_groups(pq);
          pk = sum_lane_groups(pk);
        } else {
          pq = pqg[j >= G::TL ? j - G::TL : 0];
          pk = pkg[j >= G::TL ? j - G::TL : 0];
        }
        wt[3 + j] = cdec * pq;
        wt[3 + T + j] = cdec * pk;
        cdec *= sm[(2 + j) * 16 + c];
      }
      wt[0] = cdec;
      wt[1] = sm[16 + c];
      wt[2] = sum_lane_groups(sqq);
      float* wout = reinterpret_cast<float*>(buf + G::OW) + c * G::NWT;
#pragma unroll
      for (int v = 0; v < 3 + 2 * T; ++v)
        if ((v & 3) == g) wout[v] = wt[v];
    };
    if (T > 0) lds_barrier();  // Q
    lds_barrier();  // P
    lds_barrier();  // S
    lds_barrier();  // A
    const unsigned long long d0 = stamp_now();
    dots(0);
    GDN_STAMP_AT(9, G::WDOT, stamp_now() - d0);
    lds_barrier();  // 0
    unsigned long long busy = 0, at_barrier = 0;
    for (int i = 0; i < ntiles; ++i) {
      const unsigned long long b0 = stamp_now();
      if (i + 1 < ntiles) dots(i + 1);
      const unsigned long long b1 = stamp_now();
      lds_barrier();  // i + 1
      busy += b1 - b0;
      at_barrier += stamp_now() - b1;
    }
    GDN_STAMP_AT(8, G::WDOT, busy);
    GDN_STAMP_AT(13, G::WDOT, at_barrier);
    return;
  }

  // ============================================================ consumers
  // This wave's part of S0[r, h] as bf16 planes in the MFMA A layout: lane
  // (g, c) holds key channels 32s + 8g .. +7 of value row vs0 + 16w + c, so
  // C row 4g + i is value row vs0 + 16w + 4g + i.
  // A DMA wave stages the slice in LDS (d_k <= 128), or each lane loads its
  // entries from HBM here, overlapping the schedule build (d_k = 256); the
  // planes are formed between barriers S and A.
  GDN_STAMP(0);
  GDN_STAMP_WHERE();
  float s0x[G::S0_LDS ? 1 : KS][8];
  if constexpr (!G::S0_LDS) {
    const float* Sg = a.S + ((size_t)r * a.H + h) * DK * DV + vs0 + w * 16 + c;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) s0x[s][e] = Sg[(size_t)(s * 32 + g * 8 + e) * DV];
  }
  if (T > 0) lds_barrier();  // Q
  GDN_STAMP(1);
  const int row0 = vs0 + w * 16 + 4 * g;  // first of this lane's 4 value rows

  // Store windows over the chunk's beams [b_begin, b_end): a lane whose beam
  // is past the chunk (last tile) lands outside its window.
  const int so = a.H * DV * 4, sk = a.Hk * DK * 2, sa = a.H * 4;  // bytes between beams
  const size_t tok0 = ((size_t)r * a.Wt + b_begin) * a.H + h;
  const size_t rec0 = (((size_t)T * a.R + r) * a.Wm + b_begin) * a.H + h;
  const __amdgpu_buffer_rsrc_t w_o = store_window(a.o + tok0 * DV, (nb - 1) * so + DV * 4);
  const __amdgpu_buffer_rsrc_t w_d = store_window(a.rec_delta + rec0 * DV, (nb - 1) * so + DV * 4);
  // the record key lives per key head: one of its value heads writes it
  const size_t rec0k = (((size_t)T * a.R + r) * a.Wm + b_begin) * a.Hk + h / a.gq;
  const bool key_writer = h % a.gq == 0;
  const __amdgpu_buffer_rsrc_t w_k = store_window(a.rec_k + rec0k * DK, (nb - 1) * sk + DK * 2);
  const __amdgpu_buffer_rsrc_t w_a = store_window(a.rec_alpha + rec0, (nb - 1) * sa + 4);
  // The appended key row: consumer waves w < KS store it, whole 128-byte
  // lines of 8 beams each (d_k >= 64), else channels 32w .. 32w + 31 of every
  // beam (16 bytes per lane).

  // ancestral update vectors of one tile, this lane's 4 rows of beam c
  auto load_deltas = [&](int p, f32x4* d) {
    if constexpr (T > 0) {
      const int posi = min(p * 16 + c, nb - 1);
      const u32x4 e = s_tab[posi];
      int sl[TT > 3 ? TT : 3] = {(int)e[1], (int)e[2], (int)e[3]};
#pragma unroll
      for (int j = 3; j < T; ++j) sl[j] = s_slot_hi[(j - 3) * kMaxChunkF + posi];
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const size_t rj = (((size_t)j * a.R + r) * a.Wm + sl[j]) * a.H + h;
        d[j] = *reinterpret_cast<const f32x4*>(a.rec_delta + rj * DV + row0);
      }
    }
  };

  lds_barrier();  // P: schedule table written
  GDN_STAMP(2);
  f32x4 dnext[TT];
  load_deltas(0, dnext);  // in flight while tile 0 arrives
  lds_barrier();  // S: S0 staged
  GDN_STAMP(3);
  u32x4 As[KS][NPL];
  if constexpr (G::S0_LDS) {
    const float* S = reinterpret_cast<const float*>(smem + G::OS0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = S[(s * 32 + g * 8 + e) * G::VS + w * 16 + c];
      split_planes<NPL>(x, As[s]);
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) split_planes<NPL>(s0x[s], As[s]);
  }
  lds_barrier();  // A: tile 0 resident
  GDN_STAMP(4);
  lds_barrier();  // 0
  GDN_STAMP(5);

  // Staged outputs of tile p (written by every consumer wave before the
  // barrier that ends tile p): this wave stores line block w of o and of
  // delta, value rows 32m .. 32m + 31 of beams 8 half .. 8 half + 7, lane
  // (beam 8 half + l / 8, rows 32m + 4 (l % 8) .. + 3).
  constexpr int PF = G::PITCH / 4;  // floats per staged beam row
  float* const stg = reinterpret_cast<float*>(smem + G::OSTG);
  auto store_staged = [&](int p) {
    constexpr int NM = G::VS / 32;
    const float* sb = stg + (p & 1) * (2 * 16 * PF);
    const int bl = (w / NM) * 8 + (lane >> 3);
    const int rrow = (w % NM) * 32 + (lane & 7) * 4;
    const u32x4 vo = *reinterpret_cast<const u32x4*>(sb + bl * PF + rrow);
    const u32x4 vd = *reinterpret_cast<const u32x4*>(sb + (16 + bl) * PF + rrow);
    const int pos = p * 16 + bl;
    const bool lv = pos < nb;
    const int ibb = lv ? (T > 0 ? (int)s_tab[pos][0] : pos) : 0;
    const int rb = (vs0 + rrow) * 4;
    __builtin_amdgcn_raw_buffer_store_b128(vo, w_o, lv ? ibb * so + rb : kOutside, 0, kStreamStore);
    __builtin_amdgcn_raw_buffer_store_b128(vd, w_d, lv ? pos * so + rb : kOutside, 0, kStreamStore);
  };

  unsigned long long c_busy = 0, c_barrier = 0;
  for (int it = 0; it < ntiles; ++it) {
    const unsigned long long c0 = stamp_now();
    f32x4 dcur[TT];
#pragma unroll
    for (int j = 0; j < T; ++j) dcur[j] = dnext[j];
    if (it + 1 < ntiles) load_deltas(it + 1, dnext);
    // the previous tile's outputs, issued after the next tile's loads so
    // that waiting for those loads does not wait for these stores
    if constexpr (G::STAGE)
      if (it > 0) store_staged(it - 1);

    const uint8_t* buf = smem + (it % G::NBUF) * G::BUF;
    // the tile's q and k fragments (B operands); with d_k = 256 each is read
    // at its MFMA step instead, so that 64 registers stay free for the chain
    constexpr bool kBInLoop = DK > 128;
    u32x4 qf[kBInLoop ? 1 : KS], kf[kBInLoop ? 1 : KS];
    if constexpr (!kBInLoop) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qf[s] = *reinterpret_cast<const u32x4*>(buf + G::OQ + (s * 64 + lane) * 16);
        kf[s] = *reinterpret_cast<const u32x4*>(buf + G::OKK + (s * 64 + lane) * 16);
      }
    }
    const int vch = w * 2 + (g >> 1);  // 16-byte v chunk holding rows row0 .. row0 + 3
    const u32x2 vw = *reinterpret_cast<const u32x2*>(buf + G::OV + ((vch >> 2) * 64 + (vch & 3) * 16 + c) * 16 +
                                                     (g & 1) * 8);
    float wt[G::NWT];
#pragma unroll
    for (int v = 0; v < G::NWT; v += 4) {
      const f32x4 q4 = *reinterpret_cast<const f32x4*>(buf + G::OW + (c * G::NWT + v) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) wt[v + e] = q4[e];
    }

    // S0^T [q | k] on the matrix cores, smallest plane first
    f32x4 uq = {0.f, 0.f, 0.f, 0.f}, uk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 qs, kss;
      if constexpr (kBInLoop) {
        qs = *reinterpret_cast<const u32x4*>(buf + G::OQ + (s * 64 + lane) * 16);
        kss = *reinterpret_cast<const u32x4*>(buf + G::OKK + (s * 64 + lane) * 16);
      } else {
        qs = qf[s];
        kss = kf[s];
      }
#pragma unroll
      for (int p = NPL - 1; p >= 0; --p) {
        uq = mfma16x16x32(As[s][p], qs, uq);
        uk = mfma16x16x32(As[s][p], kss, uk);
      }
    }

    // replay (§3.2) with the dot wave's weights, then the current transition
    f32x4 xq = wt[0] * uq, xk = wt[0] * uk;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      xq += wt[3 + j] * dcur[j];
      xk += wt[3 + T + j] * dcur[j];
    }
    f32x4 dt, ot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = vw[i >> 1];
      const float vv = (i & 1) ? bf16_hi(word) : bf16_lo(word);
      dt[i] = wt[1] * (vv - xk[i]);
      ot[i] = xq[i] + dt[i] * wt[2];
    }

    // output and append (§3.4): every wave issues the same four stores; a
    // position past the chunk stores outside the windows.  o goes to the
    // beam's index, the record to its position in the step's order (its
    // key: record slots follow the order, so the next steps gather them in
    // increasing slot order)
    const int posi = it * 16 + c;
    const bool live = posi < nb;
    if constexpr (G::STAGE) {
      float* sb = stg + (it & 1) * (2 * 16 * PF);
      *reinterpret_cast<f32x4*>(sb + c * PF + w * 16 + 4 * g) = ot;
      *reinterpret_cast<f32x4*>(sb + (16 + c) * PF + w * 16 + 4 * g) = dt;
    } else {
      const int ib = live ? (T > 0 ? (int)s_tab[posi][0] : posi) : 0;
      const int off_o = live ? ib * so + row0 * 4 : kOutside;
      const int off_r = live ? posi * so + row0 * 4 : kOutside;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ot), w_o, off_o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dt), w_d, off_r, 0, 0);
    }
    if constexpr (DK >= 64) {
      // whole 128-byte lines of the key rows, read from the tile buffer:
      // wave w < KS takes line w % (DK / 64) of 8 beams, lane (beam l / 8,
      // 16-byte chunk l % 8 of the line)
      constexpr int LPR = DK / 64;
      if (w < KS) {
        const int bl = (w / LPR) * 8 + (lane >> 3);
        const int ch = (w % LPR) * 8 + (lane & 7);
        const u32x4 kk = *reinterpret_cast<const u32x4*>(buf + G::OKK + ((ch >> 2) * 64 + (ch & 3) * 16 + bl) * 16);
        const int pk = it * 16 + bl;
        __builtin_amdgcn_raw_buffer_store_b128(kk, w_k, pk < nb && key_writer && slice0 ? pk * sk + ch * 16 : kOutside,
                                               0, 0);
      }
    } else if (w < KS) {
      u32x4 kk;
      if constexpr (kBInLoop) {
        kk = *reinterpret_cast<const u32x4*>(buf + G::OKK + (w * 64 + lane) * 16);
      } else {
        kk = kf[0];
#pragma unroll
        for (int s = 1; s < KS; ++s)
          if (w == s) kk = kf[s];
      }
      const int off_k = live && key_writer && slice0 ? posi * sk + (w * 32 + g * 8) * 2 : kOutside;
      __builtin_amdgcn_raw_buffer_store_b128(kk, w_k, off_k, 0, 0);
    }
    const float at = *reinterpret_cast<const float*>(buf + G::OS + c * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(at), w_a,
                                          (live && slice0 && w == G::NC - 1 && g == 0) ? posi * sa : kOutside, 0, 0);
    const unsigned long long c1 = stamp_now();
    lds_barrier();  // it + 1
    c_busy += c1 - c0;
    c_barrier += stamp_now() - c1;
  }
  if constexpr (G::STAGE)
    if (ntiles > 0) store_staged(ntiles - 1);  // the last barrier ended its tile
  GDN_STAMP(6);
  GDN_STAMP_AT(10, 0, c_busy);
  GDN_STAMP_AT(14, 0, c_barrier);
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
  a.chunk = pick_chunk(sh.R * sh.H * G::NVS, Wt, kMaxChunkF, cu_count(stream));
  a.nchunk = (Wt + a.chunk - 1) / a.chunk;
  const long grid = (long)sh.R * sh.H * G::NVS * a.nchunk;
  if (grid > 0x7FFFFFFFL) return GDN_EINVAL;
  GDN_DISPATCH(io.ev_start, io.ev_stop, (k_beam_fused<DK, DV, T>), dim3((unsigned)grid), dim3(G::NT), 0, stream, a);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_EHIP;
}

// longest chain built (the same for every d_k: with d_k = 256 the keys of
// depths past the third come from memory, not the tile buffer)
constexpr int max_steps(int) { return kFusedMaxSteps; }

template <int DK, int DV>
int launch_dims(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io, hipStream_t stream) {
  switch (t) {
    case 0: return launch<DK, DV, 0>(sh, st, Wt, io, stream);
    case 1: return launch<DK, DV, 1>(sh, st, Wt, io, stream);
    case 2: return launch<DK, DV, 2>(sh, st, Wt, io, stream);
    case 3: return launch<DK, DV, 3>(sh, st, Wt, io, stream);
    default: break;
  }
  if constexpr (max_steps(DK) >= 6) {
    switch (t) {
      case 4: return launch<DK, DV, 4>(sh, st, Wt, io, stream);
      case 5: return launch<DK, DV, 5>(sh, st, Wt, io, stream);
      case 6: return launch<DK, DV, 6>(sh, st, Wt, io, stream);
      default: break;
    }
  }
  return GDN_EUNSUPPORTED;
}

bool fused_dims(int dk, int dv) {
  return (dk == 32 && dv == 32) || (dk == 64 && dv == 64) ||
         ((dk == 128 || dk == 256) && (dv == 128 || dv == 256 || dv == 512));
}

}  // namespace

bool beam_fused_supported(const gdn_shape& sh, int t) {
  return sh.decay_kind == GDN_DECAY_SCALAR && fused_dims(sh.dk, sh.dv) && t >= 0 && t <= max_steps(sh.dk) &&
         windows_fit(sh);
}

int launch_beam_fused(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io,
                      hipStream_t stream) {
#define GDN_CASE(DK_, DV_) \
  if (sh.dk == DK_ && sh.dv == DV_) return launch_dims<DK_, DV_>(sh, st, t, Wt, io, stream);
  GDN_CASE(32, 32)
  GDN_CASE(64, 64)
  GDN_CASE(128, 128)
  GDN_CASE(128, 256)
  GDN_CASE(128, 512)
  GDN_CASE(256, 128)
  GDN_CASE(256, 256)
  GDN_CASE(256, 512)
#undef GDN_CASE
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn

#ifdef GDN_STAMPS
// Measurement builds only: rows of 16 stamps per workgroup (entry, barriers
// Q, P, S, A, 0, after the last tile, (XCD << 32 | hardware id), then clock
// ticks: the dot wave's work over the loop and on tile 0, consumer wave 0's
// work over the loop, the two DMA waves' waits, the dot wave's and consumer
// wave 0's time at the loop's barriers, and one spare), and the real-time
// clock's rate.
GDN_STAMPS_READER(gdn_stamps_read)
extern "C" int gdn_stamps_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}
#endif
