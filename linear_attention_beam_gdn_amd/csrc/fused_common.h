// Device helpers shared by the fused beam decode kernels (scalar and
// per-channel decay): LDS-DMA staging with counted waits, barriers, opaque
// LDS reads, store windows, and the ancestry-order schedule of a chunk.
#pragma once

#include "beam_common.h"

namespace gdn {
namespace fused {

constexpr int kMaxChunkF = 512;         // beams per workgroup at most
constexpr int kLdsBytes = 160 * 1024;   // LDS of one gfx950 compute unit
constexpr int kSortMax = 8192;          // largest W_max whose tree order is computed

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
__device__ __forceinline__ u32x4 lds_read128_opaque(const void* p) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

// Raw buffer resource (gfx9 layout) over `bytes` bytes at `base`: stores at
// offsets past the end are dropped by the hardware, which lets every lane
// issue the same stores whatever its beam.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_window(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}
constexpr int kOutside = 0x7FFFFFF0;  // an offset past every store window
// Cache policy of the whole-line output stores (the aux operand of the
// buffer stores): non-temporal, agent scope (nt | sc1).  The outputs stream
// on to memory instead of staying dirty in the L2 and the memory-side cache,
// where the next launch's reads would pay for writing them back.  Measured at
// 8 x 512 beams, H = 32, d = 128: back-to-back passes 9 % faster; a launch
// that follows a read-only sweep 5 % slower, since the sweep had absorbed the
// write-back that plain stores leave behind.
constexpr int kStreamStore = 2 | 16;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Schedule of a chunk for a decode step with T records per chain (run by one
// wave).  Builds the chunk's ancestry (OneLA §3.3: h_t(b, T-1) = parent,
// h_t(b, j) = h_{T-1}(parent, j)), orders the beams depth-first in the beam
// tree when the chunk holds the whole step (a counting sort of the beams by
// their parent's position in the previous step's order), and writes
//   s_tab[position]  = {beam, slot_0, slot_1, slot_2},
//   s_slot_hi[(j - 3) * kMaxChunkF + position] = slot_j for 3 <= j < T,
//   anc row T of every beam (when `anc_writer`: one workgroup per request
//   and chunk), with the beam's position in the unused last entry for the
//   next step.
// The order only decides which lanes compute a beam, never its result.
//
// Record slots.  With KEY_SLOTS (the scalar-decay kernel) a step stores each
// beam's record at the beam's order key (its position in the step's order,
// the last entry of its ancestry row) rather than at its index, so the slots
// an ancestry row holds are keys: a parent's slot is the key read from its
// row.  The tiles of a step follow its order, so they gather every depth's
// records in increasing slot order.  At step 0 (no order) a beam's key is
// its index.  Without KEY_SLOTS records stay at the beam's index.
//
// Memory: the parent pointers and, for T >= 2, the whole previous-step
// ancestry block of the request (W_max x L_max entries, staged into LDS by
// LDS DMA when it fits in `scratch`) are fetched in one batch; `mid()` runs
// once they have arrived (the caller's workgroup barrier), and the sort
// follows.  `scratch` (scratch_bytes, 16-byte aligned) holds the bucket
// counts and the staged block and is free for other use afterwards.
template <int T, bool KEY_SLOTS, class Mid>
__device__ __forceinline__ void build_schedule(const BeamArgs& a, int r, bool anc_writer, int b_begin, int nb, int lane,
                                               int scratch_bytes, uint8_t* scratch, u32x4* s_tab, int* s_slot_hi,
                                               Mid mid) {
  constexpr int TT = T > 0 ? T : 1;
  constexpr int QMAX = kMaxChunkF / 64;
  const int hist_words = (a.Wm + 63) & ~63;
  const bool sorted = a.nchunk == 1 && a.Wm <= kSortMax && hist_words * 4 <= scratch_bytes;
  const int blk_words = a.Wm * a.L;
  const bool staged = T > 1 && hist_words * 4 + ((blk_words + 63) & ~63) * 4 <= scratch_bytes;
  int* hist = reinterpret_cast<int*>(scratch);
  int* rows = reinterpret_cast<int*>(scratch) + hist_words;  // staged ancestry block
  const int32_t* blk = a.anc + ((size_t)(TT - 1) * a.R + r) * a.Wm * a.L;

  // One batch: every parent pointer (indices past the chunk repeat its last
  // beam, so every load is unconditional) and the staged block.
  int slot[QMAX][TT], key[QMAX], pos[QMAX];
#pragma unroll
  for (int qi = 0; qi < QMAX; ++qi) {
    const int i = min(lane + 64 * qi, nb - 1);
    slot[qi][TT - 1] = a.parent[(size_t)r * a.Wt + b_begin + i];
  }
  if (staged)
    for (int x = 0; x < blk_words; x += 64)  // lane l of each block fills word x + l
      dma4(blk + min(x + lane, blk_words - 1), reinterpret_cast<uint8_t*>(rows + x));
  wait_vm<0>();
  mid();
#pragma unroll
  for (int qi = 0; qi < QMAX; ++qi) {
    if (anc_writer && lane + 64 * qi < nb) check_parent(a, slot[qi][TT - 1]);
    slot[qi][TT - 1] = clampi(slot[qi][TT - 1], 0, a.Wm - 1);
  }
  // Ancestry (§3.3): h_t(b, T-1) = parent, h_t(b, j) = h_{T-1}(parent, j);
  // the parent's position in the previous step's order is the sort key (its
  // own slot when the previous step is the first).
  // (two separate paths, so that the staged rows are read as LDS, not
  // through generic pointers)
  if constexpr (T > 1) {
    if (staged) {
#pragma unroll
      for (int qi = 0; qi < QMAX; ++qi) {
        const int* prow = rows + slot[qi][TT - 1] * a.L;
#pragma unroll
        for (int j = 0; j < T - 1; ++j) slot[qi][j] = clampi(prow[j], 0, a.Wm - 1);
        key[qi] = clampi(prow[a.L - 1], 0, a.Wm - 1);
        if constexpr (KEY_SLOTS) slot[qi][TT - 1] = key[qi];
      }
    } else {
#pragma unroll
      for (int qi = 0; qi < QMAX; ++qi) {
        const int32_t* prow = blk + (size_t)slot[qi][TT - 1] * a.L;
#pragma unroll
        for (int j = 0; j < T - 1; ++j) slot[qi][j] = clampi(prow[j], 0, a.Wm - 1);
        key[qi] = clampi(prow[a.L - 1], 0, a.Wm - 1);
        if constexpr (KEY_SLOTS) slot[qi][TT - 1] = key[qi];
      }
    }
  } else {
#pragma unroll
    for (int qi = 0; qi < QMAX; ++qi) key[qi] = slot[qi][TT - 1];
  }
  if (sorted) {
    // counting sort by key (ties in any order): bucket counts with LDS
    // atomics, an exclusive scan over the buckets, then each beam's position
    // = bucket start + its rank in the bucket.  One wave: its LDS accesses
    // complete in program order.
    for (int x = lane; x < a.Wm; x += 64) hist[x] = 0;
#pragma unroll
    for (int qi = 0; qi < QMAX; ++qi)
      if (lane + 64 * qi < nb) pos[qi] = atomicAdd(&hist[key[qi]], 1);
    const int per = (a.Wm + 63) / 64;
    const int x0 = min(lane * per, a.Wm), x1 = min(x0 + per, a.Wm);
    int local = 0;
    for (int x = x0; x < x1; ++x) local += hist[x];
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    int run = incl - local;
    for (int x = x0; x < x1; ++x) {
      const int cnt = hist[x];
      hist[x] = run;
      run += cnt;
    }
#pragma unroll
    for (int qi = 0; qi < QMAX; ++qi)
      if (lane + 64 * qi < nb) pos[qi] += hist[key[qi]];
  } else {
#pragma unroll
    for (int qi = 0; qi < QMAX; ++qi) pos[qi] = lane + 64 * qi;  // chunk order
  }
  // Schedule table, this step's ancestry rows, and each beam's position
  // (read by the next step) in the unused last entry of its row.
#pragma unroll
  for (int qi = 0; qi < QMAX; ++qi) {
    const int i = lane + 64 * qi;
    if (i < nb) {
      s_tab[pos[qi]] = u32x4{(uint32_t)i, (uint32_t)slot[qi][0], (uint32_t)slot[qi][T > 1 ? 1 : 0],
                             (uint32_t)slot[qi][T > 2 ? 2 : 0]};
#pragma unroll
      for (int j = 3; j < T; ++j) s_slot_hi[(j - 3) * kMaxChunkF + pos[qi]] = slot[qi][j];
      if (anc_writer) {
        int32_t* crow = a.anc + (((size_t)T * a.R + r) * a.Wm + b_begin + i) * a.L;
#pragma unroll
        for (int j = 0; j < T; ++j) crow[j] = slot[qi][j];
        crow[a.L - 1] = sorted ? pos[qi] : b_begin + i;  // order key for the next step
      }
    }
  }
}

// The store windows and per-beam store offsets are 32-bit byte ranges over a
// chunk of up to kMaxChunkF beams: the widest per-beam stride (o and delta:
// H d_v FP32; keys: H_k d_k bf16; per-channel decays: H d_k FP32) times the
// chunk must stay below 2^31.  Shapes past that take the general kernel,
// which indexes with 64-bit offsets.
inline bool windows_fit(const gdn_shape& sh) {
  const long long hk = sh.H_k > 0 ? sh.H_k : sh.H;
  long long stride = (long long)sh.H * sh.dv * 4;
  if (hk * sh.dk * 2 > stride) stride = hk * sh.dk * 2;
  if ((long long)sh.H * sh.dk * 4 > stride) stride = (long long)sh.H * sh.dk * 4;
  return (long long)kMaxChunkF * stride + stride < (1LL << 31);
}

// Compute units of the device a stream runs on, asked of the runtime at every
// launch (no cache, so concurrent first calls share no state).
inline int cu_count(hipStream_t stream) {
  hipDevice_t dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return 256;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

}  // namespace fused
}  // namespace gdn
