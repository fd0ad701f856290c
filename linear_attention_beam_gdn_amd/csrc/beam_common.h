// Types and helpers shared by the beam decode kernels.
#pragma once

#include <stdlib.h>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

struct BeamArgs {
  const float* S;
  float* rec_delta;
  uint16_t* rec_k;
  float* rec_alpha;
  int32_t* anc;
  const int32_t* parent;
  int* bad_parents;  // parent-check builds: count of parents outside [0, W_max)
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  float* o;
  int R, Wm, H, L, t, Wt;
  int chunk, nchunk;
  // key heads: q, k and the record keys have Hk heads; value head h uses key
  // head h / gq (gq = H / Hk)
  int Hk, gq;
};

// First key channel of the 8 consecutive channels that lane group g feeds to
// MFMA step s.  Any assignment works as long as the A and B operands use the
// same one; this one gives each lane 16 (d_k >= 64) contiguous channels.
template <int DK>
__device__ __forceinline__ int kchunk(int g, int s) {
  if constexpr (DK % 64 == 0) return (s >> 1) * 64 + g * 16 + (s & 1) * 8;
  else return g * 8;
}
template <int DK>
__device__ __forceinline__ bool klive(int g) {
  if constexpr (DK == 16) return g < 2;  // lane groups 2, 3 feed zero padding
  else return true;
}

// Parent-check builds (GDN_CHECK_PARENTS): count a parent pointer outside
// [0, W_max) (the kernels clamp it into that range, so no access leaves the
// store; the result for that beam is then meaningless).  One caller per
// (request, beam) counts, so the total is the number of bad pointers.
__device__ __forceinline__ void check_parent(const BeamArgs& a, int parent) {
#ifdef GDN_CHECK_PARENTS
  if ((parent < 0 || parent >= a.Wm) && a.bad_parents != nullptr) atomicAdd(a.bad_parents, 1);
#else
  (void)a;
  (void)parent;
#endif
}

__device__ __forceinline__ void load_f32x8(const float* p, float* x) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

// Split eight FP32 values into bf16 planes: x ~= sum_p plane[p] (RNE each).
template <int NP>
__device__ __forceinline__ void split_planes(const float* x, u32x4* planes) {
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    float r0 = x[e], r1 = x[e + 1];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t hb = bf16x2_rne(r0, r1);
      planes[p][e >> 1] = hb;
      r0 -= bf16_lo(hb);
      r1 -= bf16_hi(hb);
    }
  }
}

// Beams per workgroup: a multiple of 16 and at most max_chunk, sized so that
// the grid holds about target_wgs workgroups when the beam count allows it.
// GDN_BEAM_CHUNK (a multiple of 16) overrides the choice for tuning sweeps.
inline int pick_chunk(int RH, int Wt, int max_chunk, int target_wgs) {
  const int full = (Wt + 15) / 16 * 16;
  int chunk;
  const char* e = getenv("GDN_BEAM_CHUNK");
  if (e != nullptr && atoi(e) >= 16 && atoi(e) % 16 == 0) {
    chunk = atoi(e);
  } else {
    const long want = ((long)RH * Wt + target_wgs - 1) / target_wgs;
    chunk = (int)((want + 15) / 16) * 16;
  }
  if (chunk < 16) chunk = 16;
  if (chunk > full) chunk = full;
  return chunk > max_chunk ? max_chunk : chunk;
}
}  // namespace gdn
