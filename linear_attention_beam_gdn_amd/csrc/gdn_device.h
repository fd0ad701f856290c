// Device-side helpers shared by the gfx950 kernels of libgdnbeam.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two FP32 values rounded to nearest-even bf16 in one packed word (element 0
// in the low half): gfx950's packed conversion instruction.
__device__ __forceinline__ uint32_t bf16x2_rne(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
}

// Element e (0..7) of eight bf16 packed in a u32x4.
__device__ __forceinline__ float bf16x8_elem(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// Sum over the four 16-lane groups of a wave64 (lanes l, l^16, l^32, l^48)
// with the gfx950 row-swap instructions: plain VALU work, no trip through
// the LDS crossbar.  permlane16_swap exchanges 16-lane rows 1 <-> 0 and
// 3 <-> 2 between its two operands, permlane32_swap the two 32-lane halves;
// with both operands equal, the two results of each swap hold a lane's own
// row and its partner row, so every lane of a group forms the same sum
// ((x0 + x1) + (x2 + x3)) in the same order.
__device__ __forceinline__ float sum_lane_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t v = __float_as_uint(__uint_as_float(a[0]) + __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over all 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One record applied to four entries of a state row, a s + k d, with the
// rounding spelled out (k d fused onto the rounded a s) so that every kernel
// that folds records (materialise, merge, the merge path of the sequence
// decode) produces the same bits.
__device__ __forceinline__ f32x4 apply_record(const f32x4& s, float a, float k, const f32x4& d) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = __builtin_fmaf(k, d[e], a * s[e]);
  return r;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace gdn
