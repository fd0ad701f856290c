// Clock stamps for measurement builds (compiled with GDN_STAMPS): lane 0 of
// one wave of every workgroup records the real-time clock at chosen points
// (kernel entry, prologue barriers, the end of the tile loop), the XCD and
// compute unit it ran on, and time sums over the tile loop, into a
// per-workgroup row of a device array that a reader entry point copies out.
// Every source that includes this header gets its own array (internal
// linkage) and defines its reader with GDN_STAMPS_READER.  The product build
// records nothing: the macros are empty and the clock reads return 0.
#pragma once

#include <hip/hip_runtime.h>

#ifdef GDN_STAMPS
namespace gdn {
namespace {
constexpr int kStampWgs = 4096, kStamps = 16;
__device__ unsigned long long g_stamps[kStampWgs * kStamps];
__device__ __forceinline__ unsigned long long stamp_now() { return __builtin_amdgcn_s_memrealtime(); }
}  // namespace
}  // namespace gdn
// lane 0 of wave `wave` writes `val` into slot i of its workgroup's row
#define GDN_STAMP_AT(i, wave, val)                                                    \
  do {                                                                                \
    if (w == (wave) && lane == 0 && blockIdx.x < kStampWgs)                           \
      g_stamps[blockIdx.x * kStamps + (i)] = (val);                                   \
  } while (0)
#define GDN_STAMP(i) GDN_STAMP_AT(i, 0, stamp_now())
// slot 7: (XCD << 32) | hardware id of the wave
#define GDN_STAMP_WHERE()                                                             \
  do {                                                                                \
    if (w == 0 && lane == 0 && blockIdx.x < kStampWgs) {                              \
      const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xF;           \
      const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);                  \
      g_stamps[blockIdx.x * kStamps + 7] = ((unsigned long long)xcc << 32) | hw;      \
    }                                                                                 \
  } while (0)
// Copies the first n_wg rows (16 stamps each) of this source's array to host
// memory and clears the whole array (so that rows of workgroups a launch did
// not have read zero); GDN_EINVAL for a null pointer or n_wg outside
// [0, 4096].
#define GDN_STAMPS_READER(name)                                                                          \
  extern "C" int name(unsigned long long* host, int n_wg) {                                              \
    if (host == nullptr || n_wg < 0 || n_wg > gdn::kStampWgs) return GDN_EINVAL;                         \
    if (hipMemcpyFromSymbol(host, HIP_SYMBOL(gdn::g_stamps), (size_t)n_wg * gdn::kStamps * 8, 0,         \
                            hipMemcpyDeviceToHost) != hipSuccess)                                        \
      return GDN_EHIP;                                                                                   \
    void* dev = nullptr;                                                                                 \
    if (hipGetSymbolAddress(&dev, HIP_SYMBOL(gdn::g_stamps)) != hipSuccess) return GDN_EHIP;             \
    return hipMemset(dev, 0, sizeof(gdn::g_stamps)) == hipSuccess ? GDN_OK : GDN_EHIP;                   \
  }
#else
namespace gdn {
namespace {
__device__ __forceinline__ unsigned long long stamp_now() { return 0; }
}  // namespace
}  // namespace gdn
#define GDN_STAMP_AT(i, wave, val) \
  do {                             \
  } while (0)
#define GDN_STAMP(i) \
  do {               \
  } while (0)
#define GDN_STAMP_WHERE() \
  do {                    \
  } while (0)
#endif
