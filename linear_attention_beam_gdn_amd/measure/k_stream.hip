// Streaming-rate reference kernels for gfx950 (measurement only; not part of
// the decode path).  A launch moves a fixed read:write mix through HBM with
// fully coalesced 16-byte accesses, so that the decode kernels' bandwidth can
// be set against what this GPU streams at the same mix, rather than against
// a nominal peak alone.
//
// Work unit: one workgroup of 256 lanes reads RD blocks and writes WR blocks
// of 4 KiB (256 lanes x 16 bytes each); unit u reads src blocks u*RD .. and
// writes dst blocks u*WR ..  Every lane issues the loads of UNR units before
// their stores, so each wave keeps 4*RD (or 4*WR) 16-byte accesses in flight
// (units is a multiple of UNR, so no access is conditional).
// Stored values are the xor of the unit's loaded words (a constant pattern
// when RD = 0), so no load can be dropped.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int NT = 256;
constexpr int UNR = 4;

template <int RD, int WR, bool NTS>
__global__ __launch_bounds__(NT) void k_stream(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                               long long units) {
  const long long stride = (long long)gridDim.x * UNR;
  for (long long u0 = (long long)blockIdx.x * UNR; u0 < units; u0 += stride) {
    u32x4 acc[UNR];
#pragma unroll
    for (int x = 0; x < UNR; ++x) {
      acc[x] = u32x4{0x9e3779b9u, 0x7f4a7c15u, (uint32_t)u0, (uint32_t)x};
      const long long u = u0 + x;
#pragma unroll
      for (int j = 0; j < RD; ++j) acc[x] ^= src[(u * RD + j) * NT + threadIdx.x];
    }
    if constexpr (WR == 0) {
      // reads only: keep the loads alive with a store that never happens for
      // any data (the xor would have to equal a lane-dependent constant)
      u32x4 all = acc[0];
#pragma unroll
      for (int x = 1; x < UNR; ++x) all ^= acc[x];
      if (all[0] == 0x5bd1e995u + threadIdx.x && all[1] == 0xc2b2ae35u) dst[threadIdx.x] = all;
    }
#pragma unroll
    for (int x = 0; x < UNR; ++x) {
      const long long u = u0 + x;
#pragma unroll
      for (int j = 0; j < WR; ++j) {
        u32x4* p = dst + (u * WR + j) * NT + threadIdx.x;
        if constexpr (NTS) __builtin_nontemporal_store(acc[x] + (uint32_t)j, p);
        else *p = acc[x] + (uint32_t)j;
      }
    }
  }
}

// one launch; with either event set, the runtime records ev0 as the kernel
// starts and ev1 as it completes (hipExtLaunchKernel)
template <bool NTS, int RD, int WR>
void dispatch(const void* src, void* dst, long long units, int n_wg, hipStream_t s, hipEvent_t ev0,
              hipEvent_t ev1) {
  if (ev0 != nullptr || ev1 != nullptr)
    hipExtLaunchKernelGGL((k_stream<RD, WR, NTS>), dim3(n_wg), dim3(NT), 0, s, ev0, ev1, 0, (const u32x4*)src,
                          (u32x4*)dst, units);
  else
    hipLaunchKernelGGL((k_stream<RD, WR, NTS>), dim3(n_wg), dim3(NT), 0, s, (const u32x4*)src, (u32x4*)dst, units);
}

template <int RD, int WR>
int run(const void* src, void* dst, long long units, int n_wg, bool nts, hipStream_t s, hipEvent_t ev0,
        hipEvent_t ev1) {
  if (nts)
    dispatch<true, RD, WR>(src, dst, units, n_wg, s, ev0, ev1);
  else
    dispatch<false, RD, WR>(src, dst, units, n_wg, s, ev0, ev1);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

extern "C" {

// One streaming launch: `units` work units of RD 4-KiB reads from `src` and
// WR 4-KiB writes to `dst` (so src holds units*rd*4096 bytes and dst
// units*wr*4096 bytes, both 16-byte aligned device memory owned by the
// caller; with wr = 0, dst must still hold 4096 bytes; units a multiple of 4), on n_wg workgroups; nontemporal != 0 marks the stores
// non-temporal.  ev_start and ev_stop (HIP events, either may be null) are
// recorded by the runtime as the kernel starts and completes; gdn_stream_run
// is the same launch without them.  Returns 0, -1 for a mix that is not
// built or a bad size, -3 if the launch failed.
int gdn_stream_run_timed(int rd, int wr, const void* src, void* dst, long long units, int n_wg,
                         int nontemporal, void* stream, void* ev_start, void* ev_stop) {
  if (units < 0 || units % UNR != 0 || n_wg < 1 || (rd > 0 && src == nullptr) || dst == nullptr) return -1;
  if (units == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool nts = nontemporal != 0;
  hipEvent_t ev0 = static_cast<hipEvent_t>(ev_start), ev1 = static_cast<hipEvent_t>(ev_stop);
#define GDN_MIX(R_, W_) \
  if (rd == R_ && wr == W_) return run<R_, W_>(src, dst, units, n_wg, nts, s, ev0, ev1);
  GDN_MIX(1, 0)
  GDN_MIX(0, 1)
  GDN_MIX(1, 2)
  GDN_MIX(2, 3)
  GDN_MIX(4, 5)
  GDN_MIX(1, 1)
  GDN_MIX(5, 4)
  GDN_MIX(3, 2)
  GDN_MIX(2, 1)
#undef GDN_MIX
  return -1;
}

int gdn_stream_run(int rd, int wr, const void* src, void* dst, long long units, int n_wg, int nontemporal,
                   void* stream) {
  return gdn_stream_run_timed(rd, wr, src, dst, units, n_wg, nontemporal, stream, nullptr, nullptr);
}

// Timing events for kernel-bracketing measurements (the decode library's
// gdn_beam_decode_step_timed and gdn_stream_run_timed): created without the
// system-scope fence a default event performs when it is recorded, which
// would write back and invalidate caches inside the measured interval.
// Nothing synchronises with them but hipEventSynchronize.  Null on failure.
void* gdn_timing_event_create(void) {
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

void gdn_timing_event_destroy(void* ev) {
  if (ev != nullptr) (void)hipEventDestroy(static_cast<hipEvent_t>(ev));
}

// Microseconds from `start` to `stop` once `stop` has been recorded (waits
// for it); negative if either event has not been recorded or on error.
double gdn_timing_elapsed_us(void* start, void* stop) {
  if (start == nullptr || stop == nullptr) return -1.0;
  if (hipEventSynchronize(static_cast<hipEvent_t>(stop)) != hipSuccess) return -1.0;
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)) != hipSuccess)
    return -1.0;
  return 1e3 * (double)ms;
}

}  // extern "C"
