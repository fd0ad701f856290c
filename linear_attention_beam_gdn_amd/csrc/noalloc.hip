// gdn_decode_step_split_noalloc: the split-replay decode for callers that
// cannot allocate device memory.  The shared-preparation arm's workspace is
// a buffer compiled into the library (`scratch`, one copy per GPU, alive
// until the process ends).  Its device address is asked of the runtime once
// per device, at the first call on that device, with that device current,
// and kept; kernels receive that address, never the host-side name of the
// array.  Nothing here allocates or frees memory.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn_beam.h"
#include "gdn_launch.h"

namespace {

constexpr size_t kScratchBytes = GDN_SPLIT_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (null: lookup failed)

// The device address of `scratch` on device `dev` (looked up once).
void* scratch_on(int dev) {
  std::call_once(g_once[dev], [dev] {
    int cur = -1;
    const bool switch_dev = hipGetDevice(&cur) == hipSuccess && cur != dev;
    if (switch_dev && hipSetDevice(dev) != hipSuccess) return;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch[dev] = p;
    if (switch_dev) (void)hipSetDevice(cur);
  });
  return g_scratch[dev];
}

}  // namespace

extern "C" int gdn_decode_step_split_noalloc(const gdn_shape* shape, const gdn_store* store, int32_t t,
                                             int32_t n_split, int32_t shared_prep, int32_t merge, const uint16_t* q,
                                             const uint16_t* k, const uint16_t* v, const float* alpha,
                                             const float* beta, float* o, void* stream) {
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (shared_prep == 1 && shape != nullptr && gdn_split_workspace_bytes(shape) > 0) {
    if (gdn_split_workspace_bytes(shape) > kScratchBytes) return GDN_ESCRATCH;
    hipDevice_t dev = 0;
    if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev) != hipSuccess || dev < 0 ||
        dev >= kMaxDevices)
      return GDN_EHIP;
    ws = scratch_on(dev);
    if (ws == nullptr) return GDN_EHIP;
    ws_bytes = kScratchBytes;
  }
  // every other check (and the launch) is the workspace entry point's
  return gdn_decode_step_split(shape, store, t, n_split, shared_prep, merge, q, k, v, alpha, beta, o, ws, ws_bytes,
                               stream);
}
