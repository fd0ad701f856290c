// C ABI of libgdnbeam (declared in include/gdn_beam.h): host-side argument
// validation, then dispatch to the gfx950 kernels on the caller's stream.
// Validation touches no HIP API, so every error path runs without a GPU.
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "gdn_beam.h"
#include "gdn_launch.h"

namespace gdn {

bool seq_dims_supported(int dk, int dv) {
  return (dk == 16 && dv == 16) || (dk == 32 && dv == 32) || (dk == 64 && dv == 64) ||
         (dk == 128 && dv == 128);
}

bool dims_supported(int dk, int dv, int decay_kind) {
  if (seq_dims_supported(dk, dv)) return true;
  // the wider beam geometries: d_k in {128, 256} x d_v in {128, 256, 512};
  // channel decay with d_k = 128 only, the plain rule on the square shapes only
  const bool wide = (dk == 128 || dk == 256) && (dv == 128 || dv == 256 || dv == 512);
  if (!wide) return false;
  if (decay_kind == GDN_DECAY_SCALAR) return true;
  return decay_kind == GDN_DECAY_CHANNEL && dk == 128;
}

}  // namespace gdn

namespace {

#ifdef GDN_CHECK_PARENTS
// Parent-check builds only: one device counter of parent pointers found
// outside [0, W_max) by the beam decode kernels, per GPU; its address is
// looked up once per device.
__device__ int g_bad_parents;
constexpr int kMaxDevices = 64;
std::once_flag g_bad_once[kMaxDevices];
int* g_bad_ptr[kMaxDevices];
int* bad_parents_on(hipStream_t stream) {
  hipDevice_t dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_bad_once[dev], [dev] {
    int cur = -1;
    const bool sw = hipGetDevice(&cur) == hipSuccess && cur != dev;
    if (sw && hipSetDevice(dev) != hipSuccess) return;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_bad_parents)) == hipSuccess) g_bad_ptr[dev] = static_cast<int*>(p);
    if (sw) (void)hipSetDevice(cur);
  });
  return g_bad_ptr[dev];
}
#endif

bool aligned(const void* p, uintptr_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(const gdn_shape* s) {
  if (s == nullptr) return GDN_EINVAL;
  if (s->R < 1 || s->W_max < 1 || s->H < 1 || s->L_max < 1 || s->L_max > GDN_MAX_STEPS)
    return GDN_EINVAL;
  if (s->decay_kind != GDN_DECAY_SCALAR && s->decay_kind != GDN_DECAY_CHANNEL &&
      s->decay_kind != GDN_DECAY_CHANNEL_PLAIN)
    return GDN_EUNSUPPORTED;
  if (!gdn::dims_supported(s->dk, s->dv, s->decay_kind)) return GDN_EUNSUPPORTED;
  if (s->H_k < 0 || (s->H_k > 0 && s->H % s->H_k != 0)) return GDN_EINVAL;
  // element counts of the largest arrays must stay far from 2^63
  const double recs = (double)s->L_max * s->R * s->W_max * s->H * (s->dk > s->dv ? s->dk : s->dv);
  const double anc = (double)s->L_max * s->R * s->W_max * s->L_max;
  if (recs > 4.0e18 || anc > 4.0e18) return GDN_EINVAL;
  return GDN_OK;
}

int check_store(const gdn_store* st) {
  if (st == nullptr) return GDN_EINVAL;
  if (!aligned(st->S, 16) || !aligned(st->rec_delta, 16) || !aligned(st->rec_k, 16) ||
      !aligned(st->rec_alpha, 16) || !aligned(st->anc, 16))
    return GDN_EINVAL;
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_BEAM_ABI_VERSION; }

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument (null or misaligned pointer, index or size out of range)";
    case GDN_EUNSUPPORTED: return "unsupported head dims or decay kind";
    case GDN_EHIP: return "HIP kernel launch failed";
    case GDN_ESCRATCH: return "larger than the built-in scratch buffer of the no-alloc entry point";
    default: return "unknown status";
  }
}

int gdn_beam_decode_step(const gdn_shape* shape, const gdn_store* store, int32_t t, int32_t W_t,
                         const int32_t* parent, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const float* alpha, const float* beta, float* o,
                         void* stream) {
  return gdn_beam_decode_step_timed(shape, store, t, W_t, parent, q, k, v, alpha, beta, o, stream, nullptr,
                                    nullptr);
}

int gdn_beam_decode_step_timed(const gdn_shape* shape, const gdn_store* store, int32_t t, int32_t W_t,
                               const int32_t* parent, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const float* alpha, const float* beta, float* o,
                               void* stream, void* ev_start, void* ev_stop) {
  int rc = check_shape(shape);
  if (rc != GDN_OK) return rc;
  if ((rc = check_store(store)) != GDN_OK) return rc;
  if (shape->decay_kind == GDN_DECAY_CHANNEL_PLAIN && shape->W_max != 1) return GDN_EUNSUPPORTED;
  if (t < 0 || t >= shape->L_max) return GDN_EINVAL;
  if (W_t < 1 || W_t > shape->W_max) return GDN_EINVAL;
  if (t > 0 && !aligned(parent, 4)) return GDN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(alpha, 16) ||
      !aligned(beta, 16) || !aligned(o, 16))
    return GDN_EINVAL;
  gdn::StepIO io{parent, q, k, v, alpha, beta, o};
  io.ev_start = static_cast<hipEvent_t>(ev_start);
  io.ev_stop = static_cast<hipEvent_t>(ev_stop);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
#ifdef GDN_CHECK_PARENTS
  io.bad_parents = bad_parents_on(s);
#endif
  // one beam per request takes the sequence kernel where it is built; the
  // wider geometries run it through the beam kernel (the same step at W = 1)
  if (shape->W_max == 1 && gdn::seq_dims_supported(shape->dk, shape->dv))
    return gdn::launch_seq_decode(*shape, *store, t, false, io, s);
  return gdn::launch_beam_decode(*shape, *store, t, W_t, io, s);
}

int gdn_decode_merge_step(const gdn_shape* shape, const gdn_store* store, int32_t t, const uint16_t* q,
                          const uint16_t* k, const uint16_t* v, const float* alpha, const float* beta,
                          float* o, void* stream) {
  int rc = check_shape(shape);
  if (rc != GDN_OK) return rc;
  if ((rc = check_store(store)) != GDN_OK) return rc;
  if (shape->W_max != 1 || !gdn::seq_dims_supported(shape->dk, shape->dv)) return GDN_EUNSUPPORTED;
  if (t < 0 || t >= shape->L_max) return GDN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(alpha, 16) ||
      !aligned(beta, 16) || !aligned(o, 16))
    return GDN_EINVAL;
  const gdn::StepIO io{nullptr, q, k, v, alpha, beta, o};
  return gdn::launch_seq_decode(*shape, *store, t, true, io, reinterpret_cast<hipStream_t>(stream));
}

size_t gdn_split_workspace_bytes(const gdn_shape* shape) {
  if (check_shape(shape) != GDN_OK) return 0;
  return gdn::seq_split_workspace_bytes(*shape);
}

int gdn_decode_step_split(const gdn_shape* shape, const gdn_store* store, int32_t t, int32_t n_split,
                          int32_t shared_prep, int32_t merge, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const float* alpha, const float* beta, float* o, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc != GDN_OK) return rc;
  if ((rc = check_store(store)) != GDN_OK) return rc;
  if (shape->W_max != 1 || !gdn::seq_split_supported(*shape, n_split)) return GDN_EUNSUPPORTED;
  if (t < 0 || t >= shape->L_max || (merge != 0 && merge != 1) || (shared_prep != 0 && shared_prep != 1))
    return GDN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(alpha, 16) ||
      !aligned(beta, 16) || !aligned(o, 16))
    return GDN_EINVAL;
  if (shared_prep && (!aligned(workspace, 16) || workspace_bytes < gdn::seq_split_workspace_bytes(*shape)))
    return GDN_EINVAL;
  const gdn::StepIO io{nullptr, q, k, v, alpha, beta, o};
  return gdn::launch_seq_split(*shape, *store, t, merge != 0, n_split, shared_prep != 0,
                               shared_prep ? static_cast<float*>(workspace) : nullptr, io,
                               reinterpret_cast<hipStream_t>(stream));
}

int gdn_materialize(const gdn_shape* shape, const gdn_store* store, int32_t t, const int32_t* rb,
                    int32_t n, float* S_out, void* stream) {
  int rc = check_shape(shape);
  if (rc != GDN_OK) return rc;
  if ((rc = check_store(store)) != GDN_OK) return rc;
  if (t < 0 || t >= shape->L_max || n < 0) return GDN_EINVAL;
  if (n == 0) return GDN_OK;
  if (!aligned(rb, 4) || !aligned(S_out, 16)) return GDN_EINVAL;
  return gdn::launch_fold(*shape, *store, t, rb, 0, n, store->S, S_out, true,
                          reinterpret_cast<hipStream_t>(stream));
}

int gdn_log_merge(const gdn_shape* shape, const gdn_store* store, int32_t n_rec, int32_t beam,
                  void* stream) {
  int rc = check_shape(shape);
  if (rc != GDN_OK) return rc;
  if ((rc = check_store(store)) != GDN_OK) return rc;
  if (n_rec < 1 || n_rec > shape->L_max) return GDN_EINVAL;
  if (beam < 0 || beam >= shape->W_max) return GDN_EINVAL;
  return gdn::launch_fold(*shape, *store, n_rec - 1, nullptr, beam, shape->R, store->S, store->S,
                          false, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

#ifdef GDN_CHECK_PARENTS
// Parent-check builds only (libgdnbeam_check.so): the number of parent
// pointers outside [0, W_max) that beam decode steps on this stream's GPU
// have met since the last call, which resets it.  Synchronises the stream.
// Returns a negative status if the counter cannot be read.
extern "C" int gdn_debug_bad_parents(void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int* p = bad_parents_on(s);
  if (p == nullptr) return GDN_EHIP;
  int n = 0;
  if (hipMemcpyAsync(&n, p, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess) return GDN_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return GDN_EHIP;
  const int zero = 0;
  if (hipMemcpyAsync(p, &zero, sizeof(int), hipMemcpyHostToDevice, s) != hipSuccess) return GDN_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return GDN_EHIP;
  return n;
}
#endif
