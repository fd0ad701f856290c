// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_beam.h"

namespace gdn {

// Per-step inputs and output of a decode call (layouts as in gdn_beam.h).
struct StepIO {
  const int32_t* parent;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  float* o;
  // parent-check builds (GDN_CHECK_PARENTS) only: device counter of parent
  // pointers found outside [0, W_max); null otherwise
  int* bad_parents = nullptr;
  // timed calls only: events the runtime records as the step's first kernel
  // starts and as its last kernel completes; null otherwise
  hipEvent_t ev_start = nullptr;
  hipEvent_t ev_stop = nullptr;
};

// Launches a kernel as hipLaunchKernelGGL does; with either timing event
// set, through hipExtLaunchKernel, which records ev0 as the dispatch starts
// and ev1 as it completes (no event command of its own in the stream).
#define GDN_DISPATCH(ev0, ev1, kernel, grid, block, lds, stream, ...)                     \
  do {                                                                                   \
    if ((ev0) != nullptr || (ev1) != nullptr)                                            \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev0, ev1, 0, __VA_ARGS__); \
    else                                                                                 \
      hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                 \
  } while (0)

// (d_k, d_v) pairs built for a decay kind, and those of the sequence kernel
bool dims_supported(int dk, int dv, int decay_kind);
bool seq_dims_supported(int dk, int dv);

// Key heads of a shape (H_k == 0 means one per value head).
inline int key_heads(const gdn_shape& sh) { return sh.H_k > 0 ? sh.H_k : sh.H; }

// Beams sharing one state per request (W_max > 1).
int launch_beam_decode(const gdn_shape& sh, const gdn_store& st, int t, int Wt,
                       const StepIO& io, hipStream_t stream);

// Scalar-decay beams with (d_k, d_v) = (32, 32) or (64, 64), or d_k in
// {128, 256} x d_v in {128, 256, 512}, and chains of at most kFusedMaxSteps
// records: loader/consumer pipeline through LDS.
constexpr int kFusedMaxSteps = 6;
bool beam_fused_supported(const gdn_shape& sh, int t);
int launch_beam_fused(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io,
                      hipStream_t stream);

// Channel-decay beams with d_k = d_v = 64, or d_k = 128 and d_v in {128,
// 256, 512}, and chains of at most 6 records: the same pipeline with 8-beam
// tiles.
bool beam_fused_kda_supported(const gdn_shape& sh, int t);
int launch_beam_fused_kda(const gdn_shape& sh, const gdn_store& st, int t, int Wt, const StepIO& io,
                          hipStream_t stream);

// One beam per request (W_max == 1): bounded-log decoding of sequences.
// With `merge`, the step also folds log records 0..t into S and writes it.
int launch_seq_decode(const gdn_shape& sh, const gdn_store& st, int t, bool merge, const StepIO& io,
                      hipStream_t stream);

// The same step with d_v cut into n_split value tiles per (sequence, head),
// the replay preparation formed once into `prep` (shared_prep, a workspace
// of seq_split_workspace_bytes) or by every tile.
bool seq_split_supported(const gdn_shape& sh, int n_split);
size_t seq_split_workspace_bytes(const gdn_shape& sh);
int launch_seq_split(const gdn_shape& sh, const gdn_store& st, int t, bool merge, int n_split, bool shared_prep,
                     float* prep, const StepIO& io, hipStream_t stream);

// Fold chains of records onto dense states.  Item i is the (request, beam)
// pair rb[2i], rb[2i+1] (or (i, beam) when rb is NULL); its chain is the
// ancestors in anc row t and its own record at step t.  Reads the state of
// its request from `src` and writes either dst[i] (dst_per_item) or the
// request's own state in place.
int launch_fold(const gdn_shape& sh, const gdn_store& st, int t, const int32_t* rb, int beam,
                int n, const float* src, float* dst, bool dst_per_item, hipStream_t stream);

}  // namespace gdn
