/*
 * gdn_beam.h -- C ABI of the GDN large-beam decode library (libgdnbeam.so,
 * built for AMD gfx950 / MI355X).
 *
 * The method.  Gated DeltaNet keeps one recurrent state per head and updates
 * it once per token (OneLA, "Scaling Linear-Attention Decoding to Large Beams
 * in Generative Recommendation", §2.2).  For large-beam decoding every beam of
 * a request starts from one shared post-prefill state and diverges only
 * through a few decode steps (§2.4, §3.1).  So a beam is stored as
 *   - the request's shared state S0 (kept once), plus
 *   - an append-only chain of transition records r_t = (alpha_t, delta_t, k_t),
 *     delta_t = beta_t (v_t - alpha_t S_{t-1}^T k_t)              (§3.2),
 *   - found through an ancestry index h_t(b, j): the slot written at step j by
 *     the ancestor of beam b (§3.3).
 * Each decode step replays a beam's records on the two projections S^T q and
 * S^T k it needs, never rebuilding the state (§3.2 replay equations), and
 * appends the beam's new record (§3.4).  The same store, with one beam per
 * request, is the bounded log of DeltaLog ("Deferred Materialization of
 * Recurrent States for Linear Attention Decoding", Figure 4): a dense base
 * plus up to L_max records, folded back into the base by a merge.
 *
 * Orientation.  States are stored [d_k][d_v] (d_v contiguous), the transpose
 * of OneLA's d_v x d_k notation, so o_t = S_t^T q_t and
 *   S_t = alpha_t S_{t-1} + k_t delta_t^T.
 * With per-channel decay (the KDA row of DeltaLog Table 1) alpha_t is a d_k
 * vector scaling the rows of S_{t-1}.
 *
 * Conventions for every entry point.
 *   - All tensors are row-major and contiguous, in device memory, and owned
 *     by the caller.  The library never allocates, frees or synchronises.
 *   - "bf16" means raw bfloat16 bit patterns in uint16_t.
 *   - Tensors must be 16-byte aligned; int32 index arrays 4-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; execution errors surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued and a negative status is returned.
 *   - No global mutable state: calls on different stores or streams are
 *     independent.  Calls that write the same store must be stream-ordered.
 *     The one exception is gdn_decode_step_split_noalloc, whose built-in
 *     scratch buffer (one per GPU) all its calls on that GPU share.
 *   - Three environment variables, read at every beam-decode call, exist for
 *     tests and comparisons only: GDN_BEAM_CHUNK=n (a multiple of 16, at
 *     least 16) fixes the number of beams per workgroup, which only changes
 *     which lanes compute a beam, never a result; GDN_BEAM_PAIR=0 keeps the
 *     channel-decay kernel at one head per workgroup where it would take two
 *     (the same bits either way); GDN_BEAM_GENERIC=1 makes
 *     gdn_beam_decode_step use its general kernel for every shape, whose
 *     results differ from the fused kernels' by FP32 rounding only.
 */
#ifndef GDN_BEAM_H
#define GDN_BEAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_BEAM_ABI_VERSION 7

/* status codes */
#define GDN_OK 0
#define GDN_EINVAL (-1)       /* null/misaligned pointer, index or size out of range */
#define GDN_EUNSUPPORTED (-2) /* (d_k, d_v) pair or decay kind not built in */
#define GDN_EHIP (-3)         /* the HIP runtime rejected a kernel launch */
#define GDN_ESCRATCH (-4)     /* larger than the built-in scratch buffer (no-alloc entry point) */

/* decay kinds (and update rules) */
#define GDN_DECAY_SCALAR 0  /* GDN: one alpha per (beam, head, step)      */
#define GDN_DECAY_CHANNEL 1 /* KDA: one alpha per key channel (A = d_k)   */
/* RWKV6 row of DeltaLog Table 1: one alpha per key channel (A = d_k) and the
 * update pair (k_t, v_t), no delta correction: S_t = diag(a_t) S_{t-1} +
 * k_t v_t^T, so the record's update vector is delta_t = v_t and beta is
 * ignored (its pointer is still checked).  The store keeps these update
 * vectors as bf16 (the BF16/BF16 log of DeltaLog Table 3): an exact copy of
 * the bf16 input v_t.  Bounded-log (independent sequence, W_max == 1)
 * decoding, merge and materialisation only; gdn_beam_decode_step with
 * W_max > 1 returns GDN_EUNSUPPORTED. */
#define GDN_DECAY_CHANNEL_PLAIN 2

/* largest L_max (records per chain / log capacity) */
#define GDN_MAX_STEPS 16

/* Geometry of a store.  A = 1 for GDN_DECAY_SCALAR, A = dk otherwise.
 * Built-in (dk, dv): (16,16) (32,32) (64,64) (128,128) for every decay kind;
 * and the wider recurrent geometries of the OneLA §4.1 operator suite, dk in
 * {128, 256} x dv in {128, 256, 512}: GDN_DECAY_SCALAR for all six,
 * GDN_DECAY_CHANNEL with dk = 128.  Other pairs, and the wider pairs with
 * another decay kind, make every entry point return GDN_EUNSUPPORTED, as
 * does gdn_decode_merge_step for any non-square pair. */
typedef struct gdn_shape {
  int32_t R;          /* requests (W_max == 1: independent sequences)  >= 1 */
  int32_t W_max;      /* beam slots per step                            >= 1 */
  int32_t H;          /* (value) heads                                  >= 1 */
  int32_t dk;         /* key head dim                                        */
  int32_t dv;         /* value head dim                                      */
  int32_t L_max;      /* steps held (1 .. GDN_MAX_STEPS)                     */
  int32_t decay_kind; /* GDN_DECAY_SCALAR, _CHANNEL or _CHANNEL_PLAIN        */
  int32_t H_k;        /* key heads: 0 (= H) or a divisor of H.  With H_k < H,
                         value heads g*i .. g*i + g-1 (g = H / H_k) share key
                         head i (the OneLA §4.1 geometries, H_V a multiple of
                         H_K): q, k and the record keys have H_k heads, every
                         other array H                                       */
} gdn_shape;

/* The record / ancestry store (caller-allocated device memory). */
typedef struct gdn_store {
  float* S;          /* [R][H][dk][dv]  FP32 shared state (dense base)       */
  float* rec_delta;  /* [L_max][R][W_max][H][dv]  FP32 update vectors delta;
                        with GDN_DECAY_CHANNEL_PLAIN the same index layout
                        holds bf16 bit patterns (uint16_t, 2 dv bytes per
                        record and head), the bits of v_t                    */
  uint16_t* rec_k;   /* [L_max][R][W_max][H_k][dk]  bf16 keys (bit copies)   */
  float* rec_alpha;  /* [L_max][R][W_max][H][A]   FP32 decays                */
  int32_t* anc;      /* [L_max][R][W_max][L_max]  ancestry: anc[t][r][b][j] =
                        h_t(b, j), j < t: the record slot, at step j, of
                        beam b's ancestor there.  The last entry,
                        anc[t][r][b][L_max-1] (t >= 1), is the beam's order
                        key at step t: its position in the depth-first order
                        of the beam tree (when a request's beams are
                        decoded by one workgroup) or its index.  Other
                        entries j >= t are unused.                            */
} gdn_store;

/*
 * Record slots.  Step t stores the record of beam b of request r at slot
 * (t, r, s): with scalar decay and W_max > 1, s is the beam's order key
 * anc[t][r][b][L_max-1] for t >= 1 (a permutation of 0 .. W_t-1 over the
 * step's beams, so that later steps, which take beams in that order, gather
 * each step's records in increasing slot order) and b at t == 0; with
 * channel decay, and with W_max == 1, s = b.  The ancestry rows hold slots;
 * an ancestor's beam index at step j is the beam whose order key there is
 * that slot.
 */

/*
 * One decode step t for all R requests, W_t beams and H heads (OneLA §3.3,
 * §3.4; replay equations of §3.2).  In one kernel:
 *   1. ancestry: h_t(b, t-1) = the record slot of parent[r][b] at step t-1,
 *      h_t(b, j) = h_{t-1}(parent, j) for j < t-1, written to
 *      anc[t][r][b][0..t-1] with the beam's order key (skipped at t == 0);
 *   2. u_q = S[r]^T q and u_k = S[r]^T k for every beam (for channel decay
 *      the probes are (prod_{i<=t} a_i) * q and * k over the beam's chain);
 *   3. replay of the records at (j, h_t(b, j)), j < t, on u_q and u_k;
 *   4. delta_t = beta_t (v_t - alpha_t u_k), o_t = alpha_t u_q +
 *      delta_t (k_t . q_t) (channel decay: alpha_t sits in the probes);
 *   5. writes o (at the beam's index) and appends (alpha_t, delta_t, k_t)
 *      at the beam's record slot (see "Record slots").
 * Records of steps j < t are only read.
 *
 *   t       step index, 0 <= t < L_max; the chain of step t has t records
 *   W_t     beams at this step, 1 <= W_t <= W_max
 *   parent  int32 [R][W_t]: parent slot (in step t-1) of each beam; ignored
 *           (may be NULL) at t == 0.  Precondition: 0 <= parent < W_{t-1}.
 *           Out-of-range values are clamped into [0, W_max) so no access
 *           leaves the store, but the result is then meaningless.
 *   q, k    bf16 [R][W_t][H_k][dk];  v  bf16 [R][W_t][H][dv]
 *   alpha   FP32 [R][W_t][H][A];   beta FP32 [R][W_t][H]
 *   o       FP32 [R][W_t][H][dv] (output)
 * With W_max == 1 this is one token of DeltaLog-style decoding of R
 * independent sequences: S is the dense base and t is the current log length.
 */
int gdn_beam_decode_step(const gdn_shape* shape, const gdn_store* store, int32_t t,
                         int32_t W_t, const int32_t* parent, const uint16_t* q,
                         const uint16_t* k, const uint16_t* v, const float* alpha,
                         const float* beta, float* o, void* stream);

/*
 * gdn_beam_decode_step with its kernel time taken by the runtime, for
 * callers that measure the step (throughput against HBM bandwidth, profiles)
 * without adding event commands of their own around it.  ev_start and
 * ev_stop are HIP events (hipEvent_t) created by the caller on the stream's
 * device, either of them NULL: the runtime records ev_start when the step's
 * first kernel starts executing and ev_stop when its last kernel completes
 * (hipExtLaunchKernel), so hipEventElapsedTime(ev_start, ev_stop) is the
 * step's kernel time alone.  Everything else (arguments, results, errors)
 * is exactly gdn_beam_decode_step's; with both events NULL the two calls are
 * the same.
 */
int gdn_beam_decode_step_timed(const gdn_shape* shape, const gdn_store* store, int32_t t,
                               int32_t W_t, const int32_t* parent, const uint16_t* q,
                               const uint16_t* k, const uint16_t* v, const float* alpha,
                               const float* beta, float* o, void* stream, void* ev_start,
                               void* ev_stop);

/*
 * Bounded-log decoding with the merge in the same pass (DeltaLog Figure 4: the
 * logical state is written into the dense base when the log is full; Figure 5
 * caption: the merge path has the structure of the append decode and writes
 * back base tiles).  For independent sequences (W_max == 1 only): decode
 * token t exactly as gdn_beam_decode_step(shape, store, t, 1, NULL, ...) does,
 * appending its record at log slot t, then fold log records 0..t into S in
 * place, S <- alpha_j S + k_j delta_j^T in log order (channel decay:
 * diag(a_j) S + ...), from the base values the step has already read.  The
 * result equals that decode step followed by gdn_log_merge(shape, store,
 * t + 1, 0); the caller then restarts at t = 0.
 *   t        current log length, 0 <= t < L_max
 *   q, k     bf16 [R][1][H_k][dk];  v  bf16 [R][1][H][dv]
 *   alpha    FP32 [R][1][H][A];   beta FP32 [R][1][H]
 *   o        FP32 [R][1][H][dv] (output)
 * Returns GDN_EUNSUPPORTED when W_max != 1 or (dk, dv) is not one of the
 * square pairs.
 */
int gdn_decode_merge_step(const gdn_shape* shape, const gdn_store* store, int32_t t,
                          const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const float* alpha, const float* beta, float* o, void* stream);

/*
 * Split-replay bounded-log decoding (DeltaLog Figure 5 caption: an append
 * decode in three stages, shared replay preparation, parallel append decode
 * across value tiles, single-writer metadata commit, and a merge path of the
 * same structure that writes back base tiles; Figure 9: the split-replay
 * ablation).  For independent sequences (W_max == 1) with d_k = d_v = 128:
 * decode token t exactly as gdn_beam_decode_step (merge == 0) or
 * gdn_decode_merge_step (merge == 1) define it, with the d_v columns of each
 * (sequence, head) cut into n_split value tiles (1, 2 or 4) that run as
 * separate workgroups.  Every tile needs the same replay preparation: the
 * probes c * q_t and c * k_t (c the product of the chain's per-channel
 * decays, 1 for scalar decay) and the dot products k_j . (probe) of the
 * log's records.
 *   shared_prep == 1: a first kernel forms that preparation once per
 *     (sequence, head) into `workspace` and commits the record's key, decay
 *     and ancestry row; the tiles read it there.  workspace: device memory of
 *     at least gdn_split_workspace_bytes(shape) bytes, 16-byte aligned, owned
 *     by the caller, overwritten by the call (its contents are only scratch).
 *   shared_prep == 0: every tile forms the preparation itself; tile 0
 *     commits.  workspace is ignored (may be NULL).
 * Results (o, the appended record, the merged base) agree with the unsplit
 * entry points to FP32 rounding (the projections are summed over a
 * different number of row groups); the two arms give identical bits.
 *   n_split  1, 2 or 4;  shared_prep, merge  0 or 1
 *   t, q, k, v, alpha, beta, o  as for gdn_decode_merge_step
 * Returns GDN_EUNSUPPORTED unless W_max == 1 and d_k = d_v = 128 (any decay
 * kind), GDN_EINVAL for a workspace that is missing, misaligned or too
 * small (shared_prep == 1) and for the errors of the other entry points.
 * Calls that share a workspace must be stream-ordered.
 */
size_t gdn_split_workspace_bytes(const gdn_shape* shape); /* 0 for an invalid shape */
int gdn_decode_step_split(const gdn_shape* shape, const gdn_store* store, int32_t t, int32_t n_split,
                          int32_t shared_prep, int32_t merge, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const float* alpha, const float* beta, float* o,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_decode_step_split without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving
 * loops that must not allocate, harnesses that forbid it.  The
 * shared-preparation arm keeps its workspace in a buffer built into the
 * library, one per GPU, GDN_SPLIT_SCRATCH_BYTES long and held until the
 * process ends; its device address is looked up (not allocated) once per
 * device, at the first call on that device.  Nothing is allocated or freed.
 *   Arguments, results and errors as gdn_decode_step_split; in addition
 *   GDN_ESCRATCH when shared_prep == 1 and gdn_split_workspace_bytes(shape)
 *   exceeds GDN_SPLIT_SCRATCH_BYTES (8 MiB: 7,182 (sequence, head) pairs at
 *   d_k = 128), GDN_EHIP when the buffer's address cannot be found.
 * Every call on one GPU shares that buffer and the buffer keeps the last
 * call's contents (each call writes every entry it reads before reading
 * it, so nothing needs to start at zero): calls that overlap on one GPU
 * (other streams, or host threads without ordering) race and must not be
 * issued; stream-order them.
 */
#define GDN_SPLIT_SCRATCH_BYTES (8u << 20)
int gdn_decode_step_split_noalloc(const gdn_shape* shape, const gdn_store* store, int32_t t, int32_t n_split,
                                  int32_t shared_prep, int32_t merge, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const float* alpha, const float* beta, float* o,
                                  void* stream);

/*
 * Dense states after step t of n beams (the conceptual S_{t,b} of OneLA §3.1,
 * which decoding itself never forms): S[r] folded with the beam's ancestral
 * records and its own step-t record, S <- alpha_j S + k_j delta_j^T in chain
 * order (channel decay: S <- diag(a_j) S + k_j delta_j^T).
 *   t      0 <= t < L_max (anc row t must have been written by step t)
 *   rb     int32 [n][2] device array of (request, beam) pairs, beam < W_t
 *   n      >= 0 (0: nothing is enqueued)
 *   S_out  FP32 [n][H][dk][dv] (output; must not overlap the store)
 */
int gdn_materialize(const gdn_shape* shape, const gdn_store* store, int32_t t,
                    const int32_t* rb, int32_t n, float* S_out, void* stream);

/*
 * Bounded-log merge (DeltaLog Figure 4 and Figure 5 caption): fold, for every
 * request r, the first n_rec records of beam `beam`'s chain (its ancestors at
 * steps 0..n_rec-2 and its own record at step n_rec-1) into S[r] in place.
 * The caller then restarts decoding at t = 0 on the new base.
 *   n_rec  1 <= n_rec <= L_max
 *   beam   0 <= beam < W_max (0 for independent sequences)
 */
int gdn_log_merge(const gdn_shape* shape, const gdn_store* store, int32_t n_rec,
                  int32_t beam, void* stream);

/* Static description of a status code (never NULL). */
const char* gdn_status_string(int status);

/* GDN_BEAM_ABI_VERSION of the built library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_BEAM_H */
