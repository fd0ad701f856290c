/*
 * gdn_beam_check.h -- the parent-check build of the GDN large-beam decode
 * library (libgdnbeam_check.so: the same sources as libgdnbeam.so compiled
 * with GDN_CHECK_PARENTS, for debugging callers).
 *
 * gdn_beam_decode_step takes, at step t >= 1, a parent pointer per beam
 * (OneLA §3.3: the ancestry index h_t(b, t-1) = pi_t(b)); its precondition is
 * 0 <= parent < W_{t-1}.  Every build clamps a pointer into [0, W_max), so no
 * access leaves the store, and the result for that beam is then meaningless.
 * This build also counts, on the device, every parent pointer outside
 * [0, W_max) (once per (request, beam) and step; W_{t-1} is not an argument of
 * the step, so a pointer in [W_{t-1}, W_max) is not caught).  Everything else
 * is libgdnbeam.so's C ABI (gdn_beam.h), unchanged.
 */
#ifndef GDN_BEAM_CHECK_H
#define GDN_BEAM_CHECK_H

#include "gdn_beam.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The number of out-of-range parent pointers that decode steps on the GPU of
 * `stream` (a hipStream_t; NULL = the default stream) have met since the last
 * call, which resets the count to zero.  Synchronises the stream (the only
 * call of the library that does).  Returns GDN_EHIP if the counter cannot be
 * read.  One count per GPU: concurrent decode steps on one GPU add to it.
 */
int gdn_debug_bad_parents(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_BEAM_CHECK_H */
