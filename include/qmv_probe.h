/*
 * qmv_probe.h -- measurement aid exported by libqmv.so (not part of the GEMV).
 *
 * A GEMV call of this library is bounded by HBM: it must read every code and
 * scale byte of the experts it selects once.  To relate its time to what the
 * memory system delivers for the same transfer (same sizes, same number of
 * separate regions, same 16-byte non-temporal buffer loads), this probe only
 * reads the given regions, with no decode and no dependence on expert ids.
 * Its time per call is the practical read ceiling that a benchmark divides
 * the GEMV's time by.  A clock stamp (qmv_probe_clock) lets a benchmark time
 * launches on the GPU's own clock.
 */
#ifndef QMV_PROBE_H
#define QMV_PROBE_H

#include <hip/hip_runtime_api.h>

#include "qmv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Most regions one call may read. */
#define QMV_PROBE_MAX_REGIONS 64
/* Launch shapes (threads per workgroup, 16-byte loads in flight per lane). */
#define QMV_PROBE_VARIANTS 6

/*
 * Read n_regions device regions once each: region r starts at ptrs[r]
 * (16-byte aligned) and holds bytes[r] bytes (1 <= bytes[r] < 2^31; a tail
 * that is not a multiple of 16 is read as zeros past the end).  ptrs and
 * bytes are HOST arrays of n_regions entries (1 <= n_regions <=
 * QMV_PROBE_MAX_REGIONS); their values are copied into the launch, so the
 * arrays may be reused as soon as the call returns.  variant selects the
 * launch shape, 0 <= variant < QMV_PROBE_VARIANTS.  sink is a 4-byte aligned
 * device word that the kernel writes only when the XOR of everything it read
 * equals a fixed constant (so the loads cannot be optimized away); the caller
 * owns it.  Enqueues one kernel on `stream`; returns QMV_EINVAL for a null
 * or misaligned pointer or a size out of range, QMV_EUNSUPPORTED for a bad
 * variant or region count, QMV_EHIP if the launch is refused.
 */
qmv_status_t qmv_probe_stream_read(int n_regions, const void *const *ptrs,
                                   const long long *bytes, int variant, unsigned *sink,
                                   hipStream_t stream);

/*
 * Enqueue one single-thread kernel on `stream` that stores the GPU's
 * real-time counter (a constant 100 MHz clock, independent of the shader
 * clock) to *out, a device word (8-byte aligned) the caller owns.  Two stamps
 * around a sequence of launches in a HIP graph time that sequence on the GPU
 * itself, without the graph launch's own start-up.  Returns QMV_EINVAL for a
 * null or misaligned pointer, QMV_EHIP if the launch is refused.
 */
qmv_status_t qmv_probe_clock(unsigned long long *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_PROBE_H */
