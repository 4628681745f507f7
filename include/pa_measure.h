/*
 * pa_measure.h -- calibration for the benchmark of libpa.so: a plain
 * streaming read of one device buffer.  Its rate is the practical HBM read
 * ceiling of the GPU, reported beside the published peak as context for the
 * decode kernels' bandwidth.  It is not part of the decode path and nothing
 * in the path calls it.
 */
#ifndef PA_MEASURE_H
#define PA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Words of the sink pa_measure_stream_read writes (one per workgroup). */
#define PA_MEASURE_SINK_WORDS 4096

/*
 * Read every byte of buf[0, bytes) once, in 16-byte loads through buffer
 * descriptors -- the access the decode kernels make to K/V tiles -- with the
 * non-temporal hint the decode kernels give tiles they read once
 * (nontemporal = 1) or the default cache policy (0).  The XOR of every
 * 32-bit word read is folded into sink: the XOR of sink's
 * PA_MEASURE_SINK_WORDS words equals the XOR of all 32-bit words of the
 * buffer, so a caller can check that nothing was skipped.
 *
 *   buf    device, 16-byte aligned, `bytes` a multiple of 16   (in)
 *   sink   device, PA_MEASURE_SINK_WORDS uint32                (out)
 *
 * Asynchronous on `stream`; allocates nothing.  Returns PA_OK, PA_ERR_NULL,
 * PA_ERR_ALIGN (buf or bytes not 16-byte aligned) or PA_ERR_LAUNCH.
 * bytes == 0 writes zeros to sink.
 */
int pa_measure_stream_read(const void *buf, size_t bytes, int nontemporal, uint32_t *sink,
                           void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_MEASURE_H */
