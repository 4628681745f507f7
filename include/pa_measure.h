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

/*
 * Read tiles of two pools the way the decode kernels read K and V, with no
 * arithmetic: the practical ceiling of paged reads of those exact tiles.
 * Tile i is the tile_bytes bytes at byte offset tiles[i] * tile_bytes in
 * k_pool and the same in v_pool (with the cache layout of pa.h and
 * tile_bytes = block_size * head_dim * elem_bytes, tile (block b, KV head
 * g) is index b * num_kv_heads + g).  A fixed set of persistent wavefronts
 * (one per SIMD) takes equal contiguous shares of the list and keeps
 * several tiles' 16-byte loads in flight, with the non-temporal hint; the
 * XOR of every 32-bit word read is folded into sink as for
 * pa_measure_stream_read.
 *
 *   k_pool, v_pool  device, 16-byte aligned                        (in)
 *   tiles           device int32 [num_tiles], each >= 0 and inside
 *                   both pools (not checked on the device)         (in)
 *   tile_bytes      1024, 2048, 4096 or 8192
 *   sink            device, PA_MEASURE_SINK_WORDS uint32           (out)
 *
 * Asynchronous on `stream`; allocates nothing.  Returns PA_OK, PA_ERR_NULL,
 * PA_ERR_ALIGN, PA_ERR_UNSUPPORTED (tile_bytes), PA_ERR_SHAPE
 * (num_tiles < 1) or PA_ERR_LAUNCH.
 */
int pa_measure_tile_read(const void *k_pool, const void *v_pool, const int32_t *tiles,
                         int num_tiles, int tile_bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_MEASURE_H */
