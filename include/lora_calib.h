/*
 * lora_calib.h -- a measurement aid beside the LoRA library (not an operation
 * of the method, and not used by any lora_* call).
 *
 * The decode kernel of lora.h reads each used adapter's A and B as separate
 * contiguous blocks (r x d_in and d_out x r elements) scattered over a large
 * resident pool: one work item reads A, then (after a workgroup barrier) B,
 * and reads and writes back one row of y.  lora_calib_gather_read reads blocks
 * of that shape in the same workgroup shape (256 threads, 16-byte loads,
 * eight in flight per lane) and does nothing else, so that its rate is the
 * practical HBM rate of that access pattern on the device it runs on: the
 * benchmark reports it next to the LoRA kernels' rates.
 */
#ifndef RANK_SGMV_BGMV_LORA_CALIB_H
#define RANK_SGMV_BGMV_LORA_CALIB_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "lora.h"

#ifdef __cplusplus
extern "C" {
#endif

/* n_groups workgroups; workgroup g reads blocks_per_group blocks of
 * block_bytes bytes each, one after another with a workgroup barrier between
 * them: block k of group g starts at byte offset off[g * blocks_per_group + k]
 * of `pool`.  With rmw != NULL the workgroup also reads rmw_bytes bytes at
 * rmw + g * rmw_bytes before its last block and writes the same bytes back
 * after it (the values are unchanged).  Each workgroup reserves lds_bytes of
 * LDS (0 .. 65536) that it does not use, which limits how many workgroups
 * share a compute unit (65536: two, as many as the decode kernel fits).  It
 * writes one 32-bit word,
 * sink[g] = the XOR of the 32-bit words of its blocks, so that no load can be
 * dropped.
 *   pool         device, read only; every block lies inside it
 *   off          device, n_groups * blocks_per_group byte offsets, each a multiple of 16
 *   block_bytes  a positive multiple of 32768 (256 threads x 8 loads x 16 bytes)
 *   rmw          device, n_groups * rmw_bytes bytes, or NULL
 *   rmw_bytes    4096, 8192, 12288 or 16384 (256 threads x 16 bytes, 1 to 4 times);
 *                ignored when rmw is NULL
 *   sink         device, n_groups words, written
 * Returns LORA_EINVAL for NULL pool, off or sink, or n_groups < 0;
 * LORA_ESHAPE for blocks_per_group < 1, a block size that is not a positive
 * multiple of 32768, (rmw given) an rmw_bytes other than those four, or an
 * lds_bytes outside 0 .. 65536; LORA_EHIP when the launch fails.  n_groups == 0 launches
 * nothing.  Asynchronous on `stream`. */
lora_status lora_calib_gather_read(const void *pool, const int64_t *off, int32_t n_groups, int32_t blocks_per_group,
                                   int32_t block_bytes, void *rmw, int32_t rmw_bytes, int32_t lds_bytes,
                                   uint32_t *sink, hipStream_t stream);

/* The traffic of the MFMA kernel's prefill tiles with none of their
 * arithmetic.  Workgroup t owns rows t*rows .. t*rows + rows - 1 of x and of y
 * (row stride row_bytes; 8192 for a 4096-wide bf16 layer).
 *   order 0, the MFMA kernel's stages: row_bytes / 512 shrink stages, each
 *     reading 512 bytes of every row of x and, with adapters, 32 KB of the
 *     tile's A; then row_bytes / 256 expand stages, each reading 256 bytes of
 *     every row of y and, with adapters, 16 KB of B, and writing those bytes
 *     of y back; a workgroup barrier in every stage.  Tile t reads adapter
 *     t % n_adapters: A of row_bytes / 512 * 32 KB bytes followed by B of
 *     row_bytes / 256 * 16 KB bytes (a rank-64 adapter of the layer: 512 KB
 *     each at row_bytes 8192).
 *   order 1, whole rows: each wave reads its rows of x one after another, 1 KB
 *     per load instruction, then reads and writes back its rows of y the same
 *     way; adapters are not read.
 * The values of y are unchanged.  sink[t] = the XOR of every 32-bit word the
 * tile read (x, y and adapter bytes).  lds_bytes as for lora_calib_gather_read.
 *   x, y       device, n_tiles * rows * row_bytes bytes each
 *   adapters   device, n_adapters * (row_bytes / 512 * 32768 + row_bytes / 256 * 16384)
 *              bytes, or NULL
 *   sink       device, n_tiles words, written
 * Returns LORA_EINVAL for NULL x, y or sink, n_tiles < 0, or adapters with
 * n_adapters < 1; LORA_ESHAPE for rows outside 1 .. 64, a row_bytes that is not
 * a multiple of 1024 in 1024 .. 65536, an order other than 0 or 1, or an
 * lds_bytes outside 0 .. 65536; LORA_EHIP when the launch fails.  n_tiles == 0
 * launches nothing.  Asynchronous on `stream`. */
lora_status lora_calib_tile_stream(const void *x, void *y, int32_t n_tiles, int32_t rows, int32_t row_bytes,
                                   const void *adapters, int32_t n_adapters, int32_t order, int32_t lds_bytes,
                                   uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RANK_SGMV_BGMV_LORA_CALIB_H */
