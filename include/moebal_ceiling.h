/*
 * moebal_ceiling.h — reference kernels that bound libmoebal's dispatch on
 * the GPU it runs on (libmoebal_ceiling.so, a measurement library beside
 * libmoebal.so; nothing in libmoebal calls it).
 *
 * The dispatch of MoonEP ("What MoonEP enforces and how": token rows written
 * straight into fixed-shape expert-grouped buffers) reads each token row
 * once and writes it to K rows of the dispatch buffer at the rows the plan's
 * pos gives. These kernels take that traffic apart: a contiguous fill and
 * copy of the same byte count (what HBM streams), a contiguous read (the
 * read side alone), and the dispatch's own writes with no reads — the same
 * pos, the same rows, the same 16-byte lane stores, in the two shapes of
 * libmoebal's dispatch kernels: one wave per 1 KiB of a row (k_dispatch),
 * or a workgroup of K waves per 2 KiB span, one destination row per wave
 * (k_dispatch_span). Comparing the dispatch with them says how much of its
 * time the scattered writes alone cost. For the combine (K expert-output
 * rows gathered per token, weighted and summed, one row written) one kernel
 * moves the same bytes in k_combine's shape with an XOR in place of the
 * fp32 arithmetic.
 *
 * All entry points enqueue one kernel on `stream` and return 0, or -1 for
 * invalid arguments (nothing enqueued), or the HIP error code of the launch.
 * Pointers are device memory, 16-byte aligned; byte counts and row bytes are
 * multiples of 16. Kernels never read or write outside the sizes given.
 */
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Write `bytes` bytes at dst contiguously, one 16-byte store per lane. */
int mbc_fill(void* dst, int64_t bytes, hipStream_t stream);

/* Copy `bytes` bytes from src to dst contiguously, 16 bytes per lane. */
int mbc_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* Read `bytes` bytes at src contiguously, 16 bytes per lane; a lane writes
 * its value to sink (16 bytes) only if it equals `key` in all four words,
 * so the loads cannot be dropped and, for keys absent from src, nothing is
 * stored. */
int mbc_read(const void* src, int64_t bytes, const uint32_t key[4], void* sink,
             hipStream_t stream);

/* The writes of the dispatch alone: for token t < n_tokens and k < top_k,
 * row pos[t * top_k + k] of buf (row_bytes each, `rows` rows; entries outside
 * [0, rows) are skipped) receives 16 bytes per lane from registers, in
 * k_dispatch's layout: one wave per 1 KiB of a row, four waves per
 * workgroup, the wave's K stores one after another. top_k in [1, 32]. */
int mbc_scatter_write(const int32_t* pos, void* buf, int32_t n_tokens, int32_t top_k,
                      int32_t row_bytes, int32_t rows, hipStream_t stream);

/* The same writes in k_dispatch_span's shape, one destination row per wave:
 * a workgroup of top_k waves covers 2 KiB of one token's row, wave k writing
 * that span of row pos[t * top_k + k] contiguously. top_k in [1, 16]. */
int mbc_row_write(const int32_t* pos, void* buf, int32_t n_tokens, int32_t top_k,
                  int32_t row_bytes, int32_t rows, hipStream_t stream);

/* The combine's traffic alone: for token t < n_tokens, y row t (row_bytes)
 * = XOR over k < top_k of y_exp row pos[t * top_k + k] (rows of row_bytes,
 * `rows` rows; entries outside [0, rows) are skipped), in k_combine's shape:
 * one wave per 512 bytes of an output row (8-byte lane chunks), 16 waves per
 * workgroup, a lane's top_k loads issued before their use, loads and stores
 * nontemporal. top_k in [1, 32]. */
int mbc_gather_xor(const int32_t* pos, const void* y_exp, void* y, int32_t n_tokens,
                   int32_t top_k, int32_t row_bytes, int32_t rows, hipStream_t stream);

#ifdef __cplusplus
}
#endif
