/*
 * pipe_ceiling.h -- context-only HBM ceilings (libpipeceil.so).
 *
 * Plain streaming kernels with no LDS ring, no barriers and no tiles: every
 * thread moves 16-byte vectors straight from global memory to registers and
 * (for the copy) back. They are timed beside the tile stream so that its
 * bandwidth can be read both against the chip's published HBM peak and
 * against what the same memory traffic reaches on the same device with the
 * simplest possible kernel. They are a measurement aid, not part of the tile
 * stream's interface (include/pipe_tile.h).
 *
 * Common rules:
 *   - Pointers are device pointers, 16-byte aligned; `bytes` is a positive
 *     multiple of 16. The caller owns all memory; nothing is allocated.
 *   - `grid` is the number of 256-thread workgroups (1 .. 65536); each walks
 *     the buffer with a grid-sized stride, so any grid covers all bytes.
 *   - Launches are asynchronous on `stream` (0 = the null stream).
 *   - Return 0 on success; 1 for a null pointer, 2 for a bad size or
 *     alignment, 3 for a bad grid or variant, 4 when the HIP launch or copy
 *     reports an error. Nothing is launched when validation fails.
 */
#ifndef PIPE_CEILING_H
#define PIPE_CEILING_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0:bytes) = src[0:bytes). `unroll` (1 or 4) is the number of 16-byte
 * vectors a thread loads before it stores them; `nt` (0/1) marks loads and
 * stores non-temporal. Buffers must not overlap. */
int ceil_copy(const void* src, void* dst, size_t bytes, int grid, int unroll, int nt,
              hipStream_t stream);

/* Reads src[0:bytes) and folds it with XOR into one word per thread; `sink`
 * (one uint32, device) is written only in the rare case that a thread's fold
 * equals a fixed constant, so the loads cannot be optimised away. `nt` as
 * above. */
int ceil_read(const void* src, unsigned* sink, size_t bytes, int grid, int nt,
              hipStream_t stream);

/* hipMemcpyAsync device to device of `bytes` (the runtime's own copy path). */
int ceil_memcpy(void* dst, const void* src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PIPE_CEILING_H */
