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
 *   - Pointers are device pointers, 16-byte aligned. The caller owns all
 *     memory; nothing is allocated.
 *   - ceil_copy / ceil_read: `bytes` is a positive multiple of 16; `grid` is
 *     the number of 256-thread workgroups (1 .. 65536), each walking the
 *     buffer with a grid-sized stride, so any grid covers all bytes.
 *   - Launches are asynchronous on `stream` (0 = the null stream).
 *   - Return 0 on success; 1 for a null pointer, 2 for a bad size or
 *     alignment, 3 for a bad grid or variant, 4 when the HIP launch or copy
 *     reports an error. Nothing is launched when validation fails.
 */
#ifndef PIPE_CEILING_H
#define PIPE_CEILING_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

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

/* Column-strip ceilings: the tile stream's access pattern with no LDS ring.
 * The region is `rows` x `width` bytes at a row pitch of `pitch` bytes (all
 * row-major, 16-byte aligned). It is cut into column strips `strip_bytes`
 * wide (128, 256 or 512) and into 16 KiB tiles of 16384 / strip_bytes rows;
 * `rows` must be a whole number of tiles and `width` of strips. Each strip is
 * walked by `split` workgroups of 512 threads, segment s taking tiles s,
 * s + split, ...; the grid, (width / strip_bytes) * split, must be a multiple
 * of 8 and at most 65536 (consecutive segments share an XCD). A wave moves
 * two 1 KiB pieces of a tile at a time (64 lanes x 16 bytes), non-temporally.
 * With 128-byte strips this is the access pattern of 128 x 64 fp16 tiles
 * streamed down column strips; with 512-byte strips, that of 32 x 256 tiles.
 * The region may span at most 2^40 bytes. */

/* dst <- src over the region (dst has the same pitch; buffers must not overlap). */
int ceil_strip_copy(const void* src, void* dst, int64_t rows, int64_t pitch, int64_t width,
                    int strip_bytes, int split, hipStream_t stream);

/* Reads the region and folds it per thread; `sink` (one uint32, device) as in
 * ceil_read. */
int ceil_strip_read(const void* src, unsigned* sink, int64_t rows, int64_t pitch, int64_t width,
                    int strip_bytes, int split, hipStream_t stream);

/* Writes the region: each 16-byte piece gets the words (row, byte column,
 * ~row, ~byte column) of its first byte, as uint32. */
int ceil_strip_write(void* dst, int64_t rows, int64_t pitch, int64_t width, int strip_bytes,
                     int split, hipStream_t stream);

/* LDS ceilings: one kind of LDS traffic at full rate, no other work. `grid`
 * workgroups (1 .. 65536) of 512 threads, each holding 64 KiB of LDS (two fit
 * on a CU); every wave issues 8 conflict-free instructions per iteration for
 * `iters` iterations (1 .. 2^20).
 *   op 0: ds_read_b128, 1 KiB per wave instruction;
 *   op 1: ds_read_b64_tr_b16, 512 B per wave instruction, with the address
 *         pattern of the GEMM's B operand (32 columns of 16 K-rows);
 *   op 2: global_load_lds_dwordx4, 1 KiB per wave instruction, from the first
 *         65 536 bytes of `src` (16-byte aligned; stays in L2);
 *   op 3: ds_write_b128, 1 KiB per wave instruction;
 *   op 4: waves 0-3 as op 2 while waves 4-7 as op 0 (the DMA writes and the
 *         fragment reads of the GEMM mainloop, side by side);
 *   op 5: waves 4-7 as op 0, waves 0-3 idle;
 *   op 6: waves 0-3 as op 2, waves 4-7 idle.
 * `fold` (grid * 512 uint32, device) receives each thread's fold of what it
 * read, so that no read is optimised away. `clocks` (4 * grid uint64, device)
 * receives, per workgroup, the shader-clock cycles and the 100 MHz real-time
 * ticks that wave 0 measured around its loop, then the same for wave 4.
 * `src` is ignored unless op is 2, 4 or 6. */
int ceil_lds(int op, const void* src, unsigned* fold, uint64_t* clocks, int grid, int iters,
             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PIPE_CEILING_H */
