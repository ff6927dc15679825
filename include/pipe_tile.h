/*
 * pipe_tile -- a pipelined tile stream for AMD MI355X (gfx950).
 *
 * One hot path: a producer wavefront streams 2D tiles from HBM into a ring of
 * S swizzled LDS slots; every slot carries a full/empty handshake with phase
 * parity; consumer wavefronts wait on a slot, use the tile, and release it.
 * Three uses are exported: copy the tile back out, reduce it into fp32 row
 * sums, and feed a bf16 matrix-multiply mainloop.
 *
 * Sources (pages, by title and section):
 *   "cute（12）async_pipeline" -- the ring of stages, full/empty barrier pair
 *       per stage, PipelineState cursor, producer start phase 1, producer /
 *       consumer API (sections 1-3, 6, 7), Params (section 4);
 *   "cute（11）hopper之TMA_copy" -- one 128x64 fp16 tile round trip
 *       global -> swizzled shared memory -> global (code, sections 1-4);
 *   "cuda-features-10-pipelines" 4.10 -- acquire / commit / wait / release,
 *       stage-count trade-offs (4.10.7), 16-byte alignment advice (4.10.6);
 *   "chapter_async_barriers" (mlc.ai) -- mbarrier phase semantics.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major: element (r, c) of an M x N matrix with leading
 *     dimension ld (in elements) is at base + r*ld + c.
 *   - All data pointers are DEVICE pointers owned by the caller. The library
 *     never allocates or frees memory, never synchronises the stream and keeps
 *     no per-call host state; it is safe to call from several host threads.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls are
 *     asynchronous: results are visible after the caller synchronises.
 *   - Calls that use the library's own device memory -- its status word (when
 *     cfg->status is NULL) or pipe_rowsum_noalloc's buffer -- look it up on the
 *     current device, so a non-NULL `stream` must belong to that device (else
 *     PIPE_ERR_CONFIG, nothing enqueued).
 *   - Arguments are validated before anything is launched; on any error no
 *     work is enqueued and the error code is returned.
 *   - A stalled handshake never hangs the device: each wait gives up after
 *     cfg->spin_limit polls and sets a bit in the status word (cfg->status, or
 *     the library's own word read back by pipe_device_status()).
 */
#ifndef PIPE_TILE_H
#define PIPE_TILE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PIPE_ABI_VERSION 1

typedef enum {
  PIPE_OK = 0,
  PIPE_ERR_NULL = 1,      /* a required pointer is NULL */
  PIPE_ERR_SHAPE = 2,     /* negative size, ld < width, a matrix spanning 2^62 bytes or more,
                             or a shape the op does not support */
  PIPE_ERR_ALIGN = 3,     /* base pointer or row pitch not 16-byte aligned */
  PIPE_ERR_STAGES = 4,    /* stage count out of range or the ring does not fit in LDS */
  PIPE_ERR_CONFIG = 5,    /* unsupported tile shape, wave counts, grid, split or flags */
  PIPE_ERR_WORKSPACE = 6, /* workspace missing or smaller than required */
  PIPE_ERR_HIP = 7,       /* the HIP runtime reported an error at launch */
  PIPE_ERR_TIMEOUT = 8,   /* (device status) a pipeline wait exceeded spin_limit */
  PIPE_ERR_INVARIANT = 9  /* (device status) a check of PIPE_FLAG_DEBUG_CHECKS failed */
} pipe_status_t;

/* The two sentinels give the type the range of int32, so that any int a
 * caller passes is a value of it (and is rejected with PIPE_ERR_CONFIG when it
 * names no op). */
typedef enum {
  PIPE_OP_COPY = 0,
  PIPE_OP_ROWSUM = 1,
  PIPE_OP_GEMM = 2,
  PIPE_OP_RANGE_MIN_ = -0x7fffffff - 1,
  PIPE_OP_RANGE_MAX_ = 0x7fffffff
} pipe_op_t;

/* cfg->flags */
#define PIPE_FLAG_TRACE 0x1u           /* record per-tile cursor values into cfg->trace (copy,
                                          rowsum, and gemm with fp32 C and row-major B; else
                                          PIPE_ERR_CONFIG for the gemm) */
#define PIPE_FLAG_ROW_STRIPS 0x2u      /* copy: walk tiles along rows instead of down columns */
#define PIPE_FLAG_NONTEMPORAL 0x4u     /* copy/rowsum: non-temporal hint on streamed loads/stores */
#define PIPE_FLAG_GEMM_B_LINEAR 0x8u   /* gemm: store B K-rows in LDS without the XOR swizzle */
#define PIPE_FLAG_XCD_REMAP 0x10u      /* copy/rowsum: give each XCD neighbouring strips (when the
                                          item count is a multiple of 8) */
#define PIPE_FLAG_SPLIT_INTERLEAVE 0x20u /* copy/rowsum: segment s of a strip takes every split-th
                                            tile from s on, instead of a contiguous run */
#define PIPE_FLAG_UNIFIED 0x40u        /* copy/rowsum: the unified (non-specialised) pipeline --
                                          consumer_waves waves (2, 4 or 8) each load and use their
                                          share of every tile, with per-wave batch waits and no
                                          full/empty barriers; M % 128 == N % 64 == 0 only, no
                                          checksums or trace (else PIPE_ERR_CONFIG).
                                          gemm: 256 x 256 output tiles (tile_m = tile_n = 256,
                                          no trace) whose waves all load a share of each
                                          stage and compute, with one workgroup barrier per K
                                          step; producer_waves and the commit policy do not
                                          apply. consumer_waves = 16 (64 x 64 output blocks):
                                          tile_k 64, stages 2. consumer_waves = 4 (128 x 128
                                          blocks, one wave per SIMD): tile_k 64 with stages 2, or
                                          tile_k 32 with stages 3..5 (the fastest GEMM here; its
                                          64-byte LDS rows take a fixed chunk XOR and ignore
                                          swizzle_shift; it alone also takes GEMM_C_BF16, written
                                          straight from registers). Else PIPE_ERR_CONFIG /
                                          PIPE_ERR_STAGES */
#define PIPE_FLAG_LAZY_COMMIT 0x80u    /* copy/rowsum/gemm (specialised ring): the producer commits
                                          a tile only once `lag` younger tiles are in flight, never
                                          while its acquire waits for a slot. Without this flag a
                                          producer whose acquire waits commits its oldest tile in
                                          flight (after it landed) while it has 2 or more in flight */
#define PIPE_FLAG_EAGER_NEWEST 0x400u  /* as above, but the waiting producer also commits its newest
                                          tile in flight (waits for it to land); exclusive with
                                          PIPE_FLAG_LAZY_COMMIT (else PIPE_ERR_CONFIG) */
#define PIPE_FLAG_GEMM_C_BF16 0x800u   /* gemm: C is bf16, rounded to nearest even and written
                                          through LDS staging by the MFMA waves themselves */
#define PIPE_FLAG_GEMM_STORE_WAVE 0x1000u /* gemm with bf16 C: stage through a one-slot ring per
                                             MFMA wave pair that a dedicated store wave drains
                                             (full/empty handshake); requires GEMM_C_BF16 */
#define PIPE_FLAG_GEMM_B_COLMAJOR 0x2000u /* gemm: B is column-major, element (k, n) at
                                             B[n * ldb + k] with ldb >= K; its tiles are
                                             loaded and read like A's (no transposing LDS
                                             read); exclusive with GEMM_B_LINEAR */
#define PIPE_FLAG_STRIP_GROUPS 0x4000u /* copy down column strips of 128 x 64 tiles: a strip
                                          spans G neighbouring tile columns and is walked one
                                          tile row at a time; consumers wait on the G slots of
                                          a tile row and store it as G*128-byte row runs. G = 4,
                                          else 2, where M % 128 == 0, N % 64 == 0, the
                                          tile-column count is a multiple of G, G <= stages,
                                          consumer_waves is 4 or 8, producer_waves 2 or 4, and
                                          no checksums, row strips or unified ring are asked
                                          for; elsewhere the flag changes nothing. The commit
                                          lag is then at most stages - G, and split 0 means G
                                          segments per strip (one work item per tile column) */
#define PIPE_FLAG_PRODUCER_VGPR 0x8000u /* copy/rowsum, 128 x 64 tiles: the producers load with
                                          global_load_dwordx4 into registers and write each
                                          slot with ds_write_b128 at the swizzled positions
                                          (instead of direct-to-LDS loads), loading up to 3
                                          tiles ahead (1 with one producer wave); a tile is
                                          committed once its writes have returned, so the
                                          commit policies do not apply. Rings: stages 1..4,
                                          consumer_waves 3 or 4, producer_waves 1 or 4; not
                                          with UNIFIED or DEBUG_CHECKS (else PIPE_ERR_CONFIG);
                                          STRIP_GROUPS is then ignored */
#define PIPE_FLAG_DEBUG_CHECKS 0x10000u /* copy/rowsum, 128 x 64 tiles: run the ring with its
                                          protocol checks compiled in. When a wait passes, the
                                          barrier word must hold exactly the completed phases
                                          the protocol allows and the cursor its closed form;
                                          a consumer's slot must not be committed again before
                                          it releases it. A failed check sets
                                          PIPE_STATUS_INVARIANT; the kernel carries on. Rings:
                                          stages 1..4 with 1 producer + 3 consumer waves or
                                          4 + 4; not with UNIFIED or PRODUCER_VGPR (else
                                          PIPE_ERR_CONFIG); STRIP_GROUPS is then ignored */
#define PIPE_FLAG_TEST_JITTER 0x20000u  /* test only, with DEBUG_CHECKS (else PIPE_ERR_CONFIG):
                                          every wave pauses a pseudo-random 0..15 short sleeps
                                          before each wait, to shake the waves' timing */
#define PIPE_FLAG_TEST_EARLY_RELEASE 0x40000u /* test only, with DEBUG_CHECKS (else
                                          PIPE_ERR_CONFIG): consumers release each slot before
                                          reading it and then pause, so the producer refills
                                          it under them; the checks must report it */
#define PIPE_FLAG_GROUP_LOADS 0x80000u /* copy, with STRIP_GROUPS, stages 4 or 8, producer_waves
                                          2 or 4, consumer_waves 4 or 8 (else PIPE_ERR_CONFIG):
                                          where the strips are 4 tile columns wide, the producers
                                          also fill the 4 slots of a tile row together, with loads
                                          of 2 rows x 512 contiguous bytes, and commit the 4 tiles
                                          together (lag stages - 4). The 4 slots of a group are
                                          then interleaved in LDS (row r of tile g at
                                          r * 512 + g * 128 from the group's first slot). Where
                                          the strips resolve to 2 or 1 tile columns the flag
                                          changes nothing */
#define PIPE_FLAG_TEST_START_PHASE0 0x100u /* test only: producer starts at phase 0 (the
                                              deadlock of the pages); must end in a timeout */
#define PIPE_FLAG_TEST_NO_RELEASE 0x200u   /* test only: consumers never release; the
                                              producer's first wait of lap 2 times out */

/* Status-word bits (cfg->status or pipe_device_status). */
#define PIPE_STATUS_TIMEOUT_PRODUCER 0x1u
#define PIPE_STATUS_TIMEOUT_CONSUMER 0x2u
#define PIPE_STATUS_INVARIANT 0x4u        /* a check of PIPE_FLAG_DEBUG_CHECKS failed */

/* One trace record: 8 uint32 words. Written only by workgroup 0, for the first
 * cfg->trace_capacity / 2 tiles of its stream, at record index 2*t + event.
 *   [0] event (0 = producer acquired the slot, 1 = consumer wave 0 passed its wait)
 *   [1] tile ordinal t in the workgroup's stream
 *   [2] cursor index   [3] cursor phase   [4] cursor count
 *   [5] wave id        [6] s_memrealtime low   [7] s_memrealtime high          */
#define PIPE_TRACE_WORDS 8

typedef struct {
  int32_t stages;         /* S, ring depth: copy/rowsum 1..8 (5..8 need 4 or 8 consumer
                             waves; the ring must fit 160 KiB of LDS); gemm 1..4 (unified:
                             see PIPE_FLAG_UNIFIED)                                       */
  int32_t tile_m;         /* copy/rowsum: 128, 64 or 32 (with tile_n 64, 128, 256: every
                             tile is 16 KiB; the wider two need S 2..4, producer_waves
                             2 or 4, consumer_waves 4 or 8 -- unified: 2 or 4); gemm 128,
                             or 256 with 8 consumer and 4 producer waves (S 1..3, S 1..2
                             with bf16 C; no store wave, no trace)                        */
  int32_t tile_n;         /* copy/rowsum: 64, 128 or 256 fp16 (see tile_m); gemm: 128,   
                             or 256 with PIPE_FLAG_UNIFIED                               */
  int32_t tile_k;         /* gemm only: 64, or 32 for the 4-wave unified GEMM             */
  int32_t producer_waves; /* copy/rowsum: 1, 2 or 4; gemm: 2 or 4 (each tile's loads split
                             evenly; a wave keeps up to 2, 6 or 14 tiles of commit lag)   */
  int32_t consumer_waves; /* copy/rowsum: 1, 2, 3, 4 or 8 (unified: 2, 4 or 8); gemm:
                             tile_m / 32 (4 or 8 MFMA waves, each a 64 x 64 output block);
                             unified gemm: 16 or 4                                        */
  int32_t grid;           /* workgroups; 0 = one per work item (capped by the device)     */
  int32_t split;          /* copy/rowsum: segments each strip is cut into; 0 = default:
                             copy 1 (G with PIPE_FLAG_STRIP_GROUPS), rowsum the smallest
                             power of two giving >= 256 work items                      */
  int32_t swizzle_shift;  /* row bits XOR-ed into the 16-byte chunk index: 0..3           */
  uint32_t flags;         /* PIPE_FLAG_*                                                  */
  uint32_t spin_limit;    /* polls per wait before giving up; 0 = default (1 << 22)       */
  int32_t trace_capacity; /* records available at trace                                   */
  uint32_t* trace;        /* device, nullable; used with PIPE_FLAG_TRACE                  */
  uint32_t* status;       /* device, nullable; OR-ed with PIPE_STATUS_* bits              */
} pipe_config_t;

typedef struct {
  int32_t lds_bytes;      /* LDS per workgroup (ring + barrier words)                    */
  int32_t threads;        /* threads per workgroup                                        */
  int32_t grid;           /* workgroups that would be launched                            */
  int32_t items;          /* strips x segments (copy/rowsum) or output tiles (gemm)       */
  int32_t tiles_per_item; /* tiles streamed through the ring per work item (max)          */
  int32_t split;          /* segments per strip actually used                             */
} pipe_kernel_info_t;

typedef struct {
  int32_t vgprs;          /* vector registers per lane, as the HIP runtime reports them
                             (numRegs; no kernel of this library uses AGPRs)              */
  int32_t lds_bytes;      /* static LDS per workgroup                                     */
  int32_t scratch_bytes;  /* private memory per lane (register spills); 0 when none       */
  int32_t max_threads;    /* largest workgroup the kernel can be launched with            */
} pipe_kernel_resources_t;

/* ABI version of the loaded library (PIPE_ABI_VERSION). Part of this
 * library's own interface, not an operation of the pages. */
int pipe_abi_version(void);

/* Static, human-readable name of a status code (never NULL; unknown codes
 * get a fixed string). Part of this library's own interface, not an operation
 * of the pages. */
const char* pipe_status_str(int status);

/* Fill *cfg with the defaults of an op (the pipeline parameters of
 * "cute（12）async_pipeline" section 4 -- stage count, producer and consumer
 * counts -- plus this library's tile, flag and launch choices; grid and split
 * automatic):
 *   copy:   stages 2, tile 128x64, 4 producer + 4 consumer waves,
 *           flags NONTEMPORAL | XCD_REMAP | LAZY_COMMIT, swizzle shift 0;
 *   rowsum: stages 3, tile 128x64, 4 producer + 4 consumer waves,
 *           flags NONTEMPORAL | XCD_REMAP (eager commits), swizzle shift 0;
 *   gemm:   stages 2, tile 128x128x64, 4 producer + 4 consumer waves,
 *           flags EAGER_NEWEST, swizzle shift 1. */
pipe_status_t pipe_config_default(pipe_op_t op, pipe_config_t* cfg);

/* Tile copy (configs: "cute（11）hopper之TMA_copy" round trip; "cute（12）
 * async_pipeline" ring).  dst[r][c] = src[r][c] bit for bit for r < M, c < N;
 * the 16-bit payload is opaque (fp16, bf16, raw codes). Each tile passes
 * through a swizzled LDS slot.
 *   src, dst: device, 16-byte aligned; ld_src, ld_dst: row pitch in elements,
 *   multiples of 8, >= N. N must be a multiple of 8 (16-byte chunks; else
 *   PIPE_ERR_SHAPE); M is arbitrary: the last tile row / column may be partial.
 *   M == 0 or N == 0 is a no-op.
 *   tile_checksums: device, nullable; if given, receives for every tile
 *   (i, j) of the ceil(M/128) x ceil(N/64) grid, in row-major tile order, the
 *   uint32 sum of the raw 16-bit codes of the tile's in-range elements. */
pipe_status_t pipe_tile_copy(const void* src, void* dst, int64_t M, int64_t N,
                             int64_t ld_src, int64_t ld_dst, const pipe_config_t* cfg,
                             uint32_t* tile_checksums, void* stream);

/* Bytes of workspace pipe_rowsum needs for this shape and config (0 when each
 * row strip is one segment): split x M fp32 segment partials, then, from the
 * next 256-byte boundary, one uint32 arrival ticket per row strip. A
 * diagnostic of this library's decomposition, not an operation of the pages. */
pipe_status_t pipe_rowsum_workspace_bytes(int64_t M, int64_t N, const pipe_config_t* cfg,
                                          size_t* bytes);

/* Row sums of an fp16 matrix with fp32 accumulation: out[r] = sum_c A[r][c]
 * ("cute（12）async_pipeline" 3.2: the consumer's use of each tile, here a
 * reduction; the pages leave the use open, the strip decomposition below is
 * this library's).
 * Row strips of tile_m rows are cut into cfg->split segments along the
 * columns. With more than one segment, each segment's fp32 partials go to the
 * workspace and every consumer wave counts an arrival on its strip's ticket;
 * the wave that arrives last adds the strip's partials in segment order
 * 0, 1, ..., split - 1 and writes out, inside the same kernel. The order is
 * fixed, so the result does not depend on timing and equals a plain
 * fixed-order sum of the partials. The call enqueues a small fill kernel that
 * zeroes the tickets and then the stream kernel, so the workspace may hold
 * anything on entry; two calls that share a workspace must not overlap (use
 * one stream, or one workspace per stream).
 *   A: device fp16, 16-byte aligned, lda multiple of 8 and >= N;
 *   N a multiple of 8, M arbitrary (partial edge tiles are masked);
 *   N == 0 gives out = 0; M == 0 is a no-op.
 *   out: device float[M]. workspace: device, 4-byte aligned,
 *   >= pipe_rowsum_workspace_bytes (else PIPE_ERR_WORKSPACE / PIPE_ERR_ALIGN). */
pipe_status_t pipe_rowsum(const void* A, float* out, int64_t M, int64_t N, int64_t lda,
                          const pipe_config_t* cfg, void* workspace, size_t workspace_bytes,
                          void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: pipe_rowsum
 * with its workspace in a buffer the library owns (PIPE_ROWSUM_SCRATCH_BYTES of
 * static device memory on each device it runs on, held until the process
 * ends) instead of a caller's. Same kernels and bit-identical results as
 * pipe_rowsum; the caller still passes A and out. It allocates nothing, with
 * no allocating runtime call: the buffer's device address is looked up once
 * per device (hipGetSymbolAddress) on the first call there; make that first
 * call outside stream capture, and later calls may be captured and replayed
 * (the captured launches keep the buffer's address). A shape whose
 * pipe_rowsum_workspace_bytes exceeds PIPE_ROWSUM_SCRATCH_BYTES returns
 * PIPE_ERR_WORKSPACE before anything is enqueued (a smaller cfg->split needs
 * less). Every call on one device shares that device's buffer and finds the
 * previous call's contents there; each call zeroes what must start at zero
 * (the strip tickets) itself. Calls that overlap on one device -- on two
 * streams, or from two host threads -- race on the buffer: serialise them. */
#define PIPE_ROWSUM_SCRATCH_BYTES (1u << 20)
pipe_status_t pipe_rowsum_noalloc(const void* A, float* out, int64_t M, int64_t N, int64_t lda,
                                  const pipe_config_t* cfg, void* stream);

/* GEMM mainloop ("chapter_async_barriers", section 常见的同步规则: a stage
 * whose copies have all landed is handed to the matrix-multiply consumers;
 * "cute（12）async_pipeline" ring): C = A * B with bf16 A (M x K, row-major) and B (K x N,
 * row-major; column-major with PIPE_FLAG_GEMM_B_COLMAJOR), fp32 accumulation,
 * C (M x N, row-major) in fp32 -- or, with
 * PIPE_FLAG_GEMM_C_BF16, in bf16 (each fp32 sum rounded to nearest even),
 * staged through LDS so that C is written in whole 16-byte row pieces
 * (optionally by a dedicated store wave, PIPE_FLAG_GEMM_STORE_WAVE). A and B tiles
 * of each K step (tile_k deep) pass through the LDS ring to MFMA waves.
 *   M arbitrary, N % 8 == 0 and K % 8 == 0 (whole 16-byte chunks; else
 *   PIPE_ERR_SHAPE). Shapes that are not whole tiles (M % tile_m, N % tile_n or
 *   K % tile_k non-zero) run a masked kernel: chunks outside A or B enter the ring
 *   as zeros and only C's M x N elements are written (with PIPE_FLAG_TRACE
 *   such shapes return PIPE_ERR_SHAPE). lda >= K and ldb >= N (ldb >= K for
 *   column-major B), both multiples of 8; ldc >= N (elements of C's type; a
 *   multiple of 8 for bf16 C, whose base must be 16-byte aligned); K == 0
 *   gives C = 0. */
pipe_status_t pipe_gemm_mainloop(const void* A, const void* B, void* C, int64_t M,
                                 int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                 const pipe_config_t* cfg, void* stream);

/* Launch geometry an op would use for this shape and config, computed on the
 * host (no launch, no HIP call): LDS per workgroup (ring slots of
 * "cute（12）async_pipeline" plus barrier words), threads, grid, work items,
 * tiles per item. A diagnostic of this library, not an operation of the pages. */
pipe_status_t pipe_query_kernel(pipe_op_t op, const pipe_config_t* cfg, int64_t M, int64_t N,
                                int64_t K, pipe_kernel_info_t* info);

/* Compiled resources of the main kernel that an op would launch for this
 * shape and config (the stream, unified or GEMM kernel; not a zero fill), from
 * the HIP runtime's function attributes. It
 * takes the same checks as the op's entry point minus those on pointers, with
 * the tightest pitches (ld = N, or K for A and column-major B), and launches
 * nothing. Unlike pipe_query_kernel it needs the HIP runtime and a device.
 * A diagnostic of this library, not an operation of the pages.
 *   PIPE_ERR_SHAPE also for shapes that launch no main kernel (M or N zero,
 *   or K zero for the GEMM); PIPE_ERR_HIP when the runtime cannot report. */
pipe_status_t pipe_kernel_resources(pipe_op_t op, const pipe_config_t* cfg, int64_t M, int64_t N,
                                    int64_t K, pipe_kernel_resources_t* out);

/* Blocking read of the library's own device status word on the current
 * device (used when cfg->status is NULL); clears it when `clear` != 0.
 * Part of this library's error reporting, not an operation of the pages. */
pipe_status_t pipe_device_status(uint32_t* out, int clear);

/* The error code a status word stands for, on the host (no HIP call): PIPE_OK
 * for 0, PIPE_ERR_INVARIANT when PIPE_STATUS_INVARIANT is set, else
 * PIPE_ERR_TIMEOUT when a timeout bit is set. For a word read back from
 * cfg->status or with pipe_device_status after the caller synchronised. Part
 * of this library's error reporting, not an operation of the pages. */
pipe_status_t pipe_status_from_word(uint32_t word);

#ifdef __cplusplus
}
#endif

#endif /* PIPE_TILE_H */
