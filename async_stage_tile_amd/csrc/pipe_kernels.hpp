// Kernel parameter blocks and launchers shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pipe {

enum StreamOp : int { kOpCopy = 0, kOpRowsum = 1 };

struct StreamParams {
  const uint8_t* src;     // copy source / rowsum input (fp16)
  uint8_t* dst;           // copy destination
  float* out;             // rowsum: final sums (split 1) or segment partials [split][M]
  float* final_out;       // rowsum with split > 1: the final sums, written by the last arrival
  uint32_t* tickets;      // rowsum with split > 1: one arrival counter per row strip, zero at launch
  uint32_t* checksums;    // copy: per-tile code sums (nullable)
  uint32_t* trace;        // nullable
  uint32_t* status;       // never null
  int64_t ld_src;         // row pitch, bytes
  int64_t ld_dst;         // row pitch, bytes
  int64_t M;              // rows (also the rowsum partial stride)
  int64_t N;              // columns (fp16 elements, a multiple of 8)
  int32_t tile_cols;      // ceil(N / 64)
  int32_t n_strips;
  int32_t strip_len;      // tiles per strip
  int32_t seg_len;        // tiles per segment
  int32_t split;          // segments per strip
  int32_t items;          // n_strips * split
  int32_t row_strips;     // 1: a strip is one tile row walked along the columns
  int32_t swz_shift;
  int32_t lag;            // producer commit lag in tiles (<= stages - 1, <= stream_max_lag)
  uint32_t spin_limit;
  uint32_t start_phase;   // producer start phase (1; 0 only in the deadlock test)
  int32_t no_release;     // test: consumers never release
  int32_t trace_cap;      // trace records
  int32_t nt;             // non-temporal hints on the streamed loads and stores
  int32_t xcd_remap;      // permute items so each XCD streams neighbouring strips
  int32_t interleave;     // segment s takes tiles s, s + split, s + 2 split, ...
  int32_t eager;          // eager commits while the acquire waits: min tiles in flight (0 = off)
  int32_t jitter;         // debug kernels: pseudo-random pauses before every wait
  int32_t early_release;  // debug kernels, test: consumers release before reading
};

// Ring shapes (stages S, consumer waves C, producer waves PW, tile columns TC)
// the stream kernel is instantiated for. The pages' 128 x 64 tile (TC = 64):
// PW in {1, 2, 4}; C in {1, 2, 3, 4, 8} for S = 1..4, and C in {4, 8} for the
// deep rings S = 5..8. The wider 16 KiB tiles 64 x 128 and 32 x 256
// (TC = 128, 256): S = 2..4, PW in {2, 4}, C in {4, 8}.
constexpr bool stream_shape_supported(int S, int C, int PW, int TC = 64) {
  if (S < 1 || S > 8) return false;
  if (!(PW == 1 || PW == 2 || PW == 4)) return false;
  if (TC == 128 || TC == 256)
    return S >= 2 && S <= 4 && (PW == 2 || PW == 4) && (C == 4 || C == 8);
  if (TC != 64) return false;
  if (S > 4) return C == 4 || C == 8;
  return C == 1 || C == 2 || C == 3 || C == 4 || C == 8;
}

// Grouped copy strips (128 x 64 tiles; consumers store a tile row of G
// neighbouring tiles at once): G in {2, 4} with G <= S, C in {4, 8}, PW in {2, 4}.
constexpr bool group_shape_supported(int S, int C, int PW, int G) {
  return (G == 2 || G == 4) && G <= S && S <= 8 && (C == 4 || C == 8) && (PW == 2 || PW == 4);
}

// Grouped loads (strips of 4 tile columns whose producers fill the 4 slots of a
// tile row together): S in {4, 8} (one or two interleaved groups of 4 slots),
// C in {4, 8}, PW in {2, 4}.
constexpr bool group_load_shape_supported(int S, int C, int PW) {
  return (S == 4 || S == 8) && (C == 4 || C == 8) && (PW == 2 || PW == 4);
}

// Register producer engine (128 x 64 tiles): S = 1..4, C in {3, 4}, PW in {1, 4}.
constexpr bool regs_shape_supported(int S, int C, int PW) {
  return S >= 1 && S <= 4 && (C == 3 || C == 4) && (PW == 1 || PW == 4);
}

// Debug kernels (protocol checks at run time; 128 x 64 tiles): S = 1..4 with
// 1 producer + 3 consumer waves or 4 + 4.
constexpr bool debug_shape_supported(int S, int C, int PW) {
  return S >= 1 && S <= 4 && ((C == 3 && PW == 1) || (C == 4 && PW == 4));
}

// Largest commit lag for PW producer waves: each wave issues 16 / PW loads per
// tile and (lag + 1) tiles of them must fit the 63-entry vmcnt counter.
constexpr int stream_max_lag(int PW) { return 63 / (16 / PW) - 1; }

// Launch the stream kernel for (op, stages, consumers, producers, tile
// columns). Returns hipSuccess or the launch error (hipErrorInvalidValue for a
// shape that is not instantiated). `grid` workgroups of 64 * (producers +
// consumers) threads.
hipError_t launch_stream(int op, int stages, int consumers, int producers, int tile_n, int grid,
                         const StreamParams& p, hipStream_t stream);
template <int S>
hipError_t launch_stream_stages(int op, int consumers, int producers, int tile_n, int grid,
                                const StreamParams& p, hipStream_t stream);
int stream_lds_bytes(int stages, int consumers);

// Grouped copy strips: launch the kernel for (stages, consumers, producers,
// group); hipErrorInvalidValue for a shape group_shape_supported rejects. The
// commit lag in `p` must be at most stages - group.
hipError_t launch_stream_group(int stages, int consumers, int producers, int group, int grid,
                               const StreamParams& p, hipStream_t stream);
template <int S>
hipError_t launch_group_stages(int consumers, int producers, int group, int grid,
                               const StreamParams& p, hipStream_t stream);

// Grouped loads: launch the kernel for (stages, consumers, producers);
// hipErrorInvalidValue for a shape group_load_shape_supported rejects.
hipError_t launch_stream_group_load(int stages, int consumers, int producers, int grid,
                                    const StreamParams& p, hipStream_t stream);
template <int S>
hipError_t launch_group_load_stages(int consumers, int producers, int grid, const StreamParams& p,
                                    hipStream_t stream);

// Debug kernel: the DMA ring with its protocol checks (and optional jitter);
// hipErrorInvalidValue for a shape debug_shape_supported rejects.
hipError_t launch_stream_debug(int op, int stages, int consumers, int producers, int grid,
                               const StreamParams& p, hipStream_t stream);
template <int S>
hipError_t launch_debug_stages(int op, int consumers, int producers, int grid,
                               const StreamParams& p, hipStream_t stream);

// Register producer engine: launch the stream kernel whose producers load
// into registers and write the slots with ds_write_b128 (128 x 64 tiles);
// hipErrorInvalidValue for a shape regs_shape_supported rejects.
hipError_t launch_stream_regs(int op, int stages, int consumers, int producers, int grid,
                              const StreamParams& p, hipStream_t stream);
template <int S>
hipError_t launch_regs_stages(int op, int consumers, int producers, int grid,
                              const StreamParams& p, hipStream_t stream);

// Unified variant: `waves` waves each load and consume 16 / waves blocks of
// every tile; divisible shapes only, no checksums or trace. 128 x 64 tiles:
// waves 2, 4 or 8, stages 1..8; wider tiles: waves 2 or 4, stages 2..4.
constexpr bool unified_shape_supported(int S, int W, int TC) {
  if (TC == 64) return S >= 1 && S <= 8 && (W == 2 || W == 4 || W == 8);
  if (TC == 128 || TC == 256) return S >= 2 && S <= 4 && (W == 2 || W == 4);
  return false;
}
hipError_t launch_unified(int op, int stages, int waves, int tile_n, int grid,
                          const StreamParams& p, hipStream_t stream);

hipError_t launch_fill_u32(uint32_t* out, int64_t n, uint32_t value, hipStream_t stream);
hipError_t launch_fill_f32(float* out, int64_t rows, int64_t cols, int64_t ld, float value,
                           hipStream_t stream);
hipError_t launch_fill_u16(uint16_t* out, int64_t rows, int64_t cols, int64_t ld, uint16_t value,
                           hipStream_t stream);

struct GemmParams {
  const uint8_t* A;       // bf16 M x K
  const uint8_t* B;       // bf16 K x N
  void* C;                // M x N, fp32 (or bf16 when c_bf16)
  int64_t lda, ldb, ldc;  // bytes for A, B; elements for C
  int32_t M, N, K;
  int32_t tiles_n, k_steps;  // output tile columns; 64-deep K steps
  int32_t items;          // output tiles
  int32_t swz_shift;
  int32_t b_swz;          // 1: XOR-swizzle the B K-rows (default; row-major B only)
  int32_t b_colmajor;     // B given column-major (N x K rows of K): loaded and read like A
  uint32_t spin_limit;
  uint32_t* status;
  uint32_t* trace;
  int32_t trace_cap;
  int32_t eager;          // eager commits while the acquire waits: min stages in flight (0 = off)
  int32_t c_bf16;         // C is bf16, written through an LDS-staged epilogue
  int32_t store_wave;     // bf16 C: a dedicated store wave drains the staging slots
  int32_t tile_m;         // output tile rows: 128 (4 MFMA waves) or 256 (8 MFMA waves)
  int32_t unified;        // 0, or the unified kernel's waves (16 or 4), which all load and compute
};

hipError_t launch_gemm(int stages, int producers, int grid, const GemmParams& p,
                       hipStream_t stream);

// The unified GEMM (256 x 256 tiles, PIPE_FLAG_UNIFIED): a two-slot ring of
// 64 KiB stages, 16 waves of 64 x 64 output blocks or 4 of 128 x 128.
constexpr int kGemmUnifiedWaves = 16;
constexpr int kGemmWideWaves = 4;
constexpr int kGemmUnifiedLdsBytes = 2 * (32768 + 32768);

// Kernel lookup without a launch. While the calling thread's record slot is
// set, launch_or_record stores the address of the kernel it was given there
// and launches nothing; otherwise it launches it.
const void** record_slot();
void set_record_slot(const void** slot);

template <class P>
inline hipError_t launch_or_record(void (*kernel)(P), dim3 grid, dim3 block, hipStream_t stream,
                                   const P& p) {
  if (const void** slot = record_slot()) {
    *slot = reinterpret_cast<const void*>(kernel);
    return hipSuccess;
  }
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}
int gemm_lds_bytes(int stages, bool c_bf16, bool store_wave, int tile_m);
int gemm_threads(int producers, bool c_bf16, bool store_wave, int tile_m);

}  // namespace pipe
