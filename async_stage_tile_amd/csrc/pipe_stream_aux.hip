// Stream-kernel dispatch over the stage count, small fill kernels, and the per-thread slot of kernel lookups without a launch. The stream kernels themselves are instantiated per stage
// count in the objects built from pipe_stream.hip.
#include "pipe_device.hpp"
#include "pipe_kernels.hpp"

namespace pipe {

namespace {
thread_local const void** t_record_slot = nullptr;
}  // namespace

const void** record_slot() { return t_record_slot; }
void set_record_slot(const void** slot) { t_record_slot = slot; }

hipError_t launch_stream(int op, int stages, int consumers, int producers, int tile_n, int grid,
                         const StreamParams& p, hipStream_t stream) {
  switch (stages) {
    case 1: return launch_stream_stages<1>(op, consumers, producers, tile_n, grid, p, stream);
    case 2: return launch_stream_stages<2>(op, consumers, producers, tile_n, grid, p, stream);
    case 3: return launch_stream_stages<3>(op, consumers, producers, tile_n, grid, p, stream);
    case 4: return launch_stream_stages<4>(op, consumers, producers, tile_n, grid, p, stream);
    case 5: return launch_stream_stages<5>(op, consumers, producers, tile_n, grid, p, stream);
    case 6: return launch_stream_stages<6>(op, consumers, producers, tile_n, grid, p, stream);
    case 7: return launch_stream_stages<7>(op, consumers, producers, tile_n, grid, p, stream);
    case 8: return launch_stream_stages<8>(op, consumers, producers, tile_n, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_group(int stages, int consumers, int producers, int group, int grid,
                               const StreamParams& p, hipStream_t stream) {
  switch (stages) {
    case 2: return launch_group_stages<2>(consumers, producers, group, grid, p, stream);
    case 3: return launch_group_stages<3>(consumers, producers, group, grid, p, stream);
    case 4: return launch_group_stages<4>(consumers, producers, group, grid, p, stream);
    case 5: return launch_group_stages<5>(consumers, producers, group, grid, p, stream);
    case 6: return launch_group_stages<6>(consumers, producers, group, grid, p, stream);
    case 7: return launch_group_stages<7>(consumers, producers, group, grid, p, stream);
    case 8: return launch_group_stages<8>(consumers, producers, group, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_group_load(int stages, int consumers, int producers, int grid,
                                    const StreamParams& p, hipStream_t stream) {
  switch (stages) {
    case 4: return launch_group_load_stages<4>(consumers, producers, grid, p, stream);
    case 8: return launch_group_load_stages<8>(consumers, producers, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_regs(int op, int stages, int consumers, int producers, int grid,
                              const StreamParams& p, hipStream_t stream) {
  switch (stages) {
    case 1: return launch_regs_stages<1>(op, consumers, producers, grid, p, stream);
    case 2: return launch_regs_stages<2>(op, consumers, producers, grid, p, stream);
    case 3: return launch_regs_stages<3>(op, consumers, producers, grid, p, stream);
    case 4: return launch_regs_stages<4>(op, consumers, producers, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_debug(int op, int stages, int consumers, int producers, int grid,
                               const StreamParams& p, hipStream_t stream) {
  switch (stages) {
    case 1: return launch_debug_stages<1>(op, consumers, producers, grid, p, stream);
    case 2: return launch_debug_stages<2>(op, consumers, producers, grid, p, stream);
    case 3: return launch_debug_stages<3>(op, consumers, producers, grid, p, stream);
    case 4: return launch_debug_stages<4>(op, consumers, producers, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

int stream_lds_bytes(int stages, int consumers) {
  return stages * kTileBytes + stages * 4 * (3 + consumers);
}

__global__ void __launch_bounds__(256) fill_f32(float* __restrict__ out, int64_t rows,
                                                int64_t cols, int64_t ld, float value) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  out[(i / cols) * ld + (i % cols)] = value;
}

__global__ void __launch_bounds__(256) fill_u32(uint32_t* __restrict__ out, int64_t n,
                                                uint32_t value) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = value;
}

__global__ void __launch_bounds__(256) fill_u16(uint16_t* __restrict__ out, int64_t rows,
                                                int64_t cols, int64_t ld, uint16_t value) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  out[(i / cols) * ld + (i % cols)] = value;
}

hipError_t launch_fill_u32(uint32_t* out, int64_t n, uint32_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_u32, dim3((unsigned)blocks), dim3(256), 0, stream, out, n, value);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* out, int64_t rows, int64_t cols, int64_t ld, float value,
                           hipStream_t stream) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_f32, dim3((unsigned)blocks), dim3(256), 0, stream, out, rows, cols,
                     ld, value);
  return hipGetLastError();
}

hipError_t launch_fill_u16(uint16_t* out, int64_t rows, int64_t cols, int64_t ld, uint16_t value,
                           hipStream_t stream) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_u16, dim3((unsigned)blocks), dim3(256), 0, stream, out, rows, cols, ld,
                     value);
  return hipGetLastError();
}

}  // namespace pipe
