// Context-only HBM ceilings: plain grid-stride streaming kernels (no LDS, no
// pipeline). Built into libpipeceil.so, separate from the tile-stream library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pipe_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

template <bool NT, int UNR>
__global__ void __launch_bounds__(kThreads) copy_kernel(const u32x4* __restrict__ s,
                                                         u32x4* __restrict__ d, size_t n) {
  const size_t step = (size_t)gridDim.x * kThreads * UNR;
  for (size_t i = (size_t)blockIdx.x * kThreads * UNR + threadIdx.x; i < n; i += step) {
    u32x4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (i + (size_t)u * kThreads < n) v[u] = ld<NT>(s + i + (size_t)u * kThreads);
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (i + (size_t)u * kThreads < n) st<NT>(d + i + (size_t)u * kThreads, v[u]);
  }
}

template <bool NT>
__global__ void __launch_bounds__(kThreads) read_kernel(const u32x4* __restrict__ s,
                                                         uint32_t* __restrict__ sink, size_t n) {
  const size_t step = (size_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += step) {
    const u32x4 v = ld<NT>(s + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

int check(const void* a, const void* b, size_t bytes, int grid) {
  if (a == nullptr || b == nullptr) return 1;
  if (bytes == 0 || bytes % 16 != 0) return 2;
  if (((uintptr_t)a | (uintptr_t)b) % 16 != 0) return 2;
  if (grid < 1 || grid > 65536) return 3;
  return 0;
}

}  // namespace

extern "C" int ceil_copy(const void* src, void* dst, size_t bytes, int grid, int unroll, int nt,
                         hipStream_t stream) {
  if (int e = check(src, dst, bytes, grid)) return e;
  if ((unroll != 1 && unroll != 4) || (nt != 0 && nt != 1)) return 3;
  const auto* s = static_cast<const u32x4*>(src);
  auto* d = static_cast<u32x4*>(dst);
  const size_t n = bytes / 16;
  if (nt && unroll == 4)
    hipLaunchKernelGGL((copy_kernel<true, 4>), dim3(grid), dim3(kThreads), 0, stream, s, d, n);
  else if (nt)
    hipLaunchKernelGGL((copy_kernel<true, 1>), dim3(grid), dim3(kThreads), 0, stream, s, d, n);
  else if (unroll == 4)
    hipLaunchKernelGGL((copy_kernel<false, 4>), dim3(grid), dim3(kThreads), 0, stream, s, d, n);
  else
    hipLaunchKernelGGL((copy_kernel<false, 1>), dim3(grid), dim3(kThreads), 0, stream, s, d, n);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int ceil_read(const void* src, unsigned* sink, size_t bytes, int grid, int nt,
                         hipStream_t stream) {
  if (sink == nullptr) return 1;
  if (int e = check(src, src, bytes, grid)) return e;
  if (nt != 0 && nt != 1) return 3;
  const auto* s = static_cast<const u32x4*>(src);
  const size_t n = bytes / 16;
  if (nt)
    hipLaunchKernelGGL((read_kernel<true>), dim3(grid), dim3(kThreads), 0, stream, s, sink, n);
  else
    hipLaunchKernelGGL((read_kernel<false>), dim3(grid), dim3(kThreads), 0, stream, s, sink, n);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int ceil_memcpy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (dst == nullptr || src == nullptr) return 1;
  if (bytes == 0) return 2;
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, stream) == hipSuccess ? 0 : 4;
}
