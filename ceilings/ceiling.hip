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

// Column-strip ceilings: the tile stream's access pattern without its ring.
// The region is `rows` x `width` bytes at a row pitch of `pitch` bytes, cut
// into column strips WB bytes wide and 16 KiB tiles of 16384/WB rows. Each
// 512-thread workgroup walks one strip segment (tiles seg, seg + split, ...);
// consecutive segments share an XCD. A wave moves two 1 KiB pieces of each
// tile (64 lanes x 16 bytes = 1024/WB rows of WB bytes each), one tile at a
// time, with non-temporal loads and stores.
constexpr int kStripThreads = 512;
enum StripOp { kStripRead = 0, kStripWrite = 1, kStripCopy = 2 };

template <int WB, int OP>
__global__ void __launch_bounds__(kStripThreads) strip_kernel(const uint8_t* __restrict__ src,
                                                              uint8_t* __restrict__ dst,
                                                              uint32_t* __restrict__ sink,
                                                              int64_t pitch, int64_t rows,
                                                              int split) {
  constexpr int kRowsPerPiece = 1024 / WB, kTileRows = 16384 / WB, kLanesPerRow = WB / 16;
  const int per_xcd = gridDim.x / 8;  // gridDim.x % 8 == 0
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  const int strip = item / split, seg = item % split;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t col = (int64_t)strip * WB + (lane % kLanesPerRow) * 16;
  const int lrow = lane / kLanesPerRow;
  const int64_t n_tiles = rows / kTileRows;
  uint32_t acc = 0;
  for (int64_t t = seg; t < n_tiles; t += split) {
    u32x4 v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = t * kTileRows + (2 * wave + i) * kRowsPerPiece + lrow;
      if constexpr (OP == kStripWrite) {
        v[i] = u32x4{(uint32_t)row, (uint32_t)col, ~(uint32_t)row, ~(uint32_t)col};
      } else {
        v[i] = ld<true>(reinterpret_cast<const u32x4*>(src + row * pitch + col));
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = t * kTileRows + (2 * wave + i) * kRowsPerPiece + lrow;
      if constexpr (OP == kStripRead)
        acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
      else
        st<true>(reinterpret_cast<u32x4*>(dst + row * pitch + col), v[i]);
    }
  }
  if (OP == kStripRead && acc == 0x9E3779B9u) sink[0] = acc;
}

int check_strips(int64_t rows, int64_t pitch, int64_t width, int strip_bytes, int split) {
  if (strip_bytes != 128 && strip_bytes != 256 && strip_bytes != 512) return 3;
  if (rows <= 0 || width <= 0 || pitch < width || pitch % 16 != 0) return 2;
  if (width % strip_bytes != 0 || rows % (16384 / strip_bytes) != 0) return 2;
  if (pitch > (int64_t(1) << 40) || rows > (int64_t(1) << 40) / pitch) return 2;
  const int64_t grid = width / strip_bytes * split;
  if (split < 1 || grid % 8 != 0 || grid > 65536) return 3;
  return 0;
}

template <int OP>
int launch_strips(const void* src, void* dst, unsigned* sink, int64_t rows, int64_t pitch,
                  int64_t width, int strip_bytes, int split, hipStream_t stream) {
  const dim3 grid((unsigned)(width / strip_bytes * split)), block(kStripThreads);
  const auto* s = static_cast<const uint8_t*>(src);
  auto* d = static_cast<uint8_t*>(dst);
  if (strip_bytes == 128)
    hipLaunchKernelGGL((strip_kernel<128, OP>), grid, block, 0, stream, s, d, sink, pitch, rows,
                       split);
  else if (strip_bytes == 256)
    hipLaunchKernelGGL((strip_kernel<256, OP>), grid, block, 0, stream, s, d, sink, pitch, rows,
                       split);
  else
    hipLaunchKernelGGL((strip_kernel<512, OP>), grid, block, 0, stream, s, d, sink, pitch, rows,
                       split);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// LDS ceilings: how fast one instruction kind moves bytes into or out of LDS.
// 512-thread workgroups with 64 KiB of LDS each (two per CU); every wave issues
// 8 instructions per iteration, all conflict-free. OP 0: ds_read_b128 (1 KiB
// per wave instruction); OP 1: ds_read_b64_tr_b16 (512 B), with the address
// pattern of a 32-column MFMA B operand; OP 2: global_load_lds_dwordx4 (1 KiB)
// from a 64 KiB global buffer that stays in L2; OP 3: ds_write_b128 (1 KiB);
// OP 4: waves 0-3 as OP 2 while waves 4-7 run OP 0; OP 5 and OP 6: one of the
// two halves of OP 4 with the other half idle. Waves 0 and 4 record the
// shader clock and the 100 MHz real-time clock around their loops, so the host
// can convert to bytes per clock.
enum LdsOp {
  kLdsReadB128 = 0,
  kLdsReadTr16 = 1,
  kLdsDma = 2,
  kLdsWriteB128 = 3,
  kLdsDmaAndRead = 4,  // waves 0-3 DMA, waves 4-7 ds_read_b128
  kLdsReadHalf = 5,    // waves 4-7 ds_read_b128, waves 0-3 idle
  kLdsDmaHalf = 6,     // waves 0-3 DMA, waves 4-7 idle
};
constexpr int kLdsThreads = 512;
constexpr int kLdsBytes = 65536;
typedef __attribute__((address_space(3))) uint8_t lds_byte;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int OP>
__global__ void __launch_bounds__(kLdsThreads) lds_kernel(const uint8_t* __restrict__ src,
                                                          uint32_t* __restrict__ fold,
                                                          uint64_t* __restrict__ clocks,
                                                          int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kLdsBytes / 16; i += kLdsThreads)
    reinterpret_cast<u32x4*>(lds)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t acc = 0;
  const bool idle = (OP == kLdsReadHalf && wave < 4) || (OP == kLdsDmaHalf && wave >= 4);
  for (int it = 0; it < (idle ? 0 : iters); ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (OP == kLdsWriteB128) {
        const int a = ((wave * 8 + j) * 1024 + lane * 16 + it * 64) & (kLdsBytes - 16);
        // Written as an instruction: nothing reads these bytes back, so a plain
        // store would be dropped as dead.
        const uint32_t la = (uint32_t)(uintptr_t)((lds_byte*)lds + a);
        const u32x4 v = {(uint32_t)it, (uint32_t)j, 0u, 1u};
        asm volatile("ds_write_b128 %0, %1" : : "v"(la), "v"(v) : "memory");
      } else if (OP == kLdsReadB128 || OP == kLdsReadHalf || (OP == kLdsDmaAndRead && wave >= 4)) {
        const int a = ((wave * 8 + j) * 1024 + lane * 16 + it * 64) & (kLdsBytes - 16);
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + a);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      } else if constexpr (OP == kLdsReadTr16) {
        // 16 K-rows of 256 bytes per 4 KiB; lane groups of 16 read 4 K-rows x 4 columns
        const int g = lane >> 4, i = lane & 15;
        const int k = 8 * (g >> 1) + (i >> 2) + 16 * ((j + it) & 3);
        const int col = 16 * (g & 1) + 4 * (i & 3) + 32 * (j >> 2) + 64 * (wave & 1);
        const int sw = ((k & 3) << 2) ^ (((k >> 3) & 1) << 1);
        const int a = (wave >> 1) * 16384 + k * 256 + (((col >> 3) ^ sw) << 4) + (col & 7) * 2;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_byte*)lds + a));
        acc ^= (uint32_t)(uint16_t)v[0] ^ ((uint32_t)(uint16_t)v[3] << 16);
      } else if (OP == kLdsDma || OP == kLdsDmaAndRead || OP == kLdsDmaHalf) {
        const uint8_t* g = src + (((wave * 8 + j) * 1024 + it * 4096) & (kLdsBytes - 1)) + lane * 16;
        const uint32_t base = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)((lds_byte*)lds + (((wave * 8 + j) * 1024) & (kLdsBytes - 1))));
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(base) : "memory");
      }
    }
    if constexpr (OP == kLdsDma || OP == kLdsDmaAndRead || OP == kLdsDmaHalf)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  }
  if constexpr (OP == kLdsDma || OP == kLdsDmaAndRead || OP == kLdsDmaHalf)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (OP == kLdsWriteB128) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  fold[(size_t)blockIdx.x * kLdsThreads + threadIdx.x] = acc;
  if (lane == 0 && (wave == 0 || wave == 4)) {
    clocks[4 * blockIdx.x + (wave >> 1)] = c1 - c0;
    clocks[4 * blockIdx.x + (wave >> 1) + 1] = r1 - r0;
  }
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

extern "C" int ceil_strip_copy(const void* src, void* dst, int64_t rows, int64_t pitch,
                               int64_t width, int strip_bytes, int split, hipStream_t stream) {
  if (src == nullptr || dst == nullptr) return 1;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return 2;
  if (int e = check_strips(rows, pitch, width, strip_bytes, split)) return e;
  return launch_strips<kStripCopy>(src, dst, nullptr, rows, pitch, width, strip_bytes, split,
                                   stream);
}

extern "C" int ceil_strip_read(const void* src, unsigned* sink, int64_t rows, int64_t pitch,
                               int64_t width, int strip_bytes, int split, hipStream_t stream) {
  if (src == nullptr || sink == nullptr) return 1;
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0) return 2;
  if (int e = check_strips(rows, pitch, width, strip_bytes, split)) return e;
  return launch_strips<kStripRead>(src, nullptr, sink, rows, pitch, width, strip_bytes, split,
                                   stream);
}

extern "C" int ceil_strip_write(void* dst, int64_t rows, int64_t pitch, int64_t width,
                                int strip_bytes, int split, hipStream_t stream) {
  if (dst == nullptr) return 1;
  if ((uintptr_t)dst % 16 != 0) return 2;
  if (int e = check_strips(rows, pitch, width, strip_bytes, split)) return e;
  return launch_strips<kStripWrite>(nullptr, dst, nullptr, rows, pitch, width, strip_bytes, split,
                                    stream);
}

extern "C" int ceil_lds(int op, const void* src, unsigned* fold, uint64_t* clocks, int grid,
                        int iters, hipStream_t stream) {
  const bool dma = op == kLdsDma || op == kLdsDmaAndRead || op == kLdsDmaHalf;
  if (fold == nullptr || clocks == nullptr || (dma && src == nullptr)) return 1;
  if (((uintptr_t)fold % 4) || ((uintptr_t)clocks % 8) || (dma && (uintptr_t)src % 16)) return 2;
  if (grid < 1 || grid > 65536 || iters < 1 || iters > (1 << 20)) return 3;
  const dim3 g(grid), b(kLdsThreads);
  const auto* s = static_cast<const uint8_t*>(src);
  if (op == kLdsReadB128)
    hipLaunchKernelGGL((lds_kernel<kLdsReadB128>), g, b, 0, stream, s, fold, clocks, iters);
  else if (op == kLdsReadTr16)
    hipLaunchKernelGGL((lds_kernel<kLdsReadTr16>), g, b, 0, stream, s, fold, clocks, iters);
  else if (op == kLdsDma)
    hipLaunchKernelGGL((lds_kernel<kLdsDma>), g, b, 0, stream, s, fold, clocks, iters);
  else if (op == kLdsWriteB128)
    hipLaunchKernelGGL((lds_kernel<kLdsWriteB128>), g, b, 0, stream, s, fold, clocks, iters);
  else if (op == kLdsDmaAndRead)
    hipLaunchKernelGGL((lds_kernel<kLdsDmaAndRead>), g, b, 0, stream, s, fold, clocks, iters);
  else if (op == kLdsReadHalf)
    hipLaunchKernelGGL((lds_kernel<kLdsReadHalf>), g, b, 0, stream, s, fold, clocks, iters);
  else if (op == kLdsDmaHalf)
    hipLaunchKernelGGL((lds_kernel<kLdsDmaHalf>), g, b, 0, stream, s, fold, clocks, iters);
  else
    return 3;
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
