// Unified (non-specialised) tile stream, the comparison design to the
// warp-specialised ring: every wave both loads and consumes.
//
// "cuda-features-10-pipelines" 4.10.7 describes the unified pattern: a
// prologue that prefills S-1 stages, a steady state that submits the next
// tile and then waits for and uses the current one, and an epilogue that
// drains; the batch wait is by count of outstanding batches (4.10.3,
// wait_prior). "cute（12）async_pipeline" section 7 (the comparison with lesson
// 09) contrasts it with the producer/consumer split: no empty barrier, no
// phase.
//
// Here each of the W waves moves its 16/W blocks of every tile into the LDS
// ring with direct-to-LDS loads and later consumes exactly those blocks, so a
// wave's own `s_waitcnt vmcnt(n)` is the whole handshake: n counts the vector
// memory operations the wave issued after the tile's loads (loads of younger
// tiles and, for the copy, its own stores; gfx9 counts both in issue order).
// Every operation counted must really be issued (an over-count would weaken
// the wait); operations left uncounted only make the wait stricter.
// A slot region is refilled only by the wave that read it, after its reads
// have returned (lgkmcnt), so no cross-wave barrier is needed at all.
#include "pipe_device.hpp"
#include "pipe_kernels.hpp"
#include "pipe_rowsum.hpp"

namespace pipe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The workgroup's tile sequence: items blockIdx.x, +gridDim.x, ...; each item
// is one segment of a strip (same walk as the warp-specialised kernel).
struct Walk {
  int it, item, len, k;

  __device__ __forceinline__ void start(const StreamParams& p) {
    it = blockIdx.x;
    k = 0;
    if (it < p.items) load(p);
  }
  __device__ __forceinline__ void load(const StreamParams& p) {
    item = p.xcd_remap ? ((it & 7) * (p.items >> 3) + (it >> 3)) : it;
    const int seg = item / p.n_strips;
    if (p.interleave) {
      len = (p.strip_len - seg + p.split - 1) / p.split;
    } else {
      const int left = p.strip_len - seg * p.seg_len;
      len = left < p.seg_len ? left : p.seg_len;
    }
  }
  __device__ __forceinline__ bool valid(const StreamParams& p) const { return it < p.items; }
  __device__ __forceinline__ bool last_of_item() const { return k + 1 == len; }
  __device__ __forceinline__ void next(const StreamParams& p) {
    if (++k == len) {
      k = 0;
      it += gridDim.x;
      if (it < p.items) load(p);
    }
  }
  __device__ __forceinline__ void coords(const StreamParams& p, int& tr, int& tc) const {
    const int strip = item % p.n_strips;
    const int seg = item / p.n_strips;
    const int pos = p.interleave ? seg + k * p.split : seg * p.seg_len + k;
    tr = p.row_strips ? strip : pos;
    tc = p.row_strips ? pos : strip;
  }
};

// Per-slot vmcnt marks, held as one 8-lane integer vector value (S <= 8) so
// that the runtime slot index selects a register: as a plain array the
// compiler placed the marks in LDS or in scratch memory.
template <int S>
struct Marks {
  static_assert(S >= 1 && S <= 8, "at most 8 slots");
  typedef int ivec8 __attribute__((ext_vector_type(8)));
  ivec8 m;
  __device__ __forceinline__ int get(int s) const { return m[s]; }
  __device__ __forceinline__ void set(int s, int v) { m[s] = v; }
};

template <int S, int W, int OP, int TC>
__global__ void __launch_bounds__(64 * W) unified_kernel(StreamParams p) {
  using Sh = TileShape<TC>;
  __shared__ uint8_t slots[S][kTileBytes];
  constexpr int kLoads = kBlocksPerTile / W;  // blocks loaded and consumed per wave per tile
  constexpr int kStores = OP == kOpCopy ? kLoads : 0;
  const int wave = (int)(threadIdx.x >> 6);
  const int lane = lane_id();
  const int lrow = lane >> Sh::kLog2ChunksPerRow, lpos = lane & (Sh::kChunksPerRow - 1);

  Walk iss, use;
  iss.start(p);
  use.start(p);
  Marks<S> mark;
  int vm = 0;       // vector-memory operations issued by this wave so far
  int issued = 0;   // tiles whose loads are issued
  float acc[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) acc[j] = 0.f;

  auto issue = [&]() {
    int tr, tc;
    iss.coords(p, tr, tc);
    const uint8_t* g = p.src + (int64_t)tr * Sh::kRows * p.ld_src + (int64_t)tc * Sh::kRowBytes;
    const int s = issued % S;
    const uint32_t slot = uniform(lds_addr(&slots[s][0]));
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int q = wave * kLoads + j;
      const int r = q * Sh::kRowsPerBlock + lrow;
      const int c = swz_n<Sh::kChunksPerRow>(r, lpos, p.swz_shift);
      if (p.nt)
        dma_block_nt(g + (int64_t)r * p.ld_src + c * kChunkBytes, slot + q * kBlockBytes);
      else
        dma_block(g + (int64_t)r * p.ld_src + c * kChunkBytes, slot + q * kBlockBytes);
    }
    vm += kLoads;
    mark.set(s, vm);
    ++issued;
    iss.next(p);
  };

  // Prologue: S - 1 tiles in flight.
  for (int i = 0; i < S - 1 && iss.valid(p); ++i) issue();

  for (int t = 0; use.valid(p); ++t) {
    const int s = t % S;
    if (S == 1 && iss.valid(p)) issue();
    // Batch wait: this wave's loads of tile t have landed.
    wait_vmcnt_mul<kLoads>((vm - mark.get(s)) / kLoads);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint8_t* slot = &slots[s][0];
    uint4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      v[j] = *reinterpret_cast<const uint4*>(slot + (wave * kLoads + j) * kBlockBytes +
                                             lane * kChunkBytes);
    wait_lgkmcnt0();  // reads of slot s returned: it may be refilled
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (S > 1 && iss.valid(p)) issue();  // tile t + S - 1 into the slot of tile t - 1
    int tr, tc;
    use.coords(p, tr, tc);
    if constexpr (OP == kOpCopy) {
      uint8_t* gd = p.dst + (int64_t)tr * Sh::kRows * p.ld_dst + (int64_t)tc * Sh::kRowBytes;
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int r = (wave * kLoads + j) * Sh::kRowsPerBlock + lrow;
        const int c = swz_n<Sh::kChunksPerRow>(r, lpos, p.swz_shift);
        uint8_t* a = gd + ((int64_t)r * p.ld_dst + c * kChunkBytes);
        if (p.nt) {
          const u32x4 nv = {v[j].x, v[j].y, v[j].z, v[j].w};
          __builtin_nontemporal_store(nv, reinterpret_cast<u32x4*>(a));
        } else {
          *reinterpret_cast<uint4*>(a) = v[j];
        }
      }
      vm += kStores;
    } else {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum += (float)__builtin_bit_cast(_Float16, (uint16_t)(w4[e] & 0xFFFFu));
          sum += (float)__builtin_bit_cast(_Float16, (uint16_t)(w4[e] >> 16));
        }
        acc[j] += sum;
      }
      if (use.last_of_item()) {
        const int seg = use.item / p.n_strips;
        float* o = p.out + (int64_t)seg * p.M + (int64_t)tr * Sh::kRows;
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          const float rs = sum_lanes<Sh::kChunksPerRow>(acc[j]);
          if (lpos == 0) store_partial(&o[(wave * kLoads + j) * Sh::kRowsPerBlock + lrow], rs);
          acc[j] = 0.f;
        }
        // These partial stores (and the arrival's atomic and loads) are left
        // out of `vm`: counting fewer operations than were issued only makes
        // the batch waits stricter.
        if (p.tickets != nullptr) rowsum_strip_arrive<Sh::kRows, W>(p, use.item % p.n_strips);
      }
    }
    use.next(p);
  }
  wait_vmcnt<0>();
}

template <int S, int W, int TC>
hipError_t launch_swt(int op, int grid, const StreamParams& p, hipStream_t stream) {
  if constexpr (!unified_shape_supported(S, W, TC)) {
    return hipErrorInvalidValue;
  } else {
    if (op == kOpCopy)
      return launch_or_record(unified_kernel<S, W, kOpCopy, TC>, dim3(grid), dim3(64 * W), stream,
                              p);
    return launch_or_record(unified_kernel<S, W, kOpRowsum, TC>, dim3(grid), dim3(64 * W), stream,
                            p);
  }
}

template <int S, int W>
hipError_t launch_sw(int op, int tile_n, int grid, const StreamParams& p, hipStream_t stream) {
  switch (tile_n) {
    case 64: return launch_swt<S, W, 64>(op, grid, p, stream);
    case 128: return launch_swt<S, W, 128>(op, grid, p, stream);
    case 256: return launch_swt<S, W, 256>(op, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int S>
hipError_t launch_s(int op, int waves, int tile_n, int grid, const StreamParams& p,
                    hipStream_t stream) {
  switch (waves) {
    case 2: return launch_sw<S, 2>(op, tile_n, grid, p, stream);
    case 4: return launch_sw<S, 4>(op, tile_n, grid, p, stream);
    case 8: return launch_sw<S, 8>(op, tile_n, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_unified(int op, int stages, int waves, int tile_n, int grid,
                          const StreamParams& p, hipStream_t stream) {
  switch (stages) {
    case 1: return launch_s<1>(op, waves, tile_n, grid, p, stream);
    case 2: return launch_s<2>(op, waves, tile_n, grid, p, stream);
    case 3: return launch_s<3>(op, waves, tile_n, grid, p, stream);
    case 4: return launch_s<4>(op, waves, tile_n, grid, p, stream);
    case 5: return launch_s<5>(op, waves, tile_n, grid, p, stream);
    case 6: return launch_s<6>(op, waves, tile_n, grid, p, stream);
    case 7: return launch_s<7>(op, waves, tile_n, grid, p, stream);
    case 8: return launch_s<8>(op, waves, tile_n, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pipe
