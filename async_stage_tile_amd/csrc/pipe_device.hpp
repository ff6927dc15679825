// Device primitives of the pipelined tile stream (gfx950 / CDNA4).
//
// What the pages describe and how it maps onto one gfx950 workgroup:
//   * Ring of S stage slots in shared memory, each with a "full" and an
//     "empty" barrier ("cute（12）async_pipeline", sections 1 and 6.4).
//     Here: S slots in LDS, and one 32-bit LDS word per barrier.
//   * mbarrier = pending-arrival count + phase bit; the arrival that completes
//     a phase flips the phase and reloads the count; wait(p) passes once the
//     phase is no longer p ("cute（12）async_pipeline" 6.2; mlc.ai
//     "chapter_async_barriers", section mbarrier). Here one LDS word per
//     barrier, in one of two encodings (Counter, Flip; see below). gfx950 has
//     no transaction-byte counter, so the producer arrives on "full" only
//     after `s_waitcnt vmcnt` shows that the stage's loads have landed in LDS:
//     arrivals == 0 and bytes == 0 collapse into one arrival.
//   * PipelineState (index, phase, count) with ++ wrapping the index and
//     flipping the phase; producers start at phase 1 so the first lap never
//     waits ("cute（12）async_pipeline" 2.2-2.3, 6.1). Kept in SGPRs (the
//     control path is wave-uniform, as "cuda-features-10-pipelines" 4.10.4
//     asks of the pipeline's control flow).
//   * One waiter per wave polls the barrier word (the single-poller rule of
//     "cute（11）hopper之TMA_copy" 3.4): a uniform-address ds_read_b32
//     broadcasts to all lanes, then `s_sleep` between polls. Every wait is
//     bounded: after `spin_limit` polls it records a timeout and the wave
//     abandons the stream, so a broken handshake ends the kernel instead of
//     hanging the device.
//   * The copy engine is the gfx950 direct-to-LDS load
//     (global_load_lds_dwordx4): the LDS destination is M0 + lane*16 (wave
//     uniform), only the global address is per lane. It is issued from inline
//     asm so that the compiler's wait-count pass, which cannot tell the ring
//     slots from the barrier words, does not put `s_waitcnt vmcnt(0)` in front
//     of every barrier access.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pipe {

constexpr int kWave = 64;
constexpr int kTileRows = 128;                            // tile_m
constexpr int kTileCols = 64;                             // tile_n (fp16 elements)
constexpr int kRowBytes = kTileCols * 2;                  // 128 B per tile row
constexpr int kChunkBytes = 16;                           // one b128 access
constexpr int kChunksPerRow = kRowBytes / kChunkBytes;    // 8
constexpr int kTileBytes = kTileRows * kRowBytes;         // 16384
constexpr int kBlockBytes = kWave * kChunkBytes;          // 1024 = one wave-wide DMA
constexpr int kBlocksPerTile = kTileBytes / kBlockBytes;  // 16
constexpr int kRowsPerBlock = kBlockBytes / kRowBytes;    // 8

// Tile shapes of the stream kernels. Every tile is 16 KiB: kRows x TC fp16
// with TC (tileN) in {64, 128, 256} and kRows (tileM) = 128, 64, 32. One
// wave-wide DMA moves kBlockBytes = 1 KiB, i.e. kRowsPerBlock rows of
// kChunksPerRow 16-byte chunks. TC = 64 is the pages' 128 x 64 tile.
template <int TC>
struct TileShape {
  static constexpr int kCols = TC;
  static constexpr int kRowBytes = TC * 2;
  static constexpr int kChunksPerRow = kRowBytes / kChunkBytes;
  static constexpr int kLog2ChunksPerRow = kChunksPerRow == 8 ? 3 : kChunksPerRow == 16 ? 4 : 5;
  static constexpr int kRows = kTileBytes / kRowBytes;
  static constexpr int kRowsPerBlock = kBlockBytes / kRowBytes;
  static_assert(kRowsPerBlock >= 1 && (1 << kLog2ChunksPerRow) == kChunksPerRow,
                "a tile row is 8, 16 or 32 chunks within one wave-wide DMA");
};

// Status bits written to the caller's status word.
constexpr uint32_t kStatusTimeoutProducer = 1u;
constexpr uint32_t kStatusTimeoutConsumer = 2u;
constexpr uint32_t kStatusInvariant = 4u;  // a protocol check of a debug kernel failed

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const lds_u8*)(p));
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// ---------------------------------------------------------------------------
// PipelineState: ring cursor, wave-uniform.
// ---------------------------------------------------------------------------
struct PipeState {
  int index;
  uint32_t phase;
  uint32_t count;
  int stages;

  __device__ __forceinline__ void inc() {
    ++index;
    ++count;
    if (index == stages) {
      index = 0;
      phase ^= 1u;
    }
  }
};

__device__ __forceinline__ PipeState producer_start(int stages, uint32_t start_phase) {
  return PipeState{0, start_phase, 0u, stages};
}
__device__ __forceinline__ PipeState consumer_start(int stages) {
  return PipeState{0, 0u, 0u, stages};
}

// ---------------------------------------------------------------------------
// LDS barrier words. Two encodings of the same pending-count-and-phase
// barrier, chosen per kernel (both waiters and arrivers of one barrier use the
// same one):
//
//  * Counter<E>: the word counts arrivals. A barrier that expects E arrivals
//    per phase has completed floor(count / E) phases; its phase bit is the
//    parity of that number. Arrivals for the next phase of a slot cannot start
//    before the current phase completes (the ring's handshake orders them), so
//    the count never runs ahead. An arrival is one non-returning ds_add: no
//    wave waits for it, and the phase flips with the last arrival.
//  * Flip<E>: bit 31 is the phase, bits 0..30 count the arrivals of the
//    current phase. The last arriver (it learns so from the returned count)
//    adds 2^31 - E, which clears the count and flips the phase in a second
//    atomic. Arrivals wait for their atomic to return, and the phase flips one
//    LDS round trip after the last arrival. The tile copy runs faster on this
//    slower hand-off (measured), the row sum and the GEMM on Counter.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t bar_read(uint32_t* bar) {
  return __hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <uint32_t E>
struct Counter {
  static __device__ __forceinline__ uint32_t phase(uint32_t word) { return (word / E) & 1u; }
  // The word after `phases` completed phases and no arrival of the next one.
  static __device__ __forceinline__ uint32_t settled(uint32_t phases) { return phases * E; }
  // One arrival on behalf of the whole wave (lane 0).
  static __device__ __forceinline__ void arrive(uint32_t* bar) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane_id() == 0)
      (void)__hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
};

template <uint32_t E>
struct Flip {
  static constexpr uint32_t kPhaseBit = 0x80000000u;
  static __device__ __forceinline__ uint32_t phase(uint32_t word) { return word >> 31; }
  static __device__ __forceinline__ uint32_t settled(uint32_t phases) {
    return (phases & 1u) << 31;
  }
  static __device__ __forceinline__ void arrive(uint32_t* bar) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane_id() == 0) {
      const uint32_t old = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_WORKGROUP);
      if ((old & ~kPhaseBit) + 1u == E)  // completes the phase: count to 0, phase flips
        __hip_atomic_fetch_add(bar, kPhaseBit - E, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
};

// Wait until barrier B's phase differs from `phase`. Returns false on timeout.
template <class B>
__device__ __forceinline__ bool bar_wait(uint32_t* bar, uint32_t phase, uint32_t spin_limit) {
  uint32_t polls = 0;
  while (true) {
    const uint32_t w = uniform(bar_read(bar));
    if (B::phase(w) != phase) break;
    if (++polls >= spin_limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

// ---------------------------------------------------------------------------
// Trace records (PIPE_TRACE_WORDS = 8 words each): workgroup 0 only, record
// 2 t + event for the t-th tile (stage) of its stream, while it fits `cap`.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void trace_write(uint32_t* trace, int cap, int t, int event,
                                            const PipeState& st, int wave) {
  if (trace == nullptr || blockIdx.x != 0) return;
  const int rec = 2 * t + event;
  if (rec >= cap) return;
  if (lane_id() == 0) {
    const uint64_t now = __builtin_amdgcn_s_memrealtime();
    uint32_t* r = trace + (size_t)rec * 8;
    r[0] = (uint32_t)event;
    r[1] = (uint32_t)t;
    r[2] = (uint32_t)st.index;
    r[3] = st.phase;
    r[4] = st.count;
    r[5] = (uint32_t)wave;
    r[6] = (uint32_t)now;
    r[7] = (uint32_t)(now >> 32);
  }
}

// ---------------------------------------------------------------------------
// Debug kernels: a wave-uniform pseudo-random pause (stress runs shift the
// waves' relative timing with it) and the status bit of a failed check.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void jitter_pause(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t h = a * 0x9E3779B1u ^ b * 0x85EBCA77u ^ c * 0xC2B2AE3Du;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  for (uint32_t i = uniform(h & 15u); i > 0; --i) __builtin_amdgcn_s_sleep(4);
}

__device__ __forceinline__ void flag_invariant(uint32_t* status) {
  if (lane_id() == 0) atomicOr(status, kStatusInvariant);
}

// ---------------------------------------------------------------------------
// Wait counters (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt_hi[15:14]).
// ---------------------------------------------------------------------------
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// s_waitcnt vmcnt(k * STEP) for a wave-uniform k >= 0 (a chain of scalar
// compares, since the count is an immediate). Nothing is emitted when
// k * STEP > 63: the counter never holds more than 63 operations (issue stalls
// first), so the operation waited for has already completed.
template <int STEP, int K = 0>
__device__ __forceinline__ void wait_vmcnt_mul(int k) {
  if constexpr (K * STEP <= 63) {
    if (k == K) {
      wait_vmcnt<K * STEP>();
      return;
    }
    wait_vmcnt_mul<STEP, K + 1>(k);
  }
}

// producer_acquire with eager commits. Waits until slot `index` is released
// (its EMPTY barrier left phase `phase`). While the slot is still in use and
// this wave has at least `eager_min` tiles in flight that it has not yet
// committed (eager_min = 0: never), it commits the oldest of them on its FULL
// barrier (once its LOADS loads have landed, i.e. at most
// LOADS * (pending - 1) remain outstanding) instead of idling: the consumers
// may be waiting for exactly that tile, and holding it back until the next
// issue would put a consumer release and a producer wake-up between every two
// hand-offs. With eager_min = 2 the newest tile in flight is never waited for
// here, so the producer does not stall its next issue on a load it has only
// just begun. Returns false on timeout.
template <int LOADS, int S, class EMPTY, class FULL>
__device__ __forceinline__ bool acquire_slot(uint32_t* empty_bar, uint32_t phase,
                                             uint32_t* full_bars, int index, int& pending,
                                             int eager_min, uint32_t spin_limit) {
  uint32_t polls = 0;
  while (EMPTY::phase(uniform(bar_read(empty_bar))) == phase) {
    if (eager_min > 0 && pending >= eager_min) {
      wait_vmcnt_mul<LOADS>(pending - 1);
      int oldest = index - pending;
      if (oldest < 0) oldest += S;
      FULL::arrive(&full_bars[oldest]);
      --pending;
      continue;
    }
    if (++polls >= spin_limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

// ---------------------------------------------------------------------------
// Copy engine: one wave-wide direct-to-LDS load of 64 x 16 B.
// Lane l's 16 bytes land at LDS address m0 + 16*l.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void dma_block(const void* gptr, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "{m0}"(lds_base)
               : "memory");
}

// Same, with the non-temporal hint (streamed data that is read once).
__device__ __forceinline__ void dma_block_nt(const void* gptr, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(gptr), "{m0}"(lds_base)
               : "memory");
}

// ---------------------------------------------------------------------------
// Swizzle: the 16-byte chunk c of tile row r lives at chunk position
// c ^ ((r >> shift) & 7) of that row (shift 0 = the 128-byte pattern of the
// page's Sw<3,4,3> layout). An involution, so position -> chunk is the same map.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int r, int c, int shift) {
  return c ^ ((r >> shift) & (kChunksPerRow - 1));
}

// The same XOR over a row of CPR chunks (wider tiles): position -> chunk and
// chunk -> position alike.
template <int CPR>
__device__ __forceinline__ int swz_n(int r, int c, int shift) {
  return c ^ ((r >> shift) & (CPR - 1));
}

// ---------------------------------------------------------------------------
// Cross-lane sums.
// ---------------------------------------------------------------------------
// Sum over each aligned group of 8 lanes (DPP quad permutes + half mirror).
__device__ __forceinline__ float sum8_lanes(float v) {
  int x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false)); // row_half_mirror
  return v;
}

// Sum over each aligned group of CPR lanes (8, 16 or 32), result in every lane.
template <int CPR>
__device__ __forceinline__ float sum_lanes(float v) {
  v = sum8_lanes(v);
  if constexpr (CPR >= 16) v += __shfl_xor(v, 8, kWave);
  if constexpr (CPR >= 32) v += __shfl_xor(v, 16, kWave);
  return v;
}

// Integer sum over all 64 lanes, result in every lane.
__device__ __forceinline__ uint32_t sum64_lanes_u32(uint32_t v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace pipe
