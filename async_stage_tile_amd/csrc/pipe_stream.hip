// Warp-specialised tile stream: PW producer waves fill an S-slot LDS ring with
// direct-to-LDS loads; C consumer waves copy each tile back out (with optional
// per-tile checksums) or reduce it into fp32 row sums.
//
// Follows "cute（12）async_pipeline": producer loop = acquire (wait on empty)
// -> copy into slot `index` -> commit -> ++ (section 3.1, code listing);
// consumer loop = wait on full -> use slot `index` -> release -> ++ (3.2);
// producer_tail waits S more empty phases (6.9); the producer starts at
// phase 1 (2.3). The tile use of the copy is the write-back of
// "cute（11）hopper之TMA_copy" (code step 6, section 4).
//
// Work decomposition: tiles are 16 KiB, 128 rows x 64 fp16 (the pages' tile)
// or the wider 64 x 128 and 32 x 256 (TileShape<TC>, TC = tile columns). A
// strip is one tile column walked downwards (copy default) or one tile row
// walked along the columns (rowsum, or copy with PIPE_FLAG_ROW_STRIPS). Each
// strip is cut into `split` segments; item i is segment i / n_strips of strip i % n_strips, so
// workgroups launched together touch neighbouring strips. A segment is either
// a contiguous run of the strip's tiles, or (interleaved) every split-th tile
// starting at the segment index, so that the workgroups sharing a strip read
// neighbouring tiles at the same time. A workgroup walks
// items blockIdx.x, blockIdx.x + gridDim.x, ... and its cursors run on across
// items (a persistent ring). With `xcd_remap`, the item a workgroup takes is
// permuted so that the workgroups of one XCD (dispatch is round-robin over
// the 8 XCDs) stream neighbouring strips.
//
// Ragged edges: when M or N is not a multiple of the tile, the host launches
// the MASKED instantiation. Every producer lane still issues its DMA (so each
// instruction counts once in vmcnt); a lane whose (row, chunk) lies outside
// the matrix fetches the matrix's first chunk instead, and consumers skip the
// out-of-range positions when they store, checksum or sum. Divisible shapes
// run the unmasked instantiation, which carries none of these tests.
//
// Slot layout: a tile row of CPR 16-byte chunks (CPR = 8, 16, 32 for TC = 64,
// 128, 256) holds chunk c at position c ^ ((r >> shift) & (CPR - 1)). One
// producer DMA instruction q moves the 1 KiB block of rows RPB*q ..
// RPB*(q+1) - 1 (RPB = 64 / CPR rows per block): lane l writes position
// l % CPR of row RPB*q + l / CPR, so it fetches the global chunk
// swz_n(row, l % CPR). With PW producer waves (1, 2 or 4), wave w
// issues blocks (16/PW)w .. (16/PW)(w+1)-1 of every tile and full[s] expects PW
// arrivals. A wave may keep `lag` committed-later tiles in flight as long as
// (lag + 1) * 16/PW loads fit the 63-entry vmcnt counter: lag <= 2, 6, 14.
//
// Kernel families in this file, all on this ring and slot layout:
//   stream_kernel        the ring above (every default copy and row sum);
//   stream_group_kernel  copies down strips of G neighbouring tile columns,
//                        whose consumers store a tile row of G tiles at once;
//   stream_group_load_kernel  the same strips of 4 tile columns, whose
//                        producers also load a tile row of the 4 tiles at once;
//   stream_regs_kernel   producers that load into registers and write the
//                        slots with ds_write_b128 instead of direct-to-LDS;
//   stream_debug_kernel  the ring with its protocol checks compiled in.
//
// The kernels are compiled once per stage count: this file is built several
// times, each object instantiating the stage counts PIPE_STREAM_STAGES_LO ..
// PIPE_STREAM_STAGES_HI (so the instantiations compile in parallel).
#include <type_traits>

#include "pipe_device.hpp"
#include "pipe_kernels.hpp"
#include "pipe_rowsum.hpp"

namespace pipe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int S, int C>
struct StreamLds {
  uint8_t slots[S][kTileBytes];
  uint32_t full[S];
  uint32_t empty[S];
  uint32_t fin[S];         // checksum: consumer waves done with the slot's tile
  uint32_t part[S][C];     // checksum: per-wave partial sums
};

__device__ __forceinline__ void trace_record(const StreamParams& p, int t, int event,
                                             const PipeState& st, int wave) {
  trace_write(p.trace, p.trace_cap, t, event, st, wave);
}

// Work item taken by the workgroup for its n-th item slot.
__device__ __forceinline__ int item_index(const StreamParams& p, int slot_item) {
  if (!p.xcd_remap) return slot_item;
  const int per = p.items >> 3;  // items % 8 == 0 whenever xcd_remap is set
  return (slot_item & 7) * per + (slot_item >> 3);
}

__device__ __forceinline__ void tile_coords(const StreamParams& p, int item, int k,
                                            int& tile_row, int& tile_col) {
  int strip = item % p.n_strips;
  int seg = item / p.n_strips;
  int pos = p.interleave ? seg + k * p.split : seg * p.seg_len + k;
  if (p.row_strips) {
    tile_row = strip;
    tile_col = pos;
  } else {
    tile_row = pos;
    tile_col = strip;
  }
}

__device__ __forceinline__ int item_len(const StreamParams& p, int item) {
  int seg = item / p.n_strips;
  if (p.interleave) return (p.strip_len - seg + p.split - 1) / p.split;
  int start = seg * p.seg_len;
  int len = p.strip_len - start;
  return len < p.seg_len ? len : p.seg_len;
}

// Grouped column strips (copy, 128 x 64 tiles): strip i spans the G tile
// columns G*i .. G*i + G - 1 and is walked one tile row at a time, the G tiles
// of a tile row back to back. Segments and their lengths count tile rows.
template <int G>
__device__ __forceinline__ void group_tile_coords(const StreamParams& p, int item, int k,
                                                  int& tile_row, int& tile_col) {
  const int strip = item % p.n_strips;
  const int seg = item / p.n_strips;
  const int kr = k / G;
  tile_row = p.interleave ? seg + kr * p.split : seg * p.seg_len + kr;
  tile_col = strip * G + k % G;
}

template <int G>
__device__ __forceinline__ int group_item_len(const StreamParams& p, int item) {
  return G * item_len(p, item);
}

// Rows and columns of tile (tr, tc) inside the matrix (the full tile except at
// ragged edges); wave-uniform.
template <int TC>
__device__ __forceinline__ int rows_in(const StreamParams& p, int tr) {
  constexpr int R = TileShape<TC>::kRows;
  const int64_t left = p.M - (int64_t)tr * R;
  return left < R ? (int)left : R;
}
template <int TC>
__device__ __forceinline__ int cols_in(const StreamParams& p, int tc) {
  const int64_t left = p.N - (int64_t)tc * TC;
  return left < TC ? (int)left : TC;
}

// ---------------------------------------------------------------------------
// Producer waves
// ---------------------------------------------------------------------------
// Barrier encoding per op: the copy runs faster on the two-step Flip hand-off,
// the row sum on Counter (measured on MI355X).
template <int OP, uint32_t E>
using StreamBar = typename std::conditional<OP == kOpCopy, Flip<E>, Counter<E>>::type;

template <int S, int C, int PW, int OP, bool MASKED, int TC, int G = 1, bool DBG = false>
__device__ void producer(const StreamParams& p, StreamLds<S, C>& lds, int pw) {
  using Sh = TileShape<TC>;
  using FullBar = StreamBar<OP, PW>;
  using EmptyBar = StreamBar<OP, C>;
  constexpr int kLoads = kBlocksPerTile / PW;  // DMA instructions per tile per wave
  static_assert((stream_max_lag(PW) + 1) * kLoads <= 63,
                "vmcnt counts at most 63 outstanding loads");
  const int lane = lane_id();
  const int lrow = lane >> Sh::kLog2ChunksPerRow;  // row within a 1 KiB block
  const int lpos = lane & (Sh::kChunksPerRow - 1);  // chunk position within the row
  const int lag = p.lag;
  PipeState w = producer_start(S, p.start_phase);
  int pending = 0;  // tiles issued but not yet committed (their full not arrived)
  int t = 0;
  bool ok = true;

  for (int it = blockIdx.x; ok && it < p.items; it += gridDim.x) {
    const int item = item_index(p, it);
    const int len = G == 1 ? item_len(p, item) : group_item_len<G>(p, item);
    for (int k = 0; k < len; ++k, ++t) {
      if constexpr (DBG) {
        if (p.jitter) jitter_pause(blockIdx.x, pw, t);
      }
      // producer_acquire: wait until consumers released this slot (committing
      // landed tiles meanwhile, unless commits are lazy).
      if (!acquire_slot<kLoads, S, EmptyBar, FullBar>(&lds.empty[w.index], w.phase, lds.full,
                                                      w.index, pending, p.eager,
                                                      p.spin_limit)) {
        ok = false;
        break;
      }
      if constexpr (DBG) {
        // The slot's consumers have released its previous uses and no other:
        // its next use is not committed yet. The cursor is the closed form.
        const uint32_t uses = (uint32_t)(t / S);
        if (uniform(bar_read(&lds.empty[w.index])) != EmptyBar::settled(uses) ||
            w.index != t % S || w.phase != (p.start_phase ^ (uses & 1u)))
          flag_invariant(p.status);
      }
      if (pw == 0) trace_record(p, t, 0, w, 0);
      int tr, tc;
      if constexpr (G == 1)
        tile_coords(p, item, k, tr, tc);
      else
        group_tile_coords<G>(p, item, k, tr, tc);
      const uint8_t* g =
          p.src + (int64_t)tr * Sh::kRows * p.ld_src + (int64_t)tc * Sh::kRowBytes;
      const uint32_t slot = uniform(lds_addr(&lds.slots[w.index][0]));
      if constexpr (MASKED) {
        const int rin = rows_in<TC>(p, tr), cin = cols_in<TC>(p, tc);
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          const int q = pw * kLoads + j;
          const int r = q * Sh::kRowsPerBlock + lrow;
          const int c = swz_n<Sh::kChunksPerRow>(r, lpos, p.swz_shift);
          const uint8_t* a = g + (int64_t)r * p.ld_src + c * kChunkBytes;
          dma_block((r < rin && c * 8 < cin) ? a : p.src, slot + q * kBlockBytes);
        }
      } else if (p.nt) {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          const int q = pw * kLoads + j;
          const int r = q * Sh::kRowsPerBlock + lrow;
          const int c = swz_n<Sh::kChunksPerRow>(r, lpos, p.swz_shift);
          dma_block_nt(g + (int64_t)r * p.ld_src + c * kChunkBytes, slot + q * kBlockBytes);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          const int q = pw * kLoads + j;
          const int r = q * Sh::kRowsPerBlock + lrow;
          const int c = swz_n<Sh::kChunksPerRow>(r, lpos, p.swz_shift);
          dma_block(g + (int64_t)r * p.ld_src + c * kChunkBytes, slot + q * kBlockBytes);
        }
      }
      ++pending;
      // Commit the oldest in-flight tile once `lag` newer tiles are in flight:
      // its loads are done when at most kLoads*(pending-1) remain outstanding.
      if (pending > lag) {
        wait_vmcnt_mul<kLoads>(pending - 1);
        int oldest = w.index - (pending - 1);
        if (oldest < 0) oldest += S;
        FullBar::arrive(&lds.full[oldest]);
        --pending;
      }
      w.inc();
    }
  }
  // Commit whatever is still in flight, oldest first.
  while (pending > 0) {
    wait_vmcnt_mul<kLoads>(pending - 1);
    int oldest = w.index - pending;
    if (oldest < 0) oldest += S;
    FullBar::arrive(&lds.full[oldest]);
    --pending;
  }
  // producer_tail: S more empty phases, so every slot has been drained.
  if (ok) {
    for (int i = 0; i < S; ++i) {
      if (!bar_wait<EmptyBar>(&lds.empty[w.index], w.phase, p.spin_limit)) {
        ok = false;
        break;
      }
      w.inc();
    }
  }
  wait_vmcnt<0>();
  if (!ok && lane == 0) atomicOr(p.status, kStatusTimeoutProducer);
}

// ---------------------------------------------------------------------------
// Consumer waves
// ---------------------------------------------------------------------------
template <int S, int C, int PW, int OP, bool MASKED, int TC, bool DBG = false>
__device__ void consumer(const StreamParams& p, StreamLds<S, C>& lds, int cw) {
  using Sh = TileShape<TC>;
  using FullBar = StreamBar<OP, PW>;
  using EmptyBar = StreamBar<OP, C>;
  constexpr int NB = (kBlocksPerTile + C - 1) / C;  // blocks per wave (last may idle)
  const int lane = lane_id();
  const int lrow = lane >> Sh::kLog2ChunksPerRow;
  const int lpos = lane & (Sh::kChunksPerRow - 1);
  PipeState rd = consumer_start(S);
  float acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = 0.f;
  int t = 0;
  bool ok = true;

  for (int it = blockIdx.x; ok && it < p.items; it += gridDim.x) {
    const int item = item_index(p, it);
    const int len = item_len(p, item);
    int tr = 0, tc = 0;
    for (int k = 0; k < len; ++k, ++t) {
      if constexpr (DBG) {
        if (p.jitter) jitter_pause(blockIdx.x, PW + cw, t);
      }
      // consumer_wait: the slot's full phase must have completed.
      if (!bar_wait<FullBar>(&lds.full[rd.index], rd.phase, p.spin_limit)) {
        ok = false;
        break;
      }
      uint32_t full_seen = 0;
      if constexpr (DBG) {
        // Exactly this use of the slot is committed: the next one needs this
        // wave's release first. The cursor is the closed form.
        const uint32_t uses = (uint32_t)(t / S);
        full_seen = uniform(bar_read(&lds.full[rd.index]));
        if (full_seen != FullBar::settled(uses + 1) || rd.index != t % S ||
            rd.phase != (uses & 1u))
          flag_invariant(p.status);
        if (p.early_release) {
          // Test only: release before reading (the mistake that lets the
          // producer overwrite live data), then give it time to do so.
          EmptyBar::arrive(&lds.empty[rd.index]);
          for (int i = 0; i < 64; ++i) __builtin_amdgcn_s_sleep(8);
        }
      }
      if (cw == 0) trace_record(p, t, 1, rd, 1 + cw);
      tile_coords(p, item, k, tr, tc);
      int rin = Sh::kRows, cin = TC;
      if constexpr (MASKED) {
        rin = rows_in<TC>(p, tr);
        cin = cols_in<TC>(p, tc);
      }
      const uint8_t* slot = &lds.slots[rd.index][0];
      uint4 v[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int q = cw + j * C;
        if (q < kBlocksPerTile)
          v[j] = *reinterpret_cast<const uint4*>(slot + q * kBlockBytes + lane * kChunkBytes);
      }
      if constexpr (OP == kOpCopy) {
        uint32_t csum = 0;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int q = cw + j * C;
          if (q < kBlocksPerTile) {
            const int r = q * Sh::kRowsPerBlock + lrow;
            const int c = swz_n<Sh::kChunksPerRow>(r, lpos, p.swz_shift);
            if constexpr (MASKED) {
              if (r >= rin || c * 8 >= cin) continue;
            }
            uint8_t* gd = p.dst + ((int64_t)tr * Sh::kRows + r) * p.ld_dst +
                          (int64_t)tc * Sh::kRowBytes + c * kChunkBytes;
            if (p.nt) {
              const u32x4 nv = {v[j].x, v[j].y, v[j].z, v[j].w};
              __builtin_nontemporal_store(nv, reinterpret_cast<u32x4*>(gd));
            } else {
              *reinterpret_cast<uint4*>(gd) = v[j];
            }
            if (p.checksums) {
              csum += (v[j].x & 0xFFFFu) + (v[j].x >> 16) + (v[j].y & 0xFFFFu) + (v[j].y >> 16) +
                      (v[j].z & 0xFFFFu) + (v[j].z >> 16) + (v[j].w & 0xFFFFu) + (v[j].w >> 16);
            }
          }
        }
        wait_lgkmcnt0();
        if (p.checksums) {
          // Per-wave partial -> LDS; the last wave to finish the tile adds the
          // partials and writes the tile's checksum before it releases.
          csum = sum64_lanes_u32(csum);
          if (lane == 0) lds.part[rd.index][cw] = csum;
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          uint32_t before = 0;
          if (lane == 0)
            before = __hip_atomic_fetch_add(&lds.fin[rd.index], 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_WORKGROUP);
          before = uniform(before);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          if (before % C == C - 1) {
            uint32_t tot = 0;
#pragma unroll
            for (int w2 = 0; w2 < C; ++w2) tot += lds.part[rd.index][w2];
            if (lane == 0) p.checksums[(int64_t)tr * p.tile_cols + tc] = tot;
          }
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int q = cw + j * C;
          if (q < kBlocksPerTile) {
            if constexpr (MASKED) {
              // Position lpos of row r holds logical chunk swz(r, lpos).
              const int r = q * Sh::kRowsPerBlock + lrow;
              if (r >= rin || swz_n<Sh::kChunksPerRow>(r, lpos, p.swz_shift) * 8 >= cin) continue;
            }
            const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(w4[e] & 0xFFFFu));
              const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(w4[e] >> 16));
              s += (float)lo;
              s += (float)hi;
            }
            acc[j] += s;
          }
        }
        wait_lgkmcnt0();
      }
      if constexpr (DBG) {
        // Still the same use: nothing was committed into the slot while this
        // wave read it.
        if (uniform(bar_read(&lds.full[rd.index])) != full_seen) flag_invariant(p.status);
      }
      // consumer_release.
      if (!p.no_release && !(DBG && p.early_release)) EmptyBar::arrive(&lds.empty[rd.index]);
      rd.inc();
    }
    if constexpr (OP == kOpRowsum) {
      if (ok && len > 0) {
        const int seg = item / p.n_strips;
        float* o = p.out + (int64_t)seg * p.M + (int64_t)tr * Sh::kRows;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int q = cw + j * C;
          if (q < kBlocksPerTile) {
            const float s = sum_lanes<Sh::kChunksPerRow>(acc[j]);
            const int r = q * Sh::kRowsPerBlock + lrow;
            if (lpos == 0 && (!MASKED || (int64_t)tr * Sh::kRows + r < p.M)) store_partial(&o[r], s);
          }
          acc[j] = 0.f;
        }
        if (p.tickets != nullptr) rowsum_strip_arrive<Sh::kRows, C>(p, item % p.n_strips);
      }
    }
  }
  if (!ok && lane == 0) atomicOr(p.status, kStatusTimeoutConsumer);
}

template <int S, int C, int PW, int OP, bool MASKED, int TC>
__global__ void __launch_bounds__(64 * (PW + C)) stream_kernel(StreamParams p) {
  __shared__ StreamLds<S, C> lds;
  const int wave = (int)(threadIdx.x >> 6);
  if (threadIdx.x < S) {
    lds.full[threadIdx.x] = 0u;
    lds.empty[threadIdx.x] = 0u;
    lds.fin[threadIdx.x] = 0u;
  }
  __syncthreads();
  if (wave < PW)
    producer<S, C, PW, OP, MASKED, TC>(p, lds, wave);
  else
    consumer<S, C, PW, OP, MASKED, TC>(p, lds, wave - PW);
}

// ---------------------------------------------------------------------------
// Debug kernel (PIPE_FLAG_DEBUG_CHECKS): the DMA ring of stream_kernel with
// its protocol checks compiled in. A failed check sets kStatusInvariant in the
// status word and the kernel carries on (every wait stays bounded).
// ---------------------------------------------------------------------------
template <int S, int C, int PW, int OP, bool MASKED>
__global__ void __launch_bounds__(64 * (PW + C)) stream_debug_kernel(StreamParams p) {
  __shared__ StreamLds<S, C> lds;
  const int wave = (int)(threadIdx.x >> 6);
  if (threadIdx.x < S) {
    lds.full[threadIdx.x] = 0u;
    lds.empty[threadIdx.x] = 0u;
    lds.fin[threadIdx.x] = 0u;
  }
  __syncthreads();
  if (wave < PW)
    producer<S, C, PW, OP, MASKED, 64, 1, true>(p, lds, wave);
  else
    consumer<S, C, PW, OP, MASKED, 64, true>(p, lds, wave - PW);
}

// ---------------------------------------------------------------------------
// Register producer engine (PIPE_FLAG_PRODUCER_VGPR; 128 x 64 tiles): each
// producer wave loads its blocks of a tile with global_load_dwordx4 into
// registers, 8 lanes per 128-byte row piece in natural chunk order, and writes
// them with ds_write_b128 at the swizzled slot position; the slot layout is
// the DMA engine's. The loads run D - 1 tiles ahead of the writes (D register
// buffers; the loads do not need a slot), and a tile is committed as soon as
// its writes have returned (lgkmcnt), so the commit lag and commit policies
// of the DMA engine do not apply.
// ---------------------------------------------------------------------------
struct TileWalk {
  int it;    // work-item slot: blockIdx.x + n * gridDim.x
  int item;  // the item it names (after the XCD permutation)
  int len;   // tiles of the item
  int k;     // tile within the item
};

// Move to the next tile that exists (the first of the next item when this
// item is used up).
__device__ __forceinline__ void walk_settle(const StreamParams& p, TileWalk& w) {
  while (w.it < p.items && w.k >= w.len) {
    w.it += gridDim.x;
    w.k = 0;
    if (w.it < p.items) {
      w.item = item_index(p, w.it);
      w.len = item_len(p, w.item);
    }
  }
}

__device__ __forceinline__ TileWalk walk_start(const StreamParams& p) {
  TileWalk w{(int)blockIdx.x, 0, 0, 0};
  if (w.it < p.items) {
    w.item = item_index(p, w.it);
    w.len = item_len(p, w.item);
  }
  walk_settle(p, w);
  return w;
}

// Loads of one tile's blocks for producer wave `pw`; with `valid` false (past
// the workgroup's last tile) the same number of loads re-read the matrix's
// first chunks, so that every step issues the same instructions and the
// compiler can count the loads still in flight exactly.
template <int PW, bool MASKED, bool NT>
__device__ __forceinline__ void load_tile_regs(const StreamParams& p, const TileWalk& w,
                                               bool valid, int pw,
                                               uint4 (&v)[kBlocksPerTile / PW]) {
  constexpr int kLoads = kBlocksPerTile / PW;
  const int lane = lane_id();
  const int lrow = lane >> 3, lchunk = lane & 7;
  int tr = 0, tc = 0;
  if (valid) tile_coords(p, w.item, w.k, tr, tc);
  const uint8_t* g = p.src + (int64_t)tr * kTileRows * p.ld_src + (int64_t)tc * kRowBytes +
                     lchunk * kChunkBytes;
  int rin = valid ? kTileRows : 0, cin = kTileCols;
  if constexpr (MASKED) {
    if (valid) {
      rin = rows_in<64>(p, tr);
      cin = cols_in<64>(p, tc);
    }
  }
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int r = (pw * kLoads + j) * kRowsPerBlock + lrow;
    const uint8_t* a = g + (int64_t)r * p.ld_src;
    if (r >= rin || lchunk * 8 >= cin) a = p.src;  // in bounds; nobody uses it
    u32x4 x;
    if constexpr (NT)
      x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
    else
      x = *reinterpret_cast<const u32x4*>(a);
    v[j] = uint4{x.x, x.y, x.z, x.w};
  }
}

// Register buffers per producer wave: tiles in flight, D - 1 of them ahead
// of the one being written (4 waves: 4 buffers of 16 VGPRs; 1 wave: 2 of 64).
template <int PW>
constexpr int regs_depth() { return PW == 1 ? 2 : 4; }

// One tile: issue the loads of the tile D - 1 ahead into `ahead_regs`, then
// write `cur` (whose loads the compiler waits for) into the acquired slot and
// commit it. Returns false on a timeout.
template <int S, int C, int PW, int OP, bool MASKED, bool NT>
__device__ __forceinline__ bool regs_step(const StreamParams& p, StreamLds<S, C>& lds, int pw,
                                          TileWalk& ahead, PipeState& st, int& t,
                                          const uint4 (&cur)[kBlocksPerTile / PW],
                                          uint4 (&ahead_regs)[kBlocksPerTile / PW]) {
  using FullBar = StreamBar<OP, PW>;
  using EmptyBar = StreamBar<OP, C>;
  constexpr int kLoads = kBlocksPerTile / PW;
  const bool valid = ahead.it < p.items;
  load_tile_regs<PW, MASKED, NT>(p, ahead, valid, pw, ahead_regs);
  if (valid) {
    ++ahead.k;
    walk_settle(p, ahead);
  }
  // producer_acquire (no commits pending: every earlier tile is committed).
  if (!bar_wait<EmptyBar>(&lds.empty[st.index], st.phase, p.spin_limit)) return false;
  if (pw == 0) trace_record(p, t, 0, st, 0);
  const int lane = lane_id();
  const int lrow = lane >> 3, lchunk = lane & 7;
  uint8_t* slot = &lds.slots[st.index][0];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int r = (pw * kLoads + j) * kRowsPerBlock + lrow;
    *reinterpret_cast<uint4*>(slot + r * kRowBytes + swz(r, lchunk, p.swz_shift) * kChunkBytes) =
        cur[j];
  }
  wait_lgkmcnt0();  // the tile's writes have landed: commit
  FullBar::arrive(&lds.full[st.index]);
  st.inc();
  ++t;
  return true;
}

template <int S, int C, int PW, int OP, bool MASKED, bool NT>
__device__ void producer_regs(const StreamParams& p, StreamLds<S, C>& lds, int pw) {
  using EmptyBar = StreamBar<OP, C>;
  constexpr int kLoads = kBlocksPerTile / PW;
  constexpr int D = regs_depth<PW>();
  PipeState st = producer_start(S, p.start_phase);
  int tiles = 0;  // tiles of this workgroup
  for (int it = blockIdx.x; it < p.items; it += gridDim.x) tiles += item_len(p, item_index(p, it));
  TileWalk ahead = walk_start(p);
  uint4 buf[D][kLoads];
  // Prologue: the first D - 1 tiles.
#pragma unroll
  for (int i = 0; i < D - 1; ++i) {
    const bool valid = ahead.it < p.items;
    load_tile_regs<PW, MASKED, NT>(p, ahead, valid, pw, buf[i]);
    if (valid) {
      ++ahead.k;
      walk_settle(p, ahead);
    }
  }
  bool ok = true;
  int t = 0;
  // Whole rounds of D tiles: every step runs, so each buffer's loads are
  // waited for exactly (not drained) before its writes.
  while (ok && t + D <= tiles) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      ok = regs_step<S, C, PW, OP, MASKED, NT>(p, lds, pw, ahead, st, t, buf[i],
                                               buf[(i + D - 1) % D]);
      if (!ok) break;
    }
  }
  // The last tiles (fewer than D), continuing the buffer rotation.
#pragma unroll
  for (int i = 0; i < D - 1; ++i) {
    if (ok && t < tiles)
      ok = regs_step<S, C, PW, OP, MASKED, NT>(p, lds, pw, ahead, st, t, buf[i],
                                               buf[(i + D - 1) % D]);
  }
  // producer_tail: S more empty phases, so every slot has been drained.
  if (ok) {
    for (int i = 0; i < S; ++i) {
      if (!bar_wait<EmptyBar>(&lds.empty[st.index], st.phase, p.spin_limit)) {
        ok = false;
        break;
      }
      st.inc();
    }
  }
  if (!ok && lane_id() == 0) atomicOr(p.status, kStatusTimeoutProducer);
}

template <int S, int C, int PW, int OP, bool MASKED, bool NT>
__global__ void __launch_bounds__(64 * (PW + C)) stream_regs_kernel(StreamParams p) {
  __shared__ StreamLds<S, C> lds;
  const int wave = (int)(threadIdx.x >> 6);
  if (threadIdx.x < S) {
    lds.full[threadIdx.x] = 0u;
    lds.empty[threadIdx.x] = 0u;
    lds.fin[threadIdx.x] = 0u;
  }
  __syncthreads();
  if (wave < PW)
    producer_regs<S, C, PW, OP, MASKED, NT>(p, lds, wave);
  else
    consumer<S, C, PW, OP, MASKED, 64>(p, lds, wave - PW);
}

// ---------------------------------------------------------------------------
// Grouped copy consumers (128 x 64 tiles, divisible shapes): each consumer
// wave waits on the G slots that hold one tile row of a grouped strip, stores
// its share of those G tiles, then releases all G. One store instruction
// covers 8/G rows of the group, G*128 contiguous bytes per row, where the
// per-tile consumer stores 8 rows of 128 bytes: the rows of neighbouring tiles
// reach memory as one run. Lane l takes tile (l/16) % G, rows 2*((l/16)/G) and
// 2*((l/16)/G) + 1 of the instruction's rows, chunk position l % 8; so each 16
// lanes read 256 contiguous bytes of one slot (no bank conflicts). The
// producer's commit lag must be at most S - G, or the tile that completes a
// group can be held back while the producer waits for that group's slots.
// ---------------------------------------------------------------------------
template <int S, int C, int PW, int G>
__device__ void group_consumer(const StreamParams& p, StreamLds<S, C>& lds, int cw) {
  using FullBar = StreamBar<kOpCopy, PW>;
  using EmptyBar = StreamBar<kOpCopy, C>;
  static_assert(G == 2 || G == 4, "groups of 2 or 4 tiles");
  static_assert(G <= S, "a group must fit the ring");
  constexpr int kInstr = G * kBlocksPerTile;  // 1 KiB store instructions per group
  static_assert(kInstr % C == 0, "every wave stores the same share");
  constexpr int NI = kInstr / C;
  constexpr int kRowsPerInstr = kRowsPerBlock / G;
  const int lane = lane_id();
  const int g = (lane >> 4) & (G - 1);
  const int rsub = ((lane >> 4) / G) * 2 + ((lane >> 3) & 1);
  const int pos = lane & (kChunksPerRow - 1);
  PipeState rd = consumer_start(S);
  int t = 0;
  bool ok = true;

  for (int it = blockIdx.x; ok && it < p.items; it += gridDim.x) {
    const int item = item_index(p, it);
    const int len = group_item_len<G>(p, item);
    for (int k = 0; k < len; k += G, t += G) {
      // consumer_wait on each of the group's G slots, in ring order.
      PipeState w = rd;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (!bar_wait<FullBar>(&lds.full[w.index], w.phase, p.spin_limit)) {
          ok = false;
          break;
        }
        if (cw == 0) trace_record(p, t + j, 1, w, 1 + cw);
        w.inc();
      }
      if (!ok) break;
      int tr, tc0;
      group_tile_coords<G>(p, item, k, tr, tc0);
      int si = rd.index + g;
      if (si >= S) si -= S;
      const uint8_t* slot = &lds.slots[si][0];
      uint8_t* gdst = p.dst + (int64_t)tr * kTileRows * p.ld_dst + (int64_t)(tc0 + g) * kRowBytes;
      uint4 v[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = (cw + i * C) * kRowsPerInstr + rsub;
        v[i] = *reinterpret_cast<const uint4*>(slot + r * kRowBytes + pos * kChunkBytes);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = (cw + i * C) * kRowsPerInstr + rsub;
        const int c = swz(r, pos, p.swz_shift);
        uint8_t* gd = gdst + (int64_t)r * p.ld_dst + c * kChunkBytes;
        if (p.nt) {
          const u32x4 nv = {v[i].x, v[i].y, v[i].z, v[i].w};
          __builtin_nontemporal_store(nv, reinterpret_cast<u32x4*>(gd));
        } else {
          *reinterpret_cast<uint4*>(gd) = v[i];
        }
      }
      wait_lgkmcnt0();
      // consumer_release of the G slots, in ring order.
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (!p.no_release) EmptyBar::arrive(&lds.empty[rd.index]);
        rd.inc();
      }
    }
  }
  if (!ok && lane == 0) atomicOr(p.status, kStatusTimeoutConsumer);
}

template <int S, int C, int PW, int G>
__global__ void __launch_bounds__(64 * (PW + C)) stream_group_kernel(StreamParams p) {
  __shared__ StreamLds<S, C> lds;
  const int wave = (int)(threadIdx.x >> 6);
  if (threadIdx.x < S) {
    lds.full[threadIdx.x] = 0u;
    lds.empty[threadIdx.x] = 0u;
    lds.fin[threadIdx.x] = 0u;
  }
  __syncthreads();
  if (wave < PW)
    producer<S, C, PW, kOpCopy, false, 64, G>(p, lds, wave);
  else
    group_consumer<S, C, PW, G>(p, lds, wave - PW);
}


// ---------------------------------------------------------------------------
// Grouped loads (PIPE_FLAG_GROUP_LOADS; 128 x 64 tiles, strips of G = 4 tile
// columns): the producer waits on the 4 consecutive slots that receive one
// tile row of its strip, then fills all 4 with loads that each cover 2 rows x
// 512 contiguous bytes -- the same 128-byte row piece of the 4 neighbouring
// tiles -- and commits the 4 tiles together once those loads have landed.
// Since one direct-to-LDS load writes 1 KiB of contiguous LDS, the 4 slots of
// a group are interleaved: row r of the group's tile g lives at
// slots[first] + r * 512 + g * 128 (its chunks XOR-swizzled as in every
// slot), so a group is one 64 KiB region and S is 4 or 8 (one or two groups).
// Consumers wait on the 4 slots, store 2 rows x 512 bytes per instruction
// (reading 1 KiB of contiguous LDS) and release the 4. The commit lag is at
// most S - 4 tiles, one group when S = 8: the bound that the protocol model
// proves live for a producer and consumers that both take 4 slots at a time.
// ---------------------------------------------------------------------------
constexpr int kGroupTiles = 4;
constexpr int kGroupRowBytes = kGroupTiles * kRowBytes;  // 512

template <int S, int C, int PW>
__device__ void group_load_producer(const StreamParams& p, StreamLds<S, C>& lds, int pw) {
  using FullBar = StreamBar<kOpCopy, PW>;
  using EmptyBar = StreamBar<kOpCopy, C>;
  constexpr int G = kGroupTiles;
  static_assert(S % G == 0, "whole groups of slots");
  constexpr int kLoads = G * kBlocksPerTile / PW;  // loads per group per wave
  // One group of lag when two fit the ring and (lag + 1) groups of loads fit
  // the 63-entry vmcnt counter (4 producer waves: 16 loads per group each;
  // with 2, 32 loads, so each group is committed as soon as it has landed).
  constexpr int kLagFit = 63 / kLoads - 1;
  constexpr int kLagGroups = (S / G - 1) < kLagFit ? (S / G - 1) : kLagFit;
  static_assert((kLagGroups + 1) * kLoads <= 63, "vmcnt counts at most 63 outstanding loads");
  const int lane = lane_id();
  const int lr = lane >> 5;          // row within the load's 2 rows
  const int lg = (lane >> 3) & 3;    // tile of the group
  const int lpos = lane & 7;         // chunk position within the tile row
  PipeState w = producer_start(S, p.start_phase);
  int pending = 0;  // groups issued, not yet committed
  int t = 0;
  bool ok = true;
  for (int it = blockIdx.x; ok && it < p.items; it += gridDim.x) {
    const int item = item_index(p, it);
    const int len = item_len(p, item);  // tile rows of the segment
    for (int k = 0; k < len; ++k, t += G) {
      // producer_acquire of the group's 4 slots, in ring order.
      PipeState a = w;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (!bar_wait<EmptyBar>(&lds.empty[a.index], a.phase, p.spin_limit)) {
          ok = false;
          break;
        }
        if (pw == 0) trace_record(p, t + j, 0, a, 0);
        a.inc();
      }
      if (!ok) break;
      int tr, tc0;
      group_tile_coords<G>(p, item, k * G, tr, tc0);
      const uint8_t* g = p.src + (int64_t)tr * kTileRows * p.ld_src + (int64_t)tc0 * kRowBytes;
      const uint32_t base = uniform(lds_addr(&lds.slots[w.index][0]));
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int i = pw * kLoads + j;  // 1 KiB block i of the group: rows 2i, 2i + 1
        const int r = 2 * i + lr;
        const int c = swz(r, lpos, p.swz_shift);
        const uint8_t* a2 = g + (int64_t)r * p.ld_src + lg * kRowBytes + c * kChunkBytes;
        if (p.nt)
          dma_block_nt(a2, base + i * kBlockBytes);
        else
          dma_block(a2, base + i * kBlockBytes);
      }
      ++pending;
      // Commit the oldest group once kLagGroups younger ones are in flight.
      if (pending > kLagGroups) {
        wait_vmcnt_mul<kLoads>(pending - 1);
        int oldest = w.index - (pending - 1) * G;
        if (oldest < 0) oldest += S;
#pragma unroll
        for (int j = 0; j < G; ++j) FullBar::arrive(&lds.full[oldest + j]);
        --pending;
      }
#pragma unroll
      for (int j = 0; j < G; ++j) w.inc();
    }
  }
  while (pending > 0) {
    wait_vmcnt_mul<kLoads>(pending - 1);
    int oldest = w.index - pending * G;
    if (oldest < 0) oldest += S;
#pragma unroll
    for (int j = 0; j < G; ++j) FullBar::arrive(&lds.full[oldest + j]);
    --pending;
  }
  // producer_tail: S more empty phases, so every slot has been drained.
  if (ok) {
    for (int i = 0; i < S; ++i) {
      if (!bar_wait<EmptyBar>(&lds.empty[w.index], w.phase, p.spin_limit)) {
        ok = false;
        break;
      }
      w.inc();
    }
  }
  wait_vmcnt<0>();
  if (!ok && lane == 0) atomicOr(p.status, kStatusTimeoutProducer);
}

template <int S, int C, int PW>
__device__ void group_load_consumer(const StreamParams& p, StreamLds<S, C>& lds, int cw) {
  using FullBar = StreamBar<kOpCopy, PW>;
  using EmptyBar = StreamBar<kOpCopy, C>;
  constexpr int G = kGroupTiles;
  constexpr int kInstr = G * kBlocksPerTile;  // 1 KiB blocks per group
  static_assert(kInstr % C == 0, "every wave stores the same share");
  constexpr int NI = kInstr / C;
  const int lane = lane_id();
  const int lr = lane >> 5, lg = (lane >> 3) & 3, lpos = lane & 7;
  PipeState rd = consumer_start(S);
  int t = 0;
  bool ok = true;
  for (int it = blockIdx.x; ok && it < p.items; it += gridDim.x) {
    const int item = item_index(p, it);
    const int len = item_len(p, item);
    for (int k = 0; k < len; ++k, t += G) {
      // consumer_wait on the group's 4 slots, in ring order.
      PipeState w = rd;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (!bar_wait<FullBar>(&lds.full[w.index], w.phase, p.spin_limit)) {
          ok = false;
          break;
        }
        if (cw == 0) trace_record(p, t + j, 1, w, 1 + cw);
        w.inc();
      }
      if (!ok) break;
      int tr, tc0;
      group_tile_coords<G>(p, item, k * G, tr, tc0);
      const uint8_t* base = &lds.slots[rd.index][0];
      uint8_t* gdst = p.dst + (int64_t)tr * kTileRows * p.ld_dst + (int64_t)(tc0 + lg) * kRowBytes;
      uint4 v[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        v[i] = *reinterpret_cast<const uint4*>(base + (cw + i * C) * kBlockBytes +
                                               lane * kChunkBytes);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = 2 * (cw + i * C) + lr;
        const int c = swz(r, lpos, p.swz_shift);
        uint8_t* gd = gdst + (int64_t)r * p.ld_dst + c * kChunkBytes;
        if (p.nt) {
          const u32x4 nv = {v[i].x, v[i].y, v[i].z, v[i].w};
          __builtin_nontemporal_store(nv, reinterpret_cast<u32x4*>(gd));
        } else {
          *reinterpret_cast<uint4*>(gd) = v[i];
        }
      }
      wait_lgkmcnt0();
      // consumer_release of the 4 slots, in ring order.
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (!p.no_release) EmptyBar::arrive(&lds.empty[rd.index]);
        rd.inc();
      }
    }
  }
  if (!ok && lane == 0) atomicOr(p.status, kStatusTimeoutConsumer);
}

template <int S, int C, int PW>
__global__ void __launch_bounds__(64 * (PW + C)) stream_group_load_kernel(StreamParams p) {
  __shared__ StreamLds<S, C> lds;
  const int wave = (int)(threadIdx.x >> 6);
  if (threadIdx.x < S) {
    lds.full[threadIdx.x] = 0u;
    lds.empty[threadIdx.x] = 0u;
    lds.fin[threadIdx.x] = 0u;
  }
  __syncthreads();
  if (wave < PW)
    group_load_producer<S, C, PW>(p, lds, wave);
  else
    group_load_consumer<S, C, PW>(p, lds, wave - PW);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int S, int C, int PW, int TC>
static hipError_t launch_scpt(int op, int grid, const StreamParams& p, hipStream_t stream) {
  if constexpr (!stream_shape_supported(S, C, PW, TC)) {
    return hipErrorInvalidValue;
  } else {
    constexpr int R = TileShape<TC>::kRows;
    dim3 block(64 * (PW + C));
    const bool masked = (p.M % R) != 0 || (p.N % TC) != 0;
    if (op == kOpCopy)
      return masked ? launch_or_record(stream_kernel<S, C, PW, kOpCopy, true, TC>, dim3(grid),
                                       block, stream, p)
                    : launch_or_record(stream_kernel<S, C, PW, kOpCopy, false, TC>, dim3(grid),
                                       block, stream, p);
    return masked ? launch_or_record(stream_kernel<S, C, PW, kOpRowsum, true, TC>, dim3(grid),
                                     block, stream, p)
                  : launch_or_record(stream_kernel<S, C, PW, kOpRowsum, false, TC>, dim3(grid),
                                     block, stream, p);
  }
}

template <int S, int C, int PW>
static hipError_t launch_scp(int op, int tile_n, int grid, const StreamParams& p,
                             hipStream_t stream) {
  switch (tile_n) {
    case 64: return launch_scpt<S, C, PW, 64>(op, grid, p, stream);
    case 128: return launch_scpt<S, C, PW, 128>(op, grid, p, stream);
    case 256: return launch_scpt<S, C, PW, 256>(op, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int S, int C>
static hipError_t launch_sc(int op, int pw, int tile_n, int grid, const StreamParams& p,
                            hipStream_t stream) {
  switch (pw) {
    case 1: return launch_scp<S, C, 1>(op, tile_n, grid, p, stream);
    case 2: return launch_scp<S, C, 2>(op, tile_n, grid, p, stream);
    case 4: return launch_scp<S, C, 4>(op, tile_n, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int S>
hipError_t launch_stream_stages(int op, int consumers, int producers, int tile_n, int grid,
                                const StreamParams& p, hipStream_t stream) {
  switch (consumers) {
    case 1: return launch_sc<S, 1>(op, producers, tile_n, grid, p, stream);
    case 2: return launch_sc<S, 2>(op, producers, tile_n, grid, p, stream);
    case 3: return launch_sc<S, 3>(op, producers, tile_n, grid, p, stream);
    case 4: return launch_sc<S, 4>(op, producers, tile_n, grid, p, stream);
    case 8: return launch_sc<S, 8>(op, producers, tile_n, grid, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int S>
hipError_t launch_group_stages(int consumers, int producers, int group, int grid,
                               const StreamParams& p, hipStream_t stream) {
  dim3 block(64 * (producers + consumers));
#define PIPE_GROUP_CASE(C, PW, G)                                                           \
  if constexpr (group_shape_supported(S, C, PW, G)) {                                        \
    if (consumers == C && producers == PW && group == G)                                     \
      return launch_or_record(stream_group_kernel<S, C, PW, G>, dim3(grid), block, stream, p); \
  }
  PIPE_GROUP_CASE(4, 2, 2)
  PIPE_GROUP_CASE(4, 4, 2)
  PIPE_GROUP_CASE(8, 2, 2)
  PIPE_GROUP_CASE(8, 4, 2)
  PIPE_GROUP_CASE(4, 2, 4)
  PIPE_GROUP_CASE(4, 4, 4)
  PIPE_GROUP_CASE(8, 2, 4)
  PIPE_GROUP_CASE(8, 4, 4)
#undef PIPE_GROUP_CASE
  return hipErrorInvalidValue;
}

template <int S>
hipError_t launch_group_load_stages(int consumers, int producers, int grid, const StreamParams& p,
                                    hipStream_t stream) {
  dim3 block(64 * (producers + consumers));
#define PIPE_GROUP_LOAD_CASE(C, PW)                                                           \
  if constexpr (group_load_shape_supported(S, C, PW)) {                                       \
    if (consumers == C && producers == PW)                                                    \
      return launch_or_record(stream_group_load_kernel<S, C, PW>, dim3(grid), block, stream,  \
                              p);                                                             \
  }
  PIPE_GROUP_LOAD_CASE(4, 2)
  PIPE_GROUP_LOAD_CASE(4, 4)
  PIPE_GROUP_LOAD_CASE(8, 2)
  PIPE_GROUP_LOAD_CASE(8, 4)
#undef PIPE_GROUP_LOAD_CASE
  return hipErrorInvalidValue;
}

template <int S, int C, int PW>
static hipError_t launch_debug_scp(int op, int grid, const StreamParams& p, hipStream_t stream) {
  if constexpr (!debug_shape_supported(S, C, PW)) {
    return hipErrorInvalidValue;
  } else {
    const bool masked = (p.M % kTileRows) != 0 || (p.N % kTileCols) != 0;
    const dim3 block(64 * (PW + C));
    if (op == kOpCopy)
      return masked ? launch_or_record(stream_debug_kernel<S, C, PW, kOpCopy, true>, dim3(grid),
                                       block, stream, p)
                    : launch_or_record(stream_debug_kernel<S, C, PW, kOpCopy, false>, dim3(grid),
                                       block, stream, p);
    return masked ? launch_or_record(stream_debug_kernel<S, C, PW, kOpRowsum, true>, dim3(grid),
                                     block, stream, p)
                  : launch_or_record(stream_debug_kernel<S, C, PW, kOpRowsum, false>, dim3(grid),
                                     block, stream, p);
  }
}

template <int S>
hipError_t launch_debug_stages(int op, int consumers, int producers, int grid,
                               const StreamParams& p, hipStream_t stream) {
  if (consumers == 3 && producers == 1) return launch_debug_scp<S, 3, 1>(op, grid, p, stream);
  if (consumers == 4 && producers == 4) return launch_debug_scp<S, 4, 4>(op, grid, p, stream);
  return hipErrorInvalidValue;
}

template <int S, int C, int PW, int OP, bool NT>
static hipError_t launch_regs_op(int grid, const StreamParams& p, hipStream_t stream) {
  const bool masked = (p.M % kTileRows) != 0 || (p.N % kTileCols) != 0;
  const dim3 block(64 * (PW + C));
  return masked ? launch_or_record(stream_regs_kernel<S, C, PW, OP, true, NT>, dim3(grid), block,
                                   stream, p)
                : launch_or_record(stream_regs_kernel<S, C, PW, OP, false, NT>, dim3(grid), block,
                                   stream, p);
}

template <int S, int C, int PW>
static hipError_t launch_regs_scp(int op, int grid, const StreamParams& p, hipStream_t stream) {
  if constexpr (!regs_shape_supported(S, C, PW)) {
    return hipErrorInvalidValue;
  } else {
    if (op == kOpCopy)
      return p.nt ? launch_regs_op<S, C, PW, kOpCopy, true>(grid, p, stream)
                  : launch_regs_op<S, C, PW, kOpCopy, false>(grid, p, stream);
    return p.nt ? launch_regs_op<S, C, PW, kOpRowsum, true>(grid, p, stream)
                : launch_regs_op<S, C, PW, kOpRowsum, false>(grid, p, stream);
  }
}

template <int S>
hipError_t launch_regs_stages(int op, int consumers, int producers, int grid,
                              const StreamParams& p, hipStream_t stream) {
  if (consumers == 3 && producers == 1) return launch_regs_scp<S, 3, 1>(op, grid, p, stream);
  if (consumers == 4 && producers == 1) return launch_regs_scp<S, 4, 1>(op, grid, p, stream);
  if (consumers == 3 && producers == 4) return launch_regs_scp<S, 3, 4>(op, grid, p, stream);
  if (consumers == 4 && producers == 4) return launch_regs_scp<S, 4, 4>(op, grid, p, stream);
  return hipErrorInvalidValue;
}

#if !defined(PIPE_STREAM_STAGES_LO) || !defined(PIPE_STREAM_STAGES_HI)
#error "build with -DPIPE_STREAM_STAGES_LO=<s> -DPIPE_STREAM_STAGES_HI=<s>"
#endif
#define PIPE_STREAM_INSTANTIATE(S)                                                           \
  template hipError_t launch_stream_stages<S>(int, int, int, int, int, const StreamParams&, \
                                              hipStream_t);                                 \
  template hipError_t launch_group_stages<S>(int, int, int, int, const StreamParams&,       \
                                             hipStream_t);                                 \
  template hipError_t launch_group_load_stages<S>(int, int, int, const StreamParams&,        \
                                                  hipStream_t);                            \
  template hipError_t launch_regs_stages<S>(int, int, int, int, const StreamParams&,        \
                                            hipStream_t);                                  \
  template hipError_t launch_debug_stages<S>(int, int, int, int, const StreamParams&,       \
                                             hipStream_t);
#if PIPE_STREAM_STAGES_LO <= 1 && 1 <= PIPE_STREAM_STAGES_HI
PIPE_STREAM_INSTANTIATE(1)
#endif
#if PIPE_STREAM_STAGES_LO <= 2 && 2 <= PIPE_STREAM_STAGES_HI
PIPE_STREAM_INSTANTIATE(2)
#endif
#if PIPE_STREAM_STAGES_LO <= 3 && 3 <= PIPE_STREAM_STAGES_HI
PIPE_STREAM_INSTANTIATE(3)
#endif
#if PIPE_STREAM_STAGES_LO <= 4 && 4 <= PIPE_STREAM_STAGES_HI
PIPE_STREAM_INSTANTIATE(4)
#endif
#if PIPE_STREAM_STAGES_LO <= 5 && 5 <= PIPE_STREAM_STAGES_HI
PIPE_STREAM_INSTANTIATE(5)
#endif
#if PIPE_STREAM_STAGES_LO <= 6 && 6 <= PIPE_STREAM_STAGES_HI
PIPE_STREAM_INSTANTIATE(6)
#endif
#if PIPE_STREAM_STAGES_LO <= 7 && 7 <= PIPE_STREAM_STAGES_HI
PIPE_STREAM_INSTANTIATE(7)
#endif
#if PIPE_STREAM_STAGES_LO <= 8 && 8 <= PIPE_STREAM_STAGES_HI
PIPE_STREAM_INSTANTIATE(8)
#endif

}  // namespace pipe
