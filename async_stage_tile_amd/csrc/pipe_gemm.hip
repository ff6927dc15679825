// GEMM mainloop fed by the tile ring: C = A * B, bf16 inputs, fp32 accumulate.
//
// The ring is the one of the tile stream ("cute（12）async_pipeline", sections
// 1-3 and 6): per stage two producer waves move the A tile (128 x 64) and the
// B tile (64 x 128) of one 64-deep K step into slot `index` with
// direct-to-LDS loads; each waits for its copy to land and arrives on
// full[index], which expects both arrivals (a stage is complete only when all
// its copies have landed, as in the two-copy example of
// "chapter_async_barriers", section 常见的同步规则). Four consumer waves each
// own a 64 x 64 quarter of the 128 x 128 output tile, wait on full, run
// 4 x (2 x 2) v_mfma_f32_32x32x16_bf16 per stage, release empty, and write
// their fp32 accumulators to C after the last K step.
//
// Producer waves: each stage is 32 wave-wide DMA instructions. One wave
// keeping a second stage in flight would need more than the 63 outstanding
// loads vmcnt can count, so the loads are split over PW waves (PW = 2: A and
// B; PW = 4: each half of A and of B), each committing with up to
// min(S - 1, 48 / (32 / PW) - 1) stages of lag, so that the stages in flight
// never exceed 48 outstanding loads per wave.
//
// 256 x 128 output tiles (tile_m = 256): a stage holds 256 x 64 of A (two
// 128-row halves, each laid out as above) and the same 64 x 128 of B; eight
// consumer waves each own a 64 x 64 block, so every B byte in LDS feeds twice
// the MFMAs. The stage's 48 one-KiB DMA blocks (A's 32, then B's 16) are dealt
// out 12 to each of 4 producer waves, and empty expects 8 arrivals.
//
// Consumers read fragments one 16-deep K sub-step ahead of the MFMAs (two
// register buffers), release a slot as soon as their reads of it have
// returned, and wait for the next stage while the last MFMAs still run.
//
// LDS layout of a stage: A rows of 128 B with 16-byte chunk c of row r at
// position c ^ ((r >> shift) & 7) (the MFMA A fragment reads one chunk of 32
// consecutive rows, so the XOR spreads them across banks); B rows of 256 B
// (128 bf16) with chunk c of K-row k at position c ^ fb(k),
// fb(k) = ((k & 3) << 2) ^ (((k >> 3) & 1) << 1), which puts the four K-rows
// (and the two K-halves) that one transposing read touches on different banks.
//
// Column-major B (PIPE_FLAG_GEMM_B_COLMAJOR, gemm_kernel_bcol): a B tile is
// then 128 rows (output columns) of 64 K values, the shape of an A tile, and is
// loaded, swizzled and read exactly like one (one ds_read_b128 per fragment).
//
// Row-major B fragments use the gfx950 transposing LDS read ds_read_b64_tr_b16. Within
// each group of 16 lanes, lane i receives element e (0..3) from the address
// given by lane 4e + i/4 of its group, offset by 2*(i%4) bytes (lane layout
// checked on the device by an index-coded probe). So if lane i of the group
// points at B[k0 + i/4][j0 + 4*(i%4)], it receives B[k0..k0+3][j0 + i]: four
// consecutive K values of its own column, which is half an MFMA B operand.
//
// bf16 output goes through LDS in one of two ways.
//
// Wave-private staging (the default): each MFMA wave rounds its 64 x 64
// quarter to bf16 chunk by chunk (16 rows) into its own 16 x 64 LDS buffer,
// reads it back as 16-byte row pieces and stores 128-byte row segments; no
// other wave is involved.
//
// Store wave (PIPE_FLAG_GEMM_STORE_WAVE): one more wave streams C out of LDS. Each pair of MFMA waves (the two that share 64 output rows)
// owns a one-slot staging ring with its own full/empty barriers, the same
// protocol as the input ring run in the store direction: the pair (producers,
// start phase 1) waits on empty, rounds its accumulators to bf16 and writes
// one 16-row chunk of the tile into the slot, waits for the writes to return
// and arrives on full (2 arrivals); the store wave (consumer) waits on full,
// reads the chunk back as 16-byte row pieces, releases the slot and writes
// 256-byte row segments to C. The MFMA waves thus hand the tile over in
// 4 chunks and move on to the next tile while the store wave drains it.
// Slot rows are padded to 272 bytes so the two half-waves of a fragment write
// (rows r and r + 4) fall on different banks.
//
// Ragged shapes (M not a multiple of the tile height, N of 128 or K of 64;
// N and K multiples of 8, so every 16-byte chunk is wholly inside or outside
// the operands): the host launches the MASKED instantiation. A producer lane
// whose chunk lies outside A or B (a row past M, a column past N, a K index
// past K) loads 16 bytes from a zero-filled device buffer instead, so the slot
// holds exact zeros there -- the out-of-bounds fill of a tensor copy -- and the
// MFMAs add nothing for K past K; the epilogue stores only rows below M and
// columns below N. Divisible shapes run the instantiations without these tests.
//
// MFMA 32x32x16 operand layout (lane l, element e): A[i][k] with i = l % 32,
// k = 8 * (l / 32) + e; B[k][j] with j = l % 32, k = 8 * (l / 32) + e; the
// 16 accumulators hold D[i][j] with j = l % 32,
// i = 8 * (e / 4) + 4 * (l / 32) + e % 4.
#include "pipe_device.hpp"
#include "pipe_kernels.hpp"

namespace pipe {

// The library builds this file as two objects, so that the compiler's work
// splits: PIPE_GEMM_PART=1 defines the warp-specialised rings' launchers,
// PIPE_GEMM_PART=2 the unified GEMMs' launcher (each instantiates only its own
// kernels); without the define, one object holds both.
hipError_t launch_gemm_unified(int stages, int grid, const GemmParams& p, hipStream_t stream);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Source of the zero chunks of ragged-edge stages: never written, so it holds
// the zeros of static device storage for the life of the module.
__device__ __align__(16) uint8_t g_zero_chunks[64];

constexpr int kGemmTile = 128;
constexpr int kGemmK = 64;
constexpr int kAStageBytes = kGemmTile * kGemmK * 2;  // 16 KiB
constexpr int kBStageBytes = kGemmK * kGemmTile * 2;  // 16 KiB
constexpr int kBRowBytes = kGemmTile * 2;             // 256

// MT = 1: 128 x 128 output tiles, 4 MFMA waves. MT = 2: 256 x 128 output
// tiles, 8 MFMA waves, and A stages of 256 x 64 (two 128-row halves, each laid
// out like an MT = 1 A stage), so each B byte brought into LDS feeds twice the
// MFMAs.
template <int S, int MT = 1>
struct GemmLds {
  uint8_t a[S][MT * kAStageBytes];
  uint8_t b[S][kBStageBytes];
  uint32_t full[S];
  uint32_t empty[S];
};

constexpr int kOutRows = 16;                          // rows per staged chunk
constexpr int kOutPitch = kGemmTile * 2 + 16;         // 272 B: padded bf16 row
constexpr int kOutSlotBytes = kOutRows * kOutPitch;   // 4352 B
constexpr int kOutChunks = 64 / kOutRows;             // chunks per wave pair per tile

struct OutLds {
  uint8_t slot[2][kOutSlotBytes];  // one staging slot per MFMA wave pair
  uint32_t full[2];
  uint32_t empty[2];
};

constexpr int kWaveOutPitch = 64 * 2 + 16;                // 144 B: padded 64-column bf16 row
constexpr int kWaveOutBytes = kOutRows * kWaveOutPitch;   // 2304 B per MFMA wave

template <int MT = 1>
struct WaveOutLds {
  uint8_t buf[4 * MT][kWaveOutBytes];
};
static_assert(sizeof(WaveOutLds<2>) == 8 * kWaveOutBytes, "staging buffers are unpadded");

enum GemmEpilogue : int { kEpiF32 = 0, kEpiStoreWave = 1, kEpiWaveStaged = 2 };

__device__ __forceinline__ void gemm_tile_of(const GemmParams& p, int item, int& tm, int& tn) {
  tm = item / p.tiles_n;
  tn = item % p.tiles_n;
}

// B-row chunk swizzle (positions of the 16 chunks of a 256-byte K-row).
__device__ __forceinline__ int swz_b(int k, int on) {
  return on ? (((k & 3) << 2) ^ (((k >> 3) & 1) << 1)) : 0;
}

// Global source of one 16-byte chunk: `a`, or the zero buffer where the chunk
// lies outside the operand (MASKED kernels only).
template <bool MASKED>
__device__ __forceinline__ const uint8_t* chunk_src(const uint8_t* a, bool inside) {
  if constexpr (MASKED) {
    // Selected as integers: a select of the two pointers made the compiler
    // emit an address-space check that does not assemble.
    const uint64_t zero = reinterpret_cast<uint64_t>(&g_zero_chunks[0]);
    return reinterpret_cast<const uint8_t*>(inside ? reinterpret_cast<uint64_t>(a) : zero);
  }
  return a;
}

template <int S, int PW, bool BCOL, bool TRACE = false, int MT = 1, bool MASKED = false>
__device__ __forceinline__ void gemm_producer(const GemmParams& p, GemmLds<S, MT>& lds, int pw) {
  constexpr int kABlocks = 16 * MT;                   // 1 KiB DMA blocks of an A stage
  constexpr int kLoads = (kABlocks + 16) / PW;        // DMA instructions per stage per wave
  constexpr int kMaxLag = 48 / kLoads - 1;            // (lag + 1) stages <= 48 loads
  const int lane = lane_id();
  const bool is_a = pw < PW / 2;                      // first half of the waves load A
  const int part = is_a ? pw : pw - PW / 2;           // which share of the 16 blocks
  PipeState w = producer_start(S, 1u);
  const int lag = S - 1 < kMaxLag ? S - 1 : kMaxLag;
  int pending = 0;
  int t = 0;  // stage ordinal in this workgroup's stream (for the trace)
  bool ok = true;
  for (int item = blockIdx.x; ok && item < p.items; item += gridDim.x) {
    int tm, tn;
    gemm_tile_of(p, item, tm, tn);
    const uint8_t* ga = p.A + (int64_t)tm * (kGemmTile * MT) * p.lda;
    // Row-major B: the tile's columns start tn * 256 bytes into each K-row.
    // Column-major B: its rows (one per output column) start at row tn * 128.
    const uint8_t* gb = BCOL ? p.B + (int64_t)tn * kGemmTile * p.ldb
                             : p.B + (int64_t)tn * kBRowBytes;
    // Rows of A and columns of B that lie inside the operands (MASKED).
    const int a_rows = p.M - tm * kGemmTile * MT;
    const int b_cols = p.N - tn * kGemmTile;
    for (int ks = 0; ks < p.k_steps; ++ks) {
      const int k_left = p.K - ks * kGemmK;  // K indices of this step inside the operands
      if (!acquire_slot<kLoads, S, Counter<4 * MT>, Counter<PW>>(&lds.empty[w.index], w.phase,
                                                             lds.full, w.index, pending, p.eager,
                                                             p.spin_limit)) {
        ok = false;
        break;
      }
      if constexpr (TRACE) {
        if (pw == 0) trace_write(p.trace, p.trace_cap, t, 0, w, 0);
        ++t;
      }
      if constexpr (MT > 1 || MASKED) {
        // The stage's 16 MT + 16 blocks (A first, then B) in order, kLoads
        // per wave; a wave's share may straddle A and B (uniform branch).
        // (The masked kernels take this walk for 128-row tiles too: it deals
        // the same blocks to the same waves as the A/B split below.)
        const uint32_t sa = uniform(lds_addr(&lds.a[w.index][0]));
        const uint32_t sb = uniform(lds_addr(&lds.b[w.index][0]));
        const uint8_t* a0 = ga + (int64_t)ks * kGemmK * 2;
        const uint8_t* b0 = BCOL ? gb + (int64_t)ks * kGemmK * 2 : gb + (int64_t)ks * kGemmK * p.ldb;
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          const int q = pw * kLoads + j;
          if (q < kABlocks) {
            const int r = q * 8 + (lane >> 3);
            const int c = swz(r, lane & 7, p.swz_shift);
            dma_block(chunk_src<MASKED>(a0 + (int64_t)r * p.lda + c * 16,
                                        r < a_rows && c * 8 < k_left),
                      sa + q * kBlockBytes);
          } else if constexpr (BCOL) {
            const int qb = q - kABlocks;
            const int r = qb * 8 + (lane >> 3);
            const int c = swz(r, lane & 7, p.swz_shift);
            dma_block(chunk_src<MASKED>(b0 + (int64_t)r * p.ldb + c * 16,
                                        r < b_cols && c * 8 < k_left),
                      sb + qb * kBlockBytes);
          } else {
            const int qb = q - kABlocks;
            const int r = qb * 4 + (lane >> 4);
            const int c = (lane & 15) ^ swz_b(r, p.b_swz);
            dma_block(chunk_src<MASKED>(b0 + (int64_t)r * p.ldb + c * 16,
                                        r < k_left && c * 8 < b_cols),
                      sb + qb * kBlockBytes);
          }
        }
      } else if (is_a) {
        const uint32_t sa = uniform(lds_addr(&lds.a[w.index][0]));
        const uint8_t* a0 = ga + (int64_t)ks * kGemmK * 2;
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          // A: rows 8q..8q+7, lane -> (row 8q + l/8, position l%8).
          const int q = part * kLoads + j;
          const int r = q * 8 + (lane >> 3);
          const int c = swz(r, lane & 7, p.swz_shift);
          dma_block(chunk_src<MASKED>(a0 + (int64_t)r * p.lda + c * 16,
                                      r < a_rows && c * 8 < k_left),
                    sa + q * kBlockBytes);
        }
      } else if constexpr (BCOL) {
        // Column-major B: the same 128 x 64 row layout and swizzle as A.
        const uint32_t sb = uniform(lds_addr(&lds.b[w.index][0]));
        const uint8_t* b0 = gb + (int64_t)ks * kGemmK * 2;
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          const int q = part * kLoads + j;
          const int r = q * 8 + (lane >> 3);
          const int c = swz(r, lane & 7, p.swz_shift);
          dma_block(chunk_src<MASKED>(b0 + (int64_t)r * p.ldb + c * 16,
                                      r < b_cols && c * 8 < k_left),
                    sb + q * kBlockBytes);
        }
      } else {
        const uint32_t sb = uniform(lds_addr(&lds.b[w.index][0]));
        const uint8_t* b0 = gb + (int64_t)ks * kGemmK * p.ldb;
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          // B: rows 4q..4q+3 of 256 B, lane -> (row 4q + l/16, position l%16).
          const int q = part * kLoads + j;
          const int r = q * 4 + (lane >> 4);
          const int c = (lane & 15) ^ swz_b(r, p.b_swz);
          dma_block(chunk_src<MASKED>(b0 + (int64_t)r * p.ldb + c * 16,
                                      r < k_left && c * 8 < b_cols),
                    sb + q * kBlockBytes);
        }
      }
      ++pending;
      if (pending > lag) {
        wait_vmcnt_mul<kLoads>(pending - 1);
        int oldest = w.index - (pending - 1);
        if (oldest < 0) oldest += S;
        Counter<PW>::arrive(&lds.full[oldest]);
        --pending;
      }
      w.inc();
    }
  }
  while (pending > 0) {
    wait_vmcnt_mul<kLoads>(pending - 1);
    int oldest = w.index - pending;
    if (oldest < 0) oldest += S;
    Counter<PW>::arrive(&lds.full[oldest]);
    --pending;
  }
  if (ok) {
    for (int i = 0; i < S; ++i) {
      if (!bar_wait<Counter<4 * MT>>(&lds.empty[w.index], w.phase, p.spin_limit)) {
        ok = false;
        break;
      }
      w.inc();
    }
  }
  wait_vmcnt<0>();
  if (!ok && lane == 0) atomicOr(p.status, kStatusTimeoutProducer);
}

// MFMA B operand (K 16 x N 32 block at K-rows k16.., columns col0..col0+31)
// from the row-major B slot, via two transposing reads.
__device__ __forceinline__ bf16x8 load_b_frag(const uint8_t* bslot, int k16, int col0, int lane,
                                              int b_swz) {
  const int g = lane >> 4, i = lane & 15;
  const int col = col0 + 16 * (g & 1) + 4 * (i & 3);
  const int chunk = col >> 3, within = (col & 7) * 2;
  s16x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int k = k16 + 8 * (g >> 1) + 4 * half + (i >> 2);
    const uint8_t* a = bslot + k * kBRowBytes + ((chunk ^ swz_b(k, b_swz)) << 4) + within;
    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
  }
  const s16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Fragments of one 16-deep K sub-step for one consumer wave: A (2 x 32 rows)
// and B (2 x 32 columns).
struct SubFrags {
  bf16x8 a[2];
  bf16x8 b[2];
};

// A fragment (and, for column-major B, a B fragment): lane l takes the K
// chunk kk * 2 + l / 32 of row row0 + l % 32 of a 128 x 64 slot, one b128 read.
__device__ __forceinline__ bf16x8 load_row_frag(const uint8_t* slot, int row0, int kk, int li,
                                                int lk, int shift) {
  const int r = row0 + li;
  const int c = swz(r, kk * 2 + lk, shift);
  return *reinterpret_cast<const bf16x8*>(slot + r * 128 + c * 16);
}

template <bool BCOL>
__device__ __forceinline__ void load_sub(SubFrags& f, int kk, const uint8_t* sa,
                                         const uint8_t* sb, int wm, int wn, int li, int lk,
                                         int lane, const GemmParams& p) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) f.a[mi] = load_row_frag(sa, wm * 64 + mi * 32, kk, li, lk, p.swz_shift);
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    if constexpr (BCOL)
      f.b[ni] = load_row_frag(sb, wn * 64 + ni * 32, kk, li, lk, p.swz_shift);
    else
      f.b[ni] = load_b_frag(sb, kk * 16, wn * 64 + ni * 32, lane, p.b_swz);
  }
}

__device__ __forceinline__ void mfma_sub(f32x16 (&acc)[2][2], const SubFrags& f) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
}

// Scheduling hint for a block that holds one sub-step's fragment reads (6 LDS
// reads with row-major B) and the previous sub-step's 4 MFMAs: alternate one
// MFMA with two reads, so that the reads of the next sub-step issue while the
// matrix core works, instead of being sunk next to their uses.
// Column-major B makes it 4 reads (all b128), one after each MFMA.
template <bool BCOL>
__device__ __forceinline__ void interleave_mfma_reads() {
  constexpr int kReads = BCOL ? 1 : 2;  // LDS reads after each of the first MFMAs
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);  // LDS read
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  if constexpr (BCOL) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
}

// Consumer wave. Fragment reads run one K sub-step ahead of the MFMAs through
// two register buffers. At the last sub-step of a stage the wave waits for its
// reads of the slot to return, releases the slot, then waits on full for the
// next stage (while the previous MFMAs still execute) and reads that stage's
// first sub-step before issuing the last MFMAs of the current one.
template <int S, int PW, int EPI, bool BCOL, bool TRACE = false, int MT = 1, bool MASKED = false>
__device__ __forceinline__ void gemm_consumer(const GemmParams& p, GemmLds<S, MT>& lds, void* out_lds, int cw) {
  static_assert(MT == 1 || (EPI != kEpiStoreWave && !TRACE), "256-row tiles: no store wave, no trace");
  constexpr int kTileM = kGemmTile * MT;
  OutLds* out = static_cast<OutLds*>(out_lds);
  const int lane = lane_id();
  const int wm = cw >> 1, wn = cw & 1;
  const int li = lane & 31, lk = lane >> 5;
  PipeState rd = consumer_start(S);
  PipeState ost = producer_start(1, 1u);  // staging slot of this wave's pair
  int t = 0;  // stage ordinal in this workgroup's stream (for the trace)
  bool ok = true;
  for (int item = blockIdx.x; ok && item < p.items; item += gridDim.x) {
    int tm, tn;
    gemm_tile_of(p, item, tm, tn);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    SubFrags b0, b1;
    if (!bar_wait<Counter<PW>>(&lds.full[rd.index], rd.phase, p.spin_limit)) {
      ok = false;
      break;
    }
    if constexpr (TRACE) {
      if (cw == 0) trace_write(p.trace, p.trace_cap, t, 1, rd, PW);
    }
    const uint8_t* sa = &lds.a[rd.index][0];
    const uint8_t* sb = &lds.b[rd.index][0];
    load_sub<BCOL>(b0, 0, sa, sb, wm, wn, li, lk, lane, p);
    for (int ks = 0; ks < p.k_steps; ++ks) {
      load_sub<BCOL>(b1, 1, sa, sb, wm, wn, li, lk, lane, p);
      mfma_sub(acc, b0);
      interleave_mfma_reads<BCOL>();
      load_sub<BCOL>(b0, 2, sa, sb, wm, wn, li, lk, lane, p);
      mfma_sub(acc, b1);
      interleave_mfma_reads<BCOL>();
      load_sub<BCOL>(b1, 3, sa, sb, wm, wn, li, lk, lane, p);
      mfma_sub(acc, b0);
      interleave_mfma_reads<BCOL>();
      // consumer_release: this wave's reads of the slot have all returned.
      wait_lgkmcnt0();
      Counter<4 * MT>::arrive(&lds.empty[rd.index]);
      rd.inc();
      if constexpr (TRACE) ++t;
      if (ks + 1 < p.k_steps) {
        if (!bar_wait<Counter<PW>>(&lds.full[rd.index], rd.phase, p.spin_limit)) {
          ok = false;
          break;
        }
        if constexpr (TRACE) {
          if (cw == 0) trace_write(p.trace, p.trace_cap, t, 1, rd, PW);
        }
        sa = &lds.a[rd.index][0];
        sb = &lds.b[rd.index][0];
        load_sub<BCOL>(b0, 0, sa, sb, wm, wn, li, lk, lane, p);
      }
      mfma_sub(acc, b1);
    }
    if (!ok) break;
    if constexpr (EPI == kEpiF32) {
      // Epilogue: fp32 accumulators -> C.
      float* C = static_cast<float*>(p.C);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = tn * kGemmTile + wn * 64 + ni * 32 + li;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = tm * kTileM + wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * lk + (e & 3);
            if (!MASKED || (row < p.M && col < p.N)) C[(int64_t)row * p.ldc + col] = acc[mi][ni][e];
          }
        }
    } else if constexpr (EPI == kEpiWaveStaged) {
      // Wave-private staging: chunk c = rows 16c..16c+15 of this wave's 64 rows
      // (accumulator block mi = c / 2, element groups e / 4 = 2 (c % 2) + {0, 1}).
      uint8_t* buf = &static_cast<WaveOutLds<MT>*>(out_lds)->buf[cw][0];
      uint8_t* C = static_cast<uint8_t*>(p.C);
      const int64_t ldc_bytes = p.ldc * 2;
#pragma unroll
      for (int c = 0; c < kOutChunks; ++c) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const int e = 4 * (2 * (c & 1) + g2) + m;
              const int rr = 8 * g2 + 4 * lk + m;
              *reinterpret_cast<__bf16*>(buf + rr * kWaveOutPitch + (ni * 32 + li) * 2) =
                  (__bf16)acc[c >> 1][ni][e];
            }
        wait_lgkmcnt0();
        uint4 v[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int q = i * 64 + lane;  // 16-byte piece q: row q / 8, piece q % 8
          v[i] = *reinterpret_cast<const uint4*>(buf + (q >> 3) * kWaveOutPitch + (q & 7) * 16);
        }
        wait_lgkmcnt0();  // the buffer is rewritten by the next chunk
        const int64_t row0 = (int64_t)tm * kTileM + wm * 64 + c * kOutRows;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int q = i * 64 + lane;
          const int64_t col0 = (int64_t)tn * kGemmTile + wn * 64 + (q & 7) * 8;
          if (MASKED && (row0 + (q >> 3) >= p.M || col0 >= p.N)) continue;
          uint8_t* g = C + (row0 + (q >> 3)) * ldc_bytes + col0 * 2;
          const u32x4 nv = {v[i].x, v[i].y, v[i].z, v[i].w};
          __builtin_nontemporal_store(nv, reinterpret_cast<u32x4*>(g));
        }
      }
    } else {
      // Staged epilogue: chunk c holds rows 16c..16c+15 of this pair's 64 rows,
      // i.e. accumulator block mi = c / 2, element groups e / 4 = 2 (c % 2) + {0, 1}.
      uint8_t* slot = &out->slot[wm][0];
#pragma unroll
      for (int c = 0; c < kOutChunks; ++c) {
        if (!bar_wait<Counter<1>>(&out->empty[wm], ost.phase, p.spin_limit)) {
          ok = false;
          break;
        }
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = wn * 64 + ni * 32 + li;
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const int e = 4 * (2 * (c & 1) + g2) + m;
              const int rr = 8 * g2 + 4 * lk + m;
              *reinterpret_cast<__bf16*>(slot + rr * kOutPitch + col * 2) =
                  (__bf16)acc[c >> 1][ni][e];
            }
        }
        wait_lgkmcnt0();
        Counter<2>::arrive(&out->full[wm]);
        ost.inc();
      }
      if (!ok) break;
    }
  }
  if (!ok && lane == 0) atomicOr(p.status, kStatusTimeoutConsumer);
}

// Consumer wave of a ring with three or more stages and fp32 C (one workgroup
// per CU, so registers to spare: 169 VGPRs with 128-row tiles, 148 with
// 256-row tiles, no spills).
// Fragment reads run two K sub-steps ahead of the MFMAs through four register
// buffers. A stage's last reads go out with its second sub-step's MFMAs, so the
// wave hands the slot back half-way through the stage's MFMAs, once those
// reads have returned, and the producer can refill it sooner.
template <int S, int PW, bool BCOL, bool MASKED, int MT = 1>
__device__ __forceinline__ void gemm_consumer_deep(const GemmParams& p, GemmLds<S, MT>& lds, int cw) {
  const int lane = lane_id();
  const int wm = cw >> 1, wn = cw & 1;
  const int li = lane & 31, lk = lane >> 5;
  PipeState rd = consumer_start(S);
  bool ok = true;
  for (int item = blockIdx.x; ok && item < p.items; item += gridDim.x) {
    int tm, tn;
    gemm_tile_of(p, item, tm, tn);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    SubFrags f0, f1, f2, f3;
    if (!bar_wait<Counter<PW>>(&lds.full[rd.index], rd.phase, p.spin_limit)) {
      ok = false;
      break;
    }
    const uint8_t* sa = &lds.a[rd.index][0];
    const uint8_t* sb = &lds.b[rd.index][0];
    load_sub<BCOL>(f0, 0, sa, sb, wm, wn, li, lk, lane, p);
    load_sub<BCOL>(f1, 1, sa, sb, wm, wn, li, lk, lane, p);
    for (int ks = 0; ks + 1 < p.k_steps; ++ks) {
      load_sub<BCOL>(f2, 2, sa, sb, wm, wn, li, lk, lane, p);
      mfma_sub(acc, f0);
      interleave_mfma_reads<BCOL>();
      load_sub<BCOL>(f3, 3, sa, sb, wm, wn, li, lk, lane, p);
      mfma_sub(acc, f1);
      interleave_mfma_reads<BCOL>();
      // consumer_release: every read of the slot has returned (the scheduling
      // barrier keeps the MFMAs above ahead of the wait).
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkmcnt0();
      Counter<4 * MT>::arrive(&lds.empty[rd.index]);
      rd.inc();
      if (!bar_wait<Counter<PW>>(&lds.full[rd.index], rd.phase, p.spin_limit)) {
        ok = false;
        break;
      }
      sa = &lds.a[rd.index][0];
      sb = &lds.b[rd.index][0];
      load_sub<BCOL>(f0, 0, sa, sb, wm, wn, li, lk, lane, p);
      mfma_sub(acc, f2);
      interleave_mfma_reads<BCOL>();
      load_sub<BCOL>(f1, 1, sa, sb, wm, wn, li, lk, lane, p);
      mfma_sub(acc, f3);
      interleave_mfma_reads<BCOL>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!ok) break;
    // The tile's last stage.
    load_sub<BCOL>(f2, 2, sa, sb, wm, wn, li, lk, lane, p);
    mfma_sub(acc, f0);
    interleave_mfma_reads<BCOL>();
    load_sub<BCOL>(f3, 3, sa, sb, wm, wn, li, lk, lane, p);
    mfma_sub(acc, f1);
    interleave_mfma_reads<BCOL>();
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    Counter<4 * MT>::arrive(&lds.empty[rd.index]);
    rd.inc();
    mfma_sub(acc, f2);
    mfma_sub(acc, f3);
    // Epilogue: fp32 accumulators -> C. The same loop as gemm_consumer's, kept
    // as a copy: one shared function reorders the instructions of these kernels
    // and measured about 1 % slower at S = 3.
    float* C = static_cast<float*>(p.C);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int col = tn * kGemmTile + wn * 64 + ni * 32 + li;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = tm * kGemmTile * MT + wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * lk + (e & 3);
          if (!MASKED || (row < p.M && col < p.N)) C[(int64_t)row * p.ldc + col] = acc[mi][ni][e];
        }
      }
  }
  if (!ok && lane == 0) atomicOr(p.status, kStatusTimeoutConsumer);
}

// Store wave of the staged epilogue: for every tile, drains the 4 chunks of
// each wave pair (pair 0 and pair 1 alternately) and writes them to C.
template <bool MASKED>
__device__ __forceinline__ void gemm_store_wave(const GemmParams& p, OutLds& out) {
  const int lane = lane_id();
  PipeState rd[2] = {consumer_start(1), consumer_start(1)};
  bool ok = true;
  uint8_t* C = static_cast<uint8_t*>(p.C);
  const int64_t ldc_bytes = p.ldc * 2;
  for (int item = blockIdx.x; ok && item < p.items; item += gridDim.x) {
    int tm, tn;
    gemm_tile_of(p, item, tm, tn);
    for (int c = 0; ok && c < kOutChunks; ++c) {
#pragma unroll
      for (int pair = 0; pair < 2; ++pair) {
        if (!bar_wait<Counter<2>>(&out.full[pair], rd[pair].phase, p.spin_limit)) {
          ok = false;
          break;
        }
        const uint8_t* slot = &out.slot[pair][0];
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = i * 64 + lane;  // 16-byte piece q: row q / 16, piece q % 16
          v[i] = *reinterpret_cast<const uint4*>(slot + (q >> 4) * kOutPitch + (q & 15) * 16);
        }
        wait_lgkmcnt0();
        Counter<1>::arrive(&out.empty[pair]);
        rd[pair].inc();
        const int64_t row0 = (int64_t)tm * kGemmTile + pair * 64 + c * kOutRows;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = i * 64 + lane;
          const int64_t col0 = (int64_t)tn * kGemmTile + (q & 15) * 8;
          if (MASKED && (row0 + (q >> 4) >= p.M || col0 >= p.N)) continue;
          uint8_t* g = C + (row0 + (q >> 4)) * ldc_bytes + col0 * 2;
          const u32x4 nv = {v[i].x, v[i].y, v[i].z, v[i].w};
          __builtin_nontemporal_store(nv, reinterpret_cast<u32x4*>(g));
        }
      }
    }
  }
  wait_vmcnt<0>();
  if (!ok && lane == 0) atomicOr(p.status, kStatusTimeoutConsumer);
}

template <int S, int PW, int EPI, bool BCOL, bool TRACE = false, int MT = 1, bool MASKED = false>
__device__ __forceinline__ void gemm_body(const GemmParams& p) {
  __shared__ GemmLds<S, MT> lds;
  const int wave = (int)(threadIdx.x >> 6);
  if (threadIdx.x < S) {
    lds.full[threadIdx.x] = 0u;
    lds.empty[threadIdx.x] = 0u;
  }
  if constexpr (EPI == kEpiStoreWave) {
    __shared__ OutLds out;
    if (threadIdx.x < 2) {
      out.full[threadIdx.x] = 0u;
      out.empty[threadIdx.x] = 0u;
    }
    __syncthreads();
    if (wave < PW)
      gemm_producer<S, PW, BCOL, false, 1, MASKED>(p, lds, wave);
    else if (wave < PW + 4)
      gemm_consumer<S, PW, EPI, BCOL, false, 1, MASKED>(p, lds, &out, wave - PW);
    else
      gemm_store_wave<MASKED>(p, out);
  } else if constexpr (EPI == kEpiWaveStaged) {
    __shared__ WaveOutLds<MT> out;
    __syncthreads();
    if (wave < PW)
      gemm_producer<S, PW, BCOL, false, MT, MASKED>(p, lds, wave);
    else
      gemm_consumer<S, PW, EPI, BCOL, false, MT, MASKED>(p, lds, &out, wave - PW);
  } else if constexpr (S >= 3 && !TRACE) {
    __syncthreads();
    if (wave < PW)
      gemm_producer<S, PW, BCOL, false, MT, MASKED>(p, lds, wave);
    else
      gemm_consumer_deep<S, PW, BCOL, MASKED, MT>(p, lds, wave - PW);
  } else {
    __syncthreads();
    if (wave < PW)
      gemm_producer<S, PW, BCOL, TRACE, MT, MASKED>(p, lds, wave);
    else
      gemm_consumer<S, PW, EPI, BCOL, TRACE, MT, MASKED>(p, lds, nullptr, wave - PW);
  }
}

// Waves per SIMD the GEMM kernels are compiled for (their VGPR budget): two
// workgroups share a CU where two rings fit the LDS (S <= 2 with 128-row
// tiles; 4 waves per SIMD with 4 producer waves, i.e. at most 128 VGPRs),
// else one. The store-wave variant runs one per CU anyway. Without the bound a
// few more registers (the trace's, say) can push the kernel past 128 VGPRs and
// halve its occupancy.
constexpr int gemm_waves_per_simd(int S, int PW, int EPI, int MT = 1) {
  if (EPI == kEpiStoreWave) return 1;
  const int workgroups = (S <= 2 && MT == 1) ? 2 : 1;
  return (workgroups * (PW + 4 * MT) + 3) / 4;
}

constexpr int gemm_block_threads(int PW, int EPI, int MT) {
  return 64 * (PW + 4 * MT + (EPI == kEpiStoreWave ? 1 : 0));
}

// Static LDS of one workgroup: the ring, its barrier words and the bf16 staging.
constexpr int gemm_lds_of(int S, int EPI, int MT) {
  return S * (MT * kAStageBytes + kBStageBytes + 8) +
         (EPI == kEpiStoreWave ? (int)sizeof(OutLds)
                               : EPI == kEpiWaveStaged ? 4 * MT * kWaveOutBytes : 0);
}

constexpr bool gemm_fits(int S, int EPI, int MT) { return gemm_lds_of(S, EPI, MT) <= 160 * 1024; }

// B row-major (K x N, the default) and column-major (PIPE_FLAG_GEMM_B_COLMAJOR).
template <int S, int PW, int EPI, int MT = 1, bool MASKED = false>
__global__ void __launch_bounds__(gemm_block_threads(PW, EPI, MT),
                                  gemm_waves_per_simd(S, PW, EPI, MT))
    gemm_kernel(GemmParams p) {
  gemm_body<S, PW, EPI, false, false, MT, MASKED>(p);
}

template <int S, int PW, int EPI, int MT = 1, bool MASKED = false>
__global__ void __launch_bounds__(gemm_block_threads(PW, EPI, MT),
                                  gemm_waves_per_simd(S, PW, EPI, MT))
    gemm_kernel_bcol(GemmParams p) {
  gemm_body<S, PW, EPI, true, false, MT, MASKED>(p);
}

// With PIPE_FLAG_TRACE (fp32 C, row-major B, 128-row tiles): the same
// mainloop, recording workgroup 0's acquires and waits. A separate kernel, so
// that the trace costs the other kernels no registers.
template <int S, int PW>
__global__ void __launch_bounds__(64 * (PW + 4), gemm_waves_per_simd(S, PW, kEpiF32))
    gemm_trace_kernel(GemmParams p) {
  gemm_body<S, PW, kEpiF32, false, true>(p);
}

using GemmKernel = void (*)(GemmParams);

// ---------------------------------------------------------------------------
// Unified GEMM for 256 x 256 output tiles (PIPE_FLAG_UNIFIED): no producer and
// consumer roles. All 16 waves of the workgroup (1024 threads, one workgroup
// per CU) load a share of every stage and all compute, so each SIMD holds four
// MFMA waves; the ring has two slots of 64 KiB (A: 256 x 64, B: 64 x 256).
// Per K step a wave waits for its own loads of the stage (vmcnt), one
// workgroup barrier then says that every wave's loads have landed and that
// every wave has finished reading the other slot, the stage after next is
// issued into that slot, and the wave runs its 16 MFMAs on its 64 x 64 block.
// ---------------------------------------------------------------------------
constexpr int kUniWaves = kGemmUnifiedWaves;
constexpr int kUniStageBlocks = 64;                         // 1 KiB blocks per stage
constexpr int kUniLoads = kUniStageBlocks / kUniWaves;      // per wave and stage
static_assert(kUniLoads == 4, "four DMA blocks per wave and stage");

struct UniLds {
  uint8_t a[2][2 * kAStageBytes];  // 256 rows x 64 K, rows as in the 256-row ring
  uint8_t b[2][2 * kBStageBytes];  // row-major B: two 128-column halves; column-major: 256 rows
};
static_assert(sizeof(UniLds) == kGemmUnifiedLdsBytes, "unified ring size");

// Issue this wave's LOADS DMA blocks of K step ks of output tile (tm, tn) into
// slot `slot`: blocks wave * LOADS .. wave * LOADS + LOADS - 1 of the stage's 64.
template <bool BCOL, bool MASKED, int LOADS = kUniLoads>
__device__ __forceinline__ void uni_issue(const GemmParams& p, UniLds& lds, int slot, int tm,
                                          int tn, int ks, int wave, int lane) {
  const int k_left = p.K - ks * kGemmK;
  const uint8_t* a0 = p.A + (int64_t)tm * 256 * p.lda + (int64_t)ks * kGemmK * 2;
  const int a_rows = p.M - tm * 256;
  const int b_cols = p.N - tn * 256;
  const uint32_t sa = uniform(lds_addr(&lds.a[slot][0]));
  const uint32_t sb = uniform(lds_addr(&lds.b[slot][0]));
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int q = wave * LOADS + j;  // blocks 0-31 are A, 32-63 B (uniform per wave)
    if (q < 32) {
      const int r = q * 8 + (lane >> 3);
      const int c = swz(r, lane & 7, p.swz_shift);
      dma_block(chunk_src<MASKED>(a0 + (int64_t)r * p.lda + c * 16, r < a_rows && c * 8 < k_left),
                sa + q * kBlockBytes);
    } else if constexpr (BCOL) {
      // Column-major B: 256 rows (output columns) of 64 K, laid out as A.
      const int qb = q - 32;
      const int r = qb * 8 + (lane >> 3);
      const int c = swz(r, lane & 7, p.swz_shift);
      const uint8_t* b0 = p.B + (int64_t)tn * 256 * p.ldb + (int64_t)ks * kGemmK * 2;
      dma_block(chunk_src<MASKED>(b0 + (int64_t)r * p.ldb + c * 16, r < b_cols && c * 8 < k_left),
                sb + qb * kBlockBytes);
    } else {
      // Row-major B: half h holds columns 128 h .. 128 h + 127 of the 64 K-rows.
      const int qb = q - 32;
      const int h = qb >> 4, qq = qb & 15;
      const int r = qq * 4 + (lane >> 4);
      const int c = (lane & 15) ^ swz_b(r, p.b_swz);
      const uint8_t* b0 = p.B + (int64_t)tn * 512 + (int64_t)h * kBRowBytes +
                          (int64_t)ks * kGemmK * p.ldb;
      dma_block(chunk_src<MASKED>(b0 + (int64_t)r * p.ldb + c * 16,
                                  r < k_left && h * 128 + c * 8 < b_cols),
                sb + h * kBStageBytes + qq * kBlockBytes);
    }
  }
}

template <bool BCOL, bool MASKED>
__global__ void __launch_bounds__(64 * kUniWaves, 1) gemm_unified_kernel(GemmParams p) {
  __shared__ UniLds lds;
  const int wave = (int)(threadIdx.x >> 6);
  const int lane = lane_id();
  const int wm = wave >> 2, wn = wave & 3;  // this wave's 64 x 64 block of the 256 x 256 tile
  const int li = lane & 31, lk = lane >> 5;
  // Row-major B: the wave's 64 columns lie in half wn / 2; column-major B: rows of one slot.
  const int b_off = BCOL ? 0 : (wn >> 1) * kBStageBytes;
  const int bwn = BCOL ? wn : (wn & 1);
  int slot = 0;
  int item = blockIdx.x;
  if (item < p.items) uni_issue<BCOL, MASKED>(p, lds, 0, item / p.tiles_n, item % p.tiles_n, 0, wave, lane);
  for (; item < p.items; item += gridDim.x) {
    const int tm = item / p.tiles_n, tn = item % p.tiles_n;
    const int next = item + (int)gridDim.x;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    for (int ks = 0; ks < p.k_steps; ++ks) {
      // This wave's loads of step ks have landed; after the barrier every wave's
      // have, and every wave has finished reading the other slot.
      wait_vmcnt<0>();
      __syncthreads();
      // The next stage to fetch: this tile's next K step, or the first of the
      // workgroup's next tile.
      const bool more = ks + 1 < p.k_steps;
      const int itm = more ? tm : next / p.tiles_n;
      const int itn = more ? tn : next % p.tiles_n;
      if (more || next < p.items)
        uni_issue<BCOL, MASKED>(p, lds, slot ^ 1, itm, itn, more ? ks + 1 : 0, wave, lane);
      // Four MFMA waves share each SIMD, so one wave's fragment reads are
      // covered by the others' MFMAs: one sub-step's fragments at a time.
      const uint8_t* sa = &lds.a[slot][0];
      const uint8_t* sb = &lds.b[slot][b_off];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        SubFrags f;
        load_sub<BCOL>(f, kk, sa, sb, wm, bwn, li, lk, lane, p);
        mfma_sub(acc, f);
      }
      // The slot's reads have returned before the next barrier.
      wait_lgkmcnt0();
      slot ^= 1;
    }
    float* C = static_cast<float*>(p.C);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int col = tn * 256 + wn * 64 + ni * 32 + li;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = tm * 256 + wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * lk + (e & 3);
          if (!MASKED || (row < p.M && col < p.N)) C[(int64_t)row * p.ldc + col] = acc[mi][ni][e];
        }
      }
  }
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// The same ring with 4 waves, one per SIMD, each owning a 128 x 128 block of
// the tile (4 x 4 MFMA blocks of 32 x 32). Per MFMA it reads half the fragment
// bytes of a 64 x 64 block. Its 256 fp32 accumulators per lane fit only because
// a lone wave on a SIMD may use all 512 of the SIMD's registers per lane
// (vector and accumulation registers together). The register file is split
// evenly between the waves resident on a SIMD, so a producer wave beside it
// would halve that budget: this layout exists only without warp
// specialisation. One wave per SIMD also means no other wave hides a fragment
// read, so each wave reads the next sub-step's fragments while its 16 MFMAs
// on the current one run.
// ---------------------------------------------------------------------------
constexpr int kWideWaves = kGemmWideWaves;
constexpr int kWideLoads = kUniStageBlocks / kWideWaves;  // 16 per wave and stage

struct WideFrags {
  bf16x8 a[4];
  bf16x8 b[4];
};

template <bool BCOL>
__device__ __forceinline__ void load_wide(WideFrags& f, int kk, const uint8_t* sa,
                                          const uint8_t* sb, int wm, int wn, int li, int lk,
                                          int lane, const GemmParams& p) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
    f.a[mi] = load_row_frag(sa, wm * 128 + mi * 32, kk, li, lk, p.swz_shift);
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if constexpr (BCOL)
      f.b[ni] = load_row_frag(sb, wn * 128 + ni * 32, kk, li, lk, p.swz_shift);
    else
      f.b[ni] = load_b_frag(sb, kk * 16, ni * 32, lane, p.b_swz);
  }
}

__device__ __forceinline__ void mfma_wide(f32x16 (&acc)[4][4], const WideFrags& f) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
}

// Output tile of work item `item` in an order that keeps each XCD's tiles
// together. Workgroups go to the 8 XCDs in turn, so with 8 | items the items
// are first dealt so that each XCD walks one contiguous eighth of the order;
// the order then runs down bands of kWideGroupM tile rows, column by column,
// so the tiles an XCD holds at once share few A rows and B columns (4 x 8 tiles
// for a 16 x 16 grid: 12 K-slices per step where row-major order needs 18).
// A bijection on [0, items) for every shape and grid.
constexpr int kWideGroupM = 4;
__device__ __forceinline__ void wide_tile_of(const GemmParams& p, int item, int& tm, int& tn) {
  const int per_xcd = p.items >> 3;
  const int q = (p.items & 7) ? item : (item & 7) * per_xcd + (item >> 3);
  const int band = kWideGroupM * p.tiles_n;
  const int first = (q / band) * kWideGroupM;
  const int tiles_m = p.items / p.tiles_n;
  const int rows = min(tiles_m - first, kWideGroupM);
  const int local = q - (first / kWideGroupM) * band;
  tm = first + local % rows;
  tn = local / rows;
}

template <bool BCOL, bool MASKED>
__global__ void __launch_bounds__(64 * kWideWaves, 1) gemm_wide_kernel(GemmParams p) {
  __shared__ UniLds lds;
  const int wave = (int)(threadIdx.x >> 6);
  const int lane = lane_id();
  const int wm = wave >> 1, wn = wave & 1;  // this wave's 128 x 128 block of the 256 x 256 tile
  const int li = lane & 31, lk = lane >> 5;
  // Row-major B: the wave's 128 columns are half wn of the slot; column-major B:
  // rows wn * 128 .. wn * 128 + 127 of the slot.
  const int b_off = BCOL ? 0 : wn * kBStageBytes;
  int slot = 0;
  int item = blockIdx.x;
  if (item < p.items) {
    int tm0, tn0;
    wide_tile_of(p, item, tm0, tn0);
    uni_issue<BCOL, MASKED, kWideLoads>(p, lds, 0, tm0, tn0, 0, wave, lane);
  }
  for (; item < p.items; item += gridDim.x) {
    int tm, tn, ntm = 0, ntn = 0;
    wide_tile_of(p, item, tm, tn);
    const int next = item + (int)gridDim.x;
    if (next < p.items) wide_tile_of(p, next, ntm, ntn);
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    for (int ks = 0; ks < p.k_steps; ++ks) {
      // As in the 16-wave kernel: every wave's loads of step ks have landed and
      // every wave has finished reading the other slot.
      wait_vmcnt<0>();
      __syncthreads();
      const bool more = ks + 1 < p.k_steps;
      if (more || next < p.items)
        uni_issue<BCOL, MASKED, kWideLoads>(p, lds, slot ^ 1, more ? tm : ntm, more ? tn : ntn,
                                            more ? ks + 1 : 0, wave, lane);
      const uint8_t* sa = &lds.a[slot][0];
      const uint8_t* sb = &lds.b[slot][b_off];
      WideFrags f[2];
      load_wide<BCOL>(f[0], 0, sa, sb, wm, wn, li, lk, lane, p);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < 3) load_wide<BCOL>(f[(kk + 1) & 1], kk + 1, sa, sb, wm, wn, li, lk, lane, p);
        mfma_wide(acc, f[kk & 1]);
      }
      wait_lgkmcnt0();
      slot ^= 1;
    }
    // The last MFMAs' results land before any accumulator is read (the guard of
    // the 32-K kernel's epilogue below, where a read came too early).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_sched_barrier(0);
    float* C = static_cast<float*>(p.C);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int col = tn * 256 + wn * 128 + ni * 32 + li;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = tm * 256 + wm * 128 + mi * 32 + 8 * (e >> 2) + 4 * lk + (e & 3);
          if (!MASKED || (row < p.M && col < p.N)) C[(int64_t)row * p.ldc + col] = acc[mi][ni][e];
        }
      }
  }
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// The 4-wave unified GEMM on a deeper ring: stages of 32 K instead of 64, so 3
// to 5 slots fit in LDS and up to S - 1 stages are in flight while the waves
// compute. A stage holds A as 256 rows of 64 bytes and B as two 128-column
// halves of 32 K-rows (row-major B) or as 256 rows of 64 bytes like A
// (column-major B), 32 KiB in all; each wave issues 4 of its 16 A blocks and
// 4 of its 16 B blocks. Rows of 64 bytes (4 chunks) take the chunk XOR
// (row >> 2) & 3, which spreads any 16 consecutive rows' reads of one chunk
// over all 64 banks.
//
// One workgroup barrier per step, half-way through it: once the wave has
// issued its MFMAs on the step's first 16 K, it waits until its loads of the
// next stage have landed and joins the barrier. After it, every wave's loads
// of that stage have landed, and every wave has finished reading the slot of
// the step before (its reads fed MFMAs that were issued before the barrier),
// so the stage S - 1 ahead goes into that slot. The next stage's first
// fragments are then read while the MFMAs on this step's second 16 K run.
// Between tiles, the next tile's first S - 1 stages are issued before this
// tile's C stores, and the wave drains its counter before the next tile's
// first step.
// ---------------------------------------------------------------------------
constexpr int kDeepK = 32;                        // K per stage
constexpr int kDeepHalfBytes = 256 * kDeepK * 2;  // 16 KiB: A, or B, of one stage
constexpr int kDeepStageBytes = 2 * kDeepHalfBytes;
constexpr int kDeepLoads = kDeepStageBytes / kBlockBytes / kWideWaves;  // 8 per wave and stage

// Chunk position of K chunk c (0-3) in row r of a 64-byte-row slot, and back.
__device__ __forceinline__ int swz4(int r, int c) { return c ^ ((r >> 2) & 3); }

// Sources of this wave's 8 DMA blocks of one tile, at K = 0: A blocks and B
// blocks wave * 4 .. wave * 4 + 3 of each operand's 16. Step ks adds ks * 64
// bytes (A, column-major B) or 32 ks K-rows (row-major B). In a 64-byte-row
// block, lane l writes row 16 q + l / 4 at position l % 4, which holds K
// chunk (l % 4) ^ ((l / 16) % 4) for every block q; a 256-byte K-row of
// row-major B holds chunk (l % 16) ^ swz_b(r) at position l % 16.
struct DeepSrc {
  const uint8_t* a[4];
  const uint8_t* b[4];
  uint32_t rows_in;  // MASKED: bit j: block j's A row inside M; bit 4 + j: its B row or columns inside N
};

template <bool BCOL>
__device__ __forceinline__ void deep_src(const GemmParams& p, int tm, int tn, int wave, int lane,
                                         DeepSrc& s) {
  const int c = (lane & 3) ^ ((lane >> 4) & 3);
  s.rows_in = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int qq = wave * 4 + j;
    const int r = qq * 16 + (lane >> 2);
    s.a[j] = p.A + (int64_t)(tm * 256 + r) * p.lda + c * 16;
    s.rows_in |= (r < p.M - tm * 256 ? 1u : 0u) << j;
    if constexpr (BCOL) {
      s.b[j] = p.B + (int64_t)(tn * 256 + r) * p.ldb + c * 16;
      s.rows_in |= (r < p.N - tn * 256 ? 1u : 0u) << (4 + j);
    } else {
      const int h = qq >> 3, qb = qq & 7;
      const int kr = qb * 4 + (lane >> 4);
      const int cb = (lane & 15) ^ swz_b(kr, p.b_swz);
      s.b[j] = p.B + (int64_t)kr * p.ldb + (int64_t)tn * 512 + h * kBRowBytes + cb * 16;
      s.rows_in |= (h * 128 + cb * 8 < p.N - tn * 256 ? 1u : 0u) << (4 + j);
    }
  }
}

// DMA block j (0-3: A, 4-7: B) of stage ks into the slot at `sbase`.
template <bool BCOL, bool MASKED>
__device__ __forceinline__ void deep_dma(const GemmParams& p, const DeepSrc& s, uint32_t sbase,
                                         int ks, int j, int wave, int lane) {
  const int k_left = p.K - ks * kDeepK;
  if (j < 4) {
    const int c = (lane & 3) ^ ((lane >> 4) & 3);
    dma_block(chunk_src<MASKED>(s.a[j] + (int64_t)ks * (kDeepK * 2),
                                ((s.rows_in >> j) & 1) && c * 8 < k_left),
              sbase + (wave * 4 + j) * kBlockBytes);
  } else {
    const int jb = j - 4;
    const int qq = wave * 4 + jb;
    bool inside;
    const uint8_t* src;
    if constexpr (BCOL) {
      const int c = (lane & 3) ^ ((lane >> 4) & 3);
      src = s.b[jb] + (int64_t)ks * (kDeepK * 2);
      inside = ((s.rows_in >> (4 + jb)) & 1) && c * 8 < k_left;
    } else {
      const int kr = (qq & 7) * 4 + (lane >> 4);
      src = s.b[jb] + (int64_t)ks * kDeepK * p.ldb;
      inside = ((s.rows_in >> (4 + jb)) & 1) && kr < k_left;
    }
    dma_block(chunk_src<MASKED>(src, inside), sbase + kDeepHalfBytes + qq * kBlockBytes);
  }
}

template <bool BCOL, bool MASKED>
__device__ __forceinline__ void deep_issue(const GemmParams& p, const DeepSrc& s, uint32_t sbase,
                                           int ks, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < kDeepLoads; ++j) deep_dma<BCOL, MASKED>(p, s, sbase, ks, j, wave, lane);
}

// A (or column-major B) fragment of a 64-byte-row slot: lane l takes K chunk
// kk * 2 + l / 32 of row row0 + l % 32.
__device__ __forceinline__ bf16x8 load_row_frag4(const uint8_t* slot, int row0, int kk, int li,
                                                 int lk) {
  const int r = row0 + li;
  return *reinterpret_cast<const bf16x8*>(slot + r * 64 + swz4(r, kk * 2 + lk) * 16);
}

template <bool BCOL>
__device__ __forceinline__ void load_deep(WideFrags& f, int kk, const uint8_t* sa,
                                          const uint8_t* sb, int wm, int wn, int li, int lk,
                                          int lane, const GemmParams& p) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) f.a[mi] = load_row_frag4(sa, wm * 128 + mi * 32, kk, li, lk);
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if constexpr (BCOL)
      f.b[ni] = load_row_frag4(sb, wn * 128 + ni * 32, kk, li, lk);
    else
      f.b[ni] = load_b_frag(sb, kk * 16, ni * 32, lane, p.b_swz);
  }
}

// Piece q of sub-step kk's fragments in a 64-byte-row slot: q = 0-3 the A
// fragment of row block q, q = 4-7 the B fragment of column block q - 4 (one
// b128 read, or two transposing b64 reads for row-major B).
template <bool BCOL>
__device__ __forceinline__ void load_deep_piece(WideFrags& f, int q, int kk, const uint8_t* sa,
                                                const uint8_t* sb, int wm, int wn, int li, int lk,
                                                int lane, const GemmParams& p) {
  if (q < 4) {
    f.a[q] = load_row_frag4(sa, wm * 128 + q * 32, kk, li, lk);
  } else if constexpr (BCOL) {
    f.b[q - 4] = load_row_frag4(sb, wn * 128 + (q - 4) * 32, kk, li, lk);
  } else {
    f.b[q - 4] = load_b_frag(sb, kk * 16, (q - 4) * 32, lane, p.b_swz);
  }
}

// The 16 MFMAs of one sub-step on fragments f, with the 8 pieces of the next
// sub-step's fragments g read one after each of the first 8 MFMAs, so the
// LDS queue never holds a burst that would stall the wave's MFMA issue. With
// DMA, this wave's 8 DMA blocks of stage ks go out one after every second
// MFMA as well, where `dma` holds (a wave-uniform predicate: the MFMAs are
// one sequence either way, which keeps the accumulators in one register
// chain). Unrolled by template recursion: the schedule pins take constants.
template <int I, bool BCOL, bool MASKED, bool DMA>
__device__ __forceinline__ void mfma_wide_pipelined(f32x16 (&acc)[4][4], const WideFrags& f,
                                                    WideFrags& g, int kk, const uint8_t* sa,
                                                    const uint8_t* sb, int wm, int wn, int li,
                                                    int lk, int lane, const GemmParams& p,
                                                    const DeepSrc& s, uint32_t sbase, int ks,
                                                    int wave, bool dma = true) {
  if constexpr (I < 16) {
    constexpr int kReads = (I < 4 || BCOL) ? 1 : 2;  // LDS reads of piece I
    acc[I >> 2][I & 3] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[I >> 2], f.b[I & 3], acc[I >> 2][I & 3], 0, 0, 0);
    if constexpr (I < 8) load_deep_piece<BCOL>(g, I, kk, sa, sb, wm, wn, li, lk, lane, p);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I < 8) __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
    if constexpr (DMA && (I & 1) == 1) {
      __builtin_amdgcn_sched_barrier(0);
      if (dma) deep_dma<BCOL, MASKED>(p, s, sbase, ks, I >> 1, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_wide_pipelined<I + 1, BCOL, MASKED, DMA>(acc, f, g, kk, sa, sb, wm, wn, li, lk, lane, p, s,
                                                  sbase, ks, wave, dma);
  }
}

template <int S>
struct DeepLds {
  uint8_t ring[S][kDeepStageBytes];
};

template <int S, bool BCOL, bool MASKED, bool CBF16 = false>
__global__ void __launch_bounds__(64 * kWideWaves, 1) gemm_wide_deep_kernel(GemmParams p) {
  static_assert(S >= 3, "the slot refilled at a step is the one read a step earlier");
  __shared__ DeepLds<S> lds;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = lane_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lk = lane >> 5;
  // Row-major B: the wave's columns are half wn of the B part (8 KiB each);
  // column-major B: rows wn * 128 .. of the B part.
  const int b_off = kDeepHalfBytes + (BCOL ? 0 : wn * (kDeepHalfBytes / 2));
  const int ksteps = p.k_steps;  // stages of 32 K per tile
  const int pro = ksteps < S - 1 ? ksteps : S - 1;  // stages issued ahead of a tile's first step
  const uint32_t ring = uniform(lds_addr(&lds.ring[0][0]));
  int item = blockIdx.x;
  if (item >= p.items) return;
  int tm, tn;
  wide_tile_of(p, item, tm, tn);
  DeepSrc src;
  deep_src<BCOL>(p, tm, tn, wave, lane, src);
  for (int g = 0; g < pro; ++g)
    deep_issue<BCOL, MASKED>(p, src, ring + g * kDeepStageBytes, g, wave, lane);
  // Stage 0 has landed once at most S - 2 stages' loads are younger.
  if (pro == S - 1) wait_vmcnt<(S - 2) * kDeepLoads>();
  else wait_vmcnt<0>();
  for (;;) {
    __syncthreads();
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    WideFrags f0, f1;
    load_deep<BCOL>(f0, 0, &lds.ring[0][0], &lds.ring[0][b_off], wm, wn, li, lk, lane, p);
    int slot = 0;
    for (int ks = 0; ks < ksteps; ++ks) {
      const uint8_t* sl = &lds.ring[slot][0];
      const int next_slot = slot + 1 == S ? 0 : slot + 1;
      const int fill = slot == 0 ? S - 1 : slot - 1;  // the slot of step ks - 1
      // First half: MFMAs on the step's first 16 K, reads of its second.
      mfma_wide_pipelined<0, BCOL, MASKED, false>(acc, f0, f1, 1, sl, sl + b_off, wm, wn, li, lk,
                                                  lane, p, src, 0, 0, wave);
      if (ks + 1 < ksteps) {
        // Stage ks + 1 has landed once at most S - 3 stages' loads are
        // younger; near the tile's end fewer were issued, and the wave drains.
        if (ks + S - 2 < ksteps) wait_vmcnt<(S - 3) * kDeepLoads>();
        else wait_vmcnt<0>();
        __syncthreads();
      }
      // Second half: MFMAs on the second 16 K, reads of the next stage's first
      // (after the tile's last step they read a slot nobody uses), and the
      // refill of the slot of step ks - 1 with the stage S - 1 ahead.
      const uint8_t* nl = &lds.ring[next_slot][0];
      mfma_wide_pipelined<0, BCOL, MASKED, true>(acc, f1, f0, 0, nl, nl + b_off, wm, wn, li, lk,
                                                 lane, p, src, ring + fill * kDeepStageBytes,
                                                 ks + S - 1, wave, ks + S - 1 < ksteps);
      slot = next_slot;
    }
    // Every wave has issued its last MFMAs, so every slot's reads are done:
    // the next tile's first stages may refill slots 0 .. S - 2.
    const int next = item + (int)gridDim.x;
    int ntm = 0, ntn = 0;
    if (next < p.items) {
      wide_tile_of(p, next, ntm, ntn);
      __syncthreads();
      deep_src<BCOL>(p, ntm, ntn, wave, lane, src);
      for (int g = 0; g < pro; ++g)
        deep_issue<BCOL, MASKED>(p, src, ring + g * kDeepStageBytes, g, wave, lane);
    }
    // C: each store instruction writes 32 consecutive columns of two rows,
    // 128 bytes per row in fp32 or 64 in bf16 (rounded to nearest even).
    // Before any accumulator is read the wave sleeps once: with the bf16
    // conversion the compiler read the last MFMA's result registers about a
    // dozen instructions after that MFMA issued, too early to see its sum
    // (measured: element 2 of the last block kept its previous value). The
    // schedule fences keep the accumulator reads block by block after it.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        if constexpr (CBF16) __builtin_amdgcn_sched_barrier(0);
        const int col = tn * 256 + wn * 128 + ni * 32 + li;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = tm * 256 + wm * 128 + mi * 32 + 8 * (e >> 2) + 4 * lk + (e & 3);
          if (!MASKED || (row < p.M && col < p.N)) {
            if constexpr (CBF16)
              static_cast<__bf16*>(p.C)[(int64_t)row * p.ldc + col] = (__bf16)acc[mi][ni][e];
            else
              static_cast<float*>(p.C)[(int64_t)row * p.ldc + col] = acc[mi][ni][e];
          }
        }
      }
    if (next >= p.items) break;
    item = next;
    tm = ntm;
    tn = ntn;
    wait_vmcnt<0>();
  }
  wait_vmcnt<0>();
}

#if !defined(PIPE_GEMM_PART) || PIPE_GEMM_PART == 2
}  // namespace

hipError_t launch_gemm_unified(int stages, int grid, const GemmParams& p, hipStream_t stream) {
  if (stages < 2 || stages > 5 || p.trace != nullptr) return hipErrorInvalidValue;
  if (p.c_bf16 && !(p.unified == kWideWaves && stages >= 3)) return hipErrorInvalidValue;
  const bool bcol = p.b_colmajor != 0;
  const bool masked = (p.M % 256) != 0 || (p.N % 256) != 0 || (p.K % kGemmK) != 0;
  if (p.unified == kWideWaves && stages >= 3) {
    const bool dm = (p.M % 256) != 0 || (p.N % 256) != 0 || (p.K % kDeepK) != 0;
    GemmKernel k = nullptr;
#define PIPE_DEEP_C(SS, CB)                                                               \
  if (stages == SS && p.c_bf16 == (CB ? 1 : 0))                                           \
    k = dm ? (bcol ? gemm_wide_deep_kernel<SS, true, true, CB>                            \
                   : gemm_wide_deep_kernel<SS, false, true, CB>)                          \
           : (bcol ? gemm_wide_deep_kernel<SS, true, false, CB>                           \
                   : gemm_wide_deep_kernel<SS, false, false, CB>);
#define PIPE_DEEP(SS) PIPE_DEEP_C(SS, false) PIPE_DEEP_C(SS, true)
    PIPE_DEEP(3)
    PIPE_DEEP(4)
    PIPE_DEEP(5)
#undef PIPE_DEEP
#undef PIPE_DEEP_C
    if (k == nullptr) return hipErrorInvalidValue;
    return launch_or_record(k, dim3(grid), dim3(64 * kWideWaves), stream, p);
  }
  if (p.unified == kWideWaves) {
    GemmKernel k = masked ? (bcol ? gemm_wide_kernel<true, true> : gemm_wide_kernel<false, true>)
                          : (bcol ? gemm_wide_kernel<true, false> : gemm_wide_kernel<false, false>);
    return launch_or_record(k, dim3(grid), dim3(64 * kWideWaves), stream, p);
  }
  if (p.unified != kUniWaves || stages != 2) return hipErrorInvalidValue;
  GemmKernel k = masked ? (bcol ? gemm_unified_kernel<true, true> : gemm_unified_kernel<false, true>)
                        : (bcol ? gemm_unified_kernel<true, false> : gemm_unified_kernel<false, false>);
  return launch_or_record(k, dim3(grid), dim3(64 * kUniWaves), stream, p);
}

namespace {
#endif
#if !defined(PIPE_GEMM_PART) || PIPE_GEMM_PART == 1



// The kernel for ring depth S, or null where its LDS would not fit a CU.
template <int S, int PW, int EPI, int MT>
GemmKernel gemm_pick(bool bcol, bool masked) {
  if constexpr (gemm_fits(S, EPI, MT)) {
    if (masked)
      return bcol ? gemm_kernel_bcol<S, PW, EPI, MT, true> : gemm_kernel<S, PW, EPI, MT, true>;
    return bcol ? gemm_kernel_bcol<S, PW, EPI, MT> : gemm_kernel<S, PW, EPI, MT>;
  } else {
    return nullptr;
  }
}

template <int PW, int EPI, int MT>
hipError_t launch_gemm_pw(int stages, int grid, const GemmParams& p, hipStream_t stream) {
  const dim3 g(grid), b(gemm_block_threads(PW, EPI, MT));
  const bool bcol = p.b_colmajor != 0;
  const bool masked = (p.M % (kGemmTile * MT)) != 0 || (p.N % kGemmTile) != 0 ||
                      (p.K % kGemmK) != 0;
  GemmKernel k;
  switch (stages) {
    case 1: k = gemm_pick<1, PW, EPI, MT>(bcol, masked); break;
    case 2: k = gemm_pick<2, PW, EPI, MT>(bcol, masked); break;
    case 3: k = gemm_pick<3, PW, EPI, MT>(bcol, masked); break;
    case 4: k = gemm_pick<4, PW, EPI, MT>(bcol, masked); break;
    default: return hipErrorInvalidValue;
  }
  if (p.trace != nullptr) {  // fp32 C, row-major B, 128-row tiles, whole tiles (checked by the host)
    if (EPI != kEpiF32 || bcol || MT != 1 || masked) return hipErrorInvalidValue;
    switch (stages) {
      case 1: k = gemm_trace_kernel<1, PW>; break;
      case 2: k = gemm_trace_kernel<2, PW>; break;
      case 3: k = gemm_trace_kernel<3, PW>; break;
      default: k = gemm_trace_kernel<4, PW>; break;
    }
  }
  if (k == nullptr) return hipErrorInvalidValue;
  return launch_or_record(k, g, b, stream, p);
}

template <int EPI, int MT>
hipError_t launch_gemm_epi(int stages, int producers, int grid, const GemmParams& p,
                           hipStream_t stream) {
  if (producers == 4) return launch_gemm_pw<4, EPI, MT>(stages, grid, p, stream);
  // Two producer waves would each issue 24 DMA instructions per 256-row stage
  // and spill their addresses; 256-row tiles take four.
  if constexpr (MT == 1)
    if (producers == 2) return launch_gemm_pw<2, EPI, MT>(stages, grid, p, stream);
  return hipErrorInvalidValue;
}

template <int MT>
hipError_t launch_gemm_mt(int stages, int producers, int grid, const GemmParams& p,
                          hipStream_t stream) {
  if (!p.c_bf16) return launch_gemm_epi<kEpiF32, MT>(stages, producers, grid, p, stream);
  if (p.store_wave) {
    if constexpr (MT == 1) return launch_gemm_epi<kEpiStoreWave, 1>(stages, producers, grid, p, stream);
    return hipErrorInvalidValue;
  }
  return launch_gemm_epi<kEpiWaveStaged, MT>(stages, producers, grid, p, stream);
}
#endif

}  // namespace

#if !defined(PIPE_GEMM_PART) || PIPE_GEMM_PART == 1
hipError_t launch_gemm(int stages, int producers, int grid, const GemmParams& p,
                       hipStream_t stream) {
  if (p.unified) return launch_gemm_unified(stages, grid, p, stream);
  if (p.tile_m == 256) return launch_gemm_mt<2>(stages, producers, grid, p, stream);
  if (p.tile_m == 128) return launch_gemm_mt<1>(stages, producers, grid, p, stream);
  return hipErrorInvalidValue;
}

int gemm_lds_bytes(int stages, bool c_bf16, bool store_wave, int tile_m) {
  const int mt = tile_m / kGemmTile;
  const int out = !c_bf16 ? 0
                  : store_wave ? (int)sizeof(OutLds)
                  : 4 * mt * kWaveOutBytes;
  const int ring = stages * (mt * kAStageBytes + kBStageBytes) + stages * 8;
  // A further LDS object of the kernel (the bf16 staging) starts on a 16-byte
  // boundary.
  return out > 0 ? ((ring + 15) & ~15) + out : ring;
}

int gemm_threads(int producers, bool c_bf16, bool store_wave, int tile_m) {
  return 64 * (producers + 4 * (tile_m / kGemmTile) + (c_bf16 && store_wave ? 1 : 0));
}
#endif

}  // namespace pipe
