// C ABI of the pipelined tile stream: argument validation, launch geometry and
// dispatch. Validation happens before any HIP call, so the library can be
// loaded and its argument checks exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pipe_tile.h"
#include "pipe_kernels.hpp"

namespace {

using namespace pipe;

__device__ uint32_t g_status_word;

constexpr uint32_t kDefaultSpin = 1u << 22;
// Eager commits (see acquire_slot): a producer whose acquire waits commits its
// oldest tile in flight while at least this many are uncommitted (0 = never).
int eager_min_pending(uint32_t flags) {
  if (flags & PIPE_FLAG_LAZY_COMMIT) return 0;
  return (flags & PIPE_FLAG_EAGER_NEWEST) ? 1 : 2;
}
constexpr int kMaxDevices = 64;
constexpr int kLdsLimit = 163840;
constexpr uint32_t kKnownFlags = PIPE_FLAG_TRACE | PIPE_FLAG_ROW_STRIPS | PIPE_FLAG_NONTEMPORAL |
                                 PIPE_FLAG_GEMM_B_LINEAR | PIPE_FLAG_XCD_REMAP |
                                 PIPE_FLAG_SPLIT_INTERLEAVE | PIPE_FLAG_UNIFIED |
                                 PIPE_FLAG_LAZY_COMMIT | PIPE_FLAG_EAGER_NEWEST |
                                 PIPE_FLAG_GEMM_C_BF16 | PIPE_FLAG_GEMM_STORE_WAVE |
                                 PIPE_FLAG_GEMM_B_COLMAJOR | PIPE_FLAG_STRIP_GROUPS |
                                 PIPE_FLAG_PRODUCER_VGPR | PIPE_FLAG_DEBUG_CHECKS |
                                 PIPE_FLAG_GROUP_LOADS |
                                 PIPE_FLAG_TEST_JITTER | PIPE_FLAG_TEST_EARLY_RELEASE |
                                 PIPE_FLAG_TEST_START_PHASE0 | PIPE_FLAG_TEST_NO_RELEASE;

std::mutex g_status_mu;
uint32_t* g_status_ptr[kMaxDevices] = {nullptr};

// Address of this device's library status word (looked up once per device).
pipe_status_t library_status_word(uint32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PIPE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_status_mu);
  if (g_status_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_status_word)) != hipSuccess || p == nullptr)
      return PIPE_ERR_HIP;
    g_status_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_status_ptr[dev];
  return PIPE_OK;
}

// The row sum's workspace for callers that cannot allocate
// (pipe_rowsum_noalloc): one fixed buffer per device, held until the process
// ends. In host code `scratch` names a host-side stand-in, not the device
// buffer: its device address comes from hipGetSymbolAddress, once per device
// with that device current, and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[PIPE_ROWSUM_SCRATCH_BYTES];

std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {nullptr};

pipe_status_t library_scratch(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PIPE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PIPE_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return PIPE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Defaults per op, from the launch-shape sweeps on MI355X (bandwidth of the
// 16384^2 copy and 8192 x 65536 row sum, TFLOP/s of the 4096^3 GEMM).
pipe_config_t defaults(pipe_op_t op) {
  pipe_config_t c{};
  c.tile_m = 128;
  c.tile_n = (op == PIPE_OP_GEMM) ? 128 : 64;
  c.tile_k = (op == PIPE_OP_GEMM) ? 64 : 0;
  c.grid = 0;
  c.split = 0;
  switch (op) {
    case PIPE_OP_COPY:
      c.stages = 2;
      c.producer_waves = 4;
      c.consumer_waves = 4;
      c.swizzle_shift = 0;
      c.flags = PIPE_FLAG_NONTEMPORAL | PIPE_FLAG_XCD_REMAP | PIPE_FLAG_LAZY_COMMIT;
      break;
    case PIPE_OP_ROWSUM:
      c.stages = 3;
      c.producer_waves = 4;
      c.consumer_waves = 4;
      c.swizzle_shift = 0;
      c.flags = PIPE_FLAG_NONTEMPORAL | PIPE_FLAG_XCD_REMAP;
      break;
    default:
      c.stages = 2;
      c.producer_waves = 4;
      c.consumer_waves = 4;
      c.swizzle_shift = 1;
      c.flags = PIPE_FLAG_EAGER_NEWEST;
      break;
  }
  c.spin_limit = 0;
  c.trace_capacity = 0;
  c.trace = nullptr;
  c.status = nullptr;
  return c;
}

pipe_status_t check_common(const pipe_config_t& c) {
  if (c.flags & ~kKnownFlags) return PIPE_ERR_CONFIG;
  if ((c.flags & PIPE_FLAG_LAZY_COMMIT) && (c.flags & PIPE_FLAG_EAGER_NEWEST))
    return PIPE_ERR_CONFIG;
  if (c.grid < 0 || c.split < 0 || c.swizzle_shift < 0 || c.swizzle_shift > 3)
    return PIPE_ERR_CONFIG;
  if (c.trace_capacity < 0) return PIPE_ERR_CONFIG;
  if ((c.flags & PIPE_FLAG_TRACE) && (c.trace == nullptr || c.trace_capacity == 0))
    return PIPE_ERR_NULL;
  if (c.status != nullptr && !aligned4(c.status)) return PIPE_ERR_ALIGN;
  if (c.trace != nullptr && !aligned4(c.trace)) return PIPE_ERR_ALIGN;
  return PIPE_OK;
}

pipe_status_t check_stream_cfg(const pipe_config_t& c) {
  pipe_status_t s = check_common(c);
  if (s != PIPE_OK) return s;
  if (c.flags & (PIPE_FLAG_GEMM_C_BF16 | PIPE_FLAG_GEMM_B_LINEAR | PIPE_FLAG_GEMM_STORE_WAVE |
                 PIPE_FLAG_GEMM_B_COLMAJOR))
    return PIPE_ERR_CONFIG;
  if (c.stages < 1 || c.stages > 8) return PIPE_ERR_STAGES;
  // 16 KiB tiles: the pages' 128 x 64, or the wider 64 x 128 and 32 x 256.
  if (!((c.tile_m == 128 && c.tile_n == 64) || (c.tile_m == 64 && c.tile_n == 128) ||
        (c.tile_m == 32 && c.tile_n == 256)))
    return PIPE_ERR_CONFIG;
  const int cw = c.consumer_waves, pw = c.producer_waves;
  if (c.flags & PIPE_FLAG_PRODUCER_VGPR) {
    if ((c.flags & (PIPE_FLAG_UNIFIED | PIPE_FLAG_DEBUG_CHECKS)) || c.tile_m != 128 ||
        c.tile_n != 64 || !regs_shape_supported(c.stages, cw, pw))
      return PIPE_ERR_CONFIG;
  }
  if ((c.flags & (PIPE_FLAG_TEST_JITTER | PIPE_FLAG_TEST_EARLY_RELEASE)) &&
      !(c.flags & PIPE_FLAG_DEBUG_CHECKS))
    return PIPE_ERR_CONFIG;
  if (c.flags & PIPE_FLAG_GROUP_LOADS) {
    if (!(c.flags & PIPE_FLAG_STRIP_GROUPS) ||
        (c.flags & (PIPE_FLAG_PRODUCER_VGPR | PIPE_FLAG_DEBUG_CHECKS | PIPE_FLAG_UNIFIED |
                    PIPE_FLAG_ROW_STRIPS)) ||
        !group_load_shape_supported(c.stages, cw, pw))
      return PIPE_ERR_CONFIG;
  }
  if (c.flags & PIPE_FLAG_DEBUG_CHECKS) {
    if ((c.flags & PIPE_FLAG_UNIFIED) || c.tile_m != 128 || c.tile_n != 64 ||
        !debug_shape_supported(c.stages, cw, pw))
      return PIPE_ERR_CONFIG;
  }
  if (c.flags & PIPE_FLAG_UNIFIED) {
    if (!unified_shape_supported(c.stages, cw, c.tile_n)) return PIPE_ERR_CONFIG;
    return c.stages * 16384 > kLdsLimit ? PIPE_ERR_STAGES : PIPE_OK;
  }
  if (!(pw == 1 || pw == 2 || pw == 4)) return PIPE_ERR_CONFIG;
  if (!(cw == 1 || cw == 2 || cw == 3 || cw == 4 || cw == 8)) return PIPE_ERR_CONFIG;
  if (!stream_shape_supported(c.stages, cw, pw, c.tile_n)) return PIPE_ERR_CONFIG;
  if (stream_lds_bytes(c.stages, cw) > kLdsLimit) return PIPE_ERR_STAGES;
  return PIPE_OK;
}

// The unified variant's extra constraints (see PIPE_FLAG_UNIFIED).
pipe_status_t check_unified(const pipe_config_t& c, int64_t M, int64_t N, bool checksums) {
  const int w = c.consumer_waves;
  if (!(w == 2 || w == 4 || w == 8)) return PIPE_ERR_CONFIG;
  if (checksums || (c.flags & (PIPE_FLAG_TRACE | PIPE_FLAG_TEST_START_PHASE0 |
                               PIPE_FLAG_TEST_NO_RELEASE)))
    return PIPE_ERR_CONFIG;
  if (M % c.tile_m != 0 || N % c.tile_n != 0) return PIPE_ERR_CONFIG;
  return PIPE_OK;
}

// Device code forms byte offsets in int64: a matrix of `rows` rows (plus up to
// one partial tile row) at a pitch of `ld` elements of `elem` bytes must span
// fewer than 2^62 bytes.
bool extent_fits(int64_t rows, int64_t ld, int64_t elem) {
  constexpr int64_t kMaxBytes = int64_t(1) << 62;
  if (rows < 0 || ld < 0 || rows > kMaxBytes) return false;
  return ld <= kMaxBytes / elem / (rows + 256);
}

struct StreamGeom {
  int32_t tile_rows, tile_cols, n_strips, strip_len, seg_len, split, items, grid;
  int32_t group;  // tile columns per grouped copy strip (1: plain strips)
};

// Tile columns per strip of a copy with PIPE_FLAG_STRIP_GROUPS: 4, else 2,
// where the grouped kernels take the launch; 1 (plain strips) elsewhere.
int copy_strip_group(const pipe_config_t& c, int64_t M, int64_t N, bool checksums) {
  if (!(c.flags & PIPE_FLAG_STRIP_GROUPS) ||
      (c.flags & (PIPE_FLAG_PRODUCER_VGPR | PIPE_FLAG_DEBUG_CHECKS)))
    return 1;
  if (checksums || (c.flags & (PIPE_FLAG_ROW_STRIPS | PIPE_FLAG_UNIFIED))) return 1;
  if (c.tile_m != 128 || c.tile_n != 64 || M % 128 != 0 || N % 64 != 0) return 1;
  const int64_t tile_cols = N / 64;
  for (int g = 4; g >= 2; g /= 2)
    if (tile_cols % g == 0 &&
        group_shape_supported(c.stages, c.consumer_waves, c.producer_waves, g))
      return g;
  return 1;
}

// Rowsum default split: the smallest power of two that gives >= 256 work
// items (one workgroup per CU of an MI355X).
int rowsum_default_split(int n_strips, int strip_len) {
  int split = 1;
  while ((int64_t)n_strips * split < 256 && split < strip_len) split *= 2;
  return split < strip_len ? split : strip_len;
}

pipe_status_t stream_geometry(int64_t M, int64_t N, const pipe_config_t& c, bool row_strips,
                              bool rowsum, StreamGeom* g, int group = 1) {
  // Ceiling divisions written so that M or N near INT64_MAX cannot overflow.
  const int64_t tr = M / c.tile_m + (M % c.tile_m != 0);
  const int64_t tc = N / c.tile_n + (N % c.tile_n != 0);
  if (tr > INT32_MAX || tc > INT32_MAX) return PIPE_ERR_SHAPE;
  g->tile_rows = (int32_t)tr;
  g->tile_cols = (int32_t)tc;
  g->group = group;
  g->n_strips = row_strips ? g->tile_rows : g->tile_cols / group;
  g->strip_len = row_strips ? g->tile_cols : g->tile_rows;  // tile rows of a grouped strip
  // Default split: the row sum's from rowsum_default_split; a copy keeps one
  // work item per tile column (G segments per strip of G tile columns).
  int split = c.split;
  if (split == 0) split = rowsum ? rowsum_default_split(g->n_strips, g->strip_len) : group;
  if (split > g->strip_len) split = g->strip_len;
  if (split < 1) split = 1;
  g->seg_len = (g->strip_len + split - 1) / split;
  g->split = (g->strip_len + g->seg_len - 1) / g->seg_len;  // no empty segments
  const int64_t items = (int64_t)g->n_strips * g->split;
  if (items > INT32_MAX) return PIPE_ERR_SHAPE;
  g->items = (int32_t)items;
  g->grid = (c.grid == 0 || c.grid > g->items) ? g->items : c.grid;
  // Barrier words count arrivals in 32 bits; keep every count below 2^31 (so
  // that a wrap never occurs, whatever the arrivals per phase).
  const int64_t per_wg = ((int64_t)g->items + g->grid - 1) / g->grid * g->seg_len * group;
  const int64_t arrivals = c.consumer_waves > c.producer_waves ? c.consumer_waves
                                                               : c.producer_waves;
  if (per_wg * arrivals >= (int64_t(1) << 31)) return PIPE_ERR_SHAPE;
  return PIPE_OK;
}

// Row-sum workspace: fp32 segment partials [split][M] from offset 0, then one
// uint32 arrival ticket per row strip from a 256-byte aligned offset. Nothing
// when each strip is one segment (the kernel writes `out` directly).
struct RowsumWorkspace {
  size_t ticket_offset;  // bytes
  size_t bytes;          // total
};

RowsumWorkspace rowsum_workspace(const StreamGeom& g, int64_t M) {
  RowsumWorkspace w{0, 0};
  if (g.split <= 1) return w;
  const size_t partials = (size_t)g.split * (size_t)M * sizeof(float);
  w.ticket_offset = (partials + 255) & ~(size_t)255;
  w.bytes = w.ticket_offset + (size_t)g.n_strips * sizeof(uint32_t);
  return w;
}

void fill_stream_params(const pipe_config_t& c, const StreamGeom& g, bool row_strips,
                        StreamParams* p) {
  p->tile_cols = g.tile_cols;
  p->n_strips = g.n_strips;
  p->strip_len = g.strip_len;
  p->seg_len = g.seg_len;
  p->split = g.split;
  p->items = g.items;
  p->row_strips = row_strips ? 1 : 0;
  p->swz_shift = c.swizzle_shift;
  // Commit lag: at most S-1 tiles (the protocol's liveness bound; S-G when
  // consumers hold G slots at once) and at most what the vmcnt counter can
  // track: (lag + 1) tiles of 16 / producer_waves loads.
  const int max_lag = stream_max_lag(c.producer_waves);
  const int live_lag = c.stages - g.group;
  p->lag = live_lag < max_lag ? live_lag : max_lag;
  p->xcd_remap = ((c.flags & PIPE_FLAG_XCD_REMAP) && g.items % 8 == 0) ? 1 : 0;
  p->interleave = (c.flags & PIPE_FLAG_SPLIT_INTERLEAVE) ? 1 : 0;
  p->spin_limit = c.spin_limit ? c.spin_limit : kDefaultSpin;
  p->start_phase = (c.flags & PIPE_FLAG_TEST_START_PHASE0) ? 0u : 1u;
  p->no_release = (c.flags & PIPE_FLAG_TEST_NO_RELEASE) ? 1 : 0;
  p->trace = (c.flags & PIPE_FLAG_TRACE) ? c.trace : nullptr;
  p->trace_cap = (c.flags & PIPE_FLAG_TRACE) ? c.trace_capacity : 0;
  p->nt = (c.flags & PIPE_FLAG_NONTEMPORAL) ? 1 : 0;
  p->eager = eager_min_pending(c.flags);
  p->jitter = (c.flags & PIPE_FLAG_TEST_JITTER) ? 1 : 0;
  p->early_release = (c.flags & PIPE_FLAG_TEST_EARLY_RELEASE) ? 1 : 0;
}

// The main kernel of a copy or row sum: the unified ring, the register
// producer engine, grouped strips, or the DMA ring.
hipError_t launch_stream_op(int op, const pipe_config_t& c, const StreamGeom& g,
                            const StreamParams& p, hipStream_t stream) {
  if (c.flags & PIPE_FLAG_UNIFIED)
    return launch_unified(op, c.stages, c.consumer_waves, c.tile_n, g.grid, p, stream);
  if (c.flags & PIPE_FLAG_PRODUCER_VGPR)
    return launch_stream_regs(op, c.stages, c.consumer_waves, c.producer_waves, g.grid, p, stream);
  if (c.flags & PIPE_FLAG_DEBUG_CHECKS)
    return launch_stream_debug(op, c.stages, c.consumer_waves, c.producer_waves, g.grid, p,
                               stream);
  if (g.group == 4 && (c.flags & PIPE_FLAG_GROUP_LOADS))
    return launch_stream_group_load(c.stages, c.consumer_waves, c.producer_waves, g.grid, p,
                                    stream);
  if (g.group > 1)
    return launch_stream_group(c.stages, c.consumer_waves, c.producer_waves, g.group, g.grid, p,
                               stream);
  return launch_stream(op, c.stages, c.consumer_waves, c.producer_waves, c.tile_n, g.grid, p,
                       stream);
}

// The library's own per-device memory (status word, row-sum buffer) is looked
// up for the current device, so a launch that uses it must go to a stream of
// that device; the null stream always does.
pipe_status_t check_stream_device(hipStream_t st) {
  if (st == nullptr) return PIPE_OK;
  int cur = 0;
  hipDevice_t dev = 0;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(st, &dev) != hipSuccess)
    return PIPE_ERR_HIP;
  return dev == cur ? PIPE_OK : PIPE_ERR_CONFIG;
}

pipe_status_t resolve_status(const pipe_config_t& c, hipStream_t st, uint32_t** out) {
  if (c.status != nullptr) {
    *out = c.status;
    return PIPE_OK;
  }
  const pipe_status_t s = check_stream_device(st);
  if (s != PIPE_OK) return s;
  return library_status_word(out);
}

pipe_status_t hip_status(hipError_t e) { return e == hipSuccess ? PIPE_OK : PIPE_ERR_HIP; }

// GEMM checks that need no pointers: the configuration ...
pipe_status_t gemm_check_config(const pipe_config_t& c) {
  pipe_status_t s = check_common(c);
  if (s != PIPE_OK) return s;
  // The unified kernels: 256 x 256 tiles, waves that all load and compute,
  // fp32 C (the producer count and commit policy do not apply). 16 waves:
  // 64-K stages, two slots. 4 waves: the same, or 32-K stages in three to
  // five slots.
  if (c.flags & PIPE_FLAG_UNIFIED) {
    if (c.tile_m != 256 || c.tile_n != 256) return PIPE_ERR_CONFIG;
    if (c.consumer_waves == kGemmUnifiedWaves) {
      if (c.tile_k != 64) return PIPE_ERR_CONFIG;
      if (c.stages != 2) return PIPE_ERR_STAGES;
    } else if (c.consumer_waves == kGemmWideWaves) {
      if (c.tile_k != 64 && c.tile_k != 32) return PIPE_ERR_CONFIG;
      if (c.tile_k == 64 ? c.stages != 2 : (c.stages < 3 || c.stages > 5)) return PIPE_ERR_STAGES;
    } else {
      return PIPE_ERR_CONFIG;
    }
    if (c.split > 1) return PIPE_ERR_CONFIG;
    if (c.flags & (PIPE_FLAG_ROW_STRIPS | PIPE_FLAG_TEST_NO_RELEASE | PIPE_FLAG_STRIP_GROUPS |
                   PIPE_FLAG_GROUP_LOADS | PIPE_FLAG_PRODUCER_VGPR | PIPE_FLAG_DEBUG_CHECKS |
                   PIPE_FLAG_TEST_JITTER | PIPE_FLAG_TEST_EARLY_RELEASE | PIPE_FLAG_TRACE |
                   PIPE_FLAG_GEMM_STORE_WAVE | PIPE_FLAG_TEST_START_PHASE0))
      return PIPE_ERR_CONFIG;
    // bf16 C: the 32-K kernel only.
    if ((c.flags & PIPE_FLAG_GEMM_C_BF16) && c.tile_k != 32) return PIPE_ERR_CONFIG;
    if ((c.flags & PIPE_FLAG_GEMM_B_COLMAJOR) && (c.flags & PIPE_FLAG_GEMM_B_LINEAR))
      return PIPE_ERR_CONFIG;
    return PIPE_OK;
  }
  if (c.stages < 1 || c.stages > 4) return PIPE_ERR_STAGES;
  // 128 x 128 output tiles with 4 MFMA waves, or 256 x 128 with 8.
  if ((c.tile_m != 128 && c.tile_m != 256) || c.tile_n != 128 || c.tile_k != 64)
    return PIPE_ERR_CONFIG;
  if ((c.producer_waves != 2 && c.producer_waves != 4) || c.consumer_waves != c.tile_m / 32)
    return PIPE_ERR_CONFIG;
  if (c.split > 1) return PIPE_ERR_CONFIG;
  if (c.flags & (PIPE_FLAG_ROW_STRIPS | PIPE_FLAG_TEST_NO_RELEASE | PIPE_FLAG_STRIP_GROUPS |
                 PIPE_FLAG_GROUP_LOADS |
                 PIPE_FLAG_PRODUCER_VGPR | PIPE_FLAG_DEBUG_CHECKS | PIPE_FLAG_TEST_JITTER |
                 PIPE_FLAG_TEST_EARLY_RELEASE))
    return PIPE_ERR_CONFIG;
  const bool c_bf16 = (c.flags & PIPE_FLAG_GEMM_C_BF16) != 0;
  const bool store_wave = (c.flags & PIPE_FLAG_GEMM_STORE_WAVE) != 0;
  if (store_wave && !c_bf16) return PIPE_ERR_CONFIG;
  if ((c.flags & PIPE_FLAG_GEMM_B_COLMAJOR) && (c.flags & PIPE_FLAG_GEMM_B_LINEAR))
    return PIPE_ERR_CONFIG;
  // The trace kernel: fp32 C, row-major B.
  if ((c.flags & PIPE_FLAG_TRACE) && (c.flags & (PIPE_FLAG_GEMM_C_BF16 | PIPE_FLAG_GEMM_B_COLMAJOR)))
    return PIPE_ERR_CONFIG;
  // 256-row tiles: four producer waves, no store wave, no trace kernel.
  if (c.tile_m == 256 && (c.producer_waves != 4 ||
                          (c.flags & (PIPE_FLAG_GEMM_STORE_WAVE | PIPE_FLAG_TRACE))))
    return PIPE_ERR_CONFIG;
  if (gemm_lds_bytes(c.stages, c_bf16, store_wave, c.tile_m) > kLdsLimit) return PIPE_ERR_STAGES;
  return PIPE_OK;
}

// ... the shape and pitches ...
pipe_status_t gemm_check_shape(const pipe_config_t& c, int64_t M, int64_t N, int64_t K,
                               int64_t lda, int64_t ldb, int64_t ldc) {
  const bool b_col = (c.flags & PIPE_FLAG_GEMM_B_COLMAJOR) != 0;
  if (M < 0 || N < 0 || K < 0 || lda < K || ldb < (b_col ? K : N) || ldc < N)
    return PIPE_ERR_SHAPE;
  // Whole 16-byte chunks of B's and A's rows; ragged tiles are masked (the
  // trace kernel takes whole tiles only).
  if (N % 8 != 0 || K % 8 != 0) return PIPE_ERR_SHAPE;
  if ((c.flags & PIPE_FLAG_TRACE) && (M % c.tile_m != 0 || N % 128 != 0 || K % 64 != 0))
    return PIPE_ERR_SHAPE;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return PIPE_ERR_SHAPE;
  if (!extent_fits(M, lda, 2) || !extent_fits(b_col ? N : K, ldb, 2) ||
      !extent_fits(M, ldc, (c.flags & PIPE_FLAG_GEMM_C_BF16) ? 2 : 4))
    return PIPE_ERR_SHAPE;
  return PIPE_OK;
}

// ... and the launch parameters (all but the pointers) with the grid, for
// M, N, K > 0.
pipe_status_t gemm_fill_params(const pipe_config_t& c, int64_t M, int64_t N, int64_t K,
                               int64_t lda, int64_t ldb, int64_t ldc, GemmParams* p, int* grid) {
  p->lda = lda * 2;
  p->ldb = ldb * 2;
  p->ldc = ldc;
  p->M = (int32_t)M;
  p->N = (int32_t)N;
  p->K = (int32_t)K;
  p->unified = (c.flags & PIPE_FLAG_UNIFIED) ? c.consumer_waves : 0;
  p->tiles_n = (int32_t)((N + c.tile_n - 1) / c.tile_n);
  p->k_steps = (int32_t)((K + c.tile_k - 1) / c.tile_k);
  const int64_t items = ((M + c.tile_m - 1) / c.tile_m) * (int64_t)p->tiles_n;
  p->tile_m = c.tile_m;
  if (items > INT32_MAX) return PIPE_ERR_SHAPE;
  p->items = (int32_t)items;
  p->swz_shift = c.swizzle_shift;
  p->b_swz = (c.flags & PIPE_FLAG_GEMM_B_LINEAR) ? 0 : 1;
  p->b_colmajor = (c.flags & PIPE_FLAG_GEMM_B_COLMAJOR) ? 1 : 0;
  p->eager = eager_min_pending(c.flags);
  p->c_bf16 = (c.flags & PIPE_FLAG_GEMM_C_BF16) ? 1 : 0;
  p->store_wave = (c.flags & PIPE_FLAG_GEMM_STORE_WAVE) ? 1 : 0;
  p->spin_limit = c.spin_limit ? c.spin_limit : kDefaultSpin;
  p->trace = (c.flags & PIPE_FLAG_TRACE) ? c.trace : nullptr;
  p->trace_cap = (c.flags & PIPE_FLAG_TRACE) ? c.trace_capacity : 0;
  if (c.flags & PIPE_FLAG_TEST_START_PHASE0) return PIPE_ERR_CONFIG;
  *grid = (c.grid == 0 || c.grid > p->items) ? p->items : c.grid;
  // Barrier words count arrivals in 32 bits (one per MFMA wave and stage on empty).
  if (((int64_t)p->items + *grid - 1) / *grid * p->k_steps * c.consumer_waves >= (int64_t(1) << 31))
    return PIPE_ERR_SHAPE;
  return PIPE_OK;
}

// The row sum's launches for a validated call: with segment partials, zero the
// strips' arrival tickets, then run the stream kernel, whose last arrival per
// strip writes `out`; else the stream kernel writes `out` itself.
pipe_status_t launch_rowsum(const pipe_config_t& c, const StreamGeom& g,
                            const RowsumWorkspace& ws, uint8_t* workspace, float* out,
                            StreamParams* p, hipStream_t st) {
  if (ws.bytes == 0) {
    p->out = out;
    p->final_out = nullptr;
    p->tickets = nullptr;
  } else {
    p->out = reinterpret_cast<float*>(workspace);
    p->final_out = out;
    p->tickets = reinterpret_cast<uint32_t*>(workspace + ws.ticket_offset);
    pipe_status_t s = hip_status(launch_fill_u32(p->tickets, g.n_strips, 0u, st));
    if (s != PIPE_OK) return s;
  }
  return hip_status(launch_stream_op(kOpRowsum, c, g, *p, st));
}

// pipe_rowsum and pipe_rowsum_noalloc: the caller's workspace, or (use_scratch)
// this device's library buffer, which calls no allocator.
pipe_status_t rowsum_call(const void* A, float* out, int64_t M, int64_t N, int64_t lda,
                          const pipe_config_t* cfg, void* workspace, size_t workspace_bytes,
                          bool use_scratch, void* stream) {
  const pipe_config_t c = cfg ? *cfg : defaults(PIPE_OP_ROWSUM);
  pipe_status_t s = check_stream_cfg(c);
  if (s != PIPE_OK) return s;
  if (c.flags & (PIPE_FLAG_ROW_STRIPS | PIPE_FLAG_GROUP_LOADS))
    return PIPE_ERR_CONFIG;  // always row strips; grouped loads are the copy's
  if (M < 0 || N < 0 || lda < N) return PIPE_ERR_SHAPE;
  if (N % 8 != 0 || !extent_fits(M, lda, 2)) return PIPE_ERR_SHAPE;
  if (M == 0) return PIPE_OK;
  if (out == nullptr) return PIPE_ERR_NULL;
  if (!aligned4(out)) return PIPE_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (N == 0) return hip_status(launch_fill_f32(out, M, 1, 1, 0.f, st));
  if (A == nullptr) return PIPE_ERR_NULL;
  if (!aligned16(A) || (lda % 8)) return PIPE_ERR_ALIGN;
  const bool unified = (c.flags & PIPE_FLAG_UNIFIED) != 0;
  if (unified) {
    s = check_unified(c, M, N, false);
    if (s != PIPE_OK) return s;
  }
  StreamGeom g;
  s = stream_geometry(M, N, c, true, true, &g);
  if (s != PIPE_OK) return s;
  const RowsumWorkspace ws = rowsum_workspace(g, M);
  if (use_scratch) {
    if (ws.bytes > PIPE_ROWSUM_SCRATCH_BYTES) return PIPE_ERR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
  } else if (ws.bytes > 0) {
    if (workspace == nullptr || workspace_bytes < ws.bytes) return PIPE_ERR_WORKSPACE;
    if (!aligned4(workspace)) return PIPE_ERR_ALIGN;
  }
  StreamParams p{};
  fill_stream_params(c, g, true, &p);
  p.src = static_cast<const uint8_t*>(A);
  p.dst = nullptr;
  p.checksums = nullptr;
  p.ld_src = lda * 2;
  p.ld_dst = 0;
  p.M = M;
  p.N = N;
  s = resolve_status(c, st, &p.status);
  if (s != PIPE_OK) return s;
  if (use_scratch && ws.bytes > 0) {
    s = check_stream_device(st);
    if (s != PIPE_OK) return s;
    uint8_t* buf = nullptr;
    s = library_scratch(&buf);
    if (s != PIPE_OK) return s;
    workspace = buf;
  }
  return launch_rowsum(c, g, ws, static_cast<uint8_t*>(workspace), out, &p, st);
}

// Address of the kernel that `launch` would launch, without launching it.
template <class F>
pipe_status_t record_kernel(F launch, const void** fn) {
  *fn = nullptr;
  set_record_slot(fn);
  const hipError_t e = launch();
  set_record_slot(nullptr);
  return (e == hipSuccess && *fn != nullptr) ? PIPE_OK : PIPE_ERR_CONFIG;
}

}  // namespace

extern "C" {

int pipe_abi_version(void) { return PIPE_ABI_VERSION; }

const char* pipe_status_str(int status) {
  switch (status) {
    case PIPE_OK: return "ok";
    case PIPE_ERR_NULL: return "null pointer";
    case PIPE_ERR_SHAPE: return "unsupported shape";
    case PIPE_ERR_ALIGN: return "misaligned pointer or pitch";
    case PIPE_ERR_STAGES: return "stage count out of range or ring exceeds LDS";
    case PIPE_ERR_CONFIG: return "unsupported configuration";
    case PIPE_ERR_WORKSPACE: return "workspace missing or too small";
    case PIPE_ERR_HIP: return "HIP runtime error";
    case PIPE_ERR_TIMEOUT: return "pipeline wait timed out";
    case PIPE_ERR_INVARIANT: return "pipeline invariant check failed";
    default: return "unknown status";
  }
}

pipe_status_t pipe_config_default(pipe_op_t op, pipe_config_t* cfg) {
  if (cfg == nullptr) return PIPE_ERR_NULL;
  if (op != PIPE_OP_COPY && op != PIPE_OP_ROWSUM && op != PIPE_OP_GEMM) return PIPE_ERR_CONFIG;
  *cfg = defaults(op);
  return PIPE_OK;
}

pipe_status_t pipe_tile_copy(const void* src, void* dst, int64_t M, int64_t N, int64_t ld_src,
                             int64_t ld_dst, const pipe_config_t* cfg, uint32_t* tile_checksums,
                             void* stream) {
  const pipe_config_t c = cfg ? *cfg : defaults(PIPE_OP_COPY);
  pipe_status_t s = check_stream_cfg(c);
  if (s != PIPE_OK) return s;
  if (M < 0 || N < 0 || ld_src < N || ld_dst < N) return PIPE_ERR_SHAPE;
  if (N % 8 != 0) return PIPE_ERR_SHAPE;
  if (!extent_fits(M, ld_src, 2) || !extent_fits(M, ld_dst, 2)) return PIPE_ERR_SHAPE;
  if (M == 0 || N == 0) return PIPE_OK;
  if (src == nullptr || dst == nullptr) return PIPE_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst) || (ld_src % 8) || (ld_dst % 8)) return PIPE_ERR_ALIGN;
  if (tile_checksums != nullptr && !aligned4(tile_checksums)) return PIPE_ERR_ALIGN;
  const bool row_strips = (c.flags & PIPE_FLAG_ROW_STRIPS) != 0;
  const bool unified = (c.flags & PIPE_FLAG_UNIFIED) != 0;
  if (unified) {
    s = check_unified(c, M, N, tile_checksums != nullptr);
    if (s != PIPE_OK) return s;
  }
  StreamGeom g;
  s = stream_geometry(M, N, c, row_strips, false, &g,
                      copy_strip_group(c, M, N, tile_checksums != nullptr));
  if (s != PIPE_OK) return s;

  StreamParams p{};
  fill_stream_params(c, g, row_strips, &p);
  p.src = static_cast<const uint8_t*>(src);
  p.dst = static_cast<uint8_t*>(dst);
  p.out = nullptr;
  p.checksums = tile_checksums;
  p.ld_src = ld_src * 2;
  p.ld_dst = ld_dst * 2;
  p.M = M;
  p.N = N;
  s = resolve_status(c, static_cast<hipStream_t>(stream), &p.status);
  if (s != PIPE_OK) return s;
  return hip_status(launch_stream_op(kOpCopy, c, g, p, static_cast<hipStream_t>(stream)));
}

pipe_status_t pipe_rowsum_workspace_bytes(int64_t M, int64_t N, const pipe_config_t* cfg,
                                          size_t* bytes) {
  if (bytes == nullptr) return PIPE_ERR_NULL;
  const pipe_config_t c = cfg ? *cfg : defaults(PIPE_OP_ROWSUM);
  pipe_status_t s = check_stream_cfg(c);
  if (s != PIPE_OK) return s;
  if (c.flags & (PIPE_FLAG_ROW_STRIPS | PIPE_FLAG_GROUP_LOADS)) return PIPE_ERR_CONFIG;  // as pipe_rowsum
  if (M < 0 || N < 0 || N % 8 != 0) return PIPE_ERR_SHAPE;
  *bytes = 0;
  if (M == 0 || N == 0) return PIPE_OK;
  StreamGeom g;
  s = stream_geometry(M, N, c, true, true, &g);
  if (s != PIPE_OK) return s;
  *bytes = rowsum_workspace(g, M).bytes;
  return PIPE_OK;
}

pipe_status_t pipe_rowsum(const void* A, float* out, int64_t M, int64_t N, int64_t lda,
                          const pipe_config_t* cfg, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return rowsum_call(A, out, M, N, lda, cfg, workspace, workspace_bytes, false, stream);
}

pipe_status_t pipe_rowsum_noalloc(const void* A, float* out, int64_t M, int64_t N, int64_t lda,
                                  const pipe_config_t* cfg, void* stream) {
  return rowsum_call(A, out, M, N, lda, cfg, nullptr, 0, true, stream);
}

pipe_status_t pipe_gemm_mainloop(const void* A, const void* B, void* C, int64_t M, int64_t N,
                                 int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                 const pipe_config_t* cfg, void* stream) {
  const pipe_config_t c = cfg ? *cfg : defaults(PIPE_OP_GEMM);
  pipe_status_t s = gemm_check_config(c);
  if (s != PIPE_OK) return s;
  s = gemm_check_shape(c, M, N, K, lda, ldb, ldc);
  if (s != PIPE_OK) return s;
  const bool c_bf16 = (c.flags & PIPE_FLAG_GEMM_C_BF16) != 0;
  if (M == 0 || N == 0) return PIPE_OK;
  if (C == nullptr) return PIPE_ERR_NULL;
  if (c_bf16 ? (!aligned16(C) || (ldc % 8)) : !aligned4(C)) return PIPE_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (K == 0) {
    return hip_status(c_bf16 ? launch_fill_u16(static_cast<uint16_t*>(C), M, N, ldc, 0, st)
                             : launch_fill_f32(static_cast<float*>(C), M, N, ldc, 0.f, st));
  }
  if (A == nullptr || B == nullptr) return PIPE_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || (lda % 8) || (ldb % 8)) return PIPE_ERR_ALIGN;
  GemmParams p{};
  int grid = 0;
  s = gemm_fill_params(c, M, N, K, lda, ldb, ldc, &p, &grid);
  if (s != PIPE_OK) return s;
  p.A = static_cast<const uint8_t*>(A);
  p.B = static_cast<const uint8_t*>(B);
  p.C = C;
  s = resolve_status(c, st, &p.status);
  if (s != PIPE_OK) return s;
  return hip_status(launch_gemm(c.stages, c.producer_waves, grid, p, st));
}

pipe_status_t pipe_query_kernel(pipe_op_t op, const pipe_config_t* cfg, int64_t M, int64_t N,
                                int64_t K, pipe_kernel_info_t* info) {
  if (info == nullptr) return PIPE_ERR_NULL;
  const pipe_config_t c = cfg ? *cfg : defaults(op);
  *info = pipe_kernel_info_t{};
  if (op == PIPE_OP_GEMM) {
    pipe_status_t s = gemm_check_config(c);  // rejects what pipe_gemm_mainloop rejects
    if (s != PIPE_OK) return s;
    if (c.flags & PIPE_FLAG_TEST_START_PHASE0) return PIPE_ERR_CONFIG;
    if (M < 0 || N < 0 || K < 0 || N % 8 || K % 8) return PIPE_ERR_SHAPE;
    if ((c.flags & PIPE_FLAG_TRACE) && (M % c.tile_m || N % 128 || K % 64)) return PIPE_ERR_SHAPE;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return PIPE_ERR_SHAPE;
    const int64_t items = ((M + c.tile_m - 1) / c.tile_m) * ((N + c.tile_n - 1) / c.tile_n);
    if (items > INT32_MAX) return PIPE_ERR_SHAPE;
    const bool c_bf16 = (c.flags & PIPE_FLAG_GEMM_C_BF16) != 0;
    const bool store_wave = (c.flags & PIPE_FLAG_GEMM_STORE_WAVE) != 0;
    const bool unified = (c.flags & PIPE_FLAG_UNIFIED) != 0;
    info->lds_bytes = unified ? (c.tile_k == 32 ? c.stages * 32768 : kGemmUnifiedLdsBytes)
                              : gemm_lds_bytes(c.stages, c_bf16, store_wave, c.tile_m);
    info->threads = unified ? 64 * c.consumer_waves
                            : gemm_threads(c.producer_waves, c_bf16, store_wave, c.tile_m);
    info->items = (int32_t)items;
    info->grid = (c.grid == 0 || c.grid > info->items) ? info->items : c.grid;
    info->tiles_per_item = (int32_t)((K + c.tile_k - 1) / c.tile_k);
    info->split = 1;
    return PIPE_OK;
  }
  if (op != PIPE_OP_COPY && op != PIPE_OP_ROWSUM) return PIPE_ERR_CONFIG;
  pipe_status_t s = check_stream_cfg(c);
  if (s != PIPE_OK) return s;
  const bool rowsum = op == PIPE_OP_ROWSUM;
  if (rowsum && (c.flags & (PIPE_FLAG_ROW_STRIPS | PIPE_FLAG_GROUP_LOADS)))
    return PIPE_ERR_CONFIG;  // as pipe_rowsum
  if (M < 0 || N < 0 || N % 8 || !extent_fits(M, N, 2)) return PIPE_ERR_SHAPE;
  const bool row_strips = rowsum || (c.flags & PIPE_FLAG_ROW_STRIPS);
  const bool unified = (c.flags & PIPE_FLAG_UNIFIED) != 0;
  if (unified) {
    s = check_unified(c, M, N, false);
    if (s != PIPE_OK) return s;
  }
  info->lds_bytes = unified ? c.stages * 16384 : stream_lds_bytes(c.stages, c.consumer_waves);
  info->threads = 64 * (unified ? c.consumer_waves : c.producer_waves + c.consumer_waves);
  if (M == 0 || N == 0) return PIPE_OK;
  StreamGeom g;
  s = stream_geometry(M, N, c, row_strips, rowsum, &g,
                      rowsum ? 1 : copy_strip_group(c, M, N, false));
  if (s != PIPE_OK) return s;
  info->grid = g.grid;
  info->items = g.items;
  info->tiles_per_item = g.seg_len * g.group;
  info->split = g.split;
  return PIPE_OK;
}

pipe_status_t pipe_kernel_resources(pipe_op_t op, const pipe_config_t* cfg, int64_t M, int64_t N,
                                    int64_t K, pipe_kernel_resources_t* out) {
  if (out == nullptr) return PIPE_ERR_NULL;
  *out = pipe_kernel_resources_t{};
  const pipe_config_t c = cfg ? *cfg : defaults(op);
  const void* fn = nullptr;
  pipe_status_t s;
  if (op == PIPE_OP_GEMM) {
    s = gemm_check_config(c);
    if (s != PIPE_OK) return s;
    const bool b_col = (c.flags & PIPE_FLAG_GEMM_B_COLMAJOR) != 0;
    s = gemm_check_shape(c, M, N, K, K, b_col ? K : N, N);
    if (s != PIPE_OK) return s;
    if (M == 0 || N == 0 || K == 0) return PIPE_ERR_SHAPE;
    GemmParams p{};
    int grid = 0;
    s = gemm_fill_params(c, M, N, K, K, b_col ? K : N, N, &p, &grid);
    if (s != PIPE_OK) return s;
    s = record_kernel([&] { return launch_gemm(c.stages, c.producer_waves, grid, p, nullptr); },
                      &fn);
  } else if (op == PIPE_OP_COPY || op == PIPE_OP_ROWSUM) {
    s = check_stream_cfg(c);
    if (s != PIPE_OK) return s;
    const bool rowsum = op == PIPE_OP_ROWSUM;
    if (rowsum && (c.flags & (PIPE_FLAG_ROW_STRIPS | PIPE_FLAG_GROUP_LOADS)))
      return PIPE_ERR_CONFIG;
    if (M < 0 || N < 0 || N % 8 != 0 || !extent_fits(M, N, 2)) return PIPE_ERR_SHAPE;
    if (M == 0 || N == 0) return PIPE_ERR_SHAPE;
    const bool row_strips = rowsum || (c.flags & PIPE_FLAG_ROW_STRIPS);
    const bool unified = (c.flags & PIPE_FLAG_UNIFIED) != 0;
    if (unified) {
      s = check_unified(c, M, N, false);
      if (s != PIPE_OK) return s;
    }
    StreamGeom g;
    s = stream_geometry(M, N, c, row_strips, rowsum, &g,
                        rowsum ? 1 : copy_strip_group(c, M, N, false));
    if (s != PIPE_OK) return s;
    StreamParams p{};
    fill_stream_params(c, g, row_strips, &p);
    p.ld_src = N * 2;
    p.ld_dst = rowsum ? 0 : N * 2;
    p.M = M;
    p.N = N;
    const int kop = rowsum ? kOpRowsum : kOpCopy;
    s = record_kernel([&] { return launch_stream_op(kop, c, g, p, nullptr); }, &fn);
  } else {
    return PIPE_ERR_CONFIG;
  }
  if (s != PIPE_OK) return s;
  hipFuncAttributes attr{};
  if (hipFuncGetAttributes(&attr, fn) != hipSuccess) return PIPE_ERR_HIP;
  out->vgprs = attr.numRegs;
  out->lds_bytes = (int32_t)attr.sharedSizeBytes;
  out->scratch_bytes = (int32_t)attr.localSizeBytes;
  out->max_threads = attr.maxThreadsPerBlock;
  return PIPE_OK;
}

pipe_status_t pipe_status_from_word(uint32_t word) {
  if (word & PIPE_STATUS_INVARIANT) return PIPE_ERR_INVARIANT;
  if (word & (PIPE_STATUS_TIMEOUT_PRODUCER | PIPE_STATUS_TIMEOUT_CONSUMER)) return PIPE_ERR_TIMEOUT;
  return PIPE_OK;
}

pipe_status_t pipe_device_status(uint32_t* out, int clear) {
  if (out == nullptr) return PIPE_ERR_NULL;
  uint32_t* word = nullptr;
  pipe_status_t s = library_status_word(&word);
  if (s != PIPE_OK) return s;
  if (hipMemcpy(out, word, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return PIPE_ERR_HIP;
  if (clear) {
    const uint32_t zero = 0;
    if (hipMemcpy(word, &zero, sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess)
      return PIPE_ERR_HIP;
  }
  return PIPE_OK;
}

}  // extern "C"
