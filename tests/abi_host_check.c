/*
 * Host-side check of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer (see test_host_sanitizers.py).
 *
 * Every call either fails validation (so nothing reaches the device; the
 * data pointers below are never dereferenced) or is pure host arithmetic
 * (pipe_config_default, pipe_query_kernel, pipe_status_str). A sanitizer
 * report or a wrong status code fails the run.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pipe_tile.h"

static int failures = 0;

#define EXPECT(cond)                                                 \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

/* Never dereferenced: every call using it fails validation first. */
#define FAKE ((void*)(uintptr_t)0x10000)
#define FAKE_AT(off) ((void*)(uintptr_t)(0x10000 + (off)))

static pipe_config_t dflt(pipe_op_t op) {
  pipe_config_t c;
  memset(&c, 0xA5, sizeof c); /* garbage in, defaults out */
  EXPECT(pipe_config_default(op, &c) == PIPE_OK);
  return c;
}

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(uint32_t n) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg >> 33) % n;
}

int main(void) {
  EXPECT(pipe_abi_version() == PIPE_ABI_VERSION);
  for (int s = -3; s < 12; ++s) EXPECT(pipe_status_str(s) != NULL && strlen(pipe_status_str(s)) > 0);
  EXPECT(pipe_config_default(PIPE_OP_COPY, NULL) == PIPE_ERR_NULL);
  EXPECT(pipe_config_default((pipe_op_t)7, NULL) != PIPE_OK);
  {
    pipe_config_t junk;
    EXPECT(pipe_config_default((pipe_op_t)7, &junk) == PIPE_ERR_CONFIG);
    EXPECT(pipe_config_default((pipe_op_t)-1, &junk) == PIPE_ERR_CONFIG);
  }

  /* copy: validation failures */
  pipe_config_t c = dflt(PIPE_OP_COPY);
  EXPECT(pipe_tile_copy(NULL, FAKE, 256, 128, 128, 128, &c, NULL, NULL) == PIPE_ERR_NULL);
  EXPECT(pipe_tile_copy(FAKE, FAKE, 256, 12, 128, 128, &c, NULL, NULL) == PIPE_ERR_SHAPE);
  EXPECT(pipe_tile_copy(FAKE, FAKE, -1, 128, 128, 128, &c, NULL, NULL) == PIPE_ERR_SHAPE);
  EXPECT(pipe_tile_copy(FAKE, FAKE, INT64_MAX, 128, 128, 128, &c, NULL, NULL) == PIPE_ERR_SHAPE);
  /* pitches whose byte extent would overflow int64 offsets on the device */
  EXPECT(pipe_tile_copy(FAKE, FAKE, 1024, 128, INT64_MAX & ~(int64_t)7, 128, &c, NULL, NULL) ==
         PIPE_ERR_SHAPE);
  EXPECT(pipe_tile_copy(FAKE, FAKE, 1024, 128, 128, (int64_t)1 << 60, &c, NULL, NULL) ==
         PIPE_ERR_SHAPE);
  EXPECT(pipe_tile_copy(FAKE_AT(8), FAKE, 256, 128, 128, 128, &c, NULL, NULL) == PIPE_ERR_ALIGN);
  EXPECT(pipe_tile_copy(FAKE, FAKE, 256, 128, 128, 128, &c, (uint32_t*)FAKE_AT(2), NULL) ==
         PIPE_ERR_ALIGN);
  EXPECT(pipe_tile_copy(NULL, NULL, 0, 128, 128, 128, &c, NULL, NULL) == PIPE_OK);
  pipe_config_t b = c;
  b.stages = 9;
  EXPECT(pipe_tile_copy(FAKE, FAKE, 256, 128, 128, 128, &b, NULL, NULL) == PIPE_ERR_STAGES);
  b = c;
  b.consumer_waves = 5;
  EXPECT(pipe_tile_copy(FAKE, FAKE, 256, 128, 128, 128, &b, NULL, NULL) == PIPE_ERR_CONFIG);
  b = c;
  b.flags |= PIPE_FLAG_LAZY_COMMIT | PIPE_FLAG_EAGER_NEWEST;
  EXPECT(pipe_tile_copy(FAKE, FAKE, 256, 128, 128, 128, &b, NULL, NULL) == PIPE_ERR_CONFIG);
  b = c;
  b.flags = PIPE_FLAG_TRACE; /* trace without a buffer */
  EXPECT(pipe_tile_copy(FAKE, FAKE, 256, 128, 128, 128, &b, NULL, NULL) == PIPE_ERR_NULL);
  b = c;
  b.tile_m = 64; /* 64 x 64 is not a tile shape */
  EXPECT(pipe_tile_copy(FAKE, FAKE, 256, 128, 128, 128, &b, NULL, NULL) == PIPE_ERR_CONFIG);
  b = c;
  b.stages = 2;
  b.producer_waves = 1;
  b.consumer_waves = 8;
  b.grid = 1; /* 2^28 tiles on one workgroup: 2^31 arrivals on one barrier */
  EXPECT(pipe_tile_copy(FAKE, FAKE, (int64_t)128 << 28, 64, 64, 64, &b, NULL, NULL) ==
         PIPE_ERR_SHAPE);

  /* row sum */
  pipe_config_t r = dflt(PIPE_OP_ROWSUM);
  size_t need = 0;
  EXPECT(pipe_rowsum_workspace_bytes(1024, 4096, &r, &need) == PIPE_OK);
  EXPECT(need > 0); /* the default split cuts these 8 row strips into segments */
  EXPECT(pipe_rowsum_workspace_bytes(1024, 4096, &r, NULL) == PIPE_ERR_NULL);
  EXPECT(pipe_rowsum(FAKE, (float*)FAKE, 1024, 4096, 4096, &r, NULL, 0, NULL) ==
         PIPE_ERR_WORKSPACE);
  EXPECT(pipe_rowsum(FAKE, (float*)FAKE, 1000, 4090, 4096, &r, FAKE, 1 << 20, NULL) ==
         PIPE_ERR_SHAPE);
  EXPECT(pipe_rowsum(NULL, NULL, 0, 4096, 4096, &r, NULL, 0, NULL) == PIPE_OK);
  EXPECT(pipe_rowsum(FAKE, (float*)FAKE, 4096, 4096, (int64_t)1 << 61, &r, FAKE, 1 << 20, NULL) ==
         PIPE_ERR_SHAPE);
  EXPECT(pipe_rowsum_workspace_bytes(INT64_MAX, 4096, &r, &need) == PIPE_ERR_SHAPE);

  /* GEMM */
  pipe_config_t g = dflt(PIPE_OP_GEMM);
  EXPECT(pipe_gemm_mainloop(FAKE, FAKE, FAKE, 256, 256, 100, 100, 256, 256, &g, NULL) ==
         PIPE_ERR_SHAPE);
  EXPECT(pipe_gemm_mainloop(FAKE_AT(4), FAKE, FAKE, 256, 256, 128, 128, 256, 256, &g, NULL) ==
         PIPE_ERR_ALIGN);
  pipe_config_t gb = g;
  gb.flags |= PIPE_FLAG_GEMM_C_BF16;
  EXPECT(pipe_gemm_mainloop(FAKE, FAKE, FAKE, 256, 256, 128, 128, 256, 260, &gb, NULL) ==
         PIPE_ERR_ALIGN);
  gb = g;
  gb.flags = PIPE_FLAG_GEMM_STORE_WAVE; /* needs bf16 C */
  EXPECT(pipe_gemm_mainloop(FAKE, FAKE, FAKE, 256, 256, 128, 128, 256, 256, &gb, NULL) ==
         PIPE_ERR_CONFIG);
  EXPECT(pipe_gemm_mainloop(FAKE, FAKE, FAKE, 0, 256, 128, 128, 256, 256, &g, NULL) == PIPE_OK);
  EXPECT(pipe_gemm_mainloop(FAKE, FAKE, FAKE, 256, 256, 128, (int64_t)1 << 60, 256, 256, &g,
                            NULL) == PIPE_ERR_SHAPE);
  EXPECT(pipe_gemm_mainloop(FAKE, FAKE, FAKE, 256, 256, 128, 128, 256, (int64_t)1 << 60, &g,
                            NULL) == PIPE_ERR_SHAPE);

  /* pipe_kernel_resources: every check below fails before the HIP runtime is asked */
  pipe_kernel_resources_t res;
  pipe_kernel_info_t info;
  EXPECT(pipe_kernel_resources(PIPE_OP_COPY, &c, 256, 128, 0, NULL) == PIPE_ERR_NULL);
  EXPECT(pipe_kernel_resources(PIPE_OP_COPY, &c, 0, 128, 0, &res) == PIPE_ERR_SHAPE);
  EXPECT(pipe_kernel_resources(PIPE_OP_COPY, &c, INT64_MAX, INT64_MAX & ~(int64_t)7, 0, &res) ==
         PIPE_ERR_SHAPE);
  EXPECT(pipe_kernel_resources(PIPE_OP_GEMM, &g, 256, 256, 0, &res) == PIPE_ERR_SHAPE);
  EXPECT(pipe_kernel_resources(PIPE_OP_GEMM, &g, (int64_t)1 << 40, 256, 128, &res) ==
         PIPE_ERR_SHAPE);
  EXPECT(pipe_kernel_resources((pipe_op_t)5, &c, 256, 128, 0, &res) == PIPE_ERR_CONFIG);
  EXPECT(pipe_query_kernel((pipe_op_t)9, &c, 256, 128, 0, &info) == PIPE_ERR_CONFIG);

  /* pipe_query_kernel: pure host arithmetic over many configurations and shapes */
  EXPECT(pipe_query_kernel(PIPE_OP_COPY, &c, 16, 16, 0, NULL) == PIPE_ERR_NULL);
  EXPECT(pipe_query_kernel(PIPE_OP_GEMM, &g, (int64_t)1 << 40, (int64_t)1 << 40, 64, &info) ==
         PIPE_ERR_SHAPE);
  EXPECT(pipe_query_kernel(PIPE_OP_COPY, &c, INT64_MAX, INT64_MAX & ~(int64_t)7, 0, &info) ==
         PIPE_ERR_SHAPE);
  const int32_t tms[] = {128, 64, 32, 16}, tns[] = {64, 128, 256, 32};
  const int64_t dims[] = {0, 1, 7, 8, 63, 64, 127, 128, 129, 1000, 4096, 65536, (int64_t)1 << 33};
  int accepted = 0;
  for (int i = 0; i < 20000; ++i) {
    const pipe_op_t op = (pipe_op_t)rnd(3);
    pipe_config_t q = dflt(op);
    q.stages = (int32_t)rnd(10);
    q.producer_waves = (int32_t)rnd(6);
    q.consumer_waves = (int32_t)rnd(10);
    q.split = (int32_t)rnd(20);
    q.grid = (int32_t)rnd(3) ? 0 : (int32_t)rnd(5000);
    const int sh = (int)rnd(4);
    if (op != PIPE_OP_GEMM) {
      q.tile_m = tms[sh];
      q.tile_n = tns[sh];
    }
    q.flags = rnd(2) ? q.flags : (uint32_t)rnd(0x100000);
    q.trace = NULL;
    q.status = NULL;
    const int64_t M = dims[rnd(13)], N = dims[rnd(13)] & ~(int64_t)7, K = dims[rnd(13)];
    const pipe_status_t s = pipe_query_kernel(op, &q, M, N, K, &info);
    if (s == PIPE_OK) {
      ++accepted;
      EXPECT(info.grid >= 0 && info.grid <= (info.items > 0 ? info.items : 0));
      EXPECT(info.threads == 0 || (info.threads % 64 == 0 && info.threads <= 1024));
      EXPECT(info.lds_bytes >= 0 && info.lds_bytes <= 160 * 1024);
    }
  }
  EXPECT(accepted > 100);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi host check ok (%d query configurations accepted)\n", accepted);
  return 0;
}
