/* Calls every entry point of the QLoRA NF4 C ABI with invalid arguments and
 * once with valid ones, against the host-only stand-ins of stubs.cpp, so
 * that the argument checks run under AddressSanitizer and
 * UndefinedBehaviorSanitizer. Every invalid call must fail with its error
 * code (or, where several checks could fire first, with some error other
 * than QLORA_ERR_HIP) before any launcher is reached; every valid call must
 * reach its launcher (and then fail with QLORA_ERR_HIP, as the stand-in
 * launchers do). Buffers are host memory: the layer never dereferences a
 * device pointer. Prints "reject: ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/qlora_nf4.h"

extern int qlora_stub_launches;

static int failures = 0;

static void expect(const char *what, int got, int want) {
  const int launches = qlora_stub_launches;
  (void)launches;
  if (got != want) {
    printf("FAIL %s: got %d, want %d (%s)\n", what, got, want, qlora_last_error());
    ++failures;
  }
}

/* rejected: an error other than a launch failure, no launcher reached */
static void rejected(const char *what, int got, int launches_before) {
  if (got >= 0 || got == QLORA_ERR_HIP || qlora_stub_launches != launches_before) {
    printf("FAIL %s: got %d, launches %d -> %d (%s)\n", what, got, launches_before, qlora_stub_launches,
           qlora_last_error());
    ++failures;
  } else if (qlora_last_error()[0] == '\0') {
    printf("FAIL %s: no error message\n", what);
    ++failures;
  }
}

static void reached(const char *what, int got, int launches_before) {
  if (got != QLORA_ERR_HIP || qlora_stub_launches != launches_before + 1) {
    printf("FAIL %s: got %d, launches %d -> %d (%s)\n", what, got, launches_before, qlora_stub_launches,
           qlora_last_error());
    ++failures;
  }
}

#define REJ(call)                      \
  do {                                 \
    const int n0 = qlora_stub_launches; \
    rejected(#call, (call), n0);       \
  } while (0)
#define REACH(call)                    \
  do {                                 \
    const int n0 = qlora_stub_launches; \
    reached(#call, (call), n0);        \
  } while (0)

static void *buf(size_t bytes) {
  void *p = aligned_alloc(256, (bytes + 255) / 256 * 256);
  memset(p, 0, (bytes + 255) / 256 * 256);
  return p;
}

static qlora_nf4_weight weight(int64_t rows, int64_t cols, int format, void *pool) {
  qlora_nf4_weight w;
  char *p = (char *)pool;
  w.rows = rows;
  w.cols = cols;
  w.codes = (uint8_t *)p;
  w.absmax_q = (int8_t *)(p + 4096);
  w.dq_scale = (float *)(p + 8192);
  w.dq_mean = (float *)(p + 12288);
  w.absmax = (float *)(p + 16384);
  w.format = format;
  return w;
}

int main(void) {
  float lv[16];
  char *pool = (char *)buf(1 << 16);
  char *ws = (char *)buf(1 << 22);
  char *data = (char *)buf(1 << 20);
  float *A = (float *)buf(1 << 16), *B = (float *)buf(1 << 16);
  const int64_t N = 128, K = 192, M = 40;
  const int r = 8;

  /* host-only queries */
  expect("codebook NULL", qlora_nf4_codebook(NULL), QLORA_ERR_NULL);
  expect("codebook", qlora_nf4_codebook(lv), QLORA_OK);
  if (lv[0] != -1.0f || lv[7] != 0.0f || lv[15] != 1.0f) {
    printf("FAIL codebook values\n");
    ++failures;
  }
  expect("levels NULL", qlora_format_levels(QLORA_FMT_NF4, NULL), QLORA_ERR_NULL);
  expect("levels format", qlora_format_levels(42, lv), QLORA_ERR_FORMAT);
  expect("levels fp4", qlora_format_levels(QLORA_FMT_FP4_DQ, lv), QLORA_OK);
  expect("storage 0", (int)qlora_nf4_storage_bytes(0, 64), 0);
  expect("weight storage format", (int)qlora_weight_storage_bytes(64, 64, 42), 0);
  expect("quantize ws 0", (int)qlora_nf4_quantize_workspace_bytes(-1, 64), 0);
  expect("linear ws r", (int)qlora_linear_workspace_bytes(M, N, K, 257), 0);
  expect("linear ws huge", (int)qlora_linear_workspace_bytes(M, (int64_t)1 << 24, K, 8), 0);
  expect("merge ws", (int)qlora_nf4_merge_workspace_bytes(N, K, -1), 0);
  expect("adamw ws", (int)qlora_adamw_workspace_bytes(0, 1), 0);

  /* quantize */
  qlora_nf4_weight w = weight(N, K, QLORA_FMT_NF4_DQ, pool);
  const size_t qws = qlora_nf4_quantize_workspace_bytes(N, K);
  REJ(qlora_nf4_quantize(NULL, QLORA_BF16, N, K, &w, ws, qws, NULL));
  REJ(qlora_nf4_quantize(data, 5, N, K, &w, ws, qws, NULL));
  REJ(qlora_nf4_quantize(data, QLORA_BF16, N, K, NULL, ws, qws, NULL));
  REJ(qlora_nf4_quantize(data, QLORA_BF16, N + 1, K, &w, ws, qws, NULL));
  REJ(qlora_nf4_quantize(data + 2, QLORA_BF16, N, K, &w, ws, qws, NULL));
  REJ(qlora_nf4_quantize(data, QLORA_BF16, N, K, &w, ws, qws - 1, NULL));
  REJ(qlora_nf4_quantize(data, QLORA_BF16, N, K, &w, NULL, qws, NULL));
  REJ(qlora_nf4_quantize(data, QLORA_BF16, N, K, &w, ws + 8, qws, NULL));
  {
    qlora_nf4_weight bad = w;
    bad.format = 9;
    REJ(qlora_nf4_quantize(data, QLORA_BF16, N, K, &bad, ws, qws, NULL));
    bad = w;
    bad.dq_scale = NULL;
    REJ(qlora_nf4_quantize(data, QLORA_BF16, N, K, &bad, ws, qws, NULL));
    bad = w;
    bad.codes = (uint8_t *)(pool + 4);
    REJ(qlora_nf4_quantize(data, QLORA_BF16, N, K, &bad, ws, qws, NULL));
    bad = w;
    bad.rows = 0;
    REJ(qlora_nf4_quantize(data, QLORA_BF16, 0, K, &bad, ws, qws, NULL));
  }
  REACH(qlora_nf4_quantize(data, QLORA_BF16, N, K, &w, ws, qws, NULL));
  {
    qlora_nf4_weight plain = weight(N, K, QLORA_FMT_NF4, pool);
    REACH(qlora_nf4_quantize(data, QLORA_F32, N, K, &plain, NULL, 0, NULL));
  }

  /* dequantize */
  REJ(qlora_nf4_dequantize(NULL, data, QLORA_F32, NULL));
  REJ(qlora_nf4_dequantize(&w, NULL, QLORA_F32, NULL));
  REJ(qlora_nf4_dequantize(&w, data, 3, NULL));
  REJ(qlora_nf4_dequantize(&w, data + 4, QLORA_F32, NULL));
  REACH(qlora_nf4_dequantize(&w, data, QLORA_BF16, NULL));

  /* linear forward and backward */
  const size_t lws = qlora_linear_workspace_bytes(M, N, K, r);
  void *X = data, *Y = data + 65536, *dY = data + 131072, *dX = data + 196608;
  float *dA = (float *)(data + 262144), *dB = (float *)(data + 327680);
  REJ(qlora_linear_fwd(NULL, M, &w, A, B, r, 2.0f, Y, ws, lws, NULL));
  REJ(qlora_linear_fwd(X, M, &w, A, B, r, 2.0f, NULL, ws, lws, NULL));
  REJ(qlora_linear_fwd(X, 0, &w, A, B, r, 2.0f, Y, ws, lws, NULL));
  REJ(qlora_linear_fwd(X, M, NULL, A, B, r, 2.0f, Y, ws, lws, NULL));
  REJ(qlora_linear_fwd(X, M, &w, A, B, 257, 2.0f, Y, ws, lws, NULL));
  REJ(qlora_linear_fwd(X, M, &w, NULL, B, r, 2.0f, Y, ws, lws, NULL));
  REJ(qlora_linear_fwd(X, M, &w, A, B, 0, 2.0f, Y, ws, lws, NULL));
  REJ(qlora_linear_fwd(X, M, &w, A + 1, B, r, 2.0f, Y, ws, lws, NULL));
  REJ(qlora_linear_fwd((char *)X + 2, M, &w, A, B, r, 2.0f, Y, ws, lws, NULL));
  REJ(qlora_linear_fwd(X, M, &w, A, B, r, 2.0f, Y, ws, lws - 1, NULL));
  REJ(qlora_linear_fwd(X, M, &w, A, B, r, 2.0f, Y, NULL, lws, NULL));
  REJ(qlora_linear_fwd(X, M, &w, A, B, r, 2.0f, Y, ws + 8, lws, NULL));
  REJ(qlora_linear_fwd(X, (int64_t)1 << 40, &w, A, B, r, 2.0f, Y, ws, lws, NULL));
  {
    qlora_nf4_weight odd = weight(N, K + 32, QLORA_FMT_NF4_DQ, pool);
    REJ(qlora_linear_fwd(X, M, &odd, A, B, r, 2.0f, Y, ws, lws, NULL));
    qlora_nf4_weight wide = weight(N, (int64_t)1 << 24, QLORA_FMT_NF4_DQ, pool);
    REJ(qlora_linear_fwd(X, 1, &wide, A, B, r, 2.0f, Y, ws, 1 << 22, NULL));
  }
  REACH(qlora_linear_fwd(X, M, &w, A, B, r, 2.0f, Y, ws, lws, NULL));
  REACH(qlora_linear_fwd(X, M, &w, NULL, NULL, 0, 0.0f, Y, ws, lws, NULL));
  REJ(qlora_linear_bwd(NULL, X, M, &w, A, B, r, 2.0f, dX, dA, dB, ws, lws, NULL));
  REJ(qlora_linear_bwd(dY, X, M, &w, A, B, r, 2.0f, dX, NULL, dB, ws, lws, NULL));
  REJ(qlora_linear_bwd(dY, X, M, &w, NULL, NULL, 0, 2.0f, dX, dA, NULL, ws, lws, NULL));
  REJ(qlora_linear_bwd(dY, X, M, &w, A, B, r, 2.0f, dX, dA + 1, dB, ws, lws, NULL));
  REJ(qlora_linear_bwd(dY, X, M, &w, A, B, r, 2.0f, dX, dA, dB, ws, 16, NULL));
  REACH(qlora_linear_bwd(dY, X, M, &w, A, B, r, 2.0f, dX, dA, dB, ws, lws, NULL));

  /* forward that keeps the adapter activations, backward that takes them */
  {
    void *Hs = data + 393216;
    REJ(qlora_linear_fwd_save(X, M, &w, A, B, r, 2.0f, Y, NULL, ws, lws, NULL));
    REJ(qlora_linear_fwd_save(X, M, &w, A, B, r, 2.0f, Y, (char *)Hs + 2, ws, lws, NULL));
    REJ(qlora_linear_fwd_save(X, M, &w, NULL, NULL, 0, 0.0f, Y, Hs, ws, lws, NULL));
    REJ(qlora_linear_fwd_save(X, M, &w, A, B, r, 2.0f, Y, Hs, ws, lws - 1, NULL));
    REACH(qlora_linear_fwd_save(X, M, &w, A, B, r, 2.0f, Y, Hs, ws, lws, NULL));
    REJ(qlora_linear_bwd_saved(dY, X, NULL, M, &w, A, B, r, 2.0f, dX, dA, dB, ws, lws, NULL));
    REJ(qlora_linear_bwd_saved(dY, X, Hs, M, &w, NULL, NULL, 0, 2.0f, dX, NULL, NULL, ws, lws, NULL));
    REJ(qlora_linear_bwd_saved(dY, X, Hs, M, &w, A, B, r, 2.0f, dX, NULL, dB, ws, lws, NULL));
    REJ(qlora_linear_bwd_saved(dY, X, Hs, M, &w, A, B, r, 2.0f, dX, dA, dB, ws, 16, NULL));
    REACH(qlora_linear_bwd_saved(dY, X, Hs, M, &w, A, B, r, 2.0f, dX, dA, dB, ws, lws, NULL));
  }

  /* allocation-free forward: the scratch limit, then a call that fits */
  {
    qlora_nf4_weight small = weight(64, 64, QLORA_FMT_NF4_DQ, pool);
    REJ(qlora_linear_fwd_noalloc(X, (int64_t)1 << 23, &small, A, B, r, 2.0f, Y, NULL));
    REJ(qlora_linear_fwd_noalloc(X, M, &w, A, B, r, 2.0f, NULL, NULL));
    REACH(qlora_linear_fwd_noalloc(X, M, &w, A, B, r, 2.0f, Y, NULL));
  }

  /* merge */
  {
    qlora_nf4_weight out = weight(N, K, QLORA_FMT_NF4_DQ, pool + 32768);
    const size_t mws = qlora_nf4_merge_workspace_bytes(N, K, r);
    REJ(qlora_nf4_merge(NULL, A, B, r, 1.0f, &out, ws, mws, NULL));
    REJ(qlora_nf4_merge(&w, A, B, r, 1.0f, NULL, ws, mws, NULL));
    REJ(qlora_nf4_merge(&w, NULL, B, r, 1.0f, &out, ws, mws, NULL));
    REJ(qlora_nf4_merge(&w, A, B, r, 1.0f, &out, ws, mws - 1, NULL));
    qlora_nf4_weight other = weight(N, K + 64, QLORA_FMT_NF4_DQ, pool + 32768);
    REJ(qlora_nf4_merge(&w, A, B, r, 1.0f, &other, ws, mws, NULL));
    REACH(qlora_nf4_merge(&w, A, B, r, 1.0f, &out, ws, mws, NULL));
  }

  /* AdamW */
  {
    float *p = (float *)data, *g = p + 4096, *m = p + 8192, *v = p + 12288;
    qlora_adamw_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 1};
    qlora_adamw_hparams bad;
    REJ(qlora_adamw_step(p, g, m, v, 1024, NULL, 0, NULL, 0, NULL));
    REJ(qlora_adamw_step(NULL, g, m, v, 1024, &hp, 0, NULL, 0, NULL));
    REJ(qlora_adamw_step(p, g, m, v, 0, &hp, 0, NULL, 0, NULL));
    REJ(qlora_adamw_step(p + 1, g, m, v, 1024, &hp, 0, NULL, 0, NULL));
    bad = hp;
    bad.step = 0;
    REJ(qlora_adamw_step(p, g, m, v, 1024, &bad, 0, NULL, 0, NULL));
    bad = hp;
    bad.beta1 = 1.0f;
    REJ(qlora_adamw_step(p, g, m, v, 1024, &bad, 0, NULL, 0, NULL));
    bad = hp;
    bad.eps = -1.0f;
    REJ(qlora_adamw_step(p, g, m, v, 1024, &bad, 0, NULL, 0, NULL));
    REJ(qlora_adamw_step(p, g, m, v, 1024, &hp, 1, NULL, 0, NULL));
    REACH(qlora_adamw_step(p, g, m, v, 1024, &hp, 0, NULL, 0, NULL));
    REACH(qlora_adamw_step(p, g, m, v, 1024, &hp, 1, ws, qlora_adamw_workspace_bytes(1024, 1), NULL));
  }

  /* profiling switches */
  {
    double ms;
    int64_t launches;
    expect("profile enable", qlora_profile_enable(1), QLORA_OK);
    REJ(qlora_profile_read(99, &ms, &launches));
    expect("profile reset", qlora_profile_reset(), QLORA_OK);
    expect("profile disable", qlora_profile_enable(0), QLORA_OK);
  }

  free(pool);
  free(ws);
  free(data);
  free(A);
  free(B);
  if (failures) {
    printf("reject: %d failure(s)\n", failures);
    return 1;
  }
  printf("reject: ok (%d launches reached)\n", qlora_stub_launches);
  return 0;
}
