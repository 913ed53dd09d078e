// C ABI of the QLoRA NF4 library: argument checks, workspace sizing and
// dispatch to the HIP kernels. Every check runs on the host before anything
// is launched; a failed check launches nothing.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/qlora_nf4.h"
#include "adamw.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return QLORA_OK;
}

int hip_status(hipError_t e, const char *where) {
  if (e == hipSuccess) return ok();
  return fail(QLORA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxElems = int64_t(1) << 40;
// The large-tile GEMMs address a 256-row operand tile with 32-bit byte
// offsets from its first row: 255 rows of a row-major bf16 operand with
// row length K (forward) or N (input gradient) must stay below 2^32 bytes.
constexpr int64_t kMaxLinearDim = int64_t(1) << 23;

bool valid_format(int format) { return format >= 0 && format < qnf4::kFormats; }

int check_weight(const qlora_nf4_weight *w, const char *fn) {
  if (!w) return fail(QLORA_ERR_NULL, "%s: weight struct is NULL", fn);
  if (w->rows <= 0 || w->cols <= 0 || w->rows > kMaxElems / w->cols)
    return fail(QLORA_ERR_SHAPE, "%s: invalid weight shape %lld x %lld", fn,
                static_cast<long long>(w->rows), static_cast<long long>(w->cols));
  if (!valid_format(w->format))
    return fail(QLORA_ERR_FORMAT, "%s: format %d is not a qlora_format", fn, static_cast<int>(w->format));
  if (qnf4::fmt_dq(w->format)) {
    if (!w->codes || !w->absmax_q || !w->dq_scale || !w->dq_mean)
      return fail(QLORA_ERR_NULL, "%s: a weight buffer is NULL", fn);
    if (!aligned16(w->codes) || !aligned16(w->absmax_q) || !aligned16(w->dq_scale) ||
        !aligned16(w->dq_mean))
      return fail(QLORA_ERR_ALIGN, "%s: weight buffers must be 16-byte aligned", fn);
  } else {
    if (!w->codes || !w->absmax) return fail(QLORA_ERR_NULL, "%s: a weight buffer is NULL", fn);
    if (!aligned16(w->codes) || !aligned16(w->absmax))
      return fail(QLORA_ERR_ALIGN, "%s: weight buffers must be 16-byte aligned", fn);
  }
  return QLORA_OK;
}

int check_linear_common(const char *fn, int64_t M, const qlora_nf4_weight *W, const float *A,
                        const float *B, int32_t r) {
  int st = check_weight(W, fn);
  if (st != QLORA_OK) return st;
  if (M <= 0 || M > kMaxElems / W->cols || M > kMaxElems / W->rows)
    return fail(QLORA_ERR_SHAPE, "%s: invalid M = %lld", fn, static_cast<long long>(M));
  if (W->cols % QLORA_NF4_BLOCK != 0 || W->rows % QLORA_NF4_BLOCK != 0)
    return fail(QLORA_ERR_SHAPE,
                "%s: N (%lld) and K (%lld) must be multiples of 64", fn,
                static_cast<long long>(W->rows), static_cast<long long>(W->cols));
  if (W->cols > kMaxLinearDim || W->rows > kMaxLinearDim)
    return fail(QLORA_ERR_SHAPE, "%s: N (%lld) and K (%lld) must not exceed %lld", fn,
                static_cast<long long>(W->rows), static_cast<long long>(W->cols),
                static_cast<long long>(kMaxLinearDim));
  if (r < 0 || r > 256) return fail(QLORA_ERR_SHAPE, "%s: r = %d out of [0, 256]", fn, r);
  if (r > 0 && (!A || !B)) return fail(QLORA_ERR_NULL, "%s: r > 0 needs A and B", fn);
  if (r == 0 && (A || B)) return fail(QLORA_ERR_SHAPE, "%s: r = 0 needs A = B = NULL", fn);
  if ((A && !aligned16(A)) || (B && !aligned16(B)))
    return fail(QLORA_ERR_ALIGN, "%s: A and B must be 16-byte aligned", fn);
  return QLORA_OK;
}

qnf4::LinearArgs make_args(int64_t M, const qlora_nf4_weight *W, int32_t r, float scale) {
  qnf4::LinearArgs a;
  a.M = M;
  a.N = W->rows;
  a.K = W->cols;
  a.r = r;
  a.scale = scale;
  a.format = W->format;
  a.codes = W->codes;
  a.absmax_q = W->absmax_q;
  a.dq_scale = W->dq_scale;
  a.dq_mean = W->dq_mean;
  a.absmax = W->absmax;
  return a;
}

// The checks and the call of both backward entry points (Hs = NULL: the
// backward forms the adapter activations itself).
int linear_bwd_checked(const char *fn, const void *dY, const void *X, const void *Hs, int64_t M,
                       const qlora_nf4_weight *W, const float *A, const float *B, int32_t r, float scale,
                       void *dX, float *dA, float *dB, void *ws, size_t ws_bytes, void *stream) {
  if (!dY || !X || !dX) return fail(QLORA_ERR_NULL, "%s: dY, X and dX must not be NULL", fn);
  int st = check_linear_common(fn, M, W, A, B, r);
  if (st != QLORA_OK) return st;
  if (r > 0 && (!dA || !dB)) return fail(QLORA_ERR_NULL, "%s: r > 0 needs dA and dB", fn);
  if (r == 0 && (dA || dB)) return fail(QLORA_ERR_SHAPE, "%s: r = 0 needs dA = dB = NULL", fn);
  if (!aligned16(dY) || !aligned16(X) || !aligned16(dX) || (dA && !aligned16(dA)) ||
      (dB && !aligned16(dB)))
    return fail(QLORA_ERR_ALIGN, "%s: tensors must be 16-byte aligned", fn);
  const size_t need = qnf4::linear_ws_bytes(M, W->rows, W->cols, r);
  if (!ws || ws_bytes < need)
    return fail(QLORA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need,
                ws ? ws_bytes : size_t(0));
  if (!aligned16(ws)) return fail(QLORA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  hipError_t e = qnf4::linear_bwd(make_args(M, W, r, scale), dY, X, A, B, dX, dA, dB, ws,
                                  static_cast<hipStream_t>(stream), Hs);
  return hip_status(e, fn);
}

}  // namespace

extern "C" {

size_t qlora_nf4_storage_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || rows > kMaxElems / cols) return 0;
  const int64_t n = rows * cols;
  const int64_t nb = qnf4::ceil_div(n, QLORA_NF4_BLOCK);
  const int64_t nd = qnf4::ceil_div(nb, QLORA_DQ_BLOCK);
  return static_cast<size_t>((n + 1) / 2 + nb + 4 * nd + 4);
}

int qlora_nf4_codebook(float *out) {
  if (!out) return fail(QLORA_ERR_NULL, "qlora_nf4_codebook: out is NULL");
  const qnf4::Nf4Tables &t = qnf4::nf4_tables();
  std::memcpy(out, t.lv, sizeof(t.lv));
  return ok();
}

size_t qlora_weight_storage_bytes(int64_t rows, int64_t cols, int format) {
  if (!valid_format(format)) return 0;
  if (qnf4::fmt_dq(format)) return qlora_nf4_storage_bytes(rows, cols);
  if (rows <= 0 || cols <= 0 || rows > kMaxElems / cols) return 0;
  const int64_t n = rows * cols;
  return static_cast<size_t>((n + 1) / 2 + 4 * qnf4::ceil_div(n, QLORA_NF4_BLOCK));
}

int qlora_format_levels(int format, float *out) {
  if (!out) return fail(QLORA_ERR_NULL, "qlora_format_levels: out is NULL");
  if (!valid_format(format))
    return fail(QLORA_ERR_FORMAT, "qlora_format_levels: format %d is not a qlora_format", format);
  const qnf4::Nf4Tables &t = qnf4::format_tables(format);
  std::memcpy(out, t.lv, sizeof(t.lv));
  return ok();
}

size_t qlora_nf4_quantize_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || rows > kMaxElems / cols) return 0;
  return qnf4::quantize_ws_bytes(rows * cols);
}

int qlora_nf4_quantize(const void *W, int w_dtype, int64_t rows, int64_t cols,
                       const qlora_nf4_weight *out, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "qlora_nf4_quantize";
  if (!W) return fail(QLORA_ERR_NULL, "%s: W is NULL", fn);
  if (w_dtype != QLORA_F32 && w_dtype != QLORA_BF16)
    return fail(QLORA_ERR_DTYPE, "%s: w_dtype %d is not QLORA_F32 or QLORA_BF16", fn, w_dtype);
  int st = check_weight(out, fn);
  if (st != QLORA_OK) return st;
  if (out->rows != rows || out->cols != cols)
    return fail(QLORA_ERR_SHAPE, "%s: out is %lld x %lld but W is %lld x %lld", fn,
                static_cast<long long>(out->rows), static_cast<long long>(out->cols),
                static_cast<long long>(rows), static_cast<long long>(cols));
  if (!aligned16(W)) return fail(QLORA_ERR_ALIGN, "%s: W must be 16-byte aligned", fn);
  const bool dq = qnf4::fmt_dq(out->format);
  if (dq) {   // without DQ no workspace is used
    const size_t need = qnf4::quantize_ws_bytes(rows * cols);
    if (!ws || ws_bytes < need)
      return fail(QLORA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need,
                  ws ? ws_bytes : size_t(0));
    if (!aligned16(ws)) return fail(QLORA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  }
  hipError_t e = qnf4::launch_quantize(W, w_dtype == QLORA_BF16, rows * cols, out->format, out->codes,
                                       out->absmax_q, out->dq_scale, out->dq_mean, out->absmax,
                                       dq ? ws : nullptr, static_cast<hipStream_t>(stream));
  return hip_status(e, fn);
}

int qlora_nf4_dequantize(const qlora_nf4_weight *q, void *out, int out_dtype, void *stream) {
  const char *fn = "qlora_nf4_dequantize";
  int st = check_weight(q, fn);
  if (st != QLORA_OK) return st;
  if (!out) return fail(QLORA_ERR_NULL, "%s: out is NULL", fn);
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16)
    return fail(QLORA_ERR_DTYPE, "%s: out_dtype %d is not QLORA_F32 or QLORA_BF16", fn, out_dtype);
  if (!aligned16(out)) return fail(QLORA_ERR_ALIGN, "%s: out must be 16-byte aligned", fn);
  hipError_t e = qnf4::launch_dequantize(q->codes, q->format, q->absmax_q, q->dq_scale, q->dq_mean,
                                         q->absmax, q->rows * q->cols, out, out_dtype == QLORA_BF16,
                                         static_cast<hipStream_t>(stream));
  return hip_status(e, fn);
}

size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (M <= 0 || N <= 0 || K <= 0 || r < 0 || r > 256) return 0;
  if (N % QLORA_NF4_BLOCK || K % QLORA_NF4_BLOCK) return 0;
  if (N > kMaxLinearDim || K > kMaxLinearDim) return 0;
  if (N > kMaxElems / K || M > kMaxElems / K || M > kMaxElems / N) return 0;
  return qnf4::linear_ws_bytes(M, N, K, r);
}

int qlora_linear_fwd(const void *X, int64_t M, const qlora_nf4_weight *W, const float *A,
                     const float *B, int32_t r, float scale, void *Y, void *ws, size_t ws_bytes,
                     void *stream) {
  const char *fn = "qlora_linear_fwd";
  if (!X || !Y) return fail(QLORA_ERR_NULL, "%s: X and Y must not be NULL", fn);
  int st = check_linear_common(fn, M, W, A, B, r);
  if (st != QLORA_OK) return st;
  if (!aligned16(X) || !aligned16(Y))
    return fail(QLORA_ERR_ALIGN, "%s: X and Y must be 16-byte aligned", fn);
  const size_t need = qnf4::linear_ws_bytes(M, W->rows, W->cols, r);
  if (!ws || ws_bytes < need)
    return fail(QLORA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need,
                ws ? ws_bytes : size_t(0));
  if (!aligned16(ws)) return fail(QLORA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  hipError_t e = qnf4::linear_fwd(make_args(M, W, r, scale), X, A, B, Y, ws,
                                  static_cast<hipStream_t>(stream));
  return hip_status(e, fn);
}

int qlora_linear_fwd_save(const void *X, int64_t M, const qlora_nf4_weight *W, const float *A,
                          const float *B, int32_t r, float scale, void *Y, void *Hs, void *ws,
                          size_t ws_bytes, void *stream) {
  const char *fn = "qlora_linear_fwd_save";
  if (!X || !Y) return fail(QLORA_ERR_NULL, "%s: X and Y must not be NULL", fn);
  int st = check_linear_common(fn, M, W, A, B, r);
  if (st != QLORA_OK) return st;
  if (r == 0) return fail(QLORA_ERR_SHAPE, "%s: r = 0 has no adapter activations to keep", fn);
  if (!Hs) return fail(QLORA_ERR_NULL, "%s: Hs must not be NULL", fn);
  if (!aligned16(X) || !aligned16(Y) || !aligned16(Hs))
    return fail(QLORA_ERR_ALIGN, "%s: X, Y and Hs must be 16-byte aligned", fn);
  const size_t need = qnf4::linear_ws_bytes(M, W->rows, W->cols, r);
  if (!ws || ws_bytes < need)
    return fail(QLORA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need,
                ws ? ws_bytes : size_t(0));
  if (!aligned16(ws)) return fail(QLORA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  hipError_t e = qnf4::linear_fwd(make_args(M, W, r, scale), X, A, B, Y, ws,
                                  static_cast<hipStream_t>(stream), true, Hs);
  return hip_status(e, fn);
}

int qlora_linear_bwd_saved(const void *dY, const void *X, const void *Hs, int64_t M,
                           const qlora_nf4_weight *W, const float *A, const float *B, int32_t r,
                           float scale, void *dX, float *dA, float *dB, void *ws, size_t ws_bytes,
                           void *stream) {
  const char *fn = "qlora_linear_bwd_saved";
  if (!Hs) return fail(QLORA_ERR_NULL, "%s: Hs must not be NULL", fn);
  if (!aligned16(Hs)) return fail(QLORA_ERR_ALIGN, "%s: Hs must be 16-byte aligned", fn);
  if (r == 0) return fail(QLORA_ERR_SHAPE, "%s: r = 0 has no adapter activations", fn);
  return linear_bwd_checked(fn, dY, X, Hs, M, W, A, B, r, scale, dX, dA, dB, ws, ws_bytes, stream);
}

int qlora_linear_bwd(const void *dY, const void *X, int64_t M, const qlora_nf4_weight *W,
                     const float *A, const float *B, int32_t r, float scale, void *dX, float *dA,
                     float *dB, void *ws, size_t ws_bytes, void *stream) {
  return linear_bwd_checked("qlora_linear_bwd", dY, X, nullptr, M, W, A, B, r, scale, dX, dA, dB, ws,
                            ws_bytes, stream);
}

int qlora_linear_fwd_noalloc(const void *X, int64_t M, const qlora_nf4_weight *W, const float *A,
                             const float *B, int32_t r, float scale, void *Y, void *stream) {
  const char *fn = "qlora_linear_fwd_noalloc";
  if (!X || !Y) return fail(QLORA_ERR_NULL, "%s: X and Y must not be NULL", fn);
  int st = check_linear_common(fn, M, W, A, B, r);
  if (st != QLORA_OK) return st;
  if (!aligned16(X) || !aligned16(Y))
    return fail(QLORA_ERR_ALIGN, "%s: X and Y must be 16-byte aligned", fn);
  // split partials of the large-tile forward only where they fit the scratch
  size_t need = qnf4::linear_fwd_ws_bytes(M, W->rows, W->cols, r, true);
  const bool split = need <= qnf4::kNoAllocScratchBytes;
  if (!split) need = qnf4::linear_fwd_ws_bytes(M, W->rows, W->cols, r, false);
  if (need > qnf4::kNoAllocScratchBytes)
    return fail(QLORA_ERR_WORKSPACE, "%s: these sizes need %zu bytes of scratch, more than the %zu the library holds",
                fn, need, qnf4::kNoAllocScratchBytes);
  void *scratch = nullptr;
  hipError_t e = qnf4::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, fn);
  e = qnf4::linear_fwd(make_args(M, W, r, scale), X, A, B, Y, scratch, static_cast<hipStream_t>(stream), split);
  return hip_status(e, fn);
}

size_t qlora_nf4_merge_workspace_bytes(int64_t rows, int64_t cols, int32_t r) {
  if (rows <= 0 || cols <= 0 || rows > kMaxElems / cols || r < 0 || r > 256) return 0;
  return qnf4::merge_ws_bytes(rows, cols, r);
}

int qlora_nf4_merge(const qlora_nf4_weight *W, const float *A, const float *B, int32_t r, float scale,
                    const qlora_nf4_weight *out, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "qlora_nf4_merge";
  int st = check_weight(W, fn);
  if (st != QLORA_OK) return st;
  st = check_weight(out, fn);
  if (st != QLORA_OK) return st;
  if (out->rows != W->rows || out->cols != W->cols)
    return fail(QLORA_ERR_SHAPE, "%s: out is %lld x %lld but W is %lld x %lld", fn,
                static_cast<long long>(out->rows), static_cast<long long>(out->cols),
                static_cast<long long>(W->rows), static_cast<long long>(W->cols));
  if (r < 0 || r > 256) return fail(QLORA_ERR_SHAPE, "%s: r = %d out of [0, 256]", fn, r);
  if (r > 0 && (!A || !B)) return fail(QLORA_ERR_NULL, "%s: r > 0 needs A and B", fn);
  if (r == 0 && (A || B)) return fail(QLORA_ERR_SHAPE, "%s: r = 0 needs A = B = NULL", fn);
  if ((A && !aligned16(A)) || (B && !aligned16(B)))
    return fail(QLORA_ERR_ALIGN, "%s: A and B must be 16-byte aligned", fn);
  const size_t need = qnf4::merge_ws_bytes(W->rows, W->cols, r);
  if (!ws || ws_bytes < need)
    return fail(QLORA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need,
                ws ? ws_bytes : size_t(0));
  if (!aligned16(ws)) return fail(QLORA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  hipError_t e = qnf4::launch_merge(make_args(0, W, r, scale), A, B, out->format, out->codes, out->absmax_q,
                                    out->dq_scale, out->dq_mean, out->absmax, ws,
                                    static_cast<hipStream_t>(stream));
  return hip_status(e, fn);
}

size_t qlora_adamw_workspace_bytes(int64_t n, int state_on_host) {
  if (n <= 0 || n > kMaxElems) return 0;
  return qnf4::adamw_ws_bytes(n, state_on_host != 0);
}

int qlora_adamw_step(float *param, const float *grad, float *m, float *v, int64_t n,
                     const qlora_adamw_hparams *hp, int state_on_host, void *ws, size_t ws_bytes,
                     void *stream) {
  const char *fn = "qlora_adamw_step";
  if (!param || !grad || !m || !v || !hp) return fail(QLORA_ERR_NULL, "%s: a pointer is NULL", fn);
  if (n <= 0 || n > kMaxElems) return fail(QLORA_ERR_SHAPE, "%s: invalid n = %lld", fn, static_cast<long long>(n));
  if (!aligned16(param) || !aligned16(grad) || !aligned16(m) || !aligned16(v))
    return fail(QLORA_ERR_ALIGN, "%s: param, grad, m and v must be 16-byte aligned", fn);
  if (hp->step < 1) return fail(QLORA_ERR_SHAPE, "%s: step must be >= 1", fn);
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) || !(hp->eps >= 0.0f))
    return fail(QLORA_ERR_SHAPE, "%s: need 0 <= beta < 1 and eps >= 0", fn);
  const size_t need = qnf4::adamw_ws_bytes(n, state_on_host != 0);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QLORA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, ws ? ws_bytes : size_t(0));
  if (need > 0 && !aligned16(ws)) return fail(QLORA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  const qnf4::AdamwHparams h{hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay, hp->step};
  hipError_t e = qnf4::launch_adamw(param, grad, m, v, n, h, state_on_host != 0, ws, static_cast<hipStream_t>(stream));
  return hip_status(e, fn);
}

int qlora_profile_enable(int on) {
  qnf4::prof_set(on != 0);
  return ok();
}

int qlora_profile_read(int kind, double *total_ms, int64_t *launches) {
  if (!total_ms || !launches) return fail(QLORA_ERR_NULL, "qlora_profile_read: NULL output");
  if (kind < 0 || kind >= qnf4::kProfKinds)
    return fail(QLORA_ERR_SHAPE, "qlora_profile_read: unknown kind %d", kind);
  return hip_status(qnf4::prof_read(kind, total_ms, launches), "qlora_profile_read");
}

int qlora_profile_reset(void) {
  qnf4::prof_reset();
  return ok();
}

const char *qlora_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
