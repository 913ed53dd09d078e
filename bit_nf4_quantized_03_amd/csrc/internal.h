// Private declarations shared by the C-ABI layer (api.cpp) and the kernel
// translation units. Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstddef>

#include "../../include/qlora_nf4.h"

namespace qnf4 {

constexpr int kBlock = 64;     // weight elements per absmax constant
constexpr int kDqBlock = 256;  // absmax constants per double-quantization block

// The NF4 levels and the 15 decision thresholds, passed by value to kernels.
// thr[i] is the largest fp32 <= the exact midpoint (lv[i] + lv[i+1]) / 2, so
// for any fp32 y: y > thr[i]  <=>  y is nearer to lv[i+1] than to lv[i] (a tie
// goes to the lower level).
struct Nf4Tables {
  float lv[16];
  float thr[15];
};

// Derived once on the host (normal quantiles in long double, rounded once to
// fp32). Thread-safe.
const Nf4Tables &nf4_tables();

// The weight formats: bit 0 = the absmax constants are stored as fp32 (no
// double quantization), bit 1 = FP4 levels instead of NF4.
constexpr int kFmtNoDq = 1;
constexpr int kFmtFp4 = 2;
constexpr int kFormats = 4;
inline bool fmt_dq(int format) { return (format & kFmtNoDq) == 0; }
// The 4-bit float (1 sign, 2 exponent, 1 mantissa bit) divided by its largest
// magnitude: 15 distinct levels ascending, zero at index 7 and +1 repeated at
// index 15 (never chosen by the nearest-level rule); thresholds as for NF4.
const Nf4Tables &fp4_tables();
inline const Nf4Tables &format_tables(int format) {
  return (format & kFmtFp4) ? fp4_tables() : nf4_tables();
}

// ------------------------------------------------------------- profiling
enum ProfKind { kProfFwdGemm = 0, kProfBwdDx = 1, kProfQuantize = 2, kProfDequantize = 3, kProfKinds = 4 };
bool prof_enabled();
void prof_set(bool on);
void prof_begin(int kind, hipStream_t s);
void prof_end(int kind, hipStream_t s);
hipError_t prof_read(int kind, double *total_ms, int64_t *count);
void prof_reset();

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- quantize
// Workspace: fp32 absmax [nb] | one fp64 tree partial sum per DQ block [nd].
// Without DQ (absmax != null) the fp32 constants go straight to `absmax` and
// no workspace is used.
size_t quantize_ws_bytes(int64_t n);
hipError_t launch_quantize(const void *W, bool w_bf16, int64_t n, int format, uint8_t *codes,
                           int8_t *absmax_q, float *dq_scale, float *dq_mean, float *absmax,
                           void *ws, hipStream_t s);

// -------------------------------------------------------------- dequantize
// With DQ the block scales come from absmax_q, dq_scale and dq_mean, without
// it from the fp32 `absmax`.
hipError_t launch_dequantize(const uint8_t *codes, int format, const int8_t *absmax_q,
                             const float *dq_scale, const float *dq_mean, const float *absmax,
                             int64_t n, void *out, bool out_bf16, hipStream_t s);

// ------------------------------------------------------------------ linear
struct LinearArgs {
  int64_t M, N, K;
  int r;
  float scale;
  int format;
  const uint8_t *codes;
  const int8_t *absmax_q;   // with DQ
  const float *dq_scale;
  const float *dq_mean;
  const float *absmax;      // without DQ: the fp32 block constants
};

// A linear workspace starts with kLinearSyncBytes of synchronization words
// (counters and flags of the single-launch skinny-M forward). They must be zero
// before the workspace is first used; every call leaves them zero. The other
// kernels' scratch follows them.
constexpr size_t kLinearSyncBytes = QLORA_LINEAR_SYNC_BYTES;

size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K, int r);
// Workspace of the forward call alone (the backward's buffers left out).
// allow_split as for linear_fwd below.
size_t linear_fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int r, bool allow_split = true);

// The no-allocation forward's scratch: a file-scope device array of
// kNoAllocScratchBytes, its address on the current device (taken once per
// device, with that device current).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void **ptr);
// allow_split = false keeps the large-tile forward to one pass over the
// reduction (no split partials in the workspace), for a caller whose scratch
// is bounded.
// hs_out (optional): the adapter activations bf16(s X A^T) [M][r] for a later
// linear_bwd (hs_in), so that the backward does not form them again.
hipError_t linear_fwd(const LinearArgs &a, const void *X, const float *A, const float *B,
                      void *Y, void *ws, hipStream_t s, bool allow_split = true, void *hs_out = nullptr);
hipError_t linear_bwd(const LinearArgs &a, const void *dY, const void *X, const float *A,
                      const float *B, void *dX, float *dA, float *dB, void *ws,
                      hipStream_t s, const void *hs_in = nullptr);

// ------------------------------------------------------------------- merge
// W' = fp32(w-hat + s B A) (rank sum in fp64) into the workspace, then
// quantized into the output buffers in `out_format`. Workspace: merged fp32
// [N*K] | B^T in fp64 [r*N] | quantize workspace.
size_t merge_ws_bytes(int64_t N, int64_t K, int r);
hipError_t launch_merge(const LinearArgs &w, const float *A, const float *B, int out_format, uint8_t *codes,
                        int8_t *absmax_q, float *dq_scale, float *dq_mean, float *absmax, void *ws,
                        hipStream_t s);

// Skinny-M forward (M <= 32) in one launch: sync words, then the split
// partials of Y and the pieces of X A^T. gemv_sync_fits is false when the
// shape needs more sync words than the workspace header holds (then the
// large-tile path runs instead).
bool gemv_sync_fits(int64_t M, int64_t N, int64_t K, int r);
size_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K, int r);
hipError_t launch_gemv(const LinearArgs &a, const void *X, const float *A, const float *B, void *Y,
                       void *ws, hipStream_t s);

}  // namespace qnf4
