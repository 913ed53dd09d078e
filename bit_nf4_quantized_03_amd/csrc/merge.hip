// Merging a LoRA adapter into the quantized base, then quantizing the result
// again (QLoRA vs ChatGPT page, capability on adapter composition: adapters
// trained on the quantized base are merged into its weights for a standalone
// model, and the merge handles full-precision adapters meeting a 4-bit base):
//
//   W'[n][k] = fp32( fp64(w-hat[n][k]) + fp64(s * sum_j B[n][j] A[j][k]) )
//
// The rank sum runs in fp64 with j ascending. A product of two fp32 values is
// exact in fp64, so fma(b, a, acc) rounds exactly like acc + b * a. Then one
// fp64 multiply by s, one fp64 add of w-hat and one rounding to fp32. The
// merged fp32 weight goes through the quantizer (any output format).
//
//   k_b_to_f64   B [N][r] fp32 -> Bt [r][Np] fp64, transposed and zero padded
//                to Np = N rounded up to kMgRows, so that a workgroup's B
//                values for one j are one aligned run (wide scalar loads)
//   k_merge      one column k per thread, kMgRows rows per workgroup; per j
//                one A[j][k] load and kMgRows fp64 FMAs whose B operand is
//                uniform over the workgroup (scalar loads); then w-hat from
//                the codes and the block constant, and the fp32 store.
#include "internal.h"

namespace qnf4 {
namespace {

constexpr int kMgThreads = 256;   // columns per workgroup, one per thread
constexpr int kMgRows = 32;       // rows per workgroup (fp64 accumulators per thread)

typedef double d8 __attribute__((ext_vector_type(8)));

int64_t padded_rows(int64_t N) { return ceil_div(N, kMgRows) * kMgRows; }

__global__ __launch_bounds__(256) void k_b_to_f64(const float *__restrict__ B, double *__restrict__ Bt,
                                                  int64_t N, int64_t Np, int r) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // index into Bt
  if (e >= Np * r) return;
  const int64_t j = e / Np, n = e - j * Np;
  Bt[e] = n < N ? static_cast<double>(B[n * r + j]) : 0.0;
}

struct MergeParams {
  const uint8_t *codes;
  const int8_t *absmax_q;   // with DQ
  const float *dq_scale;
  const float *dq_mean;
  const float *absmax;      // without DQ
  const float *A;           // [r][K]
  const double *Bt;         // [r][Np]
  float *out;               // [N][K]
  int64_t N, K, Np;
  int r;
  float scale;
  Nf4Tables tab;
};

template <bool kDq>
__global__ __launch_bounds__(kMgThreads) void k_merge(MergeParams p) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = p.tab.lv[threadIdx.x];
  const int64_t k_raw = static_cast<int64_t>(blockIdx.x) * kMgThreads + threadIdx.x;
  const bool k_ok = k_raw < p.K;
  const int64_t k = k_ok ? k_raw : p.K - 1;   // clamped: loads stay in bounds, no store
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kMgRows;

  double acc[kMgRows];
#pragma unroll
  for (int i = 0; i < kMgRows; ++i) acc[i] = 0.0;
  const float *ap = p.A + k;
  // Four rank steps per batch, with no branch inside, so that the four A
  // loads go out together. A step past r reads row r - 1 and multiplies by
  // a = 0, which leaves acc exactly unchanged (acc is never -0).
  for (int j0 = 0; j0 < p.r; j0 += 4) {
    float a4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a4[u] = ap[static_cast<int64_t>(min(j0 + u, p.r - 1)) * p.K];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = min(j0 + u, p.r - 1);
      const double a = j0 + u < p.r ? static_cast<double>(a4[u]) : 0.0;
      // the workgroup's 32 B values of this step: uniform, 256-byte aligned
      const d8 *bt = reinterpret_cast<const d8 *>(p.Bt + static_cast<int64_t>(j) * p.Np + n0);
      d8 bv[kMgRows / 8];
#pragma unroll
      for (int q = 0; q < kMgRows / 8; ++q) bv[q] = bt[q];
#pragma unroll
      for (int i = 0; i < kMgRows; ++i) acc[i] = __fma_rn(bv[i / 8][i % 8], a, acc[i]);
    }
  }

  const double s = static_cast<double>(p.scale);
  const float mu = kDq ? p.dq_mean[0] : 0.0f;
  __syncthreads();   // lv ready
  // w-hat and the store, eight rows at a time: every load of the eight rows
  // (code byte, block constant) is issued before the first is used; rows
  // past N are clamped for the loads and not stored.
  constexpr int kChunk = 8;
#pragma unroll
  for (int i0 = 0; i0 < kMgRows; i0 += kChunk) {
    int64_t e[kChunk];
    uint32_t byte[kChunk];
    float cv[kChunk];
    float ds[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int64_t n = min(n0 + i0 + u, p.N - 1);
      e[u] = n * p.K + k;
      const int64_t blk = e[u] / kBlock;
      byte[u] = p.codes[e[u] >> 1];
      if constexpr (kDq) {
        cv[u] = static_cast<float>(p.absmax_q[blk]);
        ds[u] = p.dq_scale[blk / kDqBlock];
      } else {
        cv[u] = p.absmax[blk];
        ds[u] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const uint32_t code = (e[u] & 1) ? (byte[u] & 0xFu) : (byte[u] >> 4);
      float c = cv[u];
      if constexpr (kDq) c = __fadd_rn(__fmul_rn(cv[u], __fdiv_rn(ds[u], 127.0f)), mu);
      const float w = __fmul_rn(lv[code], c);
      const double v = __dadd_rn(static_cast<double>(w), __dmul_rn(s, acc[i0 + u]));
      if (n0 + i0 + u < p.N && k_ok) p.out[e[u]] = static_cast<float>(v);   // round to nearest even
    }
  }
}

}  // namespace

size_t merge_ws_bytes(int64_t N, int64_t K, int r) {
  return align_up(static_cast<size_t>(N * K) * sizeof(float), 256) +
         align_up(static_cast<size_t>(padded_rows(N)) * r * sizeof(double), 256) + quantize_ws_bytes(N * K);
}

hipError_t launch_merge(const LinearArgs &w, const float *A, const float *B, int out_format, uint8_t *codes,
                        int8_t *absmax_q, float *dq_scale, float *dq_mean, float *absmax, void *ws,
                        hipStream_t s) {
  const int64_t N = w.N, K = w.K;
  char *base = static_cast<char *>(ws);
  float *merged = reinterpret_cast<float *>(base);
  double *Bt = reinterpret_cast<double *>(base + align_up(static_cast<size_t>(N * K) * sizeof(float), 256));
  const int64_t Np = padded_rows(N);
  void *qws = base + align_up(static_cast<size_t>(N * K) * sizeof(float), 256) +
              align_up(static_cast<size_t>(Np) * w.r * sizeof(double), 256);
  if (w.r > 0)
    hipLaunchKernelGGL(k_b_to_f64, dim3(static_cast<unsigned>(ceil_div(Np * w.r, 256))), dim3(256), 0, s, B, Bt, N,
                       Np, w.r);
  MergeParams p{};
  p.codes = w.codes;
  p.absmax_q = w.absmax_q;
  p.dq_scale = w.dq_scale;
  p.dq_mean = w.dq_mean;
  p.absmax = w.absmax;
  p.A = A;
  p.Bt = Bt;
  p.out = merged;
  p.N = N;
  p.K = K;
  p.Np = Np;
  p.r = w.r;
  p.scale = w.scale;
  p.tab = format_tables(w.format);
  const dim3 grid(static_cast<unsigned>(ceil_div(K, kMgThreads)), static_cast<unsigned>(ceil_div(N, kMgRows)));
  if (fmt_dq(w.format)) hipLaunchKernelGGL(k_merge<true>, grid, dim3(kMgThreads), 0, s, p);
  else hipLaunchKernelGGL(k_merge<false>, grid, dim3(kMgThreads), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_quantize(merged, false, N * K, out_format, codes, absmax_q, dq_scale, dq_mean, absmax,
                         fmt_dq(out_format) ? qws : nullptr, s);
}

}  // namespace qnf4
