// NF4 + double quantization and dequantization kernels (gfx950).
//
// Block-wise absmax NF4 quantization (QLoRA vs ChatGPT page, capability "NF4
// 4-bit quantization") followed by 8-bit double quantization of the absmax
// constants with their own scales (same page, capability "double
// quantization"), and the block-wise dequantization the training pipeline
// runs on the fly (same page, capability "training pipeline").
//
// Every floating-point step that decides a stored bit is an explicit
// round-to-nearest operation (__fdiv_rn, __fmul_rn, __fadd_rn, __fsub_rn) and
// this file is compiled with -ffp-contract=off, so the results are the exact
// fp32 values of the definition in qlora_nf4.h.
//
// Kernels
//   k_absmax_codes  one workgroup per DQ block (256 absmax blocks = 16384
//                   elements): coalesced 16-byte loads, per-64 absmax by lane
//                   shuffles, nearest-level codes, packed stores, fp32 absmax
//                   to the workspace and the fp64 tree sum of the DQ block's
//                   256 constants.
//   k_tree256       sums aligned 256-entry groups of fp64 partials in the same
//                   tree shape (repeated until one value is left).
//   k_dq_codes      one workgroup per DQ block: mean, per-block scale, int8 codes.
//   k_dequant       one workgroup per DQ block: per-block scales in LDS, then
//                   4-byte code loads expanded to fp32 or bf16 stores.
//   k_block_scales  the per-block reconstruction scale c_b for the GEMMs.
#include "internal.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kElemsPerDq = kBlock * kDqBlock;  // 16384
constexpr int kCells = 258;                      // z-cells -129 .. 128

// Exact code from an fp32 y already equal to fp32(x / a): number of
// thresholds strictly below y.
__device__ __forceinline__ int code_from_y(float y, const Nf4Tables &t) {
  int c = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) c += (y > t.thr[i]) ? 1 : 0;
  return c;
}

// The fast code search works on z = fp32(x * fp32(128 / a)), which is within
// 2^-15 of 128 * fp32(x / a) when 2^-100 <= a <= 2^100 (two roundings of
// relative size 2^-24 each on a value of magnitude <= 128, plus the rounding
// of the exact quotient). A lookup table over unit cells of z gives, for the
// cell floor(z), the number of thresholds certainly below any y whose z lies
// in the cell, and the one threshold (scaled by 128) that may lie within the
// cell or 2^-13 of it. When z is within 2^-14 of that threshold the element
// is recomputed with a correctly rounded division instead.
__device__ void build_lut(float2 *lut, const Nf4Tables &t) {
  for (int c = threadIdx.x; c < kCells; c += blockDim.x) {
    const float lo = static_cast<float>(c - 129);
    const float hi = lo + 1.0f;
    const float win = 0x1p-13f;
    int base = 0;
    float tc = __builtin_huge_valf();
    for (int i = 0; i < 15; ++i) {
      const float tz = t.thr[i] * 128.0f;  // exact (power-of-two scaling)
      if (tz < lo - win) ++base;
      else if (tz < hi + win) tc = tz;
    }
    lut[c] = make_float2(tc, static_cast<float>(base));
  }
}

template <bool kBf16>
struct InTraits;
template <>
struct InTraits<true> {  // bf16 weights: 8 elements per 16-byte load
  static constexpr int kEpl = 8;
  __device__ static void widen(const uint4 &v, float *x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct InTraits<false> {  // fp32 weights: 4 elements per 16-byte load
  static constexpr int kEpl = 4;
  __device__ static void widen(const uint4 &v, float *x) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
};

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void k_absmax_codes(const uint8_t *__restrict__ W, int64_t n,
                                                           uint8_t *__restrict__ codes,
                                                           float *__restrict__ absmax_ws,
                                                           double *__restrict__ partial,
                                                           int64_t nb, Nf4Tables tab) {
  using IT = InTraits<kBf16>;
  constexpr int kEpl = IT::kEpl;                    // elements per lane
  constexpr int kLpb = kBlock / kEpl;               // lanes per 64-block
  constexpr int kPasses = kElemsPerDq / (kThreads * kEpl);
  constexpr int kEsz = kBf16 ? 2 : 4;

  __shared__ float2 lut[kCells];
  __shared__ float sa[kDqBlock];
  __shared__ double wsum[kThreads / 64];

  build_lut(lut, tab);

  const int64_t d = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t e0 = d * kElemsPerDq;
  const int64_t nbytes = (n + 1) / 2;

  // Issue every load of the DQ block first (memory-level parallelism).
  uint4 raw[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t e = e0 + static_cast<int64_t>(p) * kThreads * kEpl + static_cast<int64_t>(tid) * kEpl;
    if (e + kEpl <= n) {
      raw[p] = *reinterpret_cast<const uint4 *>(W + e * kEsz);
    } else {
      uint32_t tmp[4] = {0u, 0u, 0u, 0u};
      for (int i = 0; i < kEpl; ++i) {
        if (e + i < n) {
          if (kBf16) {
            uint32_t h = reinterpret_cast<const uint16_t *>(W)[e + i];
            tmp[i / 2] |= h << (16 * (i % 2));
          } else {
            tmp[i] = reinterpret_cast<const uint32_t *>(W)[e + i];
          }
        }
      }
      raw[p] = make_uint4(tmp[0], tmp[1], tmp[2], tmp[3]);
    }
  }
  __syncthreads();  // LUT ready

#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t e = e0 + static_cast<int64_t>(p) * kThreads * kEpl + static_cast<int64_t>(tid) * kEpl;
    float x[kEpl];
    IT::widen(raw[p], x);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kEpl; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
    for (int off = 1; off < kLpb; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float a = m;

    const bool fast_scale = (a == 0.0f) || (a >= 0x1p-100f && a <= 0x1p100f);
    // Outside the fast range the lookup runs on z = 0 (always a valid cell)
    // and the exact path below recomputes every code of the lane.
    const float r128 = (a == 0.0f || !fast_scale) ? 0.0f : __fmul_rn(__fdiv_rn(1.0f, a), 128.0f);
    int c[kEpl];
    bool near = !fast_scale;
#pragma unroll
    for (int i = 0; i < kEpl; ++i) {
      const float z = __fmul_rn(x[i], r128);
      int cell = static_cast<int>(floorf(z)) + 129;
      cell = min(max(cell, 0), kCells - 1);
      const float2 en = lut[cell];
      c[i] = static_cast<int>(en.y) + ((z > en.x) ? 1 : 0);
      near |= fabsf(__fsub_rn(z, en.x)) <= 0x1p-14f;
    }
    if (near) {  // rare: exact division for this lane's elements
#pragma unroll
      for (int i = 0; i < kEpl; ++i) {
        const float y = (a == 0.0f) ? 0.0f : __fdiv_rn(x[i], a);
        c[i] = code_from_y(y, tab);
      }
    }
#pragma unroll
    for (int i = 0; i < kEpl; ++i)
      if (e + i >= n) c[i] = 0;  // padding nibble of an odd tail

    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < kEpl / 2; ++j)
      word |= static_cast<uint32_t>((c[2 * j] << 4) | c[2 * j + 1]) << (8 * j);
    const int64_t byte0 = e / 2;
    if (e + kEpl <= n) {
      if (kBf16) *reinterpret_cast<uint32_t *>(codes + byte0) = word;
      else *reinterpret_cast<uint16_t *>(codes + byte0) = static_cast<uint16_t>(word);
    } else {
      for (int j = 0; j < kEpl / 2; ++j)
        if (byte0 + j < nbytes) codes[byte0 + j] = static_cast<uint8_t>(word >> (8 * j));
    }

    const int64_t blk = e / kBlock;
    if ((tid % kLpb) == 0) {
      const int lb = static_cast<int>(blk - d * kDqBlock);
      sa[lb] = a;
      if (blk < nb) absmax_ws[blk] = a;
    }
  }
  __syncthreads();

  // fp64 tree sum of the 256 constants: xor butterflies give the adjacent-pair
  // tree inside each wave's 64 leaves, then (w0 + w1) + (w2 + w3).
  const int64_t myblk = d * kDqBlock + tid;
  double v = (myblk < nb) ? static_cast<double>(sa[tid]) : 0.0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = v + __shfl_xor(v, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = v;
  __syncthreads();
  if (tid == 0) partial[d] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

__global__ __launch_bounds__(kThreads) void k_tree256(const double *__restrict__ in, int64_t L,
                                                      double *__restrict__ out) {
  __shared__ double wsum[kThreads / 64];
  const int tid = threadIdx.x;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + tid;
  double v = (i < L) ? in[i] : 0.0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = v + __shfl_xor(v, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = v;
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

__global__ __launch_bounds__(kThreads) void k_dq_codes(const float *__restrict__ absmax_ws, int64_t nb,
                                                       const double *__restrict__ total,
                                                       int8_t *__restrict__ absmax_q,
                                                       float *__restrict__ dq_scale,
                                                       float *__restrict__ dq_mean) {
  __shared__ float wmax[kThreads / 64];
  const int tid = threadIdx.x;
  const int64_t d = blockIdx.x;
  const int64_t b = d * kDqBlock + tid;
  const float mu = static_cast<float>(total[0] / static_cast<double>(nb));
  const bool valid = b < nb;
  const float dv = valid ? __fsub_rn(absmax_ws[b], mu) : 0.0f;
  float m = fabsf(dv);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  const float s2 = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  int q = 0;
  if (s2 > 0.0f) {
    const float u = __fmul_rn(__fdiv_rn(dv, s2), 127.0f);
    q = static_cast<int>(rintf(u));
    q = min(max(q, -127), 127);
  }
  if (valid) absmax_q[b] = static_cast<int8_t>(q);
  if (tid == 0) dq_scale[d] = s2;
  if (d == 0 && tid == 0) dq_mean[0] = mu;
}

// ------------------------------------------------------------ dequantize

__device__ __forceinline__ float block_scale(int8_t q, float kd, float mu) {
  return __fadd_rn(__fmul_rn(static_cast<float>(q), kd), mu);
}

template <bool kOutBf16>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t *__restrict__ codes,
                                                      const int8_t *__restrict__ absmax_q,
                                                      const float *__restrict__ dq_scale,
                                                      const float *__restrict__ dq_mean, int64_t n,
                                                      void *__restrict__ out, Nf4Tables tab) {
  __shared__ float lv[16];
  __shared__ float cs[kDqBlock];
  const int tid = threadIdx.x;
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t nbytes = (n + 1) / 2;
  if (tid < 16) lv[tid] = tab.lv[tid];
  const float mu = dq_mean[0];

  for (int64_t d = blockIdx.x; d * kElemsPerDq < n; d += gridDim.x) {
    __syncthreads();  // previous iteration done with cs
    {
      const float kd = __fdiv_rn(dq_scale[d], 127.0f);
      const int64_t b = d * kDqBlock + tid;
      cs[tid] = (b < nb) ? block_scale(absmax_q[b], kd, mu) : 0.0f;
    }
    __syncthreads();
    const int64_t byte_base = d * (kElemsPerDq / 2);
    // 8 pieces of 4 code bytes (8 elements) per thread; piece p of thread t
    // starts at byte 4t + 1024p of the DQ block, so each wave touches a
    // contiguous 256-byte run of codes per piece.
    uint32_t w[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int64_t byte0 = byte_base + 4 * tid + 1024 * p;
      if (byte0 + 4 <= nbytes) {
        w[p] = *reinterpret_cast<const uint32_t *>(codes + byte0);
      } else {
        uint32_t t = 0;
        for (int j = 0; j < 4; ++j)
          if (byte0 + j < nbytes) t |= static_cast<uint32_t>(codes[byte0 + j]) << (8 * j);
        w[p] = t;
      }
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int64_t e = d * kElemsPerDq + 8 * tid + 2048 * p;  // first element of the piece
      if (e >= n) continue;
      const float c = cs[(8 * tid + 2048 * p) / kBlock];
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t byte = (w[p] >> (8 * j)) & 0xFFu;
        v[2 * j] = __fmul_rn(lv[byte >> 4], c);
        v[2 * j + 1] = __fmul_rn(lv[byte & 0xFu], c);
      }
      if (kOutBf16) {
        __bf16 *o = reinterpret_cast<__bf16 *>(out) + e;
        if (e + 8 <= n) {
          typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
          bf16x8 pk;
#pragma unroll
          for (int j = 0; j < 8; ++j) pk[j] = static_cast<__bf16>(v[j]);
          *reinterpret_cast<bf16x8 *>(o) = pk;
        } else {
          for (int j = 0; j < 8; ++j)
            if (e + j < n) o[j] = static_cast<__bf16>(v[j]);
        }
      } else {
        float *o = reinterpret_cast<float *>(out) + e;
        if (e + 8 <= n) {
          *reinterpret_cast<float4 *>(o) = make_float4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<float4 *>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
        } else {
          for (int j = 0; j < 8; ++j)
            if (e + j < n) o[j] = v[j];
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_block_scales(const int8_t *__restrict__ absmax_q,
                                                           const float *__restrict__ dq_scale,
                                                           const float *__restrict__ dq_mean,
                                                           int64_t nb, float *__restrict__ cs) {
  const int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (b >= nb) return;
  const float kd = __fdiv_rn(dq_scale[b / kDqBlock], 127.0f);
  cs[b] = block_scale(absmax_q[b], kd, dq_mean[0]);
}

}  // namespace

size_t quantize_ws_bytes(int64_t n) {
  const int64_t nb = ceil_div(n, kBlock);
  int64_t partials = 0;
  for (int64_t L = ceil_div(nb, kDqBlock);; L = ceil_div(L, kDqBlock)) {
    partials += L;
    if (L == 1) break;
  }
  return align_up(static_cast<size_t>(nb) * 4, 256) + static_cast<size_t>(partials) * 8;
}

hipError_t launch_quantize(const void *W, bool w_bf16, int64_t n, uint8_t *codes,
                           int8_t *absmax_q, float *dq_scale, float *dq_mean, void *ws,
                           hipStream_t s) {
  const int64_t nb = ceil_div(n, kBlock);
  const int64_t nd = ceil_div(nb, kDqBlock);
  float *absmax_ws = static_cast<float *>(ws);
  double *part = reinterpret_cast<double *>(static_cast<char *>(ws) +
                                            align_up(static_cast<size_t>(nb) * 4, 256));
  const Nf4Tables &tab = nf4_tables();
  prof_begin(kProfQuantize, s);
  if (w_bf16)
    hipLaunchKernelGGL(k_absmax_codes<true>, dim3(nd), dim3(kThreads), 0, s,
                       static_cast<const uint8_t *>(W), n, codes, absmax_ws, part, nb, tab);
  else
    hipLaunchKernelGGL(k_absmax_codes<false>, dim3(nd), dim3(kThreads), 0, s,
                       static_cast<const uint8_t *>(W), n, codes, absmax_ws, part, nb, tab);
  prof_end(kProfQuantize, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // Reduce the per-DQ-block partials 256 at a time until one value is left.
  double *cur = part;
  int64_t L = nd;
  while (L > 1) {
    const int64_t L2 = ceil_div(L, kDqBlock);
    double *next = cur + L;
    hipLaunchKernelGGL(k_tree256, dim3(L2), dim3(kThreads), 0, s, cur, L, next);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    cur = next;
    L = L2;
  }
  hipLaunchKernelGGL(k_dq_codes, dim3(nd), dim3(kThreads), 0, s, absmax_ws, nb, cur, absmax_q,
                     dq_scale, dq_mean);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *codes, const int8_t *absmax_q, const float *dq_scale,
                             const float *dq_mean, int64_t n, void *out, bool out_bf16,
                             hipStream_t s) {
  const int64_t nd = ceil_div(ceil_div(n, kBlock), kDqBlock);
  const int64_t grid = nd < 8192 ? nd : 8192;
  const Nf4Tables &tab = nf4_tables();
  prof_begin(kProfDequantize, s);
  if (out_bf16)
    hipLaunchKernelGGL(k_dequant<true>, dim3(grid), dim3(kThreads), 0, s, codes, absmax_q,
                       dq_scale, dq_mean, n, out, tab);
  else
    hipLaunchKernelGGL(k_dequant<false>, dim3(grid), dim3(kThreads), 0, s, codes, absmax_q,
                       dq_scale, dq_mean, n, out, tab);
  prof_end(kProfDequantize, s);
  return hipGetLastError();
}

hipError_t launch_block_scales(const int8_t *absmax_q, const float *dq_scale,
                               const float *dq_mean, int64_t nb, float *cs, hipStream_t s) {
  hipLaunchKernelGGL(k_block_scales, dim3(ceil_div(nb, kThreads)), dim3(kThreads), 0, s,
                     absmax_q, dq_scale, dq_mean, nb, cs);
  return hipGetLastError();
}

}  // namespace qnf4
