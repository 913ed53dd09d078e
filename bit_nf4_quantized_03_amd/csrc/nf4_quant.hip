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
//   k_absmax_codes  workgroups loop over DQ blocks (256 absmax blocks = 16384
//                   elements), the next block's loads in flight: coalesced
//                   16-byte loads, per-64 absmax by DPP lane exchanges, nearest-level codes, packed stores, fp32 absmax
//                   to the workspace and the fp64 tree sum of the DQ block's
//                   256 constants.
//   k_dq_codes_mean up to 1024 DQ blocks: one workgroup per DQ block, each of
//                   which completes the same fp64 tree over the per-DQ-block
//                   partials (the mean), then the block's scale and int8 codes.
//   k_tree_mean     larger tensors: one workgroup completes the tree (the mean),
//   k_dq_codes      then one wave per DQ block: scale and int8 codes.
//   k_dequant       one workgroup per DQ block: per-block scales in LDS, then
//                   4-byte code loads expanded to fp32 or bf16 stores.
#include <algorithm>
#include <cstring>

#include "internal.h"

namespace qnf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kElemsPerDq = kBlock * kDqBlock;  // 16384
constexpr int kCells = 257;                      // trunc(z) = -128 .. 128

// Exact code from an fp32 y already equal to fp32(x / a): number of
// thresholds strictly below y.
__device__ __forceinline__ int code_from_y(float y, const Nf4Tables &t) {
  int c = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) c += (y > t.thr[i]) ? 1 : 0;
  return c;
}

// The fast code search works on z = fp32(x * 128 r), r = the hardware
// reciprocal of a (within 1 ulp): |z - 128 x / a| <= 128 (2^-23 + 2^-24) and
// |128 fp32(x / a) - 128 x / a| <= 2^-17 for |x| <= a, so z is within 2^-15.5
// of 128 fp32(x / a) when 2^-100 <= a <= 2^100; and |z| < 129. A table over
// the cells of trunc(z) (cell t covers [t, t + 1) for t > 0, (t - 1, t] for
// t < 0 and (-1, 1) for t = 0) gives the number of thresholds certainly below
// any z of the cell and the one threshold tz (scaled by 128) that may lie
// within the cell or 2^-13 of it (the NF4 and FP4 thresholds are more than 10
// apart in z; the host checks that no cell window holds two). Entry: (tz or
// +inf, base count as int bits). The code is base + (z > tz); when z is within
// 2^-14 of tz the element is recomputed with a correctly rounded division
// instead. The table is built once per codebook on the host (every quantity
// in it is exact in fp32) and passed by value.
struct CodeLut {
  float2 cell[kCells];
};

struct CodeLuts {
  CodeLut lut[2];   // NF4, FP4
  bool ok;          // at most one threshold in every cell window
};

CodeLut build_code_lut(const Nf4Tables &t, bool *ok) {
  CodeLut l{};
  for (int c = 0; c < kCells; ++c) {
    const int iz = c - 128;
    const float lo = static_cast<float>(iz > 0 ? iz : iz - 1);
    const float hi = static_cast<float>(iz < 0 ? iz : iz + 1);
    const float win = 0x1p-13f;
    int base = 0, inside = 0;
    float tc = __builtin_huge_valf();
    for (int i = 0; i < 15; ++i) {
      const float tz = t.thr[i] * 128.0f;  // exact (power-of-two scaling)
      base += tz < lo - win ? 1 : 0;
      if (tz >= lo - win && tz < hi + win) {
        tc = tz;
        ++inside;
      }
    }
    if (inside > 1) *ok = false;
    float base_bits;
    std::memcpy(&base_bits, &base, sizeof(base_bits));
    l.cell[c] = make_float2(tc, base_bits);
  }
  return l;
}

const CodeLut *code_lut(int format) {
  static const CodeLuts luts = [] {
    CodeLuts l{};
    l.ok = true;
    l.lut[0] = build_code_lut(nf4_tables(), &l.ok);
    l.lut[1] = build_code_lut(fp4_tables(), &l.ok);
    return l;
  }();
  return luts.ok ? &luts.lut[(format & kFmtFp4) ? 1 : 0] : nullptr;
}

// The weight is read once and the codes are written once: streaming
// (non-temporal) loads and stores, which keep them from displacing data that
// is reused in the caches.
__device__ __forceinline__ uint4 load_stream(const uint8_t *p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
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

// Maximum of a non-negative float over aligned groups of G lanes (G = 8 or
// 16), by DPP lane exchanges on the bit patterns (for non-negative floats the
// unsigned order is the float order): quad swaps, then the half-row mirror
// (lane i with 7 - i) and, for 16, the row mirror (lane i with 15 - i).
template <int G>
__device__ __forceinline__ float block_max(float v) {
  static_assert(G == 8 || G == 16, "8 or 16 lanes per block");
  uint32_t u = __float_as_uint(v);
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0xB1, 0xF, 0xF, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x4E, 0xF, 0xF, false)));
  u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x141, 0xF, 0xF, false)));
  if (G == 16) u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x140, 0xF, 0xF, false)));
  return __uint_as_float(u);
}

// One lane's share of a pass: kEpl elements of one 64-block. Returns the
// block absmax; writes the packed codes. kGuard handles a tensor tail.
template <bool kBf16, bool kGuard>
__device__ __forceinline__ float code_lane(const uint4 &raw, int64_t e, int64_t n, uint8_t *__restrict__ codes,
                                           const float2 *lut, const Nf4Tables &tab) {
  using IT = InTraits<kBf16>;
  constexpr int kEpl = IT::kEpl;
  constexpr int kLpb = kBlock / kEpl;   // lanes per 64-block
  float x[kEpl];
  IT::widen(raw, x);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kEpl; ++i) m = fmaxf(m, fabsf(x[i]));
  const float a = block_max<kLpb>(m);

  const bool fast_scale = (a == 0.0f) || (a >= 0x1p-100f && a <= 0x1p100f);
  // Outside the fast range the lookup runs on z = 0 (always a valid cell)
  // and the exact path below recomputes every code of the lane.
  const float r128 = (a == 0.0f || !fast_scale) ? 0.0f : __fmul_rn(__builtin_amdgcn_rcpf(a), 128.0f);
  // d = tz - z, exact in sign (a difference of two floats is negative
  // exactly when the first is smaller), so z > tz is d < 0; and |d| is the
  // distance to the cell's threshold (infinite where the cell has none).
  int c[kEpl];
  float d[kEpl];
  float dmin = __builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < kEpl; ++i) {
    const float z = __fmul_rn(x[i], r128);
    const float2 en = lut[static_cast<int>(z) + 128];   // truncation: |z| < 129
    d[i] = __fsub_rn(en.x, z);
    c[i] = __float_as_int(en.y) + (d[i] < 0.0f ? 1 : 0);
    dmin = fminf(dmin, fabsf(d[i]));
  }
  // Rare: exact division, element by element, so that a wave pays only for
  // the elements some lane needs (ratios of bf16 values hit a dyadic
  // threshold such as FP4's 1/8 exactly now and then). One test on the
  // lane's nearest threshold first, so that a wave with no such element
  // skips the per-element tests.
  if (!fast_scale || dmin <= 0x1p-14f) {
#pragma unroll
    for (int i = 0; i < kEpl; ++i) {
      if (!fast_scale || fabsf(d[i]) <= 0x1p-14f) {
        const float y = (a == 0.0f) ? 0.0f : __fdiv_rn(x[i], a);
        c[i] = code_from_y(y, tab);
      }
    }
  }
  if (kGuard) {
#pragma unroll
    for (int i = 0; i < kEpl; ++i)
      if (e + i >= n) c[i] = 0;  // padding nibble of an odd tail
  }
  // two codes per byte (first in the high nibble), bytes in element order
  uint32_t byte[kEpl / 2];
#pragma unroll
  for (int j = 0; j < kEpl / 2; ++j) byte[j] = (static_cast<uint32_t>(c[2 * j]) << 4) | static_cast<uint32_t>(c[2 * j + 1]);
  uint32_t word;
  if (kEpl == 8)
    word = ((byte[3] << 8 | byte[2]) << 16) | (byte[1] << 8 | byte[0]);
  else
    word = byte[1] << 8 | byte[0];
  const int64_t byte0 = e / 2;
  if (!kGuard || e + kEpl <= n) {
    if (kBf16) __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(codes + byte0));
    else *reinterpret_cast<uint16_t *>(codes + byte0) = static_cast<uint16_t>(word);
  } else {
    const int64_t nbytes = (n + 1) / 2;
    for (int j = 0; j < kEpl / 2; ++j)
      if (byte0 + j < nbytes) codes[byte0 + j] = static_cast<uint8_t>(word >> (8 * j));
  }
  return a;
}

// Workgroups loop over DQ blocks d = blockIdx.x + i * gridDim.x (256 absmax
// blocks = 16384 elements each): absmax and codes of its 256 blocks, the fp32
// absmax to `absmax_out` (the workspace, or the stored constants without DQ)
// and, with DQ, the fp64 tree sum of the 256 constants. The next DQ block's
// loads are issued before the current one is coded.
template <bool kBf16, bool kDq>
__global__ __launch_bounds__(kThreads) void k_absmax_codes(const uint8_t *__restrict__ W, int64_t n,
                                                           uint8_t *__restrict__ codes,
                                                           float *__restrict__ absmax_out,
                                                           double *__restrict__ partial,
                                                           int64_t nb, int64_t nd, Nf4Tables tab,
                                                           CodeLut code_tab) {
  using IT = InTraits<kBf16>;
  constexpr int kEpl = IT::kEpl;                    // elements per lane
  constexpr int kLpb = kBlock / kEpl;               // lanes per 64-block
  constexpr int kPasses = kElemsPerDq / (kThreads * kEpl);
  constexpr int kEsz = kBf16 ? 2 : 4;

  __shared__ float2 lut[kCells];
  __shared__ float sa[kDqBlock];
  __shared__ double wsum[kThreads / 64];

  const int tid = threadIdx.x;
  auto elem = [&](int64_t d, int pass) {
    return d * kElemsPerDq + static_cast<int64_t>(pass) * kThreads * kEpl + static_cast<int64_t>(tid) * kEpl;
  };
  auto full = [&](int64_t d) { return (d + 1) * kElemsPerDq <= n; };
  // loads of a DQ block; a block with a tail is loaded element by element
  auto load = [&](int64_t d, uint4 *raw) {
    if (full(d)) {
#pragma unroll
      for (int p = 0; p < kPasses; ++p) raw[p] = load_stream(W + elem(d, p) * kEsz);
    } else {
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const int64_t e = elem(d, p);
        uint32_t tmp[4] = {0u, 0u, 0u, 0u};
        for (int i = 0; i < kEpl; ++i) {
          if (e + i < n) {
            if (kBf16) tmp[i / 2] |= static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(W)[e + i]) << (16 * (i % 2));
            else tmp[i] = reinterpret_cast<const uint32_t *>(W)[e + i];
          }
        }
        raw[p] = make_uint4(tmp[0], tmp[1], tmp[2], tmp[3]);
      }
    }
  };

  // the table's loads go out before the weights', so that writing it to LDS
  // does not wait for the weights
  static_assert(kCells <= 2 * kThreads, "two table cells per thread at most");
  const float2 cell0 = code_tab.cell[tid];
  const float2 cell1 = code_tab.cell[min(tid + kThreads, kCells - 1)];
  auto write_lut = [&]() {
    lut[tid] = cell0;
    if (tid + kThreads < kCells) lut[tid + kThreads] = cell1;
  };
  int64_t d = blockIdx.x;
  uint4 raw[kPasses];
  // (the table is written inside each branch: where the branches meet, the
  // compiler would wait for every load before the LDS store)
  if (d < nd && full(d)) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) raw[p] = load_stream(W + elem(d, p) * kEsz);
    write_lut();
  } else {
    if (d < nd) load(d, raw);
    write_lut();
  }
  __syncthreads();  // table ready

  for (; d < nd; d += gridDim.x) {
    uint4 nxt[kPasses];
    const int64_t dn = d + gridDim.x;
    if (dn < nd) load(dn, nxt);
    const bool f = full(d);
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int64_t e = elem(d, p);
      const float a = f ? code_lane<kBf16, false>(raw[p], e, n, codes, lut, tab)
                        : code_lane<kBf16, true>(raw[p], e, n, codes, lut, tab);
      if ((tid % kLpb) == 0) {
        const int64_t blk = e / kBlock;
        if (kDq) sa[blk - d * kDqBlock] = a;
        if (blk < nb) absmax_out[blk] = a;
      }
    }
    if constexpr (kDq) {
      __syncthreads();
      // fp64 tree sum of the 256 constants: xor butterflies give the
      // adjacent-pair tree inside each wave's 64 leaves, then (w0 + w1) + (w2 + w3).
      const int64_t myblk = d * kDqBlock + tid;
      double v = (myblk < nb) ? static_cast<double>(sa[tid]) : 0.0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) v = v + __shfl_xor(v, off);
      if ((tid & 63) == 0) wsum[tid >> 6] = v;
      __syncthreads();
      if (tid == 0) partial[d] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) raw[p] = nxt[p];
  }
}

// The sum of all per-DQ-block fp64 partials. The partials are
// the 256-leaf subtrees of the perfect binary tree over all absmax constants
// (zero padded), so the tree is completed in the same shape: aligned chunks
// of up to kTreeChunk partials, where thread t first sums its aligned run of
// S = top / 256 partials pairwise in registers and the 256 run sums are
// combined by xor butterflies inside each wave, then (w0 + w1) + (w2 + w3);
// the chunk sums are combined the same way.
constexpr int kTreeChunk = 8192;
constexpr int kTreeRun = kTreeChunk / kThreads;   // 32
constexpr int kTreeMaxChunks = kThreads * kTreeRun;
constexpr int64_t kDqFusedMaxBlocks = 1024;  // larger tensors take k_tree_mean + k_dq_codes
static_assert(kDqFusedMaxBlocks <= kTreeChunk, "the fused mean is a single-chunk tree");

// Sum of the perfect binary tree over top leaves (top a power of two <= kTreeChunk)
// src[base + i], zero past limit. Every thread gets the result.
__device__ double tree_sum(const double *src, int64_t base, int64_t limit, int top, double *wsum) {
  const int tid = threadIdx.x;
  const int run = top > kThreads ? top / kThreads : 1;
  double v[kTreeRun];
#pragma unroll
  for (int u = 0; u < kTreeRun; ++u) {
    const int64_t i = base + static_cast<int64_t>(tid) * run + u;
    v[u] = (u < run && tid * run + u < top && i < limit) ? src[i] : 0.0;
  }
#pragma unroll
  for (int len = kTreeRun; len > 1; len >>= 1) {
    if (len <= run) {
#pragma unroll
      for (int u = 0; u < len / 2; ++u) v[u] = v[2 * u] + v[2 * u + 1];
    }
  }
  double t = v[0];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) t = t + __shfl_xor(t, off);
  __syncthreads();   // wsum free
  if ((tid & 63) == 0) wsum[tid >> 6] = t;
  __syncthreads();
  return (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

// The DQ mean fp32(sum / nb) from the per-DQ-block partials: the tree over
// chunks of kTreeChunk partials, then over the chunk sums (csum in LDS).
__device__ float tree_mean(const double *__restrict__ partial, int64_t nd, int64_t nb, double *wsum,
                           double *csum) {
  const int tid = threadIdx.x;
  const int64_t nchunks = (nd + kTreeChunk - 1) / kTreeChunk;
  int top = 1;
  while (top < (nd < kTreeChunk ? nd : kTreeChunk)) top *= 2;
  double total;
  if (nchunks == 1) {
    total = tree_sum(partial, 0, nd, top, wsum);
  } else {
    for (int64_t c = 0; c < nchunks; ++c) {
      const double sc = tree_sum(partial, c * kTreeChunk, nd, kTreeChunk, wsum);
      if (tid == 0) csum[c] = sc;
    }
    __syncthreads();
    int ctop = 1;
    while (ctop < nchunks) ctop *= 2;
    total = tree_sum(csum, 0, nchunks, ctop, wsum);
  }
  return static_cast<float>(total / static_cast<double>(nb));
}

// DQ scale s2 = max |fp32(a - mean)| over DQ block d and its int8 codes, one
// thread per absmax constant.
// a = absmax_ws[d * 256 + thread] (0 past nb), loaded by the caller.
__device__ __forceinline__ void dq_block(float a, int64_t nb, int64_t d, float mu, int8_t *__restrict__ absmax_q,
                                         float *__restrict__ dq_scale, float *wmax) {
  const int tid = threadIdx.x;
  const int64_t b = d * kDqBlock + tid;
  const bool valid = b < nb;
  const float dv = valid ? __fsub_rn(a, mu) : 0.0f;
  float m = fabsf(dv);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  __syncthreads();   // wmax free
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
}

// Up to kDqFusedMaxBlocks DQ blocks, one per workgroup: every workgroup
// completes the same single-chunk fp64 tree over the per-DQ-block partials
// (the partials come from L2; the same tree as k_tree_mean) and workgroup 0
// stores the mean. The block's absmax load goes out before the tree's.
__global__ __launch_bounds__(kThreads) void k_dq_codes_mean(const float *__restrict__ absmax_ws,
                                                            const double *__restrict__ partial, int64_t nb,
                                                            int64_t nd, float *__restrict__ dq_mean,
                                                            int8_t *__restrict__ absmax_q,
                                                            float *__restrict__ dq_scale) {
  __shared__ double wsum[kThreads / 64];
  __shared__ float wmax[kThreads / 64];
  const int64_t d = blockIdx.x;
  const int64_t b = d * kDqBlock + threadIdx.x;
  const float a = b < nb ? absmax_ws[b] : 0.0f;
  int top = 1;
  while (top < nd) top *= 2;
  const float mu = static_cast<float>(tree_sum(partial, 0, nd, top, wsum) / static_cast<double>(nb));
  if (d == 0 && threadIdx.x == 0) dq_mean[0] = mu;
  dq_block(a, nb, d, mu, absmax_q, dq_scale, wmax);
}

// Larger tensors: one workgroup completes the mean ...
__global__ __launch_bounds__(kThreads) void k_tree_mean(const double *__restrict__ partial, int64_t nd,
                                                        int64_t nb, float *__restrict__ dq_mean) {
  __shared__ double wsum[kThreads / 64];
  __shared__ double csum[kTreeMaxChunks];
  const float mu = tree_mean(partial, nd, nb, wsum, csum);
  if (threadIdx.x == 0) dq_mean[0] = mu;
}

// ... and one wave per DQ block reads it: 4 constants per lane, the block's
// max |a - mean| by lane exchanges (max is exact in any order), no barrier;
// the same arithmetic per constant as dq_block.
__global__ __launch_bounds__(kThreads) void k_dq_codes(const float *__restrict__ absmax_ws, int64_t nb,
                                                       int64_t nd, const float *__restrict__ dq_mean,
                                                       int8_t *__restrict__ absmax_q,
                                                       float *__restrict__ dq_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t d = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (d >= nd) return;   // wave-uniform
  const float mu = dq_mean[0];
  const int64_t b0 = d * kDqBlock + 4 * lane;
  float a[4];
  if (b0 + 4 <= nb) {
    const float4 v = *reinterpret_cast<const float4 *>(absmax_ws + b0);
    a[0] = v.x;
    a[1] = v.y;
    a[2] = v.z;
    a[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = b0 + j < nb ? absmax_ws[b0 + j] : 0.0f;
  }
  float dv[4], m = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    dv[j] = b0 + j < nb ? __fsub_rn(a[j], mu) : 0.0f;
    m = fmaxf(m, fabsf(dv[j]));
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float s2 = m;
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int q = 0;
    if (s2 > 0.0f) {
      q = static_cast<int>(rintf(__fmul_rn(__fdiv_rn(dv[j], s2), 127.0f)));
      q = min(max(q, -127), 127);
    }
    packed |= (static_cast<uint32_t>(q) & 0xFFu) << (8 * j);
  }
  if (b0 + 4 <= nb) {
    *reinterpret_cast<uint32_t *>(absmax_q + b0) = packed;
  } else {
    for (int j = 0; j < 4; ++j)
      if (b0 + j < nb) absmax_q[b0 + j] = static_cast<int8_t>(packed >> (8 * j));
  }
  if (lane == 0) dq_scale[d] = s2;
}

// ------------------------------------------------------------ dequantize

__device__ __forceinline__ float block_scale(int8_t q, float kd, float mu) {
  return __fadd_rn(__fmul_rn(static_cast<float>(q), kd), mu);
}

// With kDq the block scales are decoded from the int8 codes, the DQ scales
// and the mean; without it they are the stored fp32 constants `absmax`.
template <bool kOutBf16, bool kDq>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t *__restrict__ codes,
                                                      const int8_t *__restrict__ absmax_q,
                                                      const float *__restrict__ dq_scale,
                                                      const float *__restrict__ dq_mean,
                                                      const float *__restrict__ absmax, int64_t n,
                                                      void *__restrict__ out, Nf4Tables tab) {
  __shared__ float lv[16];
  __shared__ float cs[kDqBlock];
  // fp32 output: each wave's 512 results of a piece pass through its own 2 KB
  // of LDS, so that every store instruction writes 1 KB contiguous (lane l
  // at 16 l) instead of every other 16 bytes of 2 KB
  __shared__ __attribute__((aligned(16))) float stage[kOutBf16 ? 1 : kThreads * 8];
  const int tid = threadIdx.x;
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t nbytes = (n + 1) / 2;
  if (tid < 16) lv[tid] = tab.lv[tid];
  const float mu = kDq ? dq_mean[0] : 0.0f;

  for (int64_t d = blockIdx.x; d * kElemsPerDq < n; d += gridDim.x) {
    // The code loads go out first: they do not depend on the scales, so the
    // codes and the scale inputs travel together.
    const int64_t byte_base = d * (kElemsPerDq / 2);
    // 8 pieces of 4 code bytes (8 elements) per thread; piece p of thread t
    // starts at byte 4t + 1024p of the DQ block, so each wave touches a
    // contiguous 256-byte run of codes per piece.
    uint32_t w[8];
    if ((d + 1) * kElemsPerDq <= n) {   // whole DQ block: every load in flight at once
#pragma unroll
      for (int p = 0; p < 8; ++p)
        w[p] = *reinterpret_cast<const uint32_t *>(codes + byte_base + 4 * tid + 1024 * p);
    } else {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int64_t byte0 = byte_base + 4 * tid + 1024 * p;
        uint32_t t = 0;
        for (int j = 0; j < 4; ++j)
          if (byte0 + j < nbytes) t |= static_cast<uint32_t>(codes[byte0 + j]) << (8 * j);
        w[p] = t;
      }
    }
    const int64_t b = d * kDqBlock + tid;
    float c;
    if constexpr (kDq) {
      const float s2 = dq_scale[d];
      const int8_t q = (b < nb) ? absmax_q[b] : static_cast<int8_t>(0);
      c = block_scale(q, __fdiv_rn(s2, 127.0f), mu);
    } else {
      c = (b < nb) ? absmax[b] : 0.0f;
    }
    __syncthreads();  // previous iteration done with cs
    cs[tid] = (b < nb) ? c : 0.0f;
    __syncthreads();
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
          // written once and not read again here: a streaming (non-temporal) store
          __builtin_nontemporal_store(pk, reinterpret_cast<bf16x8 *>(o));
        } else {
          for (int j = 0; j < 8; ++j)
            if (e + j < n) o[j] = static_cast<__bf16>(v[j]);
        }
      } else {
        float *o = reinterpret_cast<float *>(out) + e;
        // the wave's 512 elements are contiguous: [w0, w0 + 512) with w0 = e - 8 lane
        const int lane = tid & 63;
        const int64_t w0 = e - 8 * lane;
        if (w0 + 512 <= n) {
          float *st = stage + (tid - lane) * 8;
          *reinterpret_cast<float4 *>(st + 8 * lane) = make_float4(v[0], v[1], v[2], v[3]);
          *reinterpret_cast<float4 *>(st + 8 * lane + 4) = make_float4(v[4], v[5], v[6], v[7]);
          __builtin_amdgcn_wave_barrier();
          const float4 lo = *reinterpret_cast<const float4 *>(st + 4 * lane);
          const float4 hi = *reinterpret_cast<const float4 *>(st + 256 + 4 * lane);
          __builtin_amdgcn_wave_barrier();
          float *ow = reinterpret_cast<float *>(out) + w0;
          *reinterpret_cast<float4 *>(ow + 4 * lane) = lo;
          *reinterpret_cast<float4 *>(ow + 256 + 4 * lane) = hi;
        } else if (e + 8 <= n) {
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


}  // namespace

// fp32 absmax [nb], then one fp64 tree partial per DQ block [nd].
size_t quantize_ws_bytes(int64_t n) {
  const int64_t nb = ceil_div(n, kBlock);
  return align_up(static_cast<size_t>(nb) * 4, 256) + static_cast<size_t>(ceil_div(nb, kDqBlock)) * 8;
}

hipError_t launch_quantize(const void *W, bool w_bf16, int64_t n, int format, uint8_t *codes,
                           int8_t *absmax_q, float *dq_scale, float *dq_mean, float *absmax, void *ws,
                           hipStream_t s) {
  const int64_t nb = ceil_div(n, kBlock);
  const int64_t nd = ceil_div(nb, kDqBlock);
  const bool dq = fmt_dq(format);
  float *absmax_out = dq ? static_cast<float *>(ws) : absmax;
  double *part = dq ? reinterpret_cast<double *>(static_cast<char *>(ws) + align_up(static_cast<size_t>(nb) * 4, 256))
                    : nullptr;
  if (ceil_div(nd, kTreeChunk) > kTreeMaxChunks) return hipErrorInvalidValue;   // > 2^37 elements
  const Nf4Tables &tab = format_tables(format);
  const CodeLut *lut = code_lut(format);
  if (!lut) return hipErrorInvalidValue;
  prof_begin(kProfQuantize, s);
  const int64_t grid = nd;   // one DQ block per workgroup
  const uint8_t *w8 = static_cast<const uint8_t *>(W);
  if (w_bf16) {
    if (dq) hipLaunchKernelGGL((k_absmax_codes<true, true>), dim3(grid), dim3(kThreads), 0, s, w8, n, codes, absmax_out, part, nb, nd, tab, *lut);
    else hipLaunchKernelGGL((k_absmax_codes<true, false>), dim3(grid), dim3(kThreads), 0, s, w8, n, codes, absmax_out, part, nb, nd, tab, *lut);
  } else {
    if (dq) hipLaunchKernelGGL((k_absmax_codes<false, true>), dim3(grid), dim3(kThreads), 0, s, w8, n, codes, absmax_out, part, nb, nd, tab, *lut);
    else hipLaunchKernelGGL((k_absmax_codes<false, false>), dim3(grid), dim3(kThreads), 0, s, w8, n, codes, absmax_out, part, nb, nd, tab, *lut);
  }
  prof_end(kProfQuantize, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !dq) return err;
  if (nd <= kDqFusedMaxBlocks) {
    hipLaunchKernelGGL(k_dq_codes_mean, dim3(nd), dim3(kThreads), 0, s, absmax_out, part, nb, nd, dq_mean, absmax_q,
                       dq_scale);
  } else {
    hipLaunchKernelGGL(k_tree_mean, dim3(1), dim3(kThreads), 0, s, part, nd, nb, dq_mean);
    hipLaunchKernelGGL(k_dq_codes, dim3(ceil_div(nd, kThreads / 64)), dim3(kThreads), 0, s, absmax_out, nb, nd, dq_mean,
                       absmax_q, dq_scale);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *codes, int format, const int8_t *absmax_q, const float *dq_scale,
                             const float *dq_mean, const float *absmax, int64_t n, void *out, bool out_bf16,
                             hipStream_t s) {
  const int64_t nd = ceil_div(ceil_div(n, kBlock), kDqBlock);
  const int64_t grid = nd < 8192 ? nd : 8192;
  const Nf4Tables &tab = format_tables(format);
  const bool dq = fmt_dq(format);
  prof_begin(kProfDequantize, s);
  if (out_bf16) {
    if (dq) hipLaunchKernelGGL((k_dequant<true, true>), dim3(grid), dim3(kThreads), 0, s, codes, absmax_q, dq_scale, dq_mean, absmax, n, out, tab);
    else hipLaunchKernelGGL((k_dequant<true, false>), dim3(grid), dim3(kThreads), 0, s, codes, absmax_q, dq_scale, dq_mean, absmax, n, out, tab);
  } else {
    if (dq) hipLaunchKernelGGL((k_dequant<false, true>), dim3(grid), dim3(kThreads), 0, s, codes, absmax_q, dq_scale, dq_mean, absmax, n, out, tab);
    else hipLaunchKernelGGL((k_dequant<false, false>), dim3(grid), dim3(kThreads), 0, s, codes, absmax_q, dq_scale, dq_mean, absmax, n, out, tab);
  }
  prof_end(kProfDequantize, s);
  return hipGetLastError();
}

}  // namespace qnf4
