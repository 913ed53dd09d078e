// QLoRA linear layer on gfx950: forward and backward with the NF4 + DQ base
// dequantized on the fly (QLoRA vs ChatGPT page, capability "training
// pipeline": block-wise dequantization in the forward pass, gradients only
// for the LoRA parameters; capability "LoRA on the quantized base": a frozen
// 4-bit base plus a full-precision low-rank adapter).
//
//   forward    Y  = X W^T + s (X A^T) B^T
//   backward   dH = s dY B,  dX = dY W + dH A,  dA = dH^T X,  dB = s dY^T (X A^T)
//
// Kernel plan (all on the caller's stream, no host synchronization):
//   k_adapter_down    split partials of H = X A^T and (backward) of dY B,
//                     read straight from the fp32 factors
//   k_adapter_finish  Hs = bf16(s H), (backward) dHb = bf16(s dY B), the block
//                     scales c_b and the bf16 adapter operand of the GEMM below
//                     (B forward, A^T backward), one launch
//   k_fwd_big         Y tile = [X | Hs] [W-hat | Bb]^T: the NF4 weight is decoded
//                     into LDS step by step, the adapter term is 64-deep extra
//                     reduction steps on the same accumulators
//   k_dx_big          dX tile = [dY | dHb] [W-hat ; At]: the weight decoded
//                     transposed (reduction over out_features)
//   k_grad            split-M partials of dA = dHb^T X and dB = dY^T Hs
//   k_grad_finish     fixed-order sums of those partials
// Small M (decode, M <= 32) runs the weight-streaming kernels of gemv.hip instead.
#include <algorithm>

#include "gemm_big.h"

namespace qnf4 {
namespace {

// LDS table of level pairs for every code byte: (level[b >> 4], level[b & 15]),
// kLvCopies interleaved copies; returns this lane's copy.
__device__ __forceinline__ const float2 *load_level_pairs(float2 *lv2, const Nf4Tables &tab) {
  for (int i = threadIdx.x; i < 256 * kLvCopies; i += blockDim.x) {
    const int b = i / kLvCopies;
    lv2[i] = make_float2(tab.lv[b >> 4], tab.lv[b & 15]);
  }
  return lv2 + (threadIdx.x & (kLvCopies - 1));
}

// ------------------------------------------------------------------ forward

struct FwdParams {
  const void *X;        // bf16 [M, K]
  const uint8_t *codes; // NF4 codes of W [N, K]
  const float *cs;      // per-block scales
  const void *Hs;       // bf16 [M, rp] = bf16(s * X A^T), zero padded
  const void *Bb;       // bf16 [N, rp], zero padded
  void *Y;              // bf16 [M, N]
  int64_t M, N, K;
  int rp;
};

// Large-M forward: one 256 x 256 tile of Y per workgroup (XCD-aware order),
// run with eight waves (CfgBig8): two waves per SIMD cover each other's
// waits, at 128 x 64 accumulators per wave.
template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, 1) void k_fwd_big(FwdParams p, Nf4Tables tab) {
  constexpr int T = Cfg::kThreads;
  __shared__ __attribute__((aligned(16))) __bf16 sa0[Cfg::kLdsA], sa1[Cfg::kLdsA];
  __shared__ __attribute__((aligned(16))) __bf16 sb0[Cfg::kLdsB], sb1[Cfg::kLdsB];
  const BigSmem smem{sa0, sa1, sb0, sb1};
  __shared__ float2 lv_tab[256 * kLvCopies];
  const float2 *lv = load_level_pairs(lv_tab, tab);
  int tm, tn;
  tile_of(blockIdx.x, static_cast<int>((p.M + 255) / 256), static_cast<int>((p.N + 255) / 256), tm, tn);
  const int64_t n0 = static_cast<int64_t>(tn) * 256;
  const int64_t m0 = static_cast<int64_t>(tm) * 256;
  __syncthreads();
  Acc<Cfg> acc;
  acc.zero();
  {
    DirectRowsT<T> da(p.X, p.K, p.M, m0);
    Nf4RowBigT<T> l0(p.codes, p.cs, p.N, p.K, n0), l1 = l0;
    auto load = [](Nf4RowBigT<T> &l, int s) { l.load(static_cast<int64_t>(s) * kBK); };
    big_mainloop_nf4<Cfg>(acc, da, l0, l1, load, static_cast<int>(p.K / kBK), smem, lv);
  }
  if (p.rp > 0) {
    DirectRowsT<T> da(p.Hs, p.rp, p.M, m0), db(p.Bb, p.rp, p.N, n0);
    big_mainloop_dense<Cfg>(acc, da, db, p.rp / kBK, smem);
  }
  if (m0 + 256 <= p.M && n0 + 256 <= p.N)
    store_bf16<Cfg, false>(acc, static_cast<__bf16 *>(p.Y), p.N, p.M, p.N, m0, n0, 1.0f);
  else
    store_bf16<Cfg, true>(acc, static_cast<__bf16 *>(p.Y), p.N, p.M, p.N, m0, n0, 1.0f);
}

// ------------------------------------------------------------- backward dX

using CfgDx = CfgBig8;

struct DxParams {
  const void *dY;       // bf16 [M, N]
  const uint8_t *codes; // NF4 codes of W [N, K]
  const float *cs;
  const void *dHb;      // bf16 [M, rp] = bf16(s dY B)
  const void *Atb;      // bf16 [K, rp] = bf16(A^T)
  void *dX;             // bf16 [M, K]
  int64_t M, N, K;
  int rp;
};

// Input gradient: one 256 x 256 tile of dX per workgroup (XCD-aware order),
// run with eight waves as the forward is: the transposed decode gives each
// thread half an 8 x 8 unit (four rows n), which keeps the kernel within the
// registers two waves per SIMD leave.
template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, 1) void k_dx_big(DxParams p, Nf4Tables tab) {
  constexpr int T = Cfg::kThreads;
  __shared__ __attribute__((aligned(16))) __bf16 sa0[Cfg::kLdsA], sa1[Cfg::kLdsA];
  __shared__ __attribute__((aligned(16))) __bf16 sb0[Cfg::kLdsB], sb1[Cfg::kLdsB];
  const BigSmem smem{sa0, sa1, sb0, sb1};
  __shared__ float2 lv_tab[256 * kLvCopies];
  const float2 *lv = load_level_pairs(lv_tab, tab);
  int tm, tn;
  tile_of(blockIdx.x, static_cast<int>((p.M + 255) / 256), static_cast<int>((p.K + 255) / 256), tm, tn);
  const int64_t k0 = static_cast<int64_t>(tn) * 256;
  const int64_t m0 = static_cast<int64_t>(tm) * 256;
  __syncthreads();
  Acc<Cfg> acc;
  acc.zero();
  {
    DirectRowsT<T> da(p.dY, p.N, p.M, m0);
    Nf4TransBigT<T> l0(p.codes, p.cs, p.K, k0), l1 = l0;
    const int64_t K = p.K;
    auto load = [K](Nf4TransBigT<T> &l, int s) { l.load(static_cast<int64_t>(s) * kBK, K); };
    big_mainloop_nf4<Cfg>(acc, da, l0, l1, load, static_cast<int>(p.N / kBK), smem, lv);
  }
  if (p.rp > 0) {
    DirectRowsT<T> da(p.dHb, p.rp, p.M, m0), db(p.Atb, p.rp, p.K, k0);
    big_mainloop_dense<Cfg>(acc, da, db, p.rp / kBK, smem);
  }
  if (m0 + 256 <= p.M && k0 + 256 <= p.K)
    store_bf16<Cfg, false>(acc, static_cast<__bf16 *>(p.dX), p.K, p.M, p.K, m0, k0, 1.0f);
  else
    store_bf16<Cfg, true>(acc, static_cast<__bf16 *>(p.dX), p.K, p.M, p.K, m0, k0, 1.0f);
}

// ------------------------------------------------ adapter down-projection
//
// k_adapter_down computes split partials of H = X A^T and (backward) of
// dY B straight from the fp32 adapter factors; k_adapter_finish then sums
// them and, in the same launch, writes the other small operands of the big
// GEMMs:
//   Hs  [M][rp]   bf16(s H), columns >= r zero          (forward adapter step; dB)
//   dHb [M][rp]   bf16(s dY B), columns >= r zero       (backward adapter step; dA)
//   cs  [nb]      block scales c_b of the NF4 weight
//   Bb  [N][rp]   bf16(B), columns >= r zero            (forward adapter step)
//   Atb [K][rp]   bf16(A^T), columns >= r zero          (backward adapter step)

struct DownParams {
  const void *X, *dY;
  const float *A, *B;        // fp32 A [r][K], B [N][r]
  float *h_part, *dh_part;   // [splits][M][rp]
  int64_t M, N, K;
  int r, rp;
  int jt;                    // rp / 64 column tiles
  int mt;                    // row tiles of kDownRows (rounded up)
  int h_splits, h_steps, dh_splits, dh_steps;
};

// Skinny product tile of k_adapter_down: 128 rows of P (32 per wave) by the
// 64 adapter columns j0 .. j0 + 63 of Q, over a range of the reduction.
//
// P is streamed straight from memory into the MFMA A operand (no LDS): the
// reduction is processed in chunks of CS 64-deep steps, and within a chunk
// lane (row i = lane % 32, half h = lane / 32) holds the contiguous run
// k = h * 32 CS + 8 s .. + 7 for slices s = 0 .. 4 CS - 1. The Q operand is
// rounded to bf16 and staged in LDS as [64][264] (rows padded by 16 bytes, so
// that the 32 rows a fragment read touches start in different banks) and read
// with the same permutation of k, so each MFMA pairs equal k.
constexpr int kDownWaves = 4;
constexpr int kDownRows = 32 * kDownWaves;
constexpr int kDownThreads = 64 * kDownWaves;
constexpr int kDownLd = 256 + 8;         // LDS row of the Q chunk (bf16)
constexpr int kDownLds = 64 * kDownLd;   // bf16 per Q buffer

// fp32 source of the Q operand: rows j0 .. j0 + 63 of Q, rows >= r zero.
struct QSrc {
  const float *src;
  int64_t ld;
  int r;
  int j0;
};

// Q = A (row j of Q is row j of A [r][K]): 8-element runs of a row, two
// 16-byte loads each, consecutive threads along the row.
template <int CS>
struct QFromRows {
  static constexpr int kRuns = 64 * 8 * CS / kDownThreads;
  float4 v[2 * kRuns];
  __device__ __forceinline__ void load(const QSrc &q, int64_t kc) {
#pragma unroll
    for (int u = 0; u < kRuns; ++u) {
      const int idx = threadIdx.x + u * kDownThreads, j = idx / (8 * CS), c = idx % (8 * CS);
      const float *p = q.src + static_cast<int64_t>(min(q.j0 + j, q.r - 1)) * q.ld + kc + 8 * c;
      v[2 * u] = *reinterpret_cast<const float4 *>(p);
      v[2 * u + 1] = *reinterpret_cast<const float4 *>(p + 4);
    }
  }
  __device__ __forceinline__ void stage(const QSrc &q, __bf16 *lds) const {
#pragma unroll
    for (int u = 0; u < kRuns; ++u) {
      const int idx = threadIdx.x + u * kDownThreads, j = idx / (8 * CS), c = idx % (8 * CS);
      const bool ok = q.j0 + j < q.r;
      const float4 a = v[2 * u], b = v[2 * u + 1];
      const uint4 w = make_uint4(ok ? pack_bf16x2(a.x, a.y) : 0u, ok ? pack_bf16x2(a.z, a.w) : 0u,
                                 ok ? pack_bf16x2(b.x, b.y) : 0u, ok ? pack_bf16x2(b.z, b.w) : 0u);
      *reinterpret_cast<uint4 *>(lds + j * kDownLd + 8 * c) = w;
    }
  }
};

// Q = B^T (row j of Q is column j of B [N][r]): lane j of a wave reads
// B[n][j0 + j], so one load covers a row of B; wave w takes the pairs of
// reduction indices n = kc + 2 (w + 4 i), + 1 and writes each pair as one
// 4-byte LDS store.
template <int CS>
struct QFromCols {
  static constexpr int kPairs = 64 * CS / 2 / kDownWaves;
  float v[2 * kPairs];
  __device__ __forceinline__ void load(const QSrc &q, int64_t kc) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const float *p = q.src + min(q.j0 + lane, q.r - 1);
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int64_t n = kc + 2 * (w + kDownWaves * i);
      v[2 * i] = p[n * q.ld];
      v[2 * i + 1] = p[(n + 1) * q.ld];
    }
  }
  __device__ __forceinline__ void stage(const QSrc &q, __bf16 *lds) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const bool ok = q.j0 + lane < q.r;
#pragma unroll
    for (int i = 0; i < kPairs; ++i)
      *reinterpret_cast<uint32_t *>(lds + lane * kDownLd + 2 * (w + kDownWaves * i)) =
          ok ? pack_bf16x2(v[2 * i], v[2 * i + 1]) : 0u;
  }
};

template <int CS, template <int> class QL>
struct DownChunk {
  static constexpr int kSlices = 4 * CS;   // 16-deep MFMA slices
  uint4 x[kSlices];
  QL<CS> q;
  __device__ __forceinline__ const char *xptr(const char *xrow, int64_t kc, int h) const {
    return xrow + (kc + h * 32 * CS) * 2;
  }
  __device__ __forceinline__ void load_x(const char *xrow, int64_t kc, int h) {
    const char *px = xptr(xrow, kc, h);
#pragma unroll
    for (int s = 0; s < kSlices; ++s) x[s] = *reinterpret_cast<const uint4 *>(px + 16 * s);
  }
  // MFMAs of the staged chunk; with NEXT, slice s of the next chunk (at px)
  // is loaded into x[s] as soon as slice s has been consumed.
  template <bool NEXT>
  __device__ __forceinline__ void mma(f32x16 (&acc)[2], const __bf16 *lds, int lane, const char *px) {
    const __bf16 *lb = lds + (lane & 31) * kDownLd + (lane >> 5) * 32 * CS;
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, x[s]);
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const bf16x8 b = *reinterpret_cast<const bf16x8 *>(lb + jb * 32 * kDownLd + 8 * s);
        acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[jb], 0, 0, 0);
      }
      if (NEXT) x[s] = *reinterpret_cast<const uint4 *>(px + 16 * s);
    }
  }
};

// `n` chunks of CS steps from reduction offset k0. The Q chunk alternates
// between the two LDS buffers, one barrier per chunk; the P operand streams
// through the registers slice by slice. On entry and on exit the LDS is free.
template <int CS, template <int> class QL>
__device__ __forceinline__ void down_chunks(f32x16 (&acc)[2], const char *xrow, const QSrc &qs, int64_t k0,
                                            int n, __bf16 *lds) {
  if (n <= 0) return;
  const int lane = threadIdx.x & 63, h = lane >> 5;
  constexpr int64_t kLen = 64 * CS;
  DownChunk<CS, QL> c;
  c.load_x(xrow, k0, h);
  c.q.load(qs, k0);
  for (int i = 0; i < n; ++i) {
    __bf16 *buf = lds + (i & 1) * kDownLds;
    c.q.stage(qs, buf);
    __syncthreads();
    const int64_t kn = k0 + (i + 1) * kLen;
    if (i + 1 < n) {
      c.q.load(qs, kn);
      c.template mma<true>(acc, buf, lane, c.xptr(xrow, kn, h));
    } else {
      c.template mma<false>(acc, buf, lane, nullptr);
    }
  }
  __syncthreads();
}

template <template <int> class QL, int CS>
__device__ __forceinline__ void down_tile(const char *P, int64_t L, int64_t M, const QSrc &qs, int64_t m0,
                                          int s0, int steps, float *part, int rp, __bf16 *lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // rows past M read row M - 1 (always valid) and are not stored
  const int64_t row = min(m0 + 32 * w + (lane & 31), M - 1);
  const char *xrow = P + row * L * 2;
  f32x16 acc[2];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jb][v] = 0.0f;
  const int64_t k0 = static_cast<int64_t>(s0) * kBK;
  down_chunks<CS, QL>(acc, xrow, qs, k0, steps / CS, lds);
  if (CS > 1) down_chunks<1, QL>(acc, xrow, qs, k0 + (steps / CS) * CS * kBK, steps % CS, lds);
  const int h = lane >> 5;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int64_t col = qs.j0 + jb * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t r = m0 + 32 * w + 8 * (v >> 2) + 4 * h + (v & 3);
      if (r < M) part[r * rp + col] = acc[jb][v];
    }
  }
}

__global__ __launch_bounds__(kDownThreads, 2) void k_adapter_down(DownParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * kDownLds];
  int g = blockIdx.x;
  const int per = p.jt * p.mt;
  const bool is_h = g < per * p.h_splits;
  if (!is_h) g -= per * p.h_splits;
  const int z = g / per, t = g % per;
  const int j0 = (t % p.jt) * 64;
  const int64_t m0 = static_cast<int64_t>(t / p.jt) * kDownRows;
  const int64_t L = is_h ? p.K : p.N;
  const int steps_per = is_h ? p.h_steps : p.dh_steps;
  const int total = static_cast<int>(L / kBK);
  const int s0 = z * steps_per, steps = min(steps_per, total - s0);
  if (is_h) {
    const QSrc qs{p.A, p.K, p.r, j0};
    down_tile<QFromRows, 4>(static_cast<const char *>(p.X), L, p.M, qs, m0, s0, steps,
                         p.h_part + static_cast<int64_t>(z) * p.M * p.rp, p.rp, lds);
  } else {
    const QSrc qs{p.B, p.r, p.r, j0};
    down_tile<QFromCols, 2>(static_cast<const char *>(p.dY), L, p.M, qs, m0, s0, steps,
                         p.dh_part + static_cast<int64_t>(z) * p.M * p.rp, p.rp, lds);
  }
}

// sum_z part[z * plane + e] for z = 0 .. splits - 1, added in that order; the
// loads go out eight at a time (clamped indices, the extra terms dropped), so
// the sum costs a few memory round trips instead of one per split.
__device__ __forceinline__ float split_sum(const float *part, int64_t plane, int64_t e, int splits) {
  float v = 0.0f;
  for (int z0 = 0; z0 < splits; z0 += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = part[static_cast<int64_t>(min(z0 + u, splits - 1)) * plane + e];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < splits) v += t[u];
  }
  return v;
}

// The same sum for four consecutive elements (16-byte loads).
__device__ __forceinline__ float4 split_sum4(const float *part, int64_t plane, int64_t e, int splits) {
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int z0 = 0; z0 < splits; z0 += 8) {
    float4 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      t[u] = *reinterpret_cast<const float4 *>(part + static_cast<int64_t>(min(z0 + u, splits - 1)) * plane + e);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < splits) {
        v.x += t[u].x;
        v.y += t[u].y;
        v.z += t[u].z;
        v.w += t[u].w;
      }
  }
  return v;
}

// k_adapter_finish: one launch, its workgroups split into segments (each
// workgroup in one segment, one work item per thread):
//   Hs, dHb   fixed-order split sums, 4 elements per item, times s, to bf16
//   cs        4 block scales per item: c_b = fp32(fp32(absmax_q * fp32(d / 127)) + mean)
//   Bb / Atb  8 adapter columns of one row per item (one 16-byte store)
constexpr int kScaleBlocksPerThread = 4;

struct FinishParams {
  const float *h_part, *dh_part;   // [splits][M][rp]
  __bf16 *Hs, *dHb;
  int64_t M;
  int r, rp, h_splits, dh_splits;
  float scale;
  const int8_t *absmax_q;
  const float *dq_scale, *dq_mean;
  float *cs;
  int64_t nb;
  const float *A, *B;
  __bf16 *Bb, *Atb;                // one of them written (the other null)
  int64_t N, K;
  int64_t g_h, g_dh, g_cs, g_op;   // workgroups per segment
};

__global__ __launch_bounds__(256) void k_adapter_finish(FinishParams p) {
  int64_t g = blockIdx.x;
  if (g < p.g_h + p.g_dh) {   // split sums
    const bool second = g >= p.g_h;
    if (second) g -= p.g_h;
    const int64_t e = (g * 256 + threadIdx.x) * 4, n = p.M * p.rp;
    if (e >= n) return;
    const float4 v = split_sum4(second ? p.dh_part : p.h_part, n, e, second ? p.dh_splits : p.h_splits);
    const uint2 w = make_uint2(pack_bf16x2(p.scale * v.x, p.scale * v.y), pack_bf16x2(p.scale * v.z, p.scale * v.w));
    *reinterpret_cast<uint2 *>((second ? p.dHb : p.Hs) + e) = w;
    return;
  }
  g -= p.g_h + p.g_dh;
  if (g < p.g_cs) {           // block scales
    const int64_t b0 = (g * 256 + threadIdx.x) * kScaleBlocksPerThread;
    const float mu = p.dq_mean[0];
#pragma unroll
    for (int u = 0; u < kScaleBlocksPerThread; ++u) {
      const int64_t b = b0 + u;
      if (b < p.nb) {
        const float kd = __fdiv_rn(p.dq_scale[b / kDqBlock], 127.0f);
        p.cs[b] = __fadd_rn(__fmul_rn(static_cast<float>(p.absmax_q[b]), kd), mu);
      }
    }
    return;
  }
  g -= p.g_cs;
  const int64_t i = g * 256 + threadIdx.x;
  const int q8 = p.rp / 8;
  float v[8];
  __bf16 *dst;
  if (p.Bb) {                 // Bb[n][8 jq ..] = bf16(B[n][8 jq ..])
    if (i >= p.N * q8) return;
    const int64_t n = i / q8;
    const int j = static_cast<int>(i % q8) * 8;
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = p.B[n * p.r + min(j + t, p.r - 1)];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = j + t < p.r ? v[t] : 0.0f;
    dst = p.Bb + n * p.rp + j;
  } else {                    // Atb[k][8 jq ..] = bf16(A[8 jq ..][k]); consecutive threads take consecutive k
    if (i >= p.K * q8) return;
    const int64_t k = i % p.K;
    const int j = static_cast<int>(i / p.K) * 8;
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = p.A[static_cast<int64_t>(min(j + t, p.r - 1)) * p.K + k];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = j + t < p.r ? v[t] : 0.0f;
    dst = p.Atb + k * p.rp + j;
  }
  *reinterpret_cast<uint4 *>(dst) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

// ------------------------------------------------ adapter gradient products
//
// k_grad: M-split partials of dA = dHb^T X  ([rp][K] tiles first) and
// dB = dY^T Hs ([N][rp] tiles after them); k_grad_finish sums the partials in
// a fixed order into dA [r][K] and dB [N][r].
struct GradParams {
  const void *X, *dY, *Hs, *dHb;
  float *a_part, *b_part;     // [splits][rp][K], [splits][N][rp]
  int64_t M, N, K;
  int rp;
  int a_tiles_c, a_tiles, a_splits, a_steps;   // dA: 64 x 256 tiles over (rp, K)
  int b_tiles_c, b_tiles, b_splits, b_steps;   // dB: 256 x 64 tiles over (N, rp)
};

using CfgGradA = TileCfg<64, 256, 1, 4>;   // dA tile: 64 adapter rows x 256 columns of K
using CfgGradB = TileCfg<256, 64, 4, 1>;   // dB tile: 256 rows of N x 64 adapter columns

__global__ __launch_bounds__(256) void k_grad(GradParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (CfgGradA::kLdsA + CfgGradA::kLdsB)];
  int g = blockIdx.x;
  const bool is_a = g < p.a_tiles * p.a_splits;
  if (!is_a) g -= p.a_tiles * p.a_splits;
  const int tiles = is_a ? p.a_tiles : p.b_tiles;
  const int tiles_c = is_a ? p.a_tiles_c : p.b_tiles_c;
  const int per = is_a ? p.a_steps : p.b_steps;
  const int z = g / tiles, t = g % tiles;
  const int total = static_cast<int>((p.M + kBK - 1) / kBK);
  const int s0 = z * per, steps = min(per, total - s0);
  // rows of this split's range only: the two-stage loop reads past its end
  const int64_t red_end = min(p.M, static_cast<int64_t>(s0 + steps) * kBK);
  if (is_a) {
    const int64_t c0 = static_cast<int64_t>(t % tiles_c) * 256;
    const int64_t r0 = static_cast<int64_t>(t / tiles_c) * 64;
    Acc<CfgGradA> acc;
    acc.zero();
    TransBf16Narrow<64, 256> la(p.dHb, p.rp, red_end, r0), la1 = la;
    TransBf16<256, 256> lb(p.X, p.K, red_end, p.K, c0), lb1 = lb;
    mainloop2<CfgGradA>(acc, la, la1, lb, lb1, static_cast<int64_t>(s0) * kBK, steps, smem);
    store_f32<CfgGradA>(acc, p.a_part + static_cast<int64_t>(z) * p.rp * p.K, p.K, p.rp, p.K, r0, c0);
  } else {
    const int64_t c0 = static_cast<int64_t>(t % tiles_c) * 64;
    const int64_t r0 = static_cast<int64_t>(t / tiles_c) * 256;
    Acc<CfgGradB> acc;
    acc.zero();
    TransBf16<256, 256> la(p.dY, p.N, red_end, p.N, r0), la1 = la;
    TransBf16Narrow<64, 256> lb(p.Hs, p.rp, red_end, c0), lb1 = lb;
    mainloop2<CfgGradB>(acc, la, la1, lb, lb1, static_cast<int64_t>(s0) * kBK, steps, smem);
    store_f32<CfgGradB>(acc, p.b_part + static_cast<int64_t>(z) * p.N * p.rp, p.rp, p.N, p.rp, r0, c0);
  }
}

struct GradFinishParams {
  const float *a_part, *b_part;
  float *dA, *dB;
  int64_t N, K;
  int r, rp, a_splits, b_splits;
};

__global__ __launch_bounds__(256) void k_grad_finish(GradFinishParams p) {
  const int64_t na = static_cast<int64_t>(p.r) * p.K, nbb = p.N * p.r;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < na + nbb;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (i < na) {   // dA [r][K] from [splits][rp][K]
      p.dA[i] = split_sum(p.a_part, static_cast<int64_t>(p.rp) * p.K, i, p.a_splits);
    } else {        // dB [N][r] from [splits][N][rp]
      const int64_t e = i - na, row = e / p.r, col = e % p.r;
      p.dB[e] = split_sum(p.b_part, p.N * p.rp, row * p.rp + col, p.b_splits);
    }
  }
}

// ------------------------------------------------------------- tile configs
constexpr int kSmallM = 32;
constexpr int kTargetGroups = 512;
constexpr int kDownGroups = 256;

int64_t grid_blocks(int64_t n, int64_t b) { return ceil_div(n, b); }

struct Split {
  int splits;
  int steps_per_split;
};

// Split `steps` reduction steps so that tiles * splits reaches the target.
Split choose_split(int64_t tiles, int steps, int max_splits, int target = kTargetGroups) {
  int want = static_cast<int>(ceil_div(target, tiles > 0 ? tiles : 1));
  want = std::max(1, std::min({want, steps, max_splits}));
  const int per = static_cast<int>(ceil_div(steps, want));
  return {static_cast<int>(ceil_div(steps, per)), per};
}

// Workspace carve-out: sequential 256-byte-aligned regions.
struct Carve {
  char *base;
  size_t off = 0;
  template <class T>
  T *take(size_t count) {
    T *p = reinterpret_cast<T *>(base ? base + off : nullptr);
    off = align_up(off + count * sizeof(T), 256);
    return p;
  }
};

struct Plan {
  int rp;
  Split down, dh, ga, gb;
  bool small;
};

Plan make_plan(int64_t M, int64_t N, int64_t K, int r) {
  Plan pl;
  pl.rp = static_cast<int>(ceil_div(r, kBK) * kBK);
  pl.small = M <= kSmallM;
  const int ksteps = static_cast<int>(K / kBK), nsteps = static_cast<int>(N / kBK);
  const int64_t skinny_tiles = grid_blocks(M, kDownRows) * grid_blocks(pl.rp, 64);
  pl.down = choose_split(skinny_tiles, ksteps, 64, kDownGroups);
  pl.dh = choose_split(skinny_tiles, nsteps, 64, kDownGroups);
  const int msteps = static_cast<int>(ceil_div(M, kBK));
  pl.ga = choose_split(grid_blocks(pl.rp, 64) * grid_blocks(K, 256), msteps, 8);
  pl.gb = choose_split(grid_blocks(N, 256) * grid_blocks(pl.rp, 64), msteps, 8);
  return pl;
}

struct Buffers {
  float *cs;
  float *down_part;
  __bf16 *Hs;
  __bf16 *Bb;
  float *dh_part;
  __bf16 *dHb;
  __bf16 *Atb;
  float *ga_part;
  float *gb_part;
};

Buffers carve(void *ws, const Plan &pl, int64_t M, int64_t N, int64_t K, size_t *bytes) {
  Carve c{static_cast<char *>(ws)};
  Buffers b{};
  const int64_t nb = ceil_div(N * K, kBlock);
  const int rp = pl.rp;
  b.cs = c.take<float>(nb);
  if (rp > 0) {
    b.down_part = c.take<float>(static_cast<size_t>(pl.down.splits) * M * rp);
    b.Hs = c.take<__bf16>(static_cast<size_t>(M) * rp);
    b.Bb = c.take<__bf16>(static_cast<size_t>(N) * rp);
    b.dh_part = c.take<float>(static_cast<size_t>(pl.dh.splits) * M * rp);
    b.dHb = c.take<__bf16>(static_cast<size_t>(M) * rp);
    b.Atb = c.take<__bf16>(static_cast<size_t>(K) * rp);
    b.ga_part = c.take<float>(static_cast<size_t>(pl.ga.splits) * rp * K);
    b.gb_part = c.take<float>(static_cast<size_t>(pl.gb.splits) * N * rp);
  }
  if (bytes) *bytes = c.off;
  return b;
}

// The fp32 block scales the big GEMMs read: decoded into the workspace with
// DQ, the stored constants without it.
const float *block_scales(const LinearArgs &a, const Buffers &b) { return fmt_dq(a.format) ? b.cs : a.absmax; }

// The work before a big GEMM: the split partials of H = X A^T and (backward)
// dY B, then one launch with their sums, the block scales and the bf16 adapter
// operand of the GEMM (Bb forward, Atb backward).
hipError_t run_adapter_pre(const LinearArgs &a, const Plan &pl, const Buffers &b, const void *X,
                           const void *dY, const float *A, const float *B, bool backward, hipStream_t s) {
  const bool lora = pl.rp > 0;
  if (lora) {
    DownParams dp{};
    dp.X = X;
    dp.dY = dY;
    dp.A = A;
    dp.B = B;
    dp.h_part = b.down_part;
    dp.dh_part = b.dh_part;
    dp.M = a.M;
    dp.N = a.N;
    dp.K = a.K;
    dp.r = a.r;
    dp.rp = pl.rp;
    dp.jt = pl.rp / 64;
    dp.mt = static_cast<int>(ceil_div(a.M, kDownRows));
    dp.h_splits = pl.down.splits;
    dp.h_steps = pl.down.steps_per_split;
    dp.dh_splits = backward ? pl.dh.splits : 0;
    dp.dh_steps = pl.dh.steps_per_split;
    const int64_t groups = static_cast<int64_t>(dp.jt) * dp.mt * (dp.h_splits + dp.dh_splits);
    hipLaunchKernelGGL(k_adapter_down, dim3(groups), dim3(kDownThreads), 0, s, dp);
  }
  FinishParams fp{};
  fp.h_part = b.down_part;
  fp.dh_part = b.dh_part;
  fp.Hs = b.Hs;
  fp.dHb = b.dHb;
  fp.M = a.M;
  fp.r = a.r;
  fp.rp = pl.rp;
  fp.h_splits = pl.down.splits;
  fp.dh_splits = pl.dh.splits;
  fp.scale = a.scale;
  fp.absmax_q = a.absmax_q;
  fp.dq_scale = a.dq_scale;
  fp.dq_mean = a.dq_mean;
  fp.cs = b.cs;
  fp.nb = ceil_div(a.N * a.K, kBlock);
  fp.A = A;
  fp.B = B;
  fp.Bb = (lora && !backward) ? b.Bb : nullptr;
  fp.Atb = (lora && backward) ? b.Atb : nullptr;
  fp.N = a.N;
  fp.K = a.K;
  const int64_t sums = lora ? grid_blocks(a.M * pl.rp / 4, 256) : 0;
  fp.g_h = sums;
  fp.g_dh = backward ? sums : 0;
  // without DQ the stored fp32 constants are the block scales themselves
  fp.g_cs = fmt_dq(a.format) ? grid_blocks(ceil_div(fp.nb, kScaleBlocksPerThread), 256) : 0;
  fp.g_op = lora ? grid_blocks((backward ? a.K : a.N) * (pl.rp / 8), 256) : 0;
  const int64_t groups = fp.g_h + fp.g_dh + fp.g_cs + fp.g_op;
  if (groups > 0) hipLaunchKernelGGL(k_adapter_finish, dim3(groups), dim3(256), 0, s, fp);
  return hipGetLastError();
}

}  // namespace

size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K, int r) {
  size_t bytes = 0;
  const Plan pl = make_plan(M, N, K, r);
  carve(nullptr, pl, M, N, K, &bytes);
  // the skinny-M forward reuses the same workspace from its start
  return pl.small ? std::max(bytes, gemv_ws_bytes(M, N, K, r)) : bytes;
}

hipError_t linear_fwd(const LinearArgs &a, const void *X, const float *A, const float *B, void *Y,
                      void *ws, hipStream_t s) {
  const Plan pl = make_plan(a.M, a.N, a.K, a.r);
  if (pl.small) return launch_gemv(a, X, A, B, Y, ws, s);
  const Buffers b = carve(ws, pl, a.M, a.N, a.K, nullptr);
  hipError_t err = run_adapter_pre(a, pl, b, X, nullptr, A, B, false, s);
  if (err != hipSuccess) return err;
  FwdParams fp{X, a.codes, block_scales(a, b), b.Hs, b.Bb, Y, a.M, a.N, a.K, pl.rp};
  dim3 g(grid_blocks(a.N, 256) * grid_blocks(a.M, 256), 1, 1);
  prof_begin(kProfFwdGemm, s);
  hipLaunchKernelGGL(k_fwd_big<CfgBig8>, g, dim3(CfgBig8::kThreads), 0, s, fp, format_tables(a.format));
  prof_end(kProfFwdGemm, s);
  return hipGetLastError();
}

hipError_t linear_bwd(const LinearArgs &a, const void *dY, const void *X, const float *A,
                      const float *B, void *dX, float *dA, float *dB, void *ws, hipStream_t s) {
  const Plan pl = make_plan(a.M, a.N, a.K, a.r);
  const Buffers b = carve(ws, pl, a.M, a.N, a.K, nullptr);
  const Nf4Tables &tab = format_tables(a.format);
  hipError_t err = run_adapter_pre(a, pl, b, X, dY, A, B, true, s);
  if (err != hipSuccess) return err;
  {
    DxParams dp{dY, a.codes, block_scales(a, b), b.dHb, b.Atb, dX, a.M, a.N, a.K, pl.rp};
    dim3 g(grid_blocks(a.K, 256) * grid_blocks(a.M, 256), 1, 1);
    prof_begin(kProfBwdDx, s);
    hipLaunchKernelGGL(k_dx_big<CfgDx>, g, dim3(CfgDx::kThreads), 0, s, dp, tab);
    prof_end(kProfBwdDx, s);
  }
  if (pl.rp > 0) {
    GradParams gp{};
    gp.X = X;
    gp.dY = dY;
    gp.Hs = b.Hs;
    gp.dHb = b.dHb;
    gp.a_part = b.ga_part;
    gp.b_part = b.gb_part;
    gp.M = a.M;
    gp.N = a.N;
    gp.K = a.K;
    gp.rp = pl.rp;
    gp.a_tiles_c = static_cast<int>(grid_blocks(a.K, 256));
    gp.a_tiles = gp.a_tiles_c * (pl.rp / 64);
    gp.a_splits = pl.ga.splits;
    gp.a_steps = pl.ga.steps_per_split;
    gp.b_tiles_c = pl.rp / 64;
    gp.b_tiles = gp.b_tiles_c * static_cast<int>(grid_blocks(a.N, 256));
    gp.b_splits = pl.gb.splits;
    gp.b_steps = pl.gb.steps_per_split;
    const int64_t groups = static_cast<int64_t>(gp.a_tiles) * gp.a_splits +
                           static_cast<int64_t>(gp.b_tiles) * gp.b_splits;
    hipLaunchKernelGGL(k_grad, dim3(groups), dim3(256), 0, s, gp);
    GradFinishParams fp{b.ga_part, b.gb_part, dA, dB, a.N, a.K, a.r, pl.rp, pl.ga.splits, pl.gb.splits};
    const int64_t total = static_cast<int64_t>(a.r) * a.K + a.N * a.r;
    hipLaunchKernelGGL(k_grad_finish, dim3(std::min<int64_t>(grid_blocks(total, 256), 4096)), dim3(256), 0,
                       s, fp);
  }
  return hipGetLastError();
}

}  // namespace qnf4
