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
//   k_split_out       when the output tiles fill less than half the GPU, the
//                     two GEMMs above split their reduction into fp32 partials
//                     and this sums them in split order into bf16
// Small M (decode, M <= 32) runs the single-launch weight-streaming kernel of
// gemv.hip instead.
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
  float *part;          // fp32 [S][M][N] split partials (S > 1)
  int S, per;           // reduction splits, 64-deep steps per split
};

// Large-M forward: one 256 x 256 tile of Y per workgroup (XCD-aware order),
// run with eight waves (CfgBig8): two waves per SIMD cover each other's
// waits, at 128 x 64 accumulators per wave. With S > 1 the grid holds S
// copies of the tiles, copy z running reduction steps [z per, (z + 1) per)
// and writing its fp32 partial tile (z = 0 adds the adapter steps);
// k_split_out sums them.
template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, 1) void k_fwd_big(FwdParams p, Nf4Tables tab) {
  constexpr int T = Cfg::kThreads;
  __shared__ __attribute__((aligned(16))) __bf16 sa0[Cfg::kLdsA], sa1[Cfg::kLdsA];
  __shared__ __attribute__((aligned(16))) __bf16 sb0[Cfg::kLdsB], sb1[Cfg::kLdsB];
  const BigSmem smem{sa0, sa1, sb0, sb1};
  __shared__ float2 lv_tab[256 * kLvCopies];
  const float2 *lv = load_level_pairs(lv_tab, tab);
  // workgroup -> (reduction split z, output tile)
  const int tiles_m = static_cast<int>((p.M + 255) / 256), tiles_n = static_cast<int>((p.N + 255) / 256);
  const int tiles = tiles_m * tiles_n;
  const int z = static_cast<int>(blockIdx.x) / tiles;
  int tm, tn;
  tile_of(static_cast<int>(blockIdx.x) - z * tiles, tiles_m, tiles_n, tm, tn);
  const int64_t n0 = static_cast<int64_t>(tn) * 256;
  const int64_t m0 = static_cast<int64_t>(tm) * 256;
  const int s0 = z * p.per, s1 = min(static_cast<int>(p.K / kBK), s0 + p.per);
  __syncthreads();
  Acc<Cfg> acc;
  acc.zero();
  {
    DirectRowsT<T> da(static_cast<const __bf16 *>(p.X) + static_cast<int64_t>(s0) * kBK, p.K, p.M, m0);
    Nf4RowBigT<T> l0(p.codes, p.cs, p.N, p.K, n0), l1 = l0;
    auto load = [s0](Nf4RowBigT<T> &l, int s) { l.load(static_cast<int64_t>(s0 + s) * kBK); };
    big_mainloop_nf4<Cfg>(acc, da, l0, l1, load, s1 - s0, smem, lv);
  }
  if (p.rp > 0 && z == 0) {
    DirectRowsT<T> da(p.Hs, p.rp, p.M, m0), db(p.Bb, p.rp, p.N, n0);
    big_mainloop_dense<Cfg>(acc, da, db, p.rp / kBK, smem);
  }
  if (p.S > 1)
    store_f32<Cfg>(acc, p.part + static_cast<int64_t>(z) * p.M * p.N, p.N, p.M, p.N, m0, n0);
  else if (m0 + 256 <= p.M && n0 + 256 <= p.N)
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
  float *part;          // fp32 [S][M][K] split partials (S > 1)
  int S, per;           // reduction splits, 64-deep steps per split
};

// Input gradient: one 256 x 256 tile of dX per workgroup (XCD-aware order),
// run with eight waves as the forward is: the transposed decode gives each
// thread half an 8 x 8 unit (four rows n), which keeps the kernel within the
// registers two waves per SIMD leave. Split reduction (over N) as in the
// forward.
template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, 1) void k_dx_big(DxParams p, Nf4Tables tab) {
  constexpr int T = Cfg::kThreads;
  __shared__ __attribute__((aligned(16))) __bf16 sa0[Cfg::kLdsA], sa1[Cfg::kLdsA];
  __shared__ __attribute__((aligned(16))) __bf16 sb0[Cfg::kLdsB], sb1[Cfg::kLdsB];
  const BigSmem smem{sa0, sa1, sb0, sb1};
  __shared__ float2 lv_tab[256 * kLvCopies];
  const float2 *lv = load_level_pairs(lv_tab, tab);
  // workgroup -> (reduction split z, output tile)
  const int tiles_m = static_cast<int>((p.M + 255) / 256), tiles_k = static_cast<int>((p.K + 255) / 256);
  const int tiles = tiles_m * tiles_k;
  const int z = static_cast<int>(blockIdx.x) / tiles;
  int tm, tn;
  tile_of(static_cast<int>(blockIdx.x) - z * tiles, tiles_m, tiles_k, tm, tn);
  const int64_t k0 = static_cast<int64_t>(tn) * 256;
  const int64_t m0 = static_cast<int64_t>(tm) * 256;
  const int s0 = z * p.per, s1 = min(static_cast<int>(p.N / kBK), s0 + p.per);
  __syncthreads();
  Acc<Cfg> acc;
  acc.zero();
  {
    DirectRowsT<T> da(static_cast<const __bf16 *>(p.dY) + static_cast<int64_t>(s0) * kBK, p.N, p.M, m0);
    Nf4TransBigT<T> l0(p.codes, p.cs, p.K, k0), l1 = l0;
    const int64_t K = p.K;
    auto load = [K, s0](Nf4TransBigT<T> &l, int s) { l.load(static_cast<int64_t>(s0 + s) * kBK, K); };
    big_mainloop_nf4<Cfg>(acc, da, l0, l1, load, s1 - s0, smem, lv);
  }
  if (p.rp > 0 && z == 0) {
    DirectRowsT<T> da(p.dHb, p.rp, p.M, m0), db(p.Atb, p.rp, p.K, k0);
    big_mainloop_dense<Cfg>(acc, da, db, p.rp / kBK, smem);
  }
  if (p.S > 1)
    store_f32<Cfg>(acc, p.part + static_cast<int64_t>(z) * p.M * p.K, p.K, p.M, p.K, m0, k0);
  else if (m0 + 256 <= p.M && k0 + 256 <= p.K)
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

// One workgroup of k_adapter_down: kDownRows = 128 rows of P (X for H, dY
// for G) by the 64 adapter columns j0 .. j0 + 63 of Q (A^T for H, B for G),
// over a range of 64-deep reduction steps. Every global read is a copy
// straight into LDS (no registers), issued kDownAhead steps ahead into a ring
// of kDownAhead + 1 stages; a stage holds
//   the P tile  [128][64] bf16, 128 contiguous bytes a row (16-byte copies),
//               swizzled as the fragment reads expect, and
//   the Q tile  fp32: rows of A as [64 j][64 k], or rows of B as
//               [64 n][64 j] (16-byte copies when r is a multiple of 4, else
//               one 4-byte copy a lane and 256 bytes a row of B, whose rows
//               of r floats are then not 16-byte aligned).
// All four waves copy both tiles, so each wave's count of copies in flight
// covers the whole stage and one wait per step suffices. After a stage
// landed, the waves round its Q tile to the bf16 operand [64 j][64 k]
// (swizzled; columns j >= r zero) and each wave runs the MFMAs of its 32 rows.
constexpr int kDownWaves = 4;
constexpr int kDownRows = 128;
constexpr int kDownThreads = 64 * kDownWaves;
constexpr int kDownPBytes = kDownRows * kBK * 2;   // 16 KB
constexpr int kDownQBytes = 64 * kBK * 4;          // 16 KB
constexpr int kDownStageBytes = kDownPBytes + kDownQBytes;
constexpr int kDownQbBytes = 64 * kBK * 2;         // 8 KB
constexpr int kDownAhead = 3;                      // 96 KB in flight per workgroup
constexpr size_t kDownLds = static_cast<size_t>(kDownAhead + 1) * kDownStageBytes + kDownQbBytes;

using DownRows = DirectRowsT<kDownThreads, kDownRows>;   // 4 blocks of 1 KB per wave and step

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char *)p)));
}

// This wave's index, known to the compiler as wave-uniform (scalar).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)); }

__device__ __forceinline__ void copy16(uint32_t dst, uint32_t off, const void *src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(dst), "v"(off), "s"(src) : "memory", "m0");
}
__device__ __forceinline__ void copy4(uint32_t dst, uint32_t off, const void *src) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" : : "s"(dst), "v"(off), "s"(src) : "memory", "m0");
}

// A Q tile of 64 fp32 rows of 64 floats, row q of the tile at `row_ptr(q)`
// plus column offset `col` (floats): 16 blocks of 1 KB (4 rows each); wave w
// copies blocks w + 4 i, lane L of a block fetching row 4 b + L / 16,
// floats 4 (L % 16) .. + 3, which land at byte 16 L of the block, so the
// stage is row-major [64][64].
//   H (QRowsA): row q = row j0 + q of A [r][K] (rows >= r read row r - 1),
//               columns from the step's k0;
//   G (QColsB): row q = row n0 + q of B [N][r], columns j0 .. j0 + 63
//               (columns past r read the row's last aligned four; they are
//               dropped by the rounding), or with r % 4 != 0 one 4-byte copy
//               per row, lane j fetching column min(j0 + j, r - 1).
struct QRowsA {
  static constexpr int kCopies = 4;   // per wave and step
  const float *A;
  int64_t K;
  int brow[kCopies];        // first (clamped) row of each block: wave-uniform
  uint32_t off[kCopies];    // this lane's byte offset from that row
  __device__ QRowsA(const float *A_, int64_t K_, int r, int j0) : A(A_), K(K_) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int b = w + 4 * i;
      const int r0 = min(j0 + 4 * b, r - 1), rl = min(j0 + 4 * b + lane / 16, r - 1);
      brow[i] = __builtin_amdgcn_readfirstlane(r0);
      off[i] = static_cast<uint32_t>(static_cast<int64_t>(rl - r0) * K * 4 + 16 * (lane % 16));
    }
  }
  __device__ __forceinline__ int copies() const { return kCopies; }
  __device__ __forceinline__ void issue(int64_t k0, float *stage) const {
    const uint32_t dst0 = lds_addr(stage) + static_cast<uint32_t>(wave_id()) * 1024u;
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy16(dst0 + i * 4096u, off[i], A + static_cast<int64_t>(brow[i]) * K + k0);
  }
  // Stage [64 j][64 k] fp32 -> operand rows j: units (j, chunk c) of 8 floats.
  __device__ __forceinline__ static void convert(const float *st, __bf16 *qb, int r, int j0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = threadIdx.x + kDownThreads * u, j = idx >> 3, c = idx & 7;
      const float4 a = *reinterpret_cast<const float4 *>(st + j * 64 + 8 * c);
      const float4 b = *reinterpret_cast<const float4 *>(st + j * 64 + 8 * c + 4);
      const bool ok = j0 + j < r;
      *reinterpret_cast<uint4 *>(qb + lds_off(j, c)) =
          ok ? make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w))
             : make_uint4(0u, 0u, 0u, 0u);
    }
  }
};

struct QColsB {
  const float *B;
  int r;
  bool wide;         // r % 4 == 0: 16-byte copies
  uint32_t off;      // wide: row (lane / 16) and column; else column only
  __device__ QColsB(const float *B_, int r_, int j0) : B(B_), r(r_), wide(r_ % 4 == 0) {
    const int lane = threadIdx.x & 63;
    if (wide)
      off = static_cast<uint32_t>(((lane / 16) * r_ + min(j0 + 4 * (lane % 16), r_ - 4)) * 4);
    else
      off = static_cast<uint32_t>(4 * min(j0 + lane, r_ - 1));
  }
  __device__ __forceinline__ int copies() const { return wide ? 4 : 16; }
  __device__ __forceinline__ void issue(int64_t n0, float *stage) const {
    const int w = wave_id();
    const uint32_t dst0 = lds_addr(stage);
    if (wide) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = w + 4 * i;   // rows 4 b .. 4 b + 3
        copy16(dst0 + b * 1024u, off, B + (n0 + 4 * b) * r);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int n = w + 4 * i;
        copy4(dst0 + n * 256u, off, B + (n0 + n) * r);
      }
    }
  }
  // Stage [64 n][64 j] fp32 -> operand rows j: chunk c of row j holds
  // n = 8 c .. 8 c + 7 of column j.
  __device__ __forceinline__ static void convert(const float *st, __bf16 *qb, int r, int j0) {
    const int j = threadIdx.x & 63;
    const bool ok = j0 + j < r;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = (threadIdx.x >> 6) + 4 * u;
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = st[(8 * c + i) * 64 + j];
      *reinterpret_cast<uint4 *>(qb + lds_off(j, c)) =
          ok ? make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7]))
             : make_uint4(0u, 0u, 0u, 0u);
    }
  }
};

// Wait until at most `k` copies of this wave are in flight; k is a multiple
// of the copies per step (8 or 20) below kDownAhead steps' worth.
__device__ __forceinline__ void wait_down_copies(int k) {
  switch (k) {
    case 8: DownRows::wait_copies<8>(); break;
    case 16: DownRows::wait_copies<16>(); break;
    case 20: DownRows::wait_copies<20>(); break;
    case 40: DownRows::wait_copies<40>(); break;
    default: DownRows::wait_copies<0>(); break;
  }
}

template <class QL>
__device__ __forceinline__ void down_tile(const void *P, int64_t L, int64_t M, const QL &ql, int r, int j0,
                                          int64_t m0, int s0, int n, float *part, int rp, char *smem) {
  static_assert(kDownAhead == 3, "wait_down_copies covers two steps in flight");
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  constexpr int kRing = kDownAhead + 1;
  __bf16 *qb = reinterpret_cast<__bf16 *>(smem + kRing * kDownStageBytes);
  auto ptile = [&](int st) { return reinterpret_cast<__bf16 *>(smem + st * kDownStageBytes); };
  auto qtile = [&](int st) { return reinterpret_cast<float *>(smem + st * kDownStageBytes + kDownPBytes); };
  const DownRows pr(P, L, M, m0);
  const int64_t k0 = static_cast<int64_t>(s0) * kBK;
  const int per_step = DownRows::kPerWave + ql.copies();
  for (int i = 0; i < min(kDownAhead, n); ++i) {
    pr.issue(k0 + i * kBK, ptile(i));
    ql.issue(k0 + i * kBK, qtile(i));
  }
  // fragment offsets of this wave's 32 rows and of the Q operand rows
  int fa[4], fb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    fa[kk] = lds_off(32 * w + (lane & 31), 2 * kk + (lane >> 5));
    fb[kk] = lds_off(lane & 31, 2 * kk + (lane >> 5));
  }
  f32x16 acc[2];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jb][v] = 0.0f;
  for (int s = 0; s < n; ++s) {
    wait_down_copies(min(kDownAhead - 1, n - 1 - s) * per_step);
    __syncthreads();   // stage s landed; every wave is done with step s - 1
    if (s + kDownAhead < n) {
      const int st = (s + kDownAhead) % kRing;
      pr.issue(k0 + (s + kDownAhead) * kBK, ptile(st));
      ql.issue(k0 + (s + kDownAhead) * kBK, qtile(st));
    }
    QL::convert(qtile(s % kRing), qb, r, j0);
    __syncthreads();
    const __bf16 *pt = ptile(s % kRing);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(pt + fa[kk]);
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const bf16x8 b = *reinterpret_cast<const bf16x8 *>(qb + fb[kk] + jb * 32 * kLDK);
        acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[jb], 0, 0, 0);
      }
    }
  }
  const int h = lane >> 5;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int64_t col = j0 + jb * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + 32 * w + 8 * (v >> 2) + 4 * h + (v & 3);
      if (row < M) part[row * rp + col] = acc[jb][v];
    }
  }
}

__global__ __launch_bounds__(kDownThreads, 1) void k_adapter_down(DownParams p) {
  extern __shared__ __attribute__((aligned(16))) char down_smem[];
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
    const QRowsA ql(p.A, p.K, p.r, j0);
    down_tile(p.X, L, p.M, ql, p.r, j0, m0, s0, steps, p.h_part + static_cast<int64_t>(z) * p.M * p.rp, p.rp,
              down_smem);
  } else {
    const QColsB ql(p.B, p.r, j0);
    down_tile(p.dY, L, p.M, ql, p.r, j0, m0, s0, steps, p.dh_part + static_cast<int64_t>(z) * p.M * p.rp, p.rp,
              down_smem);
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

// Split reduction of the large-tile GEMMs when few output tiles would leave
// most of the GPU idle: out = bf16(sum of the S fp32 partials, in split
// order), four elements per thread.
__global__ __launch_bounds__(256) void k_split_out(const float *part, int S, int64_t plane, __bf16 *out) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e >= plane) return;
  const float4 v = split_sum4(part, plane, e, S);
  *reinterpret_cast<uint2 *>(out + e) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

// dst[m][j] = src[m][j] for j < ncopy, 0 for ncopy <= j < ndst (the saved
// adapter activations between the caller's [M][r] and the kernels' [M][rp]).
__global__ __launch_bounds__(256) void k_cols_copy(const __bf16 *src, int64_t sld, __bf16 *dst, int64_t dld,
                                                   int64_t M, int ncopy, int ndst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= M * ndst) return;
  const int64_t m = i / ndst;
  const int j = static_cast<int>(i - m * ndst);
  dst[m * dld + j] = j < ncopy ? src[m * sld + j] : static_cast<__bf16>(0.0f);
}

hipError_t cols_copy(const __bf16 *src, int64_t sld, __bf16 *dst, int64_t dld, int64_t M, int ncopy, int ndst,
                     hipStream_t s) {
  hipLaunchKernelGGL(k_cols_copy, dim3(static_cast<unsigned>(ceil_div(M * ndst, static_cast<int64_t>(256)))),
                     dim3(256), 0, s, src, sld, dst, dld, M, ncopy, ndst);
  return hipGetLastError();
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
  Split down, hb, dh, ga, gb;   // forward H; backward H and dY B; dA; dB
  Split dhs;                    // backward dY B alone (H saved by the forward)
  Split fs, xs;                 // reduction splits of the forward and dX GEMMs
  bool small;
};

constexpr int kCus = 256;                             // compute units of the GPU
constexpr int kMinSplitSteps = 4;                     // 64-deep steps per split at least
constexpr size_t kSplitPartMax = size_t(128) << 20;   // bytes of fp32 partials at most

// Reduction splits of a large-tile GEMM with `tiles` 256 x 256 output tiles
// of an M x cols output over `steps` 64-deep steps: none while the tiles fill
// half the GPU or more; otherwise as many as keep every workgroup in one
// round on the compute units, each split at least kMinSplitSteps long.
Split gemm_split(int64_t tiles, int steps, int64_t M, int64_t cols, bool allow) {
  int S = 1;
  if (allow && tiles * 2 <= kCus) {
    S = static_cast<int>(std::min<int64_t>(kCus / tiles, steps / kMinSplitSteps));
    while (S > 1 && static_cast<size_t>(S) * M * cols * sizeof(float) > kSplitPartMax) --S;
    S = std::max(S, 1);
  }
  const int per = static_cast<int>(ceil_div(steps, S));
  return {static_cast<int>(ceil_div(steps, per)), per};
}

Plan make_plan(int64_t M, int64_t N, int64_t K, int r, bool allow_split = true) {
  Plan pl;
  pl.rp = static_cast<int>(ceil_div(r, kBK) * kBK);
  pl.small = M <= kSmallM && gemv_sync_fits(M, N, K, r);
  const int ksteps = static_cast<int>(K / kBK), nsteps = static_cast<int>(N / kBK);
  const int64_t skinny_tiles = grid_blocks(M, kDownRows) * grid_blocks(pl.rp, 64);
  // one down-projection workgroup per CU (its LDS ring takes most of a CU):
  // the forward's H fills the GPU alone, the backward shares it with dY B
  pl.down = choose_split(skinny_tiles, ksteps, 64, kDownGroups);
  pl.hb = choose_split(skinny_tiles, ksteps, 64, kDownGroups / 2);
  pl.dh = choose_split(skinny_tiles, nsteps, 64, kDownGroups / 2);
  pl.dhs = choose_split(skinny_tiles, nsteps, 64, kDownGroups);
  const int msteps = static_cast<int>(ceil_div(M, kBK));
  pl.ga = choose_split(grid_blocks(pl.rp, 64) * grid_blocks(K, 256), msteps, 8);
  pl.gb = choose_split(grid_blocks(N, 256) * grid_blocks(pl.rp, 64), msteps, 8);
  pl.fs = gemm_split(grid_blocks(M, 256) * grid_blocks(N, 256), ksteps, M, N, allow_split);
  pl.xs = gemm_split(grid_blocks(M, 256) * grid_blocks(K, 256), nsteps, M, K, allow_split);
  return pl;
}

struct Buffers {
  float *part;   // split partials of the large-tile GEMMs
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
  // the sync words at the start of the workspace belong to the skinny-M path
  Carve c{static_cast<char *>(ws), kLinearSyncBytes};
  Buffers b{};
  const int64_t nb = ceil_div(N * K, kBlock);
  const int rp = pl.rp;
  b.cs = c.take<float>(nb);
  const size_t part = std::max(pl.fs.splits > 1 ? static_cast<size_t>(pl.fs.splits) * M * N : 0,
                               pl.xs.splits > 1 ? static_cast<size_t>(pl.xs.splits) * M * K : 0);
  b.part = part ? c.take<float>(part) : nullptr;
  if (rp > 0) {
    b.down_part = c.take<float>(static_cast<size_t>(std::max(pl.down.splits, pl.hb.splits)) * M * rp);
    b.Hs = c.take<__bf16>(static_cast<size_t>(M) * rp);
    b.Bb = c.take<__bf16>(static_cast<size_t>(N) * rp);
    b.dh_part = c.take<float>(static_cast<size_t>(std::max(pl.dh.splits, pl.dhs.splits)) * M * rp);
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
// With h_given (backward only) the forward's bf16(s H) is supplied by the
// caller: no H partials or sums, and dY B takes every down-projection
// workgroup.
hipError_t run_adapter_pre(const LinearArgs &a, const Plan &pl, const Buffers &b, const void *X,
                           const void *dY, const float *A, const float *B, bool backward, hipStream_t s,
                           bool h_given = false) {
  const bool skip_h = backward && h_given;
  const Split &dhp = skip_h ? pl.dhs : pl.dh;
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
    const Split &hs = backward ? pl.hb : pl.down;
    dp.h_splits = skip_h ? 0 : hs.splits;
    dp.h_steps = hs.steps_per_split;
    dp.dh_splits = backward ? dhp.splits : 0;
    dp.dh_steps = dhp.steps_per_split;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(k_adapter_down),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       static_cast<int>(kDownLds));
    if (attr != hipSuccess) return attr;
    const int64_t groups = static_cast<int64_t>(dp.jt) * dp.mt * (dp.h_splits + dp.dh_splits);
    hipLaunchKernelGGL(k_adapter_down, dim3(groups), dim3(kDownThreads), kDownLds, s, dp);
  }
  FinishParams fp{};
  fp.h_part = b.down_part;
  fp.dh_part = b.dh_part;
  fp.Hs = b.Hs;
  fp.dHb = b.dHb;
  fp.M = a.M;
  fp.r = a.r;
  fp.rp = pl.rp;
  fp.h_splits = backward ? pl.hb.splits : pl.down.splits;
  fp.dh_splits = dhp.splits;
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
  fp.g_h = skip_h ? 0 : sums;
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

size_t linear_fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int r, bool allow_split) {
  const Plan pl = make_plan(M, N, K, r, allow_split);
  if (pl.small) return gemv_ws_bytes(M, N, K, r);
  size_t bytes = 0;
  carve(nullptr, pl, M, N, K, &bytes);
  return bytes;
}

hipError_t linear_fwd(const LinearArgs &a, const void *X, const float *A, const float *B, void *Y,
                      void *ws, hipStream_t s, bool allow_split, void *hs_out) {
  const Plan pl = make_plan(a.M, a.N, a.K, a.r, allow_split);
  const bool save = hs_out != nullptr && pl.rp > 0;
  if (pl.small) {
    hipError_t err = launch_gemv(a, X, A, B, Y, ws, s);
    if (err != hipSuccess || !save) return err;
    // the decode kernel forms H inside; the saved activations come from the
    // down-projection kernels, after it (they reuse its workspace)
    const Buffers b = carve(ws, pl, a.M, a.N, a.K, nullptr);
    err = run_adapter_pre(a, pl, b, X, nullptr, A, B, false, s);
    if (err != hipSuccess) return err;
    return cols_copy(b.Hs, pl.rp, static_cast<__bf16 *>(hs_out), a.r, a.M, a.r, a.r, s);
  }
  Buffers b = carve(ws, pl, a.M, a.N, a.K, nullptr);
  // with r a multiple of 64 the caller's [M][r] is the kernels' [M][rp]
  const bool direct = save && a.r == pl.rp;
  if (direct) b.Hs = static_cast<__bf16 *>(hs_out);
  hipError_t err = run_adapter_pre(a, pl, b, X, nullptr, A, B, false, s);
  if (err != hipSuccess) return err;
  if (save && !direct) {
    err = cols_copy(b.Hs, pl.rp, static_cast<__bf16 *>(hs_out), a.r, a.M, a.r, a.r, s);
    if (err != hipSuccess) return err;
  }
  FwdParams fp{X, a.codes, block_scales(a, b), b.Hs, b.Bb, Y, a.M, a.N, a.K, pl.rp, b.part, pl.fs.splits,
               pl.fs.steps_per_split};
  dim3 g(grid_blocks(a.N, 256) * grid_blocks(a.M, 256) * pl.fs.splits, 1, 1);
  prof_begin(kProfFwdGemm, s);
  hipLaunchKernelGGL(k_fwd_big<CfgBig8>, g, dim3(CfgBig8::kThreads), 0, s, fp, format_tables(a.format));
  prof_end(kProfFwdGemm, s);
  if (pl.fs.splits > 1) {
    const int64_t plane = a.M * a.N;
    hipLaunchKernelGGL(k_split_out, dim3(grid_blocks(plane / 4, 256)), dim3(256), 0, s, b.part, pl.fs.splits,
                       plane, static_cast<__bf16 *>(Y));
  }
  return hipGetLastError();
}

hipError_t linear_bwd(const LinearArgs &a, const void *dY, const void *X, const float *A,
                      const float *B, void *dX, float *dA, float *dB, void *ws, hipStream_t s,
                      const void *hs_in) {
  const Plan pl = make_plan(a.M, a.N, a.K, a.r);
  Buffers b = carve(ws, pl, a.M, a.N, a.K, nullptr);
  const Nf4Tables &tab = format_tables(a.format);
  const bool given = hs_in != nullptr && pl.rp > 0;
  hipError_t err = run_adapter_pre(a, pl, b, X, dY, A, B, true, s, given);
  if (err != hipSuccess) return err;
  if (given) {   // the forward's bf16(s H): used in place, or padded to rp columns
    if (a.r == pl.rp) {
      b.Hs = const_cast<__bf16 *>(static_cast<const __bf16 *>(hs_in));
    } else {
      err = cols_copy(static_cast<const __bf16 *>(hs_in), a.r, b.Hs, pl.rp, a.M, a.r, pl.rp, s);
      if (err != hipSuccess) return err;
    }
  }
  {
    DxParams dp{dY, a.codes, block_scales(a, b), b.dHb, b.Atb, dX, a.M, a.N, a.K, pl.rp, b.part, pl.xs.splits,
                pl.xs.steps_per_split};
    dim3 g(grid_blocks(a.K, 256) * grid_blocks(a.M, 256) * pl.xs.splits, 1, 1);
    prof_begin(kProfBwdDx, s);
    hipLaunchKernelGGL(k_dx_big<CfgDx>, g, dim3(CfgDx::kThreads), 0, s, dp, tab);
    prof_end(kProfBwdDx, s);
    if (pl.xs.splits > 1) {
      const int64_t plane = a.M * a.K;
      hipLaunchKernelGGL(k_split_out, dim3(grid_blocks(plane / 4, 256)), dim3(256), 0, s, b.part, pl.xs.splits,
                         plane, static_cast<__bf16 *>(dX));
    }
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
