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
//   k_block_scales   c_b for every quantization block (fp32, workspace)
//   k_skinny<Down>   partials of H = X A^T over a K split       -> Hs = bf16(s H)
//   k_skinny<DH>     partials of dY B over an N split            -> dHb = bf16(s dY B)
//   k_fwd            Y tile = [X | Hs] [W-hat | Bb]^T: the NF4 weight is decoded
//                    into LDS step by step, the adapter term is 64-deep extra
//                    reduction steps on the same accumulators (fused epilogue)
//   k_bwd_dx         dX tile = [dY | dHb] [W-hat ; At]: the weight decoded
//                    transposed (reduction over out_features)
//   k_grad           split-M partials of dA = dHb^T X and dB = dY^T Hs
//   k_reduce_*       fixed-order sums of the split partials
// Small M (decode) runs k_fwd with a 32-row tile and a K split instead.
#include <algorithm>

#include "gemm_big.h"

namespace qnf4 {
namespace {

// LDS table of level pairs for every code byte: (level[b >> 4], level[b & 15]).
__device__ __forceinline__ void load_level_pairs(float2 *lv2, const Nf4Tables &tab) {
  for (int b = threadIdx.x; b < 256; b += blockDim.x) lv2[b] = make_float2(tab.lv[b >> 4], tab.lv[b & 15]);
}

// ------------------------------------------------------------------ forward

struct FwdParams {
  const void *X;        // bf16 [M, K]
  const uint8_t *codes; // NF4 codes of W [N, K]
  const float *cs;      // per-block scales
  const void *Hs;       // bf16 [M, rp] = bf16(s * X A^T), zero padded
  const void *Bb;       // bf16 [N, rp], zero padded
  void *Y;              // bf16 [M, N] (splits == 1) or fp32 partials [splits][M][N]
  int64_t M, N, K;
  int rp;
  int steps_per_split;  // 64-deep reduction steps per split of K
};

template <class Cfg, bool GUARD>
__device__ __forceinline__ void fwd_tile(const FwdParams &p, const float2 *lv, __bf16 *smem,
                                         int64_t m0, int64_t n0, int z) {
  const int total_steps = static_cast<int>(p.K / kBK);
  const int s0 = z * p.steps_per_split;
  const int steps = min(p.steps_per_split, total_steps - s0);
  Acc<Cfg> acc;
  acc.zero();
  {
    RowBf16<Cfg::BM, Cfg::kThreads, GUARD> la(p.X, p.K, p.M, m0);
    Nf4Row<Cfg::BN, Cfg::kThreads, GUARD> lb(p.codes, p.cs, lv, p.N, p.K, n0);
    mainloop<Cfg>(acc, la, lb, static_cast<int64_t>(s0) * kBK, steps, smem);
  }
  if (z == 0 && p.rp > 0) {
    RowBf16<Cfg::BM, Cfg::kThreads, GUARD> la(p.Hs, p.rp, p.M, m0);
    RowBf16<Cfg::BN, Cfg::kThreads, GUARD> lb(p.Bb, p.rp, p.N, n0);
    mainloop<Cfg>(acc, la, lb, 0, p.rp / kBK, smem);
  }
  if (gridDim.z == 1)
    store_bf16<Cfg, GUARD>(acc, static_cast<__bf16 *>(p.Y), p.N, p.M, p.N, m0, n0, 1.0f);
  else
    store_f32<Cfg>(acc, static_cast<float *>(p.Y) + static_cast<int64_t>(z) * p.M * p.N, p.N, p.M,
                   p.N, m0, n0);
}

// Large-M forward: one 256 x 256 tile of Y per workgroup (XCD-aware order).
__global__ __launch_bounds__(kBigThreads, 1) void k_fwd_big(FwdParams p, Nf4Tables tab) {
  __shared__ __attribute__((aligned(16))) __bf16 sa0[CfgBig::kLdsA], sa1[CfgBig::kLdsA];
  __shared__ __attribute__((aligned(16))) __bf16 sb0[CfgBig::kLdsB], sb1[CfgBig::kLdsB];
  const BigSmem smem{sa0, sa1, sb0, sb1};
  __shared__ float2 lv[256];
  load_level_pairs(lv, tab);
  int tm, tn;
  tile_of(blockIdx.x, static_cast<int>((p.M + 255) / 256), static_cast<int>((p.N + 255) / 256), tm, tn);
  const int64_t n0 = static_cast<int64_t>(tn) * 256;
  const int64_t m0 = static_cast<int64_t>(tm) * 256;
  __syncthreads();
  Acc<CfgBig> acc;
  acc.zero();
  {
    DirectRows da(p.X, p.K, p.M, m0);
    Nf4RowBig l0(p.codes, p.cs, p.N, p.K, n0), l1 = l0;
    auto load = [](Nf4RowBig &l, int s) { l.load(static_cast<int64_t>(s) * kBK); };
    big_mainloop_nf4(acc, da, l0, l1, load, static_cast<int>(p.K / kBK), smem, lv);
  }
  if (p.rp > 0) {
    DirectRows da(p.Hs, p.rp, p.M, m0), db(p.Bb, p.rp, p.N, n0);
    big_mainloop_dense(acc, da, db, p.rp / kBK, smem);
  }
  if (m0 + 256 <= p.M && n0 + 256 <= p.N)
    store_bf16<CfgBig, false>(acc, static_cast<__bf16 *>(p.Y), p.N, p.M, p.N, m0, n0, 1.0f);
  else
    store_bf16<CfgBig, true>(acc, static_cast<__bf16 *>(p.Y), p.N, p.M, p.N, m0, n0, 1.0f);
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::kThreads / 256) void k_fwd(FwdParams p, Nf4Tables tab) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (Cfg::kLdsA + Cfg::kLdsB)];
  __shared__ float2 lv[256];
  load_level_pairs(lv, tab);
  __syncthreads();
  int tm, tn;
  tile_of(blockIdx.x, static_cast<int>((p.M + Cfg::BM - 1) / Cfg::BM),
          static_cast<int>((p.N + Cfg::BN - 1) / Cfg::BN), tm, tn);
  const int64_t n0 = static_cast<int64_t>(tn) * Cfg::BN;
  const int64_t m0 = static_cast<int64_t>(tm) * Cfg::BM;
  if (m0 + Cfg::BM <= p.M && n0 + Cfg::BN <= p.N)
    fwd_tile<Cfg, false>(p, lv, smem, m0, n0, blockIdx.z);
  else
    fwd_tile<Cfg, true>(p, lv, smem, m0, n0, blockIdx.z);
}

// ------------------------------------------------------------- backward dX

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

template <class Cfg, bool GUARD>
__device__ __forceinline__ void dx_tile(const DxParams &p, const float2 *lv, __bf16 *smem,
                                        int64_t m0, int64_t k0) {
  Acc<Cfg> acc;
  acc.zero();
  {
    RowBf16<Cfg::BM, Cfg::kThreads, GUARD> la(p.dY, p.N, p.M, m0);
    Nf4Trans<Cfg::BN, Cfg::kThreads, GUARD> lb(p.codes, p.cs, lv, p.N, p.K, k0);
    mainloop<Cfg>(acc, la, lb, 0, static_cast<int>(p.N / kBK), smem);
  }
  if (p.rp > 0) {
    RowBf16<Cfg::BM, Cfg::kThreads, GUARD> la(p.dHb, p.rp, p.M, m0);
    RowBf16<Cfg::BN, Cfg::kThreads, GUARD> lb(p.Atb, p.rp, p.K, k0);
    mainloop<Cfg>(acc, la, lb, 0, p.rp / kBK, smem);
  }
  store_bf16<Cfg, GUARD>(acc, static_cast<__bf16 *>(p.dX), p.K, p.M, p.K, m0, k0, 1.0f);
}

// Input gradient: one 256 x 256 tile of dX per workgroup (XCD-aware order).
__global__ __launch_bounds__(kBigThreads, 1) void k_dx_big(DxParams p, Nf4Tables tab) {
  __shared__ __attribute__((aligned(16))) __bf16 sa0[CfgBig::kLdsA], sa1[CfgBig::kLdsA];
  __shared__ __attribute__((aligned(16))) __bf16 sb0[CfgBig::kLdsB], sb1[CfgBig::kLdsB];
  const BigSmem smem{sa0, sa1, sb0, sb1};
  __shared__ float2 lv[256];
  load_level_pairs(lv, tab);
  int tm, tn;
  tile_of(blockIdx.x, static_cast<int>((p.M + 255) / 256), static_cast<int>((p.K + 255) / 256), tm, tn);
  const int64_t k0 = static_cast<int64_t>(tn) * 256;
  const int64_t m0 = static_cast<int64_t>(tm) * 256;
  __syncthreads();
  Acc<CfgBig> acc;
  acc.zero();
  {
    DirectRows da(p.dY, p.N, p.M, m0);
    Nf4TransBig l0(p.codes, p.cs, p.K, k0), l1 = l0;
    const int64_t K = p.K;
    auto load = [K](Nf4TransBig &l, int s) { l.load(static_cast<int64_t>(s) * kBK, K); };
    big_mainloop_nf4(acc, da, l0, l1, load, static_cast<int>(p.N / kBK), smem, lv);
  }
  if (p.rp > 0) {
    DirectRows da(p.dHb, p.rp, p.M, m0), db(p.Atb, p.rp, p.K, k0);
    big_mainloop_dense(acc, da, db, p.rp / kBK, smem);
  }
  if (m0 + 256 <= p.M && k0 + 256 <= p.K)
    store_bf16<CfgBig, false>(acc, static_cast<__bf16 *>(p.dX), p.K, p.M, p.K, m0, k0, 1.0f);
  else
    store_bf16<CfgBig, true>(acc, static_cast<__bf16 *>(p.dX), p.K, p.M, p.K, m0, k0, 1.0f);
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::kThreads / 256) void k_bwd_dx(DxParams p, Nf4Tables tab) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (Cfg::kLdsA + Cfg::kLdsB)];
  __shared__ float2 lv[256];
  load_level_pairs(lv, tab);
  __syncthreads();
  int tm, tn;
  tile_of(blockIdx.x, static_cast<int>((p.M + Cfg::BM - 1) / Cfg::BM),
          static_cast<int>((p.K + Cfg::BN - 1) / Cfg::BN), tm, tn);
  const int64_t k0 = static_cast<int64_t>(tn) * Cfg::BN;
  const int64_t m0 = static_cast<int64_t>(tm) * Cfg::BM;
  if (m0 + Cfg::BM <= p.M && k0 + Cfg::BN <= p.K)
    dx_tile<Cfg, false>(p, lv, smem, m0, k0);
  else
    dx_tile<Cfg, true>(p, lv, smem, m0, k0);
}

// ------------------------------------------------- skinny adapter products

enum SkinnyKind { kDown = 0, kDH = 1 };

struct SkinnyParams {
  const void *P;    // bf16 [M, L]: X (L = K) or dY (L = N)
  const float *Q;   // fp32: A [r, K] (kDown) or B [N, r] (kDH)
  float *part;      // fp32 partials [splits][M][rp]
  int64_t M, L;
  int r, rp;
  int steps_per_split;
};

template <class Cfg, int KIND>
__global__ __launch_bounds__(Cfg::kThreads) void k_skinny(SkinnyParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (Cfg::kLdsA + Cfg::kLdsB)];
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * Cfg::BN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * Cfg::BM;
  const int z = blockIdx.z;
  const int total_steps = static_cast<int>(p.L / kBK);
  const int s0 = z * p.steps_per_split;
  const int steps = min(p.steps_per_split, total_steps - s0);
  Acc<Cfg> acc;
  acc.zero();
  RowBf16<Cfg::BM, Cfg::kThreads> la(p.P, p.L, p.M, m0);
  if (KIND == kDown) {
    RowF32<Cfg::BN, Cfg::kThreads> lb(p.Q, p.L, p.r, j0);
    mainloop<Cfg>(acc, la, lb, static_cast<int64_t>(s0) * kBK, steps, smem);
  } else {
    TransF32<Cfg::BN, Cfg::kThreads> lb(p.Q, p.r, p.L, p.r, j0);
    mainloop<Cfg>(acc, la, lb, static_cast<int64_t>(s0) * kBK, steps, smem);
  }
  store_f32<Cfg>(acc, p.part + static_cast<int64_t>(z) * p.M * p.rp, p.rp, p.M, p.rp, m0, j0);
}

// ------------------------------------------------ adapter gradient products

struct GradParams {
  const void *P1;   // bf16 [M, R1]: operand whose columns are the output rows
  const void *P2;   // bf16 [M, R2]: operand whose columns are the output cols
  float *part;      // fp32 partials [splits][R1][R2]
  int64_t M, R1, R2;
  int steps_per_split;
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::kThreads) void k_grad(GradParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (Cfg::kLdsA + Cfg::kLdsB)];
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * Cfg::BN;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * Cfg::BM;
  const int z = blockIdx.z;
  const int total_steps = static_cast<int>((p.M + kBK - 1) / kBK);
  const int s0 = z * p.steps_per_split;
  const int steps = min(p.steps_per_split, total_steps - s0);
  Acc<Cfg> acc;
  acc.zero();
  TransBf16<Cfg::BM, Cfg::kThreads> la(p.P1, p.R1, p.M, p.R1, r0);
  TransBf16<Cfg::BN, Cfg::kThreads> lb(p.P2, p.R2, p.M, p.R2, c0);
  mainloop<Cfg>(acc, la, lb, static_cast<int64_t>(s0) * kBK, steps, smem);
  store_f32<Cfg>(acc, p.part + static_cast<int64_t>(z) * p.R1 * p.R2, p.R2, p.R1, p.R2, r0, c0);
}

// ------------------------------------------------------------ small kernels

// out bf16 [rows][rp] = bf16(alpha * sum_z part[z][rows][rp]) for col < r, 0 beyond.
__global__ void k_reduce_bf16(const float *__restrict__ part, int splits, int64_t rows, int rp,
                              int r, float alpha, __bf16 *__restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = rows * rp;
  if (i >= total) return;
  const int col = static_cast<int>(i % rp);
  float s = 0.0f;
  if (col < r)
    for (int z = 0; z < splits; ++z) s += part[static_cast<int64_t>(z) * total + i];
  out[i] = static_cast<__bf16>(alpha * s);
}

// out fp32 [rows][ldo] = alpha * sum_z part[z * stride + row * ldp + col], col < cols.
__global__ void k_reduce_f32(const float *__restrict__ part, int splits, int64_t stride,
                             int64_t rows, int64_t cols, int64_t ldp, float alpha,
                             float *__restrict__ out, int64_t ldo) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t row = i / cols, col = i % cols;
  float s = 0.0f;
  for (int z = 0; z < splits; ++z) s += part[z * stride + row * ldp + col];
  out[row * ldo + col] = alpha * s;
}

// Y bf16 [M][N] = bf16(sum_z part[z][M][N]).
__global__ void k_reduce_out(const float *__restrict__ part, int splits, int64_t total,
                             __bf16 *__restrict__ Y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  float s = 0.0f;
  for (int z = 0; z < splits; ++z) s += part[z * total + i];
  Y[i] = static_cast<__bf16>(s);
}

// dst bf16 [rows][rp] = bf16(src fp32 [rows][r]), zero padded.
__global__ void k_pad_bf16(const float *__restrict__ src, int64_t rows, int r, int rp,
                           __bf16 *__restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * rp) return;
  const int64_t row = i / rp;
  const int col = static_cast<int>(i % rp);
  dst[i] = static_cast<__bf16>(col < r ? src[row * r + col] : 0.0f);
}

// dst bf16 [K][rp] = bf16(A[j][k]) for j < r, 0 beyond (transpose of A [r][K]).
__global__ void k_transpose_pad_bf16(const float *__restrict__ A, int64_t K, int r, int rp,
                                     __bf16 *__restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= K * rp) return;
  const int64_t k = i / rp;
  const int j = static_cast<int>(i % rp);
  dst[i] = static_cast<__bf16>(j < r ? A[static_cast<int64_t>(j) * K + k] : 0.0f);
}

// ------------------------------------------------------------- tile configs
using CfgDecode = TileCfg<32, 64, 1, 2>;   // M <= 32 forward, split over K
using CfgSkinny = TileCfg<64, 64, 2, 2>;   // adapter down / dH products
using CfgGrad = TileCfg<64, 64, 2, 2>;     // adapter gradients

constexpr int kSmallM = 32;
constexpr int kTargetGroups = 512;

int64_t grid_blocks(int64_t n, int64_t b) { return ceil_div(n, b); }

struct Split {
  int splits;
  int steps_per_split;
};

// Split `steps` reduction steps so that tiles * splits reaches the target.
Split choose_split(int64_t tiles, int steps, int max_splits) {
  int want = static_cast<int>(ceil_div(kTargetGroups, tiles > 0 ? tiles : 1));
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
  Split down, dh, ga, gb, dec;
  bool small;
};

Plan make_plan(int64_t M, int64_t N, int64_t K, int r) {
  Plan pl;
  pl.rp = static_cast<int>(ceil_div(r, kBK) * kBK);
  pl.small = M <= kSmallM;
  const int ksteps = static_cast<int>(K / kBK), nsteps = static_cast<int>(N / kBK);
  const int64_t skinny_tiles = grid_blocks(M, CfgSkinny::BM) * grid_blocks(pl.rp, CfgSkinny::BN);
  pl.down = choose_split(skinny_tiles, ksteps, 64);
  pl.dh = choose_split(skinny_tiles, nsteps, 64);
  const int msteps = static_cast<int>(ceil_div(M, kBK));
  pl.ga = choose_split(grid_blocks(pl.rp, CfgGrad::BM) * grid_blocks(K, CfgGrad::BN), msteps, 16);
  pl.gb = choose_split(grid_blocks(N, CfgGrad::BM) * grid_blocks(pl.rp, CfgGrad::BN), msteps, 16);
  pl.dec = choose_split(grid_blocks(N, CfgDecode::BN), ksteps, 32);
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
  float *y_part;
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
  if (pl.small && pl.dec.splits > 1) b.y_part = c.take<float>(static_cast<size_t>(pl.dec.splits) * M * N);
  if (bytes) *bytes = c.off;
  return b;
}

hipError_t run_down(const LinearArgs &a, const Plan &pl, const Buffers &b, const void *X,
                    const float *A, hipStream_t s) {
  SkinnyParams sp{X, A, b.down_part, a.M, a.K, a.r, pl.rp, pl.down.steps_per_split};
  dim3 g(grid_blocks(pl.rp, CfgSkinny::BN), grid_blocks(a.M, CfgSkinny::BM), pl.down.splits);
  hipLaunchKernelGGL((k_skinny<CfgSkinny, kDown>), g, dim3(CfgSkinny::kThreads), 0, s, sp);
  const int64_t total = a.M * pl.rp;
  hipLaunchKernelGGL(k_reduce_bf16, dim3(grid_blocks(total, 256)), dim3(256), 0, s, b.down_part,
                     pl.down.splits, a.M, pl.rp, a.r, a.scale, b.Hs);
  return hipGetLastError();
}

}  // namespace

size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K, int r) {
  size_t bytes = 0;
  carve(nullptr, make_plan(M, N, K, r), M, N, K, &bytes);
  return bytes;
}

hipError_t linear_fwd(const LinearArgs &a, const void *X, const float *A, const float *B, void *Y,
                      void *ws, hipStream_t s) {
  const Plan pl = make_plan(a.M, a.N, a.K, a.r);
  const Buffers b = carve(ws, pl, a.M, a.N, a.K, nullptr);
  const Nf4Tables &tab = nf4_tables();
  hipError_t err = launch_block_scales(a.absmax_q, a.dq_scale, a.dq_mean, ceil_div(a.N * a.K, kBlock),
                                       b.cs, s);
  if (err != hipSuccess) return err;
  if (pl.rp > 0) {
    err = run_down(a, pl, b, X, A, s);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_pad_bf16, dim3(grid_blocks(a.N * pl.rp, 256)), dim3(256), 0, s, B, a.N, a.r,
                       pl.rp, b.Bb);
  }
  FwdParams fp{X, a.codes, b.cs, b.Hs, b.Bb, Y, a.M, a.N, a.K, pl.rp, 0};
  if (pl.small) {
    fp.steps_per_split = pl.dec.steps_per_split;
    if (pl.dec.splits > 1) fp.Y = b.y_part;
    dim3 g(grid_blocks(a.N, CfgDecode::BN) * grid_blocks(a.M, CfgDecode::BM), 1, pl.dec.splits);
    prof_begin(kProfFwdGemm, s);
    hipLaunchKernelGGL(k_fwd<CfgDecode>, g, dim3(CfgDecode::kThreads), 0, s, fp, tab);
    prof_end(kProfFwdGemm, s);
    if (pl.dec.splits > 1)
      hipLaunchKernelGGL(k_reduce_out, dim3(grid_blocks(a.M * a.N, 256)), dim3(256), 0, s, b.y_part,
                         pl.dec.splits, a.M * a.N, static_cast<__bf16 *>(Y));
  } else {
    fp.steps_per_split = static_cast<int>(a.K / kBK);
    dim3 g(grid_blocks(a.N, 256) * grid_blocks(a.M, 256), 1, 1);
    prof_begin(kProfFwdGemm, s);
    hipLaunchKernelGGL(k_fwd_big, g, dim3(kBigThreads), 0, s, fp, tab);
    prof_end(kProfFwdGemm, s);
  }
  return hipGetLastError();
}

hipError_t linear_bwd(const LinearArgs &a, const void *dY, const void *X, const float *A,
                      const float *B, void *dX, float *dA, float *dB, void *ws, hipStream_t s) {
  const Plan pl = make_plan(a.M, a.N, a.K, a.r);
  const Buffers b = carve(ws, pl, a.M, a.N, a.K, nullptr);
  const Nf4Tables &tab = nf4_tables();
  hipError_t err = launch_block_scales(a.absmax_q, a.dq_scale, a.dq_mean, ceil_div(a.N * a.K, kBlock),
                                       b.cs, s);
  if (err != hipSuccess) return err;
  if (pl.rp > 0) {
    // Hs = bf16(s X A^T)
    err = run_down(a, pl, b, X, A, s);
    if (err != hipSuccess) return err;
    // dHb = bf16(s dY B)
    SkinnyParams sp{dY, B, b.dh_part, a.M, a.N, a.r, pl.rp, pl.dh.steps_per_split};
    dim3 g(grid_blocks(pl.rp, CfgSkinny::BN), grid_blocks(a.M, CfgSkinny::BM), pl.dh.splits);
    hipLaunchKernelGGL((k_skinny<CfgSkinny, kDH>), g, dim3(CfgSkinny::kThreads), 0, s, sp);
    hipLaunchKernelGGL(k_reduce_bf16, dim3(grid_blocks(a.M * pl.rp, 256)), dim3(256), 0, s,
                       b.dh_part, pl.dh.splits, a.M, pl.rp, a.r, a.scale, b.dHb);
    hipLaunchKernelGGL(k_transpose_pad_bf16, dim3(grid_blocks(a.K * pl.rp, 256)), dim3(256), 0, s, A,
                       a.K, a.r, pl.rp, b.Atb);
  }
  {
    DxParams dp{dY, a.codes, b.cs, b.dHb, b.Atb, dX, a.M, a.N, a.K, pl.rp};
    dim3 g(grid_blocks(a.K, 256) * grid_blocks(a.M, 256), 1, 1);
    prof_begin(kProfBwdDx, s);
    hipLaunchKernelGGL(k_dx_big, g, dim3(kBigThreads), 0, s, dp, tab);
    prof_end(kProfBwdDx, s);
  }
  if (pl.rp > 0) {
    // dA [r, K] = dHb^T X
    GradParams gp{b.dHb, X, b.ga_part, a.M, pl.rp, a.K, pl.ga.steps_per_split};
    dim3 g(grid_blocks(a.K, CfgGrad::BN), grid_blocks(pl.rp, CfgGrad::BM), pl.ga.splits);
    hipLaunchKernelGGL(k_grad<CfgGrad>, g, dim3(CfgGrad::kThreads), 0, s, gp);
    hipLaunchKernelGGL(k_reduce_f32, dim3(grid_blocks(static_cast<int64_t>(a.r) * a.K, 256)), dim3(256),
                       0, s, b.ga_part, pl.ga.splits, static_cast<int64_t>(pl.rp) * a.K,
                       static_cast<int64_t>(a.r), a.K, a.K, 1.0f, dA, a.K);
    // dB [N, r] = dY^T Hs   (Hs already carries the factor s)
    GradParams gq{dY, b.Hs, b.gb_part, a.M, a.N, pl.rp, pl.gb.steps_per_split};
    dim3 g2(grid_blocks(pl.rp, CfgGrad::BN), grid_blocks(a.N, CfgGrad::BM), pl.gb.splits);
    hipLaunchKernelGGL(k_grad<CfgGrad>, g2, dim3(CfgGrad::kThreads), 0, s, gq);
    hipLaunchKernelGGL(k_reduce_f32, dim3(grid_blocks(a.N * a.r, 256)), dim3(256), 0, s, b.gb_part,
                       pl.gb.splits, a.N * pl.rp, a.N, static_cast<int64_t>(a.r),
                       static_cast<int64_t>(pl.rp), 1.0f, dB, static_cast<int64_t>(a.r));
  }
  return hipGetLastError();
}

}  // namespace qnf4
