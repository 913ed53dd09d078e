// MFMA tile engine and operand loaders shared by the QLoRA linear kernels.
//
// Every product of the layer is written as
//     C[i, j] = sum_t  P[i, t] * Q[j, t]
// with both operands staged in LDS as bf16 tiles whose reduction index t is
// contiguous ("row = output index, 64 reduction elements per row"), which is
// the operand layout of v_mfma_f32_32x32x16_bf16: lane l supplies 8
// consecutive reduction elements of row (l % 32), at offset 8 * (l / 32) of a
// 16-element slice; the 32x32 fp32 result lands in 16 registers per lane,
// register v holding row 8*(v/4) + 4*(l/32) + (v%4), column l % 32.
//
// LDS layout: a tile row is 64 bf16 = 128 bytes = eight 16-byte chunks, with
// no padding; logical chunk c of row r is stored at chunk c ^ swz(r),
// swz(r) = (r & 7) ^ ((r >> 3) & 3). The swizzle depends only on r mod 32, so
// the fragment reads of one wave (rows 32i + l, i = 0..3) differ by immediate
// offsets. Eight consecutive rows read at one logical chunk (a fragment read),
// a row written chunk by chunk, and the transposed 8x8 stores (see
// TransUnits) all land on eight distinct chunk slots per group of eight lanes,
// so none of them serializes on LDS banks.
//
#pragma once

#include "internal.h"

namespace qnf4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;   // reduction elements per pipeline step
constexpr int kLDK = 64;  // LDS row length in bf16 (swizzled, unpadded)

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 3); }
// Offset (in bf16 elements) of logical 16-byte chunk `chunk` of tile row `row`.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kLDK + ((chunk ^ swz(row)) << 3);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// Low / high 16-bit halves of two words combined: (a.lo, b.lo) and (a.hi, b.hi).
__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int kLdsA = BM * kLDK, kLdsB = BN * kLDK;  // bf16 per buffer
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
};

template <class Cfg>
struct Acc {
  f32x16 v[Cfg::TM][Cfg::TN];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) v[i][j][e] = 0.0f;
  }
};

// Per-lane LDS offsets (bf16 elements) of the four 16-deep fragment slices of
// a wave's first fragment row; fragment i adds 32 * 64 * i (an immediate).
template <int WT>
struct FragAddr {
  int off[4];
  __device__ FragAddr(int row0, int lane) {
    const int r = lane & 31, half = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) off[kk] = lds_off(row0 + r, 2 * kk + half);
  }
};

// One 64-deep step of MFMAs from the LDS tiles sA [BM][64], sB [BN][64].
template <class Cfg>
__device__ __forceinline__ void mma_step(Acc<Cfg> &acc, const __bf16 *sA, const __bf16 *sB,
                                         const FragAddr<Cfg::WTM> &fa, const FragAddr<Cfg::WTN> &fb) {
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    bf16x8 a[Cfg::TM], b[Cfg::TN];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
      a[i] = *reinterpret_cast<const bf16x8 *>(sA + fa.off[kk] + i * 32 * kLDK);
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
      b[j] = *reinterpret_cast<const bf16x8 *>(sB + fb.off[kk] + j * 32 * kLDK);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.v[i][j], 0, 0, 0);
  }
}

// Main loop with two register stages: while step s runs on the MFMAs, the
// global reads of steps s + 1 and s + 2 are in flight (loaders la0 / lb0 and
// la1 / lb1 alternate). The loop runs an even number of steps with no
// branches inside; the loaders must read rows at or past red0 + 64 steps as
// zero (their reduction bound), so the steps past the end add nothing. smem
// holds the double-buffered tiles [A0 | A1 | B0 | B1]. On entry the caller has
// synchronized (LDS free); on exit every LDS read is complete.
template <class Cfg, class LA, class LB>
__device__ __forceinline__ void mainloop2(Acc<Cfg> &acc, LA &la0, LA &la1, LB &lb0, LB &lb1, int64_t red0,
                                          int steps, __bf16 *smem) {
  if (steps <= 0) return;
  __bf16 *sA0 = smem, *sA1 = smem + Cfg::kLdsA;
  __bf16 *sB0 = smem + 2 * Cfg::kLdsA, *sB1 = sB0 + Cfg::kLdsB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
  const FragAddr<Cfg::WTM> fa(wm * Cfg::WTM, lane);
  const FragAddr<Cfg::WTN> fb(wn * Cfg::WTN, lane);
  auto red = [&](int s) { return red0 + static_cast<int64_t>(s) * kBK; };
  la0.load(red(0));
  lb0.load(red(0));
  la1.load(red(1));
  lb1.load(red(1));
  la0.store(sA0);
  lb0.store(sB0);
  __syncthreads();
  for (int s = 0; s < steps; s += 2) {
    // buffer 0: step s; stage 1: step s + 1 in flight
    la0.load(red(s + 2));
    lb0.load(red(s + 2));
    mma_step<Cfg>(acc, sA0, sB0, fa, fb);
    la1.store(sA1);
    lb1.store(sB1);
    __syncthreads();
    // buffer 1: step s + 1; stage 0: step s + 2 in flight
    la1.load(red(s + 3));
    lb1.load(red(s + 3));
    mma_step<Cfg>(acc, sA1, sB1, fa, fb);
    la0.store(sA0);
    lb0.store(sB0);
    __syncthreads();
  }
}

// ----------------------------------------------------------------- loaders
// Each loader covers ROWS output rows of one operand and a 64-deep reduction
// step. load() issues the global reads into registers, store() writes the
// LDS tile [ROWS][64].

// Units of the transposed loaders: 8 reduction rows x 8 output rows. For a
// tile of ROWS output rows there are UPR = ROWS / 8 column groups cc and 8
// reduction-row groups rg per 64-deep step. A unit is written as eight 16-byte
// LDS stores (output rows 8 cc + j, logical chunk rg). Thread t takes cc from
// bits 0-1 and 3.. of t and rg from bit 2 and the bits above, so each group of
// eight lanes holds four consecutive cc and two rg four apart: with the
// swizzle above, its eight stores hit eight distinct chunk slots.
template <int ROWS, int T>
struct TransUnits {
  static constexpr int UPR = ROWS / 8;
  static constexpr int UNITS = UPR * 8;
  static constexpr int CH = (UNITS + T - 1) / T;
  static constexpr int kHiBits = (UPR == 4) ? 0 : (UPR == 8) ? 1 : (UPR == 16) ? 2 : (UPR == 32) ? 3 : 4;
  static_assert(UPR >= 4 && UPR <= 64 && (UPR & (UPR - 1)) == 0, "unsupported tile height");
  __device__ static bool active(int idx) { return UNITS % T == 0 || idx < UNITS; }
  __device__ static int cc(int idx) { return (idx & 3) | (((idx >> 3) & (UPR / 4 - 1)) << 2); }
  __device__ static int rg(int idx) { return (((idx >> 2) & 1) << 2) | ((idx >> (3 + kHiBits)) & 3); }
};

// Transposed bf16 source S[t][col] (reduction along the source's rows, cols
// contiguous, ld and ncols multiples of 8): output row = col. Reduction rows
// >= nred and columns >= ncols read as 0.
template <int ROWS, int T>
struct TransBf16 {
  using U = TransUnits<ROWS, T>;
  const __bf16 *src;
  int64_t ld, nred, ncols, col0;
  int64_t red_in = 0;   // red0 of the registers' contents
  uint4 reg[U::CH][8];
  __device__ TransBf16(const void *s, int64_t ld_, int64_t nred_, int64_t ncols_, int64_t col0_)
      : src(static_cast<const __bf16 *>(s)), ld(ld_), nred(nred_), ncols(ncols_), col0(col0_) {}
  // Out-of-range elements: a clamped (valid) address is read here and the
  // value replaced by 0 in store(), so the loads need no branches and nothing
  // waits for them before the store.
  __device__ __forceinline__ void load(int64_t red0) {
    red_in = red0;
#pragma unroll
    for (int u = 0; u < U::CH; ++u) {
      const int idx = threadIdx.x + u * T;
      if (!U::active(idx)) continue;
      const int cc = U::cc(idx), rg = U::rg(idx);
      const int64_t cl = min(col0 + cc * 8, ncols - 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t t = red0 + rg * 8 + i;
        reg[u][i] = *reinterpret_cast<const uint4 *>(src + min(t, nred - 1) * ld + cl);
      }
    }
  }
  __device__ __forceinline__ void store(__bf16 *lds) const {
#pragma unroll
    for (int u = 0; u < U::CH; ++u) {
      const int idx = threadIdx.x + u * T;
      if (!U::active(idx)) continue;
      const int cc = U::cc(idx), rg = U::rg(idx);
      const bool col_ok = col0 + cc * 8 < ncols;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 &v = reg[u][i];
          const bool ok = col_ok && red_in + rg * 8 + i < nred;
          w[i] = ok ? (q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w) : 0u;
        }
        // output rows 2q (low halves) and 2q+1 (high halves), 8 reduction values each
        uint4 even = make_uint4(lo16x2(w[0], w[1]), lo16x2(w[2], w[3]), lo16x2(w[4], w[5]),
                                lo16x2(w[6], w[7]));
        uint4 odd = make_uint4(hi16x2(w[0], w[1]), hi16x2(w[2], w[3]), hi16x2(w[4], w[5]),
                               hi16x2(w[6], w[7]));
        *reinterpret_cast<uint4 *>(lds + lds_off(cc * 8 + 2 * q, rg)) = even;
        *reinterpret_cast<uint4 *>(lds + lds_off(cc * 8 + 2 * q + 1, rg)) = odd;
      }
    }
  }
};

// Transposed bf16 source S[t][col] for small tiles (UNITS = 4 ROWS a multiple
// of T): units of 8 reduction rows x 2 output rows, one 4-byte load per
// reduction row, so every thread has whole units and the loads need no
// branches. ncols (the source's column count) is even; reduction rows >= nred
// read as 0 (a clamped, valid row is loaded and replaced in store()).
template <int ROWS, int T>
struct TransBf16Narrow {
  static constexpr int UPR = ROWS / 2;          // column pairs
  static constexpr int UNITS = UPR * 8;         // x 8 reduction-row groups
  static constexpr int CH = UNITS / T;
  static_assert(UNITS % T == 0, "whole units per thread");
  const __bf16 *src;
  int64_t ld, nred, col0;
  int64_t red_in = 0;   // red0 of the registers' contents
  uint32_t reg[CH][8];
  __device__ TransBf16Narrow(const void *s, int64_t ld_, int64_t nred_, int64_t col0_)
      : src(static_cast<const __bf16 *>(s)), ld(ld_), nred(nred_), col0(col0_) {}
  __device__ __forceinline__ void load(int64_t red0) {
    red_in = red0;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = threadIdx.x + u * T;
      const int cp = idx % UPR, rg = idx / UPR;
      const int64_t c = col0 + 2 * cp;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t t = red0 + rg * 8 + i;
        reg[u][i] = *reinterpret_cast<const uint32_t *>(src + min(t, nred - 1) * ld + c);
      }
    }
  }
  __device__ __forceinline__ void store(__bf16 *lds) const {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = threadIdx.x + u * T;
      const int cp = idx % UPR, rg = idx / UPR;
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = red_in + rg * 8 + i < nred ? reg[u][i] : 0u;
      const uint4 lo = make_uint4(lo16x2(w[0], w[1]), lo16x2(w[2], w[3]), lo16x2(w[4], w[5]), lo16x2(w[6], w[7]));
      const uint4 hi = make_uint4(hi16x2(w[0], w[1]), hi16x2(w[2], w[3]), hi16x2(w[4], w[5]), hi16x2(w[6], w[7]));
      *reinterpret_cast<uint4 *>(lds + lds_off(2 * cp, rg)) = lo;
      *reinterpret_cast<uint4 *>(lds + lds_off(2 * cp + 1, rg)) = hi;
    }
  }
};

// bf16 C[row][col] = bf16(alpha * acc), rows < nrows, cols < ncols (checked
// only when GUARD).
template <class Cfg, bool GUARD = true>
__device__ __forceinline__ void store_bf16(const Acc<Cfg> &acc, __bf16 *C, int64_t ldc, int64_t nrows,
                                           int64_t ncols, int64_t m0, int64_t n0, float alpha) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int64_t col = n0 + wn * Cfg::WTN + j * 32 + (lane & 31);
      if (GUARD && col >= ncols) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * Cfg::WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (!GUARD || row < nrows) C[row * ldc + col] = static_cast<__bf16>(alpha * acc.v[i][j][v]);
      }
    }
}

// fp32 C[row][col] = acc, rows < nrows, cols < ncols.
template <class Cfg>
__device__ __forceinline__ void store_f32(const Acc<Cfg> &acc, float *C, int64_t ldc, int64_t nrows,
                                          int64_t ncols, int64_t m0, int64_t n0) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int64_t col = n0 + wn * Cfg::WTN + j * 32 + (lane & 31);
      if (col >= ncols) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * Cfg::WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < nrows) C[row * ldc + col] = acc.v[i][j][v];
      }
    }
}

// Workgroup -> output tile. Consecutive workgroup ids are dispatched round
// robin over the 8 XCDs (each with its own L2), so id b runs on XCD b % 8.
// Tiles are numbered in groups of 4 tile-rows (grouped raster order) and each
// XCD takes a contiguous range of tile numbers: the workgroups sharing an L2
// then cover a compact block of tiles that reuse the same rows of both
// operands.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int T = tiles_m * tiles_n;
  const int base = T / 8, extra = T % 8;
  const int x = bid % 8, slot = bid / 8;
  const int t = x * base + min(x, extra) + slot;
  constexpr int G = 4;
  const int group = t / (G * tiles_n);
  const int first_m = group * G;
  const int gm = min(tiles_m - first_m, G);
  const int in = t - group * G * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

}  // namespace qnf4
