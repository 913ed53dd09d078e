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
// Loaders turn a 64-wide reduction step of a source tensor into that LDS
// layout: plain bf16 rows, fp32 rows rounded to bf16, transposed bf16 or
// fp32 (reduction along the source's rows), and the NF4 + DQ weight decoded on
// the fly either along its rows (forward: reduction over in_features) or
// transposed (input gradient: reduction over out_features). Decoding follows
// the format's reconstruction w = fp32(level[code] * c_b) and rounds w to bf16
// (round to nearest even) as the matrix-core operand.
#pragma once

#include "internal.h"

namespace qnf4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;          // reduction elements per pipeline step
constexpr int kLDK = kBK + 8;    // LDS row length in bf16 (padding vs bank conflicts)

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

// One 64-deep step of MFMAs from the LDS tiles sA [BM][kLDK], sB [BN][kLDK].
template <class Cfg>
__device__ __forceinline__ void mma_step(Acc<Cfg> &acc, const __bf16 *sA, const __bf16 *sB,
                                         int wm, int wn, int lane) {
  const int r = lane & 31;
  const int koff = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    bf16x8 a[Cfg::TM], b[Cfg::TN];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
      a[i] = *reinterpret_cast<const bf16x8 *>(sA + (wm * Cfg::WTM + i * 32 + r) * kLDK + kk * 16 + koff);
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
      b[j] = *reinterpret_cast<const bf16x8 *>(sB + (wn * Cfg::WTN + j * 32 + r) * kLDK + kk * 16 + koff);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
        acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.v[i][j], 0, 0, 0);
  }
}

// Pipelined main loop over `steps` reduction steps starting at `red0`, stride
// 64. LDS is double buffered; one barrier per step. On entry the caller has
// synchronized (LDS free); on exit all LDS reads are complete.
template <class Cfg, class LA, class LB>
__device__ __forceinline__ void mainloop(Acc<Cfg> &acc, LA &la, LB &lb, int64_t red0, int steps,
                                         __bf16 *sA0, __bf16 *sA1, __bf16 *sB0, __bf16 *sB1) {
  if (steps <= 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
  la.load(red0);
  lb.load(red0);
  la.store(sA0);
  lb.store(sB0);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    __bf16 *cA = (s & 1) ? sA1 : sA0;
    __bf16 *cB = (s & 1) ? sB1 : sB0;
    __bf16 *nA = (s & 1) ? sA0 : sA1;
    __bf16 *nB = (s & 1) ? sB0 : sB1;
    const bool more = s + 1 < steps;
    if (more) {
      la.load(red0 + static_cast<int64_t>(s + 1) * kBK);
      lb.load(red0 + static_cast<int64_t>(s + 1) * kBK);
    }
    mma_step<Cfg>(acc, cA, cB, wm, wn, lane);
    if (more) {
      la.store(nA);
      lb.store(nB);
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------- loaders
// Each loader covers ROWS output rows of one operand and a 64-deep reduction
// step. load() issues the global reads into registers, store() writes the
// LDS tile [ROWS][kLDK].

// bf16 source S[row][t] (t contiguous), row stride ld, rows >= nrows read as 0.
template <int ROWS, int T>
struct RowBf16 {
  static constexpr int CH = ROWS * 8 / T;
  static_assert(ROWS * 8 % T == 0, "tile/threads mismatch");
  const __bf16 *src;
  int64_t ld, nrows, row0;
  uint4 reg[CH];
  __device__ RowBf16(const void *s, int64_t ld_, int64_t nrows_, int64_t row0_)
      : src(static_cast<const __bf16 *>(s)), ld(ld_), nrows(nrows_), row0(row0_) {}
  __device__ __forceinline__ void load(int64_t red0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * T;
      const int64_t r = row0 + (idx >> 3);
      reg[i] = (r < nrows) ? *reinterpret_cast<const uint4 *>(src + r * ld + red0 + (idx & 7) * 8)
                           : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(__bf16 *lds) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * T;
      *reinterpret_cast<uint4 *>(lds + (idx >> 3) * kLDK + (idx & 7) * 8) = reg[i];
    }
  }
};

// fp32 source S[row][t], row stride ld (multiple of 4), rows >= nrows read as 0.
template <int ROWS, int T>
struct RowF32 {
  static constexpr int CH = ROWS * 16 / T;
  static_assert(ROWS * 16 % T == 0, "tile/threads mismatch");
  const float *src;
  int64_t ld, nrows, row0;
  float4 reg[CH];
  __device__ RowF32(const void *s, int64_t ld_, int64_t nrows_, int64_t row0_)
      : src(static_cast<const float *>(s)), ld(ld_), nrows(nrows_), row0(row0_) {}
  __device__ __forceinline__ void load(int64_t red0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * T;
      const int64_t r = row0 + (idx >> 4);
      reg[i] = (r < nrows) ? *reinterpret_cast<const float4 *>(src + r * ld + red0 + (idx & 15) * 4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void store(__bf16 *lds) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * T;
      uint2 v = make_uint2(pack_bf16x2(reg[i].x, reg[i].y), pack_bf16x2(reg[i].z, reg[i].w));
      *reinterpret_cast<uint2 *>(lds + (idx >> 4) * kLDK + (idx & 15) * 4) = v;
    }
  }
};

// Transposed bf16 source S[t][col] (reduction along the source's rows, cols
// contiguous, ld multiple of 8): output row = col. Units of 4 reduction rows x
// 8 columns; reduction rows >= nred and columns >= ncols read as 0 (ncols is
// a multiple of 8).
template <int ROWS, int T>
struct TransBf16 {
  static constexpr int UPR = ROWS / 8;           // units per reduction-row group
  static constexpr int UNITS = 16 * UPR;
  static constexpr int CH = (UNITS + T - 1) / T;
  const __bf16 *src;
  int64_t ld, nred, ncols, col0;
  uint4 reg[CH][4];
  __device__ TransBf16(const void *s, int64_t ld_, int64_t nred_, int64_t ncols_, int64_t col0_)
      : src(static_cast<const __bf16 *>(s)), ld(ld_), nred(nred_), ncols(ncols_), col0(col0_) {}
  __device__ __forceinline__ void load(int64_t red0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = threadIdx.x + u * T;
      if (UNITS % T != 0 && idx >= UNITS) continue;
      const int cc = idx % UPR, rg = idx / UPR;
      const int64_t c = col0 + cc * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = red0 + rg * 4 + i;
        reg[u][i] = (t < nred && c < ncols) ? *reinterpret_cast<const uint4 *>(src + t * ld + c)
                                            : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(__bf16 *lds) const {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = threadIdx.x + u * T;
      if (UNITS % T != 0 && idx >= UNITS) continue;
      const int cc = idx % UPR, rg = idx / UPR;
      const uint32_t w[4][4] = {{reg[u][0].x, reg[u][0].y, reg[u][0].z, reg[u][0].w},
                                {reg[u][1].x, reg[u][1].y, reg[u][1].z, reg[u][1].w},
                                {reg[u][2].x, reg[u][2].y, reg[u][2].z, reg[u][2].w},
                                {reg[u][3].x, reg[u][3].y, reg[u][3].z, reg[u][3].w}};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // columns 2q (low halves) and 2q+1 (high halves) of the four rows
        uint2 even = make_uint2(lo16x2(w[0][q], w[1][q]), lo16x2(w[2][q], w[3][q]));
        uint2 odd = make_uint2(hi16x2(w[0][q], w[1][q]), hi16x2(w[2][q], w[3][q]));
        *reinterpret_cast<uint2 *>(lds + (cc * 8 + 2 * q) * kLDK + rg * 4) = even;
        *reinterpret_cast<uint2 *>(lds + (cc * 8 + 2 * q + 1) * kLDK + rg * 4) = odd;
      }
    }
  }
};

// Transposed fp32 source S[t][col] with any row stride: scalar loads, rounded
// to bf16. Units of 4 reduction rows x 8 columns; out-of-range reads as 0.
template <int ROWS, int T>
struct TransF32 {
  static constexpr int UPR = ROWS / 8;
  static constexpr int UNITS = 16 * UPR;
  static constexpr int CH = (UNITS + T - 1) / T;
  const float *src;
  int64_t ld, nred, ncols, col0;
  float reg[CH][4][8];
  __device__ TransF32(const void *s, int64_t ld_, int64_t nred_, int64_t ncols_, int64_t col0_)
      : src(static_cast<const float *>(s)), ld(ld_), nred(nred_), ncols(ncols_), col0(col0_) {}
  __device__ __forceinline__ void load(int64_t red0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = threadIdx.x + u * T;
      if (UNITS % T != 0 && idx >= UNITS) continue;
      const int cc = idx % UPR, rg = idx / UPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = red0 + rg * 4 + i;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t c = col0 + cc * 8 + j;
          reg[u][i][j] = (t < nred && c < ncols) ? src[t * ld + c] : 0.0f;
        }
      }
    }
  }
  __device__ __forceinline__ void store(__bf16 *lds) const {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = threadIdx.x + u * T;
      if (UNITS % T != 0 && idx >= UNITS) continue;
      const int cc = idx % UPR, rg = idx / UPR;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint2 v = make_uint2(pack_bf16x2(reg[u][0][j], reg[u][1][j]),
                             pack_bf16x2(reg[u][2][j], reg[u][3][j]));
        *reinterpret_cast<uint2 *>(lds + (cc * 8 + j) * kLDK + rg * 4) = v;
      }
    }
  }
};

// NF4 + DQ weight W [N][K] decoded along its rows: output row = n, reduction
// over k. K is a multiple of 64, so a 64-step of one row is exactly one
// quantization block with scale cs[(n*K + k0)/64]. lv: the 16 levels in LDS.
template <int ROWS, int T>
struct Nf4Row {
  static constexpr int CH = ROWS * 2 / T;       // 16-byte code chunks per thread
  static_assert(ROWS * 2 % T == 0, "tile/threads mismatch");
  const uint8_t *codes;
  const float *cs;
  const float *lv;
  int64_t N, K, row0;
  uint4 reg[CH];
  float sc[CH];
  __device__ Nf4Row(const uint8_t *c, const float *s, const float *lv_, int64_t N_, int64_t K_,
                    int64_t row0_)
      : codes(c), cs(s), lv(lv_), N(N_), K(K_), row0(row0_) {}
  __device__ __forceinline__ void load(int64_t red0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * T;
      const int64_t n = row0 + (idx >> 1);
      if (n < N) {
        const int64_t e = n * K + red0;
        reg[i] = *reinterpret_cast<const uint4 *>(codes + e / 2 + (idx & 1) * 16);
        sc[i] = cs[e / kBlock];
      } else {
        reg[i] = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
        sc[i] = 0.0f;
      }
    }
  }
  __device__ __forceinline__ void store(__bf16 *lds) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * T;
      const uint32_t w[4] = {reg[i].x, reg[i].y, reg[i].z, reg[i].w};
      __bf16 *dst = lds + (idx >> 1) * kLDK + (idx & 1) * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 o;
        uint32_t ow[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t byte = (w[q] >> (8 * b)) & 0xFFu;
          ow[b] = pack_bf16x2(__fmul_rn(lv[byte >> 4], sc[i]), __fmul_rn(lv[byte & 15u], sc[i]));
        }
        o = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        *reinterpret_cast<uint4 *>(dst + q * 8) = o;
      }
    }
  }
};

// NF4 + DQ weight W [N][K] decoded transposed: output row = k, reduction over
// n. Units of 4 rows n x 8 columns k (one 32-bit word of codes per row, inside
// one quantization block). Rows n >= N read as 0.
template <int ROWS, int T>
struct Nf4Trans {
  static constexpr int UPR = ROWS / 8;
  static constexpr int UNITS = 16 * UPR;
  static constexpr int CH = (UNITS + T - 1) / T;
  const uint8_t *codes;
  const float *cs;
  const float *lv;
  int64_t N, K, col0;
  uint32_t reg[CH][4];
  float sc[CH][4];
  __device__ Nf4Trans(const uint8_t *c, const float *s, const float *lv_, int64_t N_, int64_t K_,
                      int64_t col0_)
      : codes(c), cs(s), lv(lv_), N(N_), K(K_), col0(col0_) {}
  __device__ __forceinline__ void load(int64_t red0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = threadIdx.x + u * T;
      if (UNITS % T != 0 && idx >= UNITS) continue;
      const int cc = idx % UPR, rg = idx / UPR;
      const int64_t k = col0 + cc * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = red0 + rg * 4 + i;
        if (n < N && k < K) {
          const int64_t e = n * K + k;
          reg[u][i] = *reinterpret_cast<const uint32_t *>(codes + e / 2);
          sc[u][i] = cs[e / kBlock];
        } else {
          reg[u][i] = 0x77777777u;
          sc[u][i] = 0.0f;
        }
      }
    }
  }
  __device__ __forceinline__ void store(__bf16 *lds) const {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int idx = threadIdx.x + u * T;
      if (UNITS % T != 0 && idx >= UNITS) continue;
      const int cc = idx % UPR, rg = idx / UPR;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // element j of a word: byte j/2, high nibble for even j
        const int sh = 8 * (j >> 1) + ((j & 1) ? 0 : 4);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __fmul_rn(lv[(reg[u][i] >> sh) & 15u], sc[u][i]);
        uint2 o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        *reinterpret_cast<uint2 *>(lds + (cc * 8 + j) * kLDK + rg * 4) = o;
      }
    }
  }
};

// ----------------------------------------------------------------- epilogues

// bf16 C[row][col] = bf16(alpha * acc), rows < nrows, cols < ncols.
template <class Cfg>
__device__ __forceinline__ void store_bf16(const Acc<Cfg> &acc, __bf16 *C, int64_t ldc, int64_t nrows,
                                           int64_t ncols, int64_t m0, int64_t n0, float alpha) {
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
        if (row < nrows) C[row * ldc + col] = static_cast<__bf16>(alpha * acc.v[i][j][v]);
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

}  // namespace qnf4
