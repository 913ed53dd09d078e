// Large-tile main loop for the two dequant-GEMMs (forward Y and input
// gradient dX): a 256 x 256 output tile per workgroup of four waves, each
// wave a 128 x 128 block of 4 x 4 v_mfma_f32_32x32x16_bf16 tiles whose 256
// fp32 accumulators live in the accumulation registers.
//
// Per 64-deep reduction step s:
//   * the dense operand (X, dY or an adapter factor) of step s + 1 is copied
//     straight from global memory into the other LDS buffer with
//     global_load_lds_dwordx4 (no registers, no LDS store instructions);
//   * the NF4 codes of step s + 2 are loaded into registers;
//   * the codes of step s + 1 (loaded one step earlier) are decoded into the
//     other LDS buffer in four quarters, each issued after the MFMAs of one
//     16-deep slice of step s, so decode and matrix work overlap;
//   * one barrier.
// Rows past the end of M, N or K are read from a clamped (valid) row: they
// only feed output rows or columns that are never stored.
#pragma once

#include "gemm_core.h"

namespace qnf4 {

constexpr int kBigThreads = 256;
constexpr int kBigRows = 256;
using CfgBig = TileCfg<256, 256, 2, 2>;

typedef __attribute__((address_space(3))) void lds_void;

// Dense bf16 operand rows [256][64] of src (row stride ld) via LDS DMA. Each
// wave copies eight 1 KB blocks (8 rows each); lane L of a block fetches the
// global chunk that the swizzle places at byte 16 L of the block.
struct DirectRows {
  static constexpr int kPerWave = kBigRows / 8 / (kBigThreads / 64);  // 8
  const char *base;
  uint32_t off[kPerWave];
  __device__ DirectRows(const void *src, int64_t ld, int64_t nrows, int64_t row0) {
    base = static_cast<const char *>(src) + row0 * ld * 2;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rb = lane >> 3, p = lane & 7;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int b = w + 4 * i;
      const int row = 8 * b + rb;
      const int c = p ^ swz(row);
      int64_t r = row0 + row;
      if (r >= nrows) r = nrows - 1;
      off[i] = static_cast<uint32_t>(((r - row0) * ld + 8 * c) * 2);
    }
  }
  // Issue the copies of reduction step red0 into the LDS tile `lds`.
  __device__ __forceinline__ void issue(int64_t red0, __bf16 *lds) const {
    const char *p = base + red0 * 2;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int b = w + 4 * i;
      __builtin_amdgcn_global_load_lds(p + off[i], (lds_void *)(lds + b * 512), 16, 0, 0);
    }
  }
};

// Forward B operand: NF4 rows n (reduction along k). Thread t decodes the
// 16-byte code chunks of rows t/2 and 128 + t/2, half t&1 of the 64-step.
struct Nf4RowBig {
  static constexpr int CH = 2;
  const uint8_t *cbase;
  const float *sbase;
  uint32_t coff[CH], soff[CH];
  uint4 reg[CH];
  float sc[CH];
  __device__ Nf4RowBig(const uint8_t *c, const float *s, int64_t N, int64_t K, int64_t row0)
      : cbase(c + row0 * K / 2), sbase(s + row0 * K / kBlock) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * kBigThreads;
      int64_t n = row0 + (idx >> 1);
      if (n >= N) n = N - 1;
      coff[i] = static_cast<uint32_t>((n - row0) * K / 2 + (idx & 1) * 16);
      soff[i] = static_cast<uint32_t>((n - row0) * K / kBlock);
    }
  }
  __device__ __forceinline__ void load(int64_t red0) {
    const uint8_t *cp = cbase + red0 / 2;
    const float *sp = sbase + red0 / kBlock;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      reg[i] = *reinterpret_cast<const uint4 *>(cp + coff[i]);
      sc[i] = sp[soff[i]];
    }
  }
  static constexpr int kLoads = 2 * CH;   // VMEM instructions issued by load()
  // Decode quarter q (code word q of each chunk: 8 elements per chunk).
  __device__ __forceinline__ void store_part(__bf16 *lds, const float2 *lv2, int q) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * kBigThreads;
      const uint32_t w = q == 0 ? reg[i].x : q == 1 ? reg[i].y : q == 2 ? reg[i].z : reg[i].w;
      uint32_t ow[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float2 pr = lv2[(w >> (8 * b)) & 0xFFu];
        ow[b] = pack_bf16x2(__fmul_rn(pr.x, sc[i]), __fmul_rn(pr.y, sc[i]));
      }
      *reinterpret_cast<uint4 *>(lds + lds_off(idx >> 1, (idx & 1) * 4 + q)) =
          make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
  }
};

// Input-gradient B operand: NF4 decoded transposed (output row k, reduction
// along n). One unit of 8 rows n x 8 columns k per thread (see TransUnits);
// quarter q decodes output rows 8 cc + 2q and 8 cc + 2q + 1.
struct Nf4TransBig {
  using U = TransUnits<kBigRows, kBigThreads>;
  const uint8_t *cbase;
  const float *sbase;
  uint32_t coff, soff, rowc, rows;
  uint32_t reg[8];
  float sc[8];
  __device__ Nf4TransBig(const uint8_t *c, const float *s, int64_t K, int64_t col0)
      : cbase(c + col0 / 2), sbase(s + col0 / kBlock) {
    const int idx = threadIdx.x;
    const int cc = U::cc(idx), rg = U::rg(idx);
    int64_t k = col0 + cc * 8;
    if (k >= K) k = K - 8;
    coff = static_cast<uint32_t>((rg * 8) * K / 2 + (k - col0) / 2);
    soff = static_cast<uint32_t>((rg * 8) * K / kBlock + (k - col0) / kBlock);
    rowc = static_cast<uint32_t>(K / 2);
    rows = static_cast<uint32_t>(K / kBlock);
  }
  __device__ __forceinline__ void load(int64_t red0, int64_t K) {
    const uint8_t *cp = cbase + red0 * K / 2;
    const float *sp = sbase + red0 * K / kBlock;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      reg[i] = *reinterpret_cast<const uint32_t *>(cp + coff + i * rowc);
      sc[i] = sp[soff + i * rows];
    }
  }
  static constexpr int kLoads = 16;
  __device__ __forceinline__ void store_part(__bf16 *lds, const float2 *lv2, int q) const {
    const int idx = threadIdx.x;
    const int cc = U::cc(idx), rg = U::rg(idx);
    float v0[8], v1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float2 pr = lv2[(reg[i] >> (8 * q)) & 0xFFu];
      v0[i] = __fmul_rn(pr.x, sc[i]);
      v1[i] = __fmul_rn(pr.y, sc[i]);
    }
    *reinterpret_cast<uint4 *>(lds + lds_off(cc * 8 + 2 * q, rg)) =
        make_uint4(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v0[4], v0[5]),
                   pack_bf16x2(v0[6], v0[7]));
    *reinterpret_cast<uint4 *>(lds + lds_off(cc * 8 + 2 * q + 1, rg)) =
        make_uint4(pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3]), pack_bf16x2(v1[4], v1[5]),
                   pack_bf16x2(v1[6], v1[7]));
  }
};

// Wait until at most `n` vector-memory operations of this wave are still in
// flight (the LDS DMA copies were issued before the last n code loads).
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// MFMAs of one 16-deep slice kk of the current tiles.
__device__ __forceinline__ void mma_slice(Acc<CfgBig> &acc, const __bf16 *sA, const __bf16 *sB,
                                          const FragAddr<128> &fa, const FragAddr<128> &fb, int kk) {
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(sA + fa.off[kk] + i * 32 * kLDK);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8 *>(sB + fb.off[kk] + j * 32 * kLDK);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.v[i][j], 0, 0, 0);
}

// The four LDS tiles of the large-tile kernels, as distinct objects so that
// alias analysis can tell the DMA target of a step from the tiles it reads.
struct BigSmem {
  __bf16 *a0, *a1, *b0, *b1;
};

// One step of the NF4 main loop: MFMAs on (aCur, bCur); the dense operand of
// step sn1 is copied into aNxt; the codes in ldec (step sn1) are decoded into
// bNxt; lload receives the codes of step sn2. The caller clamps sn1 and sn2
// to the last step, so the body has no branches; extra copies and decodes
// at the end land in the buffer nobody reads any more.
template <class LB, class LoadFn>
__device__ __forceinline__ void big_step(Acc<CfgBig> &acc, const DirectRows &da, LB &ldec, LB &lload,
                                         LoadFn &load, int sn1, int sn2, __bf16 *aCur, __bf16 *bCur,
                                         __bf16 *aNxt, __bf16 *bNxt, const FragAddr<128> &fa,
                                         const FragAddr<128> &fb, const float2 *lv2) {
  da.issue(static_cast<int64_t>(sn1) * kBK, aNxt);
  __builtin_amdgcn_sched_barrier(0);
  load(lload, sn2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    mma_slice(acc, aCur, bCur, fa, fb, kk);
    ldec.store_part(bNxt, lv2, kk);
  }
  wait_vmem_below<LB::kLoads>();
  __syncthreads();
}

template <class LB, class LoadFn>
__device__ __forceinline__ void big_mainloop_nf4(Acc<CfgBig> &acc, const DirectRows &da, LB &l0, LB &l1,
                                                 LoadFn load, int steps, const BigSmem &sm,
                                                 const float2 *lv2) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / CfgBig::WAVES_N, wn = w % CfgBig::WAVES_N;
  const FragAddr<128> fa(wm * 128, lane);
  const FragAddr<128> fb(wn * 128, lane);
  const int last = steps - 1;

  // prologue: step 0 into buffers 0, codes of step 1 in l1
  da.issue(0, sm.a0);
  load(l0, 0);
  load(l1, min(1, last));
#pragma unroll
  for (int q = 0; q < 4; ++q) l0.store_part(sm.b0, lv2, q);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // steps come in pairs (buffers 0, then 1); the codes of step s + 1 are in l1
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    big_step(acc, da, l1, l0, load, min(s + 1, last), min(s + 2, last), sm.a0, sm.b0, sm.a1, sm.b1,
             fa, fb, lv2);
    big_step(acc, da, l0, l1, load, min(s + 2, last), min(s + 3, last), sm.a1, sm.b1, sm.a0, sm.b0,
             fa, fb, lv2);
  }
  if (s < steps)
    big_step(acc, da, l1, l0, load, last, last, sm.a0, sm.b0, sm.a1, sm.b1, fa, fb, lv2);
  __builtin_amdgcn_s_waitcnt(0);   // no copy may still be landing in LDS
  __syncthreads();
}

// Both operands dense bf16 (the adapter steps): plain double-buffered loop.
__device__ __forceinline__ void big_mainloop_dense(Acc<CfgBig> &acc, const DirectRows &da,
                                                   const DirectRows &db, int steps, const BigSmem &sm) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / CfgBig::WAVES_N, wn = w % CfgBig::WAVES_N;
  const FragAddr<128> fa(wm * 128, lane);
  const FragAddr<128> fb(wn * 128, lane);
  for (int s = 0; s < steps; ++s) {
    da.issue(static_cast<int64_t>(s) * kBK, sm.a0);
    db.issue(static_cast<int64_t>(s) * kBK, sm.b0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) mma_slice(acc, sm.a0, sm.b0, fa, fb, kk);
    __syncthreads();
  }
}

}  // namespace qnf4
