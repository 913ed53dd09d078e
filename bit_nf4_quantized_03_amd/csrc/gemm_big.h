// Large-tile main loop for the two dequant-GEMMs (forward Y and input
// gradient dX): a 256 x 256 output tile per workgroup, built on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators in registers. Both kernels
// run eight waves of 128 x 64 (CfgBig8, two waves per SIMD, 128 accumulators
// each, so one wave's waits are covered by the other's MFMAs); the loaders
// and the main loop also take the four-wave layout of 128 x 128 per wave
// (256 threads, one wave per SIMD, 256 accumulators), which ran 5-10 %
// slower.
//
// Per 64-deep reduction step s:
//   * the dense operand (X, dY or an adapter factor) of step s + 1 is copied
//     straight from global memory into the other LDS buffer with
//     global_load_lds_dwordx4 (no registers, no LDS store instructions),
//     spread over the first three of the step's four MFMA groups;
//   * the NF4 codes of step s + 2 are loaded into registers;
//   * the codes of step s + 1 (loaded one step earlier) are decoded into the
//     other LDS buffer in four quarters, one per MFMA group, so decode and
//     matrix work overlap;
//   * one barrier.
// Rows past the end of M, N or K are read from a clamped (valid) row: they
// only feed output rows or columns that are never stored.
#pragma once

#include "gemm_core.h"

namespace qnf4 {

// Copies of the 256-entry level-pair table in LDS, interleaved entry by entry
// (entry e of copy c at e * kLvCopies + c); lane l reads copy l % kLvCopies,
// so two lanes of one 32-lane LDS pass meet in a bank only when they share a
// copy and their entries have the same parity.
constexpr int kLvCopies = 16;
constexpr int kBigRows = 256;
using CfgBig8 = TileCfg<256, 256, 2, 4>;   // eight waves: 128 x 64 per wave

typedef __attribute__((address_space(3))) void lds_void;

// Dense bf16 operand rows [ROWS][64] of src (row stride ld) via LDS DMA. The
// tile is ROWS / 8 blocks of 1 KB (8 rows each); wave w of the W = T / 64
// copying waves copies blocks w + W i, and lane L of a block fetches the
// global chunk that the swizzle places at byte 16 L of the block.
//
// The swizzle of row 8 b + rb is rb ^ (b & 3). With W a multiple of 4 every
// block of a wave has the same b & 3, so one chunk serves all of its blocks;
// otherwise the chunk is recomputed per block.
template <int T, int ROWS = kBigRows>
struct DirectRowsT {
  static constexpr int kWaves = T / 64;
  static constexpr int kPerWave = ROWS / 8 / kWaves;
  static constexpr bool kOneChunk = kWaves % 4 == 0;
  const char *base;
  uint32_t off;     // block 0 of this wave; block i adds i * bstride
  uint32_t bstride; // bytes between the wave's blocks (8 W rows)
  uint32_t clamp;   // largest valid row offset (bytes), for a tile crossing the end
  int prb;          // p ^ rb: the chunk of block b is prb ^ (b & 3)
  __device__ DirectRowsT(const void *src, int64_t ld, int64_t nrows, int64_t row0) {
    base = static_cast<const char *>(src) + row0 * ld * 2;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rb = lane >> 3, p = lane & 7;
    const int row = 8 * w + rb;
    const int c = p ^ swz(row);
    prb = p ^ rb;
    const int64_t last = (nrows - 1 - row0) < ROWS - 1 ? (nrows - 1 - row0) : ROWS - 1;
    bstride = static_cast<uint32_t>(8 * kWaves * ld * 2);
    if constexpr (kOneChunk) {
      off = static_cast<uint32_t>((row * ld + 8 * c) * 2);
      clamp = static_cast<uint32_t>((last * ld + 8 * c) * 2);
    } else {
      // row parts only; the chunk is added per block after the clamp
      off = static_cast<uint32_t>(row * ld * 2);
      clamp = static_cast<uint32_t>(last * ld * 2);
    }
  }
  // Issue the copies of reduction step red0 into the LDS tile `lds`. They are
  // written as inline assembly so that the compiler does not treat every
  // later LDS access and barrier as depending on them: the kernels wait for
  // the copies explicitly (wait_copies) before the barrier that publishes
  // the tile. The instruction returns nothing into registers.
  __device__ __forceinline__ void issue(int64_t red0, __bf16 *lds) const { issue_range(red0, lds, 0, kPerWave); }
  // Copies i0 .. i0 + n - 1 of the wave's blocks only.
  __device__ __forceinline__ void issue_range(int64_t red0, __bf16 *lds, int i0, int n) const {
    const char *p = base + red0 * 2;
    const int w = threadIdx.x >> 6;
    // LDS byte address of this wave's block 0 (wave-uniform)
    const uint32_t dst0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) __bf16 *)lds)) +
        static_cast<uint32_t>(w) * 1024u);
#pragma unroll
    for (int i = i0; i < i0 + n; ++i) {
      uint32_t o = min(off + static_cast<uint32_t>(i) * bstride, clamp);
      if constexpr (!kOneChunk) o += 16u * static_cast<uint32_t>(prb ^ ((w + kWaves * i) & 3));
      const uint32_t dst = dst0 + static_cast<uint32_t>(i) * (1024u * kWaves);   // block w + W i
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(dst), "v"(o), "s"(p)
                   : "memory", "m0");
    }
  }
  // Wait until the copies issued before the last N vector-memory
  // instructions of this wave have landed in LDS. The wait is the builtin,
  // so the compiler knows the register loads before it are complete too;
  // the empty statement keeps memory accesses from moving across it.
  template <int N>
  __device__ __forceinline__ static void wait_copies() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");
  }
};

// Forward B operand: NF4 rows n (reduction along k). Thread t decodes the
// 16-byte code chunks of rows t/2 + (T/2) i (i < 512/T), half t&1 of the
// 64-step.
template <int T>
struct Nf4RowBigT {
  static constexpr int CH = 512 / T;
  const uint8_t *cbase;
  const float *sbase;
  uint32_t coff[CH], soff[CH];
  uint4 reg[CH];
  float sc[CH];
  __device__ Nf4RowBigT(const uint8_t *c, const float *s, int64_t N, int64_t K, int64_t row0)
      : cbase(c + row0 * K / 2), sbase(s + row0 * K / kBlock) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * T;
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
  static constexpr int kWrites = CH;      // LDS stores per decode quarter
  // Quarter q = code word q of each chunk (8 elements per chunk): the level
  // pairs are fetched by lookup(), scaled, rounded and stored by finish().
  struct Pairs {
    float2 pr[CH][4];
  };
  __device__ __forceinline__ void lookup(Pairs &p, const float2 *lv2, int q) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint32_t w = q == 0 ? reg[i].x : q == 1 ? reg[i].y : q == 2 ? reg[i].z : reg[i].w;
#pragma unroll
      for (int b = 0; b < 4; ++b) p.pr[i][b] = lv2[((w >> (8 * b)) & 0xFFu) * kLvCopies];
    }
  }
  __device__ __forceinline__ void finish(__bf16 *lds, const Pairs &p, int q) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = threadIdx.x + i * T;
      uint32_t ow[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        ow[b] = pack_bf16x2(__fmul_rn(p.pr[i][b].x, sc[i]), __fmul_rn(p.pr[i][b].y, sc[i]));
      *reinterpret_cast<uint4 *>(lds + lds_off(idx >> 1, (idx & 1) * 4 + q)) =
          make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
  }
  __device__ __forceinline__ void store_part(__bf16 *lds, const float2 *lv2, int q) const {
    Pairs p;
    lookup(p, lv2, q);
    finish(lds, p, q);
  }
};

// Input-gradient B operand: NF4 decoded transposed (output row k, reduction
// along n), in units of 8 rows n x 8 columns k (see TransUnits). With 256
// threads a thread decodes a whole unit; with 512, thread t takes rows
// 4 (t / 256) .. + 3 of unit t % 256 (so a wave's lanes hold eight whole
// units' halves and its 8-byte stores still land on distinct chunk slots).
// Quarter q decodes output rows 8 cc + 2q and 8 cc + 2q + 1.
template <int T>
struct Nf4TransBigT {
  static_assert(T == 256 || T == 512, "256 or 512 threads");
  static constexpr int R = 8 * 256 / T;   // rows n per thread
  using U = TransUnits<kBigRows, 256>;
  const uint8_t *cbase;
  const float *sbase;
  // byte offset of the thread's first code word from cbase; the scale index
  // of that word's block is coff / 32 (K is a multiple of 64, so n K / 2 is a
  // multiple of 32 and the column part cc * 4 < 128 adds cc / 8)
  uint32_t coff;
  uint32_t reg[R];
  float sc[R];
  __device__ Nf4TransBigT(const uint8_t *c, const float *s, int64_t K, int64_t col0)
      : cbase(c + col0 / 2), sbase(s + col0 / kBlock) {
    const int idx = threadIdx.x & 255, hh = threadIdx.x >> 8;
    const int cc = U::cc(idx), rg = U::rg(idx);
    int64_t k = col0 + cc * 8;
    if (k >= K) k = K - 8;
    const int64_t n = rg * 8 + hh * R;
    coff = static_cast<uint32_t>(n * K / 2 + (k - col0) / 2);
  }
  __device__ __forceinline__ void load(int64_t red0, int64_t K) {
    // the row parts of the addresses are wave-uniform
    const uint8_t *cp = cbase + red0 * K / 2;
    const float *sp = sbase + red0 * K / kBlock;
    const uint32_t so = coff >> 5;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      reg[i] = *reinterpret_cast<const uint32_t *>(cp + i * (K / 2) + coff);
      sc[i] = (sp + i * (K / kBlock))[so];
    }
  }
  static constexpr int kLoads = 2 * R;
  static constexpr int kWrites = 2;
  struct Pairs {
    float2 pr[R];
  };
  __device__ __forceinline__ void lookup(Pairs &p, const float2 *lv2, int q) const {
#pragma unroll
    for (int i = 0; i < R; ++i) p.pr[i] = lv2[((reg[i] >> (8 * q)) & 0xFFu) * kLvCopies];
  }
  __device__ __forceinline__ void store_part(__bf16 *lds, const float2 *lv2, int q) const {
    Pairs p;
    lookup(p, lv2, q);
    finish(lds, p, q);
  }
  __device__ __forceinline__ void finish(__bf16 *lds, const Pairs &p, int q) const {
    const int idx = threadIdx.x & 255, hh = threadIdx.x >> 8;
    const int cc = U::cc(idx), rg = U::rg(idx);
    float v0[R], v1[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      v0[i] = __fmul_rn(p.pr[i].x, sc[i]);
      v1[i] = __fmul_rn(p.pr[i].y, sc[i]);
    }
    // rows 8 cc + j have swz = j ^ (cc & 3), so logical chunk rg of row
    // 8 cc + j sits at chunk rg ^ (cc & 3) ^ j
    const int x = rg ^ (cc & 3);
    __bf16 *d0 = lds + (cc * 8 + 2 * q) * kLDK + ((x ^ (2 * q)) << 3) + hh * R;
    __bf16 *d1 = lds + (cc * 8 + 2 * q + 1) * kLDK + ((x ^ (2 * q + 1)) << 3) + hh * R;
    if constexpr (R == 8) {
      *reinterpret_cast<uint4 *>(d0) = make_uint4(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                                                  pack_bf16x2(v0[4], v0[5]), pack_bf16x2(v0[6], v0[7]));
      *reinterpret_cast<uint4 *>(d1) = make_uint4(pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3]),
                                                  pack_bf16x2(v1[4], v1[5]), pack_bf16x2(v1[6], v1[7]));
    } else {
      *reinterpret_cast<uint2 *>(d0) = make_uint2(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]));
      *reinterpret_cast<uint2 *>(d1) = make_uint2(pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3]));
    }
  }
};

// Fragments of one 16-deep slice for a wave's WTM x WTN block.
template <class Cfg>
struct Frags {
  bf16x8 a[Cfg::TM], b[Cfg::TN];
};

template <class Cfg>
__device__ __forceinline__ void load_frags(Frags<Cfg> &f, const __bf16 *sA, const __bf16 *sB,
                                           const FragAddr<Cfg::WTM> &fa, const FragAddr<Cfg::WTN> &fb, int kk) {
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) f.a[i] = *reinterpret_cast<const bf16x8 *>(sA + fa.off[kk] + i * 32 * kLDK);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) f.b[j] = *reinterpret_cast<const bf16x8 *>(sB + fb.off[kk] + j * 32 * kLDK);
}

template <class Cfg>
__device__ __forceinline__ void mma_frags(Acc<Cfg> &acc, const Frags<Cfg> &f) {
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
      acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc.v[i][j], 0, 0, 0);
}

// MFMAs of one 16-deep slice kk of the current tiles.
template <class Cfg>
__device__ __forceinline__ void mma_slice(Acc<Cfg> &acc, const __bf16 *sA, const __bf16 *sB,
                                          const FragAddr<Cfg::WTM> &fa, const FragAddr<Cfg::WTN> &fb, int kk) {
  Frags<Cfg> f;
  load_frags(f, sA, sB, fa, fb, kk);
  mma_frags(acc, f);
}

// Interleave one slice's MFMAs with the rest of its work: the LDS reads for
// the next slice ride two to an MFMA on the first MFMAs (so they are in
// flight early), the VALU work (read addresses, scale / round of a decode
// quarter) fills the gaps, the decode stores come last. kLead puts most of
// the VALU work ahead of the first MFMA.
template <class Cfg, int kReads, int kWrites, bool kLead>
__device__ __forceinline__ void interleave_group() {
  constexpr int kMfma = Cfg::TM * Cfg::TN;
  constexpr int kWithReads = (kReads + 1) / 2 < kMfma ? (kReads + 1) / 2 : kMfma;
  __builtin_amdgcn_sched_group_barrier(0x002, kLead ? 28 : 4, 0);   // VALU
#pragma unroll
  for (int g = 0; g < kWithReads; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // 2 VALU
  }
#pragma unroll
  for (int g = kWithReads; g < kMfma; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // 3 VALU
  }
  __builtin_amdgcn_sched_group_barrier(0x200, kWrites, 0);   // LDS stores
}

// Wait until at most N LDS operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_lds_below() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
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
//
// The wave issues its instructions in order, so a wait on memory stalls the
// MFMAs queued behind it; everything a group of MFMAs consumes is therefore
// read one group earlier. The MFMA groups are shifted by one 16-deep slice
// against the barrier: a step starts with the MFMAs of the previous step's
// last slice (fragments f1, read before the barrier), which cover the reads
// of this step's first slice; then slices 0, 1, 2 follow. Decode quarter q
// runs with group q (group 0 being the previous step's last slice), its
// codebook pairs read one group earlier (pe even quarters, po odd ones; the
// pairs of quarter 0 come from the codes loaded at the start of this step).
// The copies for the next dense tile are spread over the first three groups.
template <class Cfg, bool kFirst, class DA, class LB, class LoadFn>
__device__ __forceinline__ void big_step(Acc<Cfg> &acc, const DA &da, LB &ldec, LB &lload, LoadFn &load, int sn1,
                                         int sn2, const __bf16 *aCur, const __bf16 *bCur, __bf16 *aNxt,
                                         __bf16 *bNxt, const FragAddr<Cfg::WTM> &fa,
                                         const FragAddr<Cfg::WTN> &fb, const float2 *lv2, Frags<Cfg> &f0,
                                         Frags<Cfg> &f1, typename LB::Pairs &pe, typename LB::Pairs &po) {
  // copies of the next dense tile per group (group 0, 1, 2), so that few
  // vector-memory instructions queue up behind each other in any one group
  constexpr int kDmaA = DA::kPerWave / 4, kDma0 = (DA::kPerWave - kDmaA + 1) / 2;
  constexpr int kDma1 = DA::kPerWave - kDmaA - kDma0;
  constexpr int kReads = Cfg::TM + Cfg::TN + 4 * sizeof(typename LB::Pairs) / sizeof(float2) / 4;
  const int64_t red1 = static_cast<int64_t>(sn1) * kBK;
  // group 0: last slice of the previous step; reads for slice 0
  load_frags(f0, aCur, bCur, fa, fb, 0);
  load(lload, sn2);
  da.issue_range(red1, aNxt, 0, kDmaA);
  ldec.lookup(po, lv2, 1);
  if (!kFirst) mma_frags(acc, f1);
  ldec.finish(bNxt, pe, 0);
  interleave_group<Cfg, kReads, LB::kWrites, kFirst>();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    Frags<Cfg> &cur = (kk & 1) ? f1 : f0;
    Frags<Cfg> &nxt = (kk & 1) ? f0 : f1;
    typename LB::Pairs &pc = (kk & 1) ? pe : po;   // quarter kk + 1
    typename LB::Pairs &pn = (kk & 1) ? po : pe;   // quarter kk + 2 (mod 4)
    // what this group consumes was read one group ago; only the stores of
    // the last quarter may stay in flight
    wait_lds_below<LB::kWrites>();
    if (kk == 0) da.issue_range(red1, aNxt, kDmaA, kDma0);
    if (kk == 1 && kDma1 > 0) da.issue_range(red1, aNxt, kDmaA + kDma0, kDma1);
    if (kk < 2)
      ldec.lookup(pn, lv2, kk + 2);
    else
      lload.lookup(pn, lv2, 0);
    load_frags(nxt, aCur, bCur, fa, fb, kk + 1);
    mma_frags(acc, cur);
    ldec.finish(bNxt, pc, kk + 1);
    interleave_group<Cfg, kReads, LB::kWrites, false>();
    __builtin_amdgcn_sched_barrier(0);
  }
  DA::template wait_copies<0>();
  __syncthreads();
}

template <class Cfg, class DA, class LB, class LoadFn>
__device__ __forceinline__ void big_mainloop_nf4(Acc<Cfg> &acc, const DA &da, LB &l0, LB &l1, LoadFn load,
                                                 int steps, const BigSmem &sm, const float2 *lv2) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
  const FragAddr<Cfg::WTM> fa(wm * Cfg::WTM, lane);
  const FragAddr<Cfg::WTN> fb(wn * Cfg::WTN, lane);
  const int last = steps - 1;
  typename LB::Pairs pe, po;
  Frags<Cfg> f0, f1;

  // prologue: step 0 into buffers 0, codes of step 1 in l1 and the pairs of
  // its first decode quarter in pe
  da.issue(0, sm.a0);
  load(l0, 0);
  load(l1, min(1, last));
#pragma unroll
  for (int q = 0; q < 4; ++q) l0.store_part(sm.b0, lv2, q);
  l1.lookup(pe, lv2, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // step 0 has no previous slice; then pairs of steps (buffers 1, then 0)
  big_step<Cfg, true>(acc, da, l1, l0, load, min(1, last), min(2, last), sm.a0, sm.b0, sm.a1, sm.b1, fa, fb, lv2,
                      f0, f1, pe, po);
  int s = 1;
  for (; s + 1 < steps; s += 2) {
    big_step<Cfg, false>(acc, da, l0, l1, load, min(s + 1, last), min(s + 2, last), sm.a1, sm.b1, sm.a0,
                         sm.b0, fa, fb, lv2, f0, f1, pe, po);
    big_step<Cfg, false>(acc, da, l1, l0, load, min(s + 2, last), min(s + 3, last), sm.a0, sm.b0, sm.a1,
                         sm.b1, fa, fb, lv2, f0, f1, pe, po);
  }
  if (s < steps)
    big_step<Cfg, false>(acc, da, l0, l1, load, last, last, sm.a1, sm.b1, sm.a0, sm.b0, fa, fb, lv2, f0, f1, pe,
                         po);
  mma_frags(acc, f1);   // last slice of the last step
  __builtin_amdgcn_s_waitcnt(0);   // no copy may still be landing in LDS
  __syncthreads();
}

// Both operands dense bf16 (the adapter steps): plain double-buffered loop.
template <class Cfg, class DA>
__device__ __forceinline__ void big_mainloop_dense(Acc<Cfg> &acc, const DA &da, const DA &db, int steps,
                                                   const BigSmem &sm) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / Cfg::WAVES_N, wn = w % Cfg::WAVES_N;
  const FragAddr<Cfg::WTM> fa(wm * Cfg::WTM, lane);
  const FragAddr<Cfg::WTN> fb(wn * Cfg::WTN, lane);
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
