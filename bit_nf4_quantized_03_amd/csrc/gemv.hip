// Skinny-M QLoRA forward (decode):
//   Y = X W^T + s (X A^T) B^T
// with the NF4 + DQ weight streamed from HBM once and decoded on the fly
// (QLoRA vs ChatGPT page, capability "training pipeline": block-wise
// dequantization of the 4-bit base in the forward pass; capability "LoRA on
// the quantized base": a frozen base plus a full-precision adapter).
//
// One pass handles up to 16 rows of X (more rows run as further passes).
// Two launches per pass:
//   k_gemv         grid = (column strips of 128) x (K splits of 1024). A wave
//                  owns 16 output columns. The workgroup first loads its X
//                  chunk, absmax bytes and DQ constants and stages X and a
//                  byte table in LDS; then each lane streams the code words of
//                  its split, two to six super-blocks ahead of their use (the
//                  stream starts after X is staged, so X is not queued behind
//                  it). Per 64-element block, a lane maps its code bytes to
//                  bf16 level pairs (table lookups = MFMA B operands), runs
//                  v_mfma_f32_16x16x32_bf16 into a temporary and adds
//                  c_b * temporary to its accumulator: the block scale is
//                  applied once per block and output, not once per weight.
//                  The workgroups then form the split partials of H = X A^T.
//   k_gemv_finish  per output: the fixed-order sum of the split partials plus
//                  the adapter term bf16(s H) bf16(B)^T (MFMA), rounded to bf16.
// For M <= 4 (M <= 8) one MFMA spans 4 (2) blocks in block-diagonal row
// groups (see k_gemv). Within a block the reduction order is free: each lane
// group takes contiguous code bytes and reads X in the same order. Levels
// enter the MFMA as bf16 and c_b is applied in fp32, so Y differs from
// bf16(X bf16(W-hat)^T) at the bf16 operand level.
#include <algorithm>

#include "gemm_core.h"

namespace qnf4 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGvRows = 16;                  // rows of X per pass
constexpr int kGvWaves = 8;
constexpr int kGvThreads = 64 * kGvWaves;    // 512; two workgroups per CU
constexpr int kGvCols = 16 * kGvWaves;       // output columns per workgroup
constexpr int kGvMaxBlocks = 16;             // most 64-element blocks per split
constexpr int kGvChunk = kGvMaxBlocks * kBlock;
constexpr int kGvXStride = kGvChunk + 8;     // bf16; +16 bytes keeps b128 reads conflict-free
constexpr int kLutCopies = 32;               // one table copy per LDS bank: conflict-free lookups
constexpr int kFinWaves = 8;                 // finish kernel: 128 columns per workgroup
constexpr int kFinThreads = 64 * kFinWaves;
constexpr int kFinCols = 16 * kFinWaves;

struct GemvParams {
  const __bf16 *X;        // [M][K]
  const uint8_t *codes;   // [N][K/2]
  const int8_t *absmax_q; // [N*K/64] (with DQ)
  const float *dq_scale;  // [nd]
  const float *dq_mean;   // [1]
  const float *absmax;    // [N*K/64] fp32 block constants (without DQ)
  const float *A;         // [r][K] fp32, or null when r == 0
  const float *B;         // [N][r] fp32, or null when r == 0
  float *part;            // [splits][M][N] fp32
  float *hpart;           // [splits][M][r] fp32
  __bf16 *Y;              // [M][N]
  int64_t M, N, K;        // M <= 16
  int r, splits;
  int split_blocks;       // 64-element blocks per split (the last split may have fewer)
  float scale;
  Nf4Tables tab;
};

// Code words of one lane for one super-block (BD consecutive 64-blocks).
template <int BD> struct CodeWords;
template <> struct CodeWords<1> {
  uint2 v;
  __device__ uint32_t word(int q) const { return q == 0 ? v.x : v.y; }
  __device__ void load(const uint8_t *p) { v = *reinterpret_cast<const uint2 *>(p); }
};
template <> struct CodeWords<2> {
  uint4 v;
  __device__ uint32_t word(int q) const { return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w; }
  __device__ void load(const uint8_t *p) { v = *reinterpret_cast<const uint4 *>(p); }
};
template <> struct CodeWords<4> {
  uint4 v0, v1;
  __device__ uint32_t word(int q) const {
    const uint4 &v = q < 4 ? v0 : v1;
    const int e = q & 3;
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
  }
  __device__ void load(const uint8_t *p) {
    v0 = *reinterpret_cast<const uint4 *>(p);
    v1 = *reinterpret_cast<const uint4 *>(p + 16);
  }
};

// One pass of at most 16 / BD rows of X. BD is the number of 64-blocks one
// MFMA spans: the 16 MFMA rows are BD row groups of 16 / BD rows, and row
// group b multiplies block b of the super-block while the other rows of the
// A operand are zero. Lane group g (lane / 16) then always holds 8 BD
// contiguous code bytes of one block (b = g BD / 4) and one block scale, and
// its accumulator rows all belong to that block; the row groups are summed
// across lanes once at the end. BD = 1, 2, 4 serve M <= 16, 8, 4: larger BD
// reads 16 or 32 contiguous bytes per lane and fewer X fragments.
// kAligned: K is a multiple of 256, so each lane's absmax bytes are whole dwords.
// kDq: block scales decoded from int8 codes + DQ; else the stored fp32 constants.
template <int BD, bool kAligned, bool kDq>
__global__ __launch_bounds__(kGvThreads, 2) void k_gemv(GemvParams p) {
  constexpr int NB = kGvMaxBlocks;
  constexpr int NS = NB / BD;                       // super-blocks per split
  constexpr int G = 4 / BD;                         // lane groups per block
  constexpr int RB = 16 / BD;                       // rows per row group
  constexpr int NW = 2 * BD;                        // code words (= MFMAs) per lane per super-block
  constexpr int P = BD == 1 ? 6 : BD == 2 ? 3 : 2;  // super-blocks in flight per lane
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * kLutCopies];   // 32 KB
  __shared__ __attribute__((aligned(16))) __bf16 xs[kGvRows * kGvXStride];
  __shared__ __attribute__((aligned(16))) float as_[2][kGvChunk];          // two rows of A

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int z = blockIdx.y;
  const int64_t k0 = static_cast<int64_t>(z) * p.split_blocks * kBlock;
  const int kc = static_cast<int>(min<int64_t>(p.split_blocks * kBlock, p.K - k0));   // a multiple of 64
  const int nblk = kc / kBlock;
  const int M = static_cast<int>(p.M);
  const int gx = gridDim.x, jr0 = blockIdx.x;

  const int64_t n_raw = static_cast<int64_t>(blockIdx.x) * kGvCols + w * 16 + (lane & 15);
  const bool n_ok = n_raw < p.N;
  const int64_t n = n_ok ? n_raw : p.N - 1;
  const int g = lane >> 4;
  const int bg = g / G, sub = g % G;               // block of this lane group, part of it
  const int64_t kb = p.K / kBlock;                 // blocks per weight row (a multiple of 4 if kAligned)
  const int64_t b0 = n * kb + k0 / kBlock;         // first block of this lane's split
  const uint8_t *crow = p.codes + b0 * (kBlock / 2) + 8 * BD * sub;
  // Super-block s covers blocks s BD .. s BD + BD - 1 of the split; blocks past
  // the end of a short split are clamped to its last block (in bounds, scale
  // zero), so the load sequence has no branches.
  auto cptr = [&](int s) { return crow + (kBlock / 2) * min(s * BD + bg, nblk - 1); };

  // ---- global loads, in the order they are waited for: one level, the X
  // chunk (16-byte pieces in named registers; columns past the end of a short
  // split are staged as zero, so blocks past the end contribute exactly
  // nothing), absmax bytes, DQ scales, two rows of A.
  constexpr int pieces = kGvChunk / 8;
  static_assert(kGvRows * pieces == 4 * kGvThreads, "X chunk = 4 pieces per thread");
  const int kpieces = kc / 8, xtotal = M * pieces;
  uint4 x0, x1, x2, x3;
#define QNF4_XLOAD(u, v)                                                                        \
  {                                                                                            \
    const int i = min(tid + (u) * kGvThreads, xtotal - 1);                                     \
    const int xm = i / pieces, c = i - xm * pieces;                                            \
    v = *reinterpret_cast<const uint4 *>(p.X + static_cast<int64_t>(xm) * p.K + k0 + 8 * min(c, kpieces - 1)); \
  }
  QNF4_XLOAD(0, x0) QNF4_XLOAD(1, x1) QNF4_XLOAD(2, x2) QNF4_XLOAD(3, x3)
#undef QNF4_XLOAD
  // absmax bytes (packed dwords, or one per entry) with DQ; without it the
  // fp32 constant of this lane's block in each super-block
  uint32_t am[kDq ? (kAligned ? NB / 4 : NB) : 1];
  float af[kDq ? 1 : NS];
  if constexpr (!kDq) {
#pragma unroll
    for (int s = 0; s < NS; ++s) af[s] = p.absmax[b0 + min(s * BD + bg, nblk - 1)];
  } else if constexpr (kAligned) {
    const uint32_t *ap = reinterpret_cast<const uint32_t *>(p.absmax_q + b0);
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) am[i] = ap[min(i, nblk / 4 - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < NB; ++j) am[j] = static_cast<uint8_t>(p.absmax_q[b0 + min(j, nblk - 1)]);
  }
  const int64_t d0 = b0 / kDqBlock;                // a split spans at most two DQ blocks
  const float s0 = kDq ? p.dq_scale[d0] : 0.0f;
  const float s1 = kDq ? p.dq_scale[(b0 + nblk - 1) / kDqBlock] : 0.0f;
  const float mu = kDq ? p.dq_mean[0] : 0.0f;
  // thread t holds A[jr, k0 + 2t .. +1] of rows jr0 and jr0 + gx (last: only
  // the H partials at the end use them)
  const int ka = min(2 * tid, kc - 2);
  auto aload = [&](int jr) {
    return *reinterpret_cast<const float2 *>(p.A + static_cast<int64_t>(min(jr, p.r - 1)) * p.K + k0 + ka);
  };
  float2 a0 = make_float2(0.f, 0.f), a1 = a0;
  if (jr0 < p.r) {
    a0 = aload(jr0);
    a1 = aload(jr0 + gx);
  }

  // ---- LDS: byte table (entry (b, copy) = (level[b >> 4], level[b & 15]);
  // thread t writes b = t / 32 + 16 i for i < 16 into copy t % 32: the high
  // nibble i is a constant and the low nibble t / 32 takes one value per half
  // wave, so the levels come from kernel arguments without a vector load) and
  // the X chunk (clamped pieces rewrite their own value)
  {
    const float lv_lo = p.tab.lv[2 * w], lv_hi = p.tab.lv[2 * w + 1];
    const float lv_low = lane < 32 ? lv_lo : lv_hi;   // level[t / 32]
#pragma unroll
    for (int i = 0; i < 16; ++i) lut[tid + kGvThreads * i] = pack_bf16x2(p.tab.lv[i], lv_low);
  }
#define QNF4_XSTORE(u, v)                                                                       \
  {                                                                                            \
    const int i = min(tid + (u) * kGvThreads, xtotal - 1);                                     \
    const int xm = i / pieces, c = i - xm * pieces;                                            \
    *reinterpret_cast<uint4 *>(xs + xm * kGvXStride + 8 * c) = c < kpieces ? v : make_uint4(0, 0, 0, 0); \
  }
  QNF4_XSTORE(0, x0) QNF4_XSTORE(1, x1) QNF4_XSTORE(2, x2) QNF4_XSTORE(3, x3)
#undef QNF4_XSTORE
  __syncthreads();

  // The code stream starts only now: loads issued before the barrier would
  // queue ahead of, or beside, every workgroup's X chunk and delay it.
  CodeWords<BD> cw[NS];
#pragma unroll
  for (int s = 0; s < P; ++s) cw[s].load(cptr(s));
  // block scale of this lane's block in each super-block (0 past the end);
  // formed after the barrier, so that nothing before it waits for the
  // code words issued behind the DQ scales
  const float kd0 = __fdiv_rn(s0, 127.0f);
  const float kd1 = __fdiv_rn(s1, 127.0f);
  float cs[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int j = s * BD + bg;
    if constexpr (!kDq) {
      cs[s] = j < nblk ? af[s] : 0.0f;
    } else {
      const float kd = (b0 + j) / kDqBlock == d0 ? kd0 : kd1;
      int q;
      if constexpr (kAligned) {
        uint32_t word = am[0];
#pragma unroll
        for (int i = 1; i < NB / 4; ++i) word = (j >> 2) == i ? am[i] : word;
        q = static_cast<int8_t>(word >> (8 * (j & 3)));
      } else {
        uint32_t byte = am[0];
#pragma unroll
        for (int i = 1; i < NB; ++i) byte = j == i ? am[i] : byte;
        q = static_cast<int8_t>(byte);
      }
      cs[s] = j < nblk ? __fadd_rn(__fmul_rn(static_cast<float>(q), kd), mu) : 0.0f;
    }
  }
  // ---- decode + MFMA, one super-block at a time, P super-blocks of code
  // words in flight. The A operand of lane (row rho, group g) is X row
  // rho % RB when its row group rho / RB is this lane group's block, else 0.
  const int rho = lane & 15;
  const bool xact = rho / RB == bg && rho % RB < M;
  const __bf16 *xrow = xs + (rho % RB) * kGvXStride + kBlock * bg + 16 * BD * sub;
  const uint32_t *lt = lut + (lane & (kLutCopies - 1));
  bf16x8 xv[NW];
#pragma unroll
  for (int q = 0; q < NW; ++q) xv[q] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4 zero = acc;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    asm volatile("" ::: "memory");   // keep the prefetch distance: no load moves across
    if (s + P < NS) cw[s + P].load(cptr(s + P));
    if (s * BD >= nblk) continue;    // uniform: the rest of a short split
    if (xact) {
#pragma unroll
      for (int q = 0; q < NW; ++q) xv[q] = *reinterpret_cast<const bf16x8 *>(xrow + kBlock * BD * s + 8 * q);
    }
    f32x4 t = zero;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      const uint32_t wq = cw[s].word(q);
      const uint4 wv = make_uint4(lt[(wq & 0xFFu) * kLutCopies], lt[((wq >> 8) & 0xFFu) * kLutCopies],
                                  lt[((wq >> 16) & 0xFFu) * kLutCopies], lt[(wq >> 24) * kLutCopies]);
      t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[q], __builtin_bit_cast(bf16x8, wv), t, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(cs[s], t[v], acc[v]);
  }
  // Accumulator register v holds MFMA row 4 g + v: row group bg, X row
  // (4 g + v) % RB. Sum the row groups (lanes 16 and 32 apart), fixed order.
  if constexpr (BD == 4) {
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += __shfl_xor(acc[v], 16, 64);
  }
  if constexpr (BD >= 2) {
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += __shfl_xor(acc[v], 32, 64);
  }
  if (n_ok && g < G) {
    float *out = p.part + static_cast<int64_t>(z) * p.M * p.N + n;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = (4 * g + v) % RB;
      if (row < M) out[static_cast<int64_t>(row) * p.N] = acc[v];
    }
  }

  // ---- split partials of H = X A^T for the adapter rows jr0 + i gx: thread
  // (row hm, slice sl) forms a 32-long dot product over the chunk, the 32
  // slices of a row (consecutive lanes) are summed by an xor butterfly. The
  // first two rows of A were loaded at the start; they are staged only now,
  // so that nothing before the main loop waits for them.
  const int hm = tid >> 5, sl = tid & 31;
  const bool kin = 2 * tid < kc;
  for (int jp = jr0; jp < p.r; jp += 2 * gx) {
    const float2 b0v = jp == jr0 ? a0 : aload(jp), b1v = jp == jr0 ? a1 : aload(jp + gx);
    __syncthreads();   // every wave is past the main loop / the previous pair
    *reinterpret_cast<float2 *>(&as_[0][2 * tid]) = kin ? b0v : make_float2(0.f, 0.f);
    *reinterpret_cast<float2 *>(&as_[1][2 * tid]) = kin && jp + gx < p.r ? b1v : make_float2(0.f, 0.f);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int jr = jp + i * gx;
      if (jr >= p.r) break;
      const uint4 *xp = reinterpret_cast<const uint4 *>(xs + hm * kGvXStride + 32 * sl);
      const float4 *ap = reinterpret_cast<const float4 *>(&as_[i][32 * sl]);
      float acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 xq = xp[u];
        const float4 av0 = ap[2 * u], av1 = ap[2 * u + 1];
        acc4[0] = __builtin_fmaf(av0.x, __uint_as_float(xq.x << 16), acc4[0]);
        acc4[1] = __builtin_fmaf(av0.y, __uint_as_float(xq.x & 0xFFFF0000u), acc4[1]);
        acc4[2] = __builtin_fmaf(av0.z, __uint_as_float(xq.y << 16), acc4[2]);
        acc4[3] = __builtin_fmaf(av0.w, __uint_as_float(xq.y & 0xFFFF0000u), acc4[3]);
        acc4[0] = __builtin_fmaf(av1.x, __uint_as_float(xq.z << 16), acc4[0]);
        acc4[1] = __builtin_fmaf(av1.y, __uint_as_float(xq.z & 0xFFFF0000u), acc4[1]);
        acc4[2] = __builtin_fmaf(av1.z, __uint_as_float(xq.w << 16), acc4[2]);
        acc4[3] = __builtin_fmaf(av1.w, __uint_as_float(xq.w & 0xFFFF0000u), acc4[3]);
      }
      float hsum = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) hsum += __shfl_xor(hsum, o, 64);
      if (sl == 0 && hm < M) p.hpart[(static_cast<int64_t>(z) * p.M + hm) * p.r + jr] = hsum;
    }
  }
}

// Y = bf16(sum_z part[z] + bf16(s H) bf16(B)^T), H = sum_z hpart[z].
// Split partials are summed in index order, in groups of four whose loads are
// all issued before the first add (clamped indices, zero weight past the end).
__global__ __launch_bounds__(kFinThreads) void k_gemv_finish(GemvParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 hs[kGvRows * (256 + 8)];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int M = static_cast<int>(p.M);
  const int r = p.r, splits = p.splits;
  const int rp = (r + 31) / 32 * 32;
  const int hstride = rp + 8;
  const int64_t n_raw = static_cast<int64_t>(blockIdx.x) * kFinCols + w * 16 + (lane & 15);
  const int64_t n = n_raw < p.N ? n_raw : p.N - 1;
  const int g = lane >> 4;
  const int64_t plane = p.M * p.N;

  // Every load that does not depend on another goes out first: B for the
  // first 64 adapter columns, the first four Y partials, then the H partials.
  // Columns of B past r are clamped to column r - 1: they meet zeros in bf16(s H).
  const float *brow = p.B + n * r;
  auto bload = [&](int j0, float *b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = brow[min(j0 + 8 * g + i, r - 1)];
  };
  float bA[8], bB[8];
  if (r > 0) {
    bload(0, bA);
    bload(32, bB);
  }
  float y0[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t zz = min(u, splits - 1);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      y0[u][v] = p.part[zz * plane + static_cast<int64_t>(min(4 * g + v, M - 1)) * p.N + n];
  }

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (r > 0) {
    // bf16(s H) into LDS, two entries per thread per pass, their split
    // partials loaded together (clamped entries are computed and dropped)
    const int ne = M * rp;
    for (int e0 = tid; e0 < ne; e0 += 2 * kFinThreads) {
      int ie[2], je[2], jc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int e = min(e0 + t * kFinThreads, ne - 1);
        ie[t] = e / rp;
        je[t] = e - ie[t] * rp;
        jc[t] = min(je[t], r - 1);
      }
      float v[2] = {0.0f, 0.0f};
      for (int z0 = 0; z0 < splits; z0 += 4) {
        float gq[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            gq[t][u] = p.hpart[(static_cast<int64_t>(min(z0 + u, splits - 1)) * p.M + ie[t]) * r + jc[t]];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int u = 0; u < 4; ++u) v[t] += z0 + u < splits ? gq[t][u] : 0.0f;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (e0 + t * kFinThreads < ne)
          hs[ie[t] * hstride + je[t]] = static_cast<__bf16>(je[t] < r ? p.scale * v[t] : 0.0f);
    }
    __syncthreads();
    const __bf16 *hrow = hs + (lane & 15) * hstride + 8 * g;   // rows >= M feed unstored outputs
    auto mma = [&](int j0, const float *b) {
      const uint4 bv = make_uint4(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]), pack_bf16x2(b[4], b[5]),
                                  pack_bf16x2(b[6], b[7]));
      const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(hrow + j0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    };
    mma(0, bA);
    if (rp > 32) mma(32, bB);
    for (int j0 = 64; j0 < rp; j0 += 32) {
      float b[8];
      bload(j0, b);
      mma(j0, b);
    }
  }

  float y[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    y[v] = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) y[v] += u < splits ? y0[u][v] : 0.0f;
  }
  for (int z0 = 4; z0 < splits; z0 += 4) {
    float gq[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t zz = min(z0 + u, splits - 1);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        gq[u][v] = p.part[zz * plane + static_cast<int64_t>(min(4 * g + v, M - 1)) * p.N + n];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int u = 0; u < 4; ++u) y[v] += z0 + u < splits ? gq[u][v] : 0.0f;
  }
  if (n_raw >= p.N) return;
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (4 * g + v < M) p.Y[static_cast<int64_t>(4 * g + v) * p.N + n] = static_cast<__bf16>(y[v] + acc[v]);
}

// Splits of K: kGvMaxBlocks blocks each (the last one may be shorter).
struct GemvSplit {
  int splits, blocks;
};
GemvSplit gemv_split(int64_t N, int64_t K) {
  (void)N;
  return {static_cast<int>(ceil_div(K / kBlock, kGvMaxBlocks)), kGvMaxBlocks};
}

template <int BD>
void launch_stream(bool aligned, bool dq, dim3 grid, hipStream_t s, const GemvParams &p) {
  if (dq) {
    if (aligned) hipLaunchKernelGGL((k_gemv<BD, true, true>), grid, dim3(kGvThreads), 0, s, p);
    else hipLaunchKernelGGL((k_gemv<BD, false, true>), grid, dim3(kGvThreads), 0, s, p);
  } else {
    if (aligned) hipLaunchKernelGGL((k_gemv<BD, true, false>), grid, dim3(kGvThreads), 0, s, p);
    else hipLaunchKernelGGL((k_gemv<BD, false, false>), grid, dim3(kGvThreads), 0, s, p);
  }
}

size_t part_bytes(int64_t N, int64_t K) {
  return align_up(static_cast<size_t>(gemv_split(N, K).splits * kGvRows * N) * sizeof(float), 256);
}

}  // namespace

size_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K, int r) {
  (void)M;
  return part_bytes(N, K) + align_up(static_cast<size_t>(gemv_split(N, K).splits * kGvRows * r) * sizeof(float), 256);
}

hipError_t launch_gemv(const LinearArgs &a, const void *X, const float *A, const float *B, void *Y, void *ws,
                       hipStream_t s) {
  GemvParams p{};
  p.codes = a.codes;
  p.absmax_q = a.absmax_q;
  p.dq_scale = a.dq_scale;
  p.dq_mean = a.dq_mean;
  p.absmax = a.absmax;
  p.A = A;
  p.B = B;
  p.N = a.N;
  p.K = a.K;
  p.r = a.r;
  p.scale = a.scale;
  p.tab = format_tables(a.format);
  const GemvSplit sp = gemv_split(a.N, a.K);
  p.splits = sp.splits;
  p.split_blocks = sp.blocks;
  p.part = static_cast<float *>(ws);
  p.hpart = reinterpret_cast<float *>(static_cast<char *>(ws) + part_bytes(a.N, a.K));
  const dim3 grid(static_cast<unsigned>(ceil_div(a.N, kGvCols)), static_cast<unsigned>(p.splits));
  // passes of up to 16 rows, in order on the stream (they share the workspace)
  const bool aligned = a.K % 256 == 0, dq = fmt_dq(a.format);
  for (int64_t row0 = 0; row0 < a.M; row0 += kGvRows) {
    p.M = std::min<int64_t>(kGvRows, a.M - row0);
    p.X = static_cast<const __bf16 *>(X) + row0 * a.K;
    p.Y = static_cast<__bf16 *>(Y) + row0 * a.N;
    prof_begin(kProfFwdGemm, s);
    if (p.M <= 4) launch_stream<4>(aligned, dq, grid, s, p);
    else if (p.M <= 8) launch_stream<2>(aligned, dq, grid, s, p);
    else launch_stream<1>(aligned, dq, grid, s, p);
    prof_end(kProfFwdGemm, s);
    hipLaunchKernelGGL(k_gemv_finish, dim3(static_cast<unsigned>(ceil_div(a.N, kFinCols))), dim3(kFinThreads), 0,
                       s, p);
  }
  return hipGetLastError();
}

}  // namespace qnf4
