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
//                  owns 16 output columns. Each lane issues every code and
//                  absmax load of its split up front, so the whole weight is in
//                  flight at once; while those loads travel the workgroup
//                  stages its X chunk in LDS, forms its share of the split
//                  partials of H = X A^T and builds a byte table. Then, per
//                  64-element block, a lane maps its 8 code bytes to bf16 level
//                  pairs (8 table lookups = two MFMA operands), runs two
//                  v_mfma_f32_16x16x32_bf16 into a temporary and adds
//                  c_b * temporary to its accumulator: the block scale is
//                  applied once per block and output, not once per weight.
//   k_gemv_finish  per output: the fixed-order sum of the split partials plus
//                  the adapter term bf16(s H) bf16(B)^T (MFMA), rounded to bf16.
// Within a block the reduction order is free: lane group g (lane / 16) takes
// elements 16g .. 16g + 15 (8 contiguous code bytes) and reads X in the same
// order. Levels enter the MFMA as bf16 and c_b is applied in fp32, so Y
// differs from bf16(X bf16(W-hat)^T) at the bf16 operand level.
#include <algorithm>

#include "gemm_core.h"

namespace qnf4 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGvRows = 16;                  // rows of X per pass
constexpr int kGvWaves = 8;
constexpr int kGvThreads = 64 * kGvWaves;    // 512
constexpr int kGvCols = 16 * kGvWaves;       // output columns per workgroup
constexpr int kGvBlocks = 16;                // 64-element blocks per split
constexpr int kGvChunk = kGvBlocks * kBlock; // K elements per split
constexpr int kGvXStride = kGvChunk + 8;     // bf16; +16 bytes keeps b128 reads conflict-free
constexpr int kLutCopies = 32;               // one table copy per LDS bank: conflict-free lookups

struct GemvParams {
  const __bf16 *X;        // [M][K]
  const uint8_t *codes;   // [N][K/2]
  const int8_t *absmax_q; // [N*K/64]
  const float *dq_scale;  // [nd]
  const float *dq_mean;   // [1]
  const float *A;         // [r][K] fp32, or null when r == 0
  const float *B;         // [N][r] fp32, or null when r == 0
  float *part;            // [splits][M][N] fp32
  float *hpart;           // [splits][M][r] fp32
  __bf16 *Y;              // [M][N]
  int64_t M, N, K;        // M <= 16
  int r, splits;
  float scale;
  Nf4Tables tab;
};

// kAligned: K is a multiple of 256, so each lane's absmax bytes are whole dwords.
template <bool kAligned>
__global__ __launch_bounds__(kGvThreads, 2) void k_gemv(GemvParams p) {
  constexpr int NB = kGvBlocks;
  constexpr int kEarly = 4;   // code words loaded before the X chunk is staged
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * kLutCopies];   // 32 KB
  __shared__ __attribute__((aligned(16))) __bf16 xs[kGvRows * kGvXStride];
  __shared__ __attribute__((aligned(16))) float as_[2][kGvChunk];          // two rows of A

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int z = blockIdx.y;
  const int64_t k0 = static_cast<int64_t>(z) * kGvChunk;
  const int kc = static_cast<int>(min<int64_t>(kGvChunk, p.K - k0));   // a multiple of 64
  const int nblk = kc / kBlock;
  const int M = static_cast<int>(p.M);
  const int gx = gridDim.x, jr0 = blockIdx.x;

  // ---- the first code words of this lane's split (they keep HBM busy while
  // the small operands make their round trip). Loads past the end of a short
  // split are clamped to its last block (in bounds, weight zero), so the load
  // sequence has no branches.
  const int64_t n_raw = static_cast<int64_t>(blockIdx.x) * kGvCols + w * 16 + (lane & 15);
  const bool n_ok = n_raw < p.N;
  const int64_t n = n_ok ? n_raw : p.N - 1;
  const int g = lane >> 4;
  const int64_t kb = p.K / kBlock;                 // blocks per weight row (a multiple of 4 if kAligned)
  const int64_t b0 = n * kb + k0 / kBlock;         // first block of this lane's split
  const uint2 *cp = reinterpret_cast<const uint2 *>(p.codes + b0 * (kBlock / 2) + 8 * g);
  uint2 cw[NB];
#pragma unroll
  for (int j = 0; j < kEarly; ++j) cw[j] = cp[4 * min(j, nblk - 1)];

  // ---- X chunk (16-byte pieces in named registers), two rows of A, absmax
  // bytes, DQ scales. Columns past the end of a short split are staged as
  // zero, so blocks past the end contribute exactly nothing.
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
  // thread t stages A[jr, k0 + 2t .. +1] of rows jr0 and jr0 + gx
  const int ka = min(2 * tid, kc - 2);
  auto aload = [&](int jr) {
    return *reinterpret_cast<const float2 *>(p.A + static_cast<int64_t>(min(jr, p.r - 1)) * p.K + k0 + ka);
  };
  float2 a0 = make_float2(0.f, 0.f), a1 = a0;
  if (jr0 < p.r) {
    a0 = aload(jr0);
    a1 = aload(jr0 + gx);
  }
  uint32_t am[kAligned ? NB / 4 : NB];   // absmax bytes: packed dwords, or one per entry
  if constexpr (kAligned) {
    const uint32_t *ap = reinterpret_cast<const uint32_t *>(p.absmax_q + b0);
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) am[i] = ap[min(i, nblk / 4 - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < NB; ++j) am[j] = static_cast<uint8_t>(p.absmax_q[b0 + min(j, nblk - 1)]);
  }
  const int64_t d0 = b0 / kDqBlock;                // a split spans at most two DQ blocks
  const float s0 = p.dq_scale[d0];
  const float s1 = p.dq_scale[(b0 + nblk - 1) / kDqBlock];
  const float mu = p.dq_mean[0];

  // ---- LDS: byte table (entry (b, copy) = (level[b >> 4], level[b & 15]);
  // thread t writes b = t / 32 + 16 i for i < 16 into copy t % 32), the X
  // chunk (clamped pieces rewrite their own value) and the two A rows
  const float lv_low = p.tab.lv[tid >> 5];
#pragma unroll
  for (int i = 0; i < 16; ++i) lut[tid + kGvThreads * i] = pack_bf16x2(p.tab.lv[i], lv_low);
#define QNF4_XSTORE(u, v)                                                                       \
  {                                                                                            \
    const int i = min(tid + (u) * kGvThreads, xtotal - 1);                                     \
    const int xm = i / pieces, c = i - xm * pieces;                                            \
    *reinterpret_cast<uint4 *>(xs + xm * kGvXStride + 8 * c) = c < kpieces ? v : make_uint4(0, 0, 0, 0); \
  }
  QNF4_XSTORE(0, x0) QNF4_XSTORE(1, x1) QNF4_XSTORE(2, x2) QNF4_XSTORE(3, x3)
#undef QNF4_XSTORE
  const bool kin = 2 * tid < kc;
  *reinterpret_cast<float2 *>(&as_[0][2 * tid]) = kin && jr0 < p.r ? a0 : make_float2(0.f, 0.f);
  *reinterpret_cast<float2 *>(&as_[1][2 * tid]) = kin && jr0 + gx < p.r ? a1 : make_float2(0.f, 0.f);
  const float kd0 = __fdiv_rn(s0, 127.0f);
  const float kd1 = __fdiv_rn(s1, 127.0f);
  __syncthreads();

  // ---- the rest of the code words, then decode + MFMA one block at a time
#pragma unroll
  for (int j = kEarly; j < NB; ++j) cw[j] = cp[4 * min(j, nblk - 1)];
  float cs[NB];               // block scales; 0 past the end of a short split
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const float kd = (b0 + j) / kDqBlock == d0 ? kd0 : kd1;
    const int q = kAligned ? static_cast<int8_t>(am[j / 4] >> (8 * (j % 4))) : static_cast<int8_t>(am[j]);
    cs[j] = j < nblk ? __fadd_rn(__fmul_rn(static_cast<float>(q), kd), mu) : 0.0f;
  }
  // Lanes of rows >= M read rows of the chunk that feed only unstored outputs.
  const __bf16 *xrow = xs + (lane & 15) * kGvXStride + 16 * g;
  const uint32_t *lt = lut + (lane & (kLutCopies - 1));
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4 zero = acc;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const uint32_t w0 = cw[j].x, w1 = cw[j].y;
    const uint4 wv0 = make_uint4(lt[(w0 & 0xFFu) * kLutCopies], lt[((w0 >> 8) & 0xFFu) * kLutCopies],
                                 lt[((w0 >> 16) & 0xFFu) * kLutCopies], lt[(w0 >> 24) * kLutCopies]);
    const uint4 wv1 = make_uint4(lt[(w1 & 0xFFu) * kLutCopies], lt[((w1 >> 8) & 0xFFu) * kLutCopies],
                                 lt[((w1 >> 16) & 0xFFu) * kLutCopies], lt[(w1 >> 24) * kLutCopies]);
    const bf16x8 xv0 = *reinterpret_cast<const bf16x8 *>(xrow + kBlock * j);
    const bf16x8 xv1 = *reinterpret_cast<const bf16x8 *>(xrow + kBlock * j + 8);
    f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv0, __builtin_bit_cast(bf16x8, wv0), zero, 0, 0, 0);
    t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv1, __builtin_bit_cast(bf16x8, wv1), t, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(cs[j], t[v], acc[v]);
  }
  // accumulator register v holds row 4 g + v of column n
  if (n_ok) {
    float *out = p.part + static_cast<int64_t>(z) * p.M * p.N + n;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (4 * g + v < M) out[static_cast<int64_t>(4 * g + v) * p.N] = acc[v];
  }

  // ---- split partials of H = X A^T for the adapter rows jr0 + i gx: thread
  // (row hm, slice sl) forms a 32-long dot product over the chunk, the 32
  // slices of a row (consecutive lanes) are summed by an xor butterfly.
  const int hm = tid >> 5, sl = tid & 31;
  for (int jp = jr0; jp < p.r; jp += 2 * gx) {
    if (jp != jr0) {   // further row pairs (narrow N): stage them first
      __syncthreads();
      const float2 b0v = aload(jp), b1v = aload(jp + gx);
      *reinterpret_cast<float2 *>(&as_[0][2 * tid]) = kin ? b0v : make_float2(0.f, 0.f);
      *reinterpret_cast<float2 *>(&as_[1][2 * tid]) = kin && jp + gx < p.r ? b1v : make_float2(0.f, 0.f);
      __syncthreads();
    }
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
__global__ __launch_bounds__(kGvThreads) void k_gemv_finish(GemvParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 hs[kGvRows * (256 + 8)];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int M = static_cast<int>(p.M);
  const int r = p.r, splits = p.splits;
  const int rp = (r + 31) / 32 * 32;
  const int hstride = rp + 8;
  const int64_t n_raw = static_cast<int64_t>(blockIdx.x) * kGvCols + w * 16 + (lane & 15);
  const int64_t n = n_raw < p.N ? n_raw : p.N - 1;
  const int g = lane >> 4;
  const int64_t plane = p.M * p.N;

  // first group of Y partials: in flight while the adapter term is formed
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
#pragma unroll 2
    for (int e = tid; e < M * rp; e += kGvThreads) {
      const int i = e / rp, j = e - i * rp;
      const int jc = min(j, r - 1);
      float v = 0.0f;
      for (int z0 = 0; z0 < splits; z0 += 4) {
        float gq[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          gq[u] = p.hpart[(static_cast<int64_t>(min(z0 + u, splits - 1)) * p.M + i) * r + jc];
#pragma unroll
        for (int u = 0; u < 4; ++u) v += z0 + u < splits ? gq[u] : 0.0f;
      }
      hs[i * hstride + j] = static_cast<__bf16>(j < r ? p.scale * v : 0.0f);
    }
    __syncthreads();
    const float *brow = p.B + n * r;
    const __bf16 *hrow = hs + (lane & 15) * hstride + 8 * g;   // rows >= M feed unstored outputs
    for (int j0 = 0; j0 < rp; j0 += 32) {
      float b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int col = j0 + 8 * g + i;
        const float bv = brow[min(col, r - 1)];
        b[i] = col < r ? bv : 0.0f;
      }
      const uint4 bv = make_uint4(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]), pack_bf16x2(b[4], b[5]),
                                  pack_bf16x2(b[6], b[7]));
      const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(hrow + j0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
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

int64_t gemv_splits(int64_t K) { return ceil_div(K, kGvChunk); }

size_t part_bytes(int64_t K, int64_t N) {
  return align_up(static_cast<size_t>(gemv_splits(K) * kGvRows * N) * sizeof(float), 256);
}

}  // namespace

size_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K, int r) {
  (void)M;
  return part_bytes(K, N) + align_up(static_cast<size_t>(gemv_splits(K) * kGvRows * r) * sizeof(float), 256);
}

hipError_t launch_gemv(const LinearArgs &a, const void *X, const float *A, const float *B, void *Y, void *ws,
                       hipStream_t s) {
  GemvParams p{};
  p.codes = a.codes;
  p.absmax_q = a.absmax_q;
  p.dq_scale = a.dq_scale;
  p.dq_mean = a.dq_mean;
  p.A = A;
  p.B = B;
  p.N = a.N;
  p.K = a.K;
  p.r = a.r;
  p.scale = a.scale;
  p.tab = nf4_tables();
  p.splits = static_cast<int>(gemv_splits(a.K));
  p.part = static_cast<float *>(ws);
  p.hpart = reinterpret_cast<float *>(static_cast<char *>(ws) + part_bytes(a.K, a.N));
  const dim3 grid(static_cast<unsigned>(ceil_div(a.N, kGvCols)), static_cast<unsigned>(p.splits));
  // passes of up to 16 rows, in order on the stream (they share the workspace)
  for (int64_t row0 = 0; row0 < a.M; row0 += kGvRows) {
    p.M = std::min<int64_t>(kGvRows, a.M - row0);
    p.X = static_cast<const __bf16 *>(X) + row0 * a.K;
    p.Y = static_cast<__bf16 *>(Y) + row0 * a.N;
    prof_begin(kProfFwdGemm, s);
    if (a.K % 256 == 0)
      hipLaunchKernelGGL(k_gemv<true>, grid, dim3(kGvThreads), 0, s, p);
    else
      hipLaunchKernelGGL(k_gemv<false>, grid, dim3(kGvThreads), 0, s, p);
    prof_end(kProfFwdGemm, s);
    hipLaunchKernelGGL(k_gemv_finish, dim3(grid.x), dim3(kGvThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace qnf4
