// Skinny-M QLoRA forward (decode, M <= 32 rows of X):
//   Y = X W^T + s (X A^T) B^T
// in ONE launch per call, with the 4-bit weight streamed from HBM once and
// decoded on the fly (QLoRA vs ChatGPT page, capability "training pipeline":
// block-wise dequantization of the 4-bit base in the forward pass; capability
// "LoRA on the quantized base": a frozen base plus a full-precision adapter).
//
// Two kernels. One row of X with K <= 16384 (single-token decode) takes the
// row-stream kernel k_gemv_rows further down: no matrix cores, X in
// registers, the levels through a byte-indexed table and v_dot2_f32_bf16.
// Everything else (M = 2 .. 32, longer rows, or an adapter whose published
// columns would not fit the synchronization words) takes k_gemv, below.
//
// k_gemv: grid = U adapter workgroups, then S x C weight workgroups.
//
// Weight workgroups. Strip s owns 16 T consecutive weight rows (outputs n);
// its C workgroups split the reduction into chunks whose slice of X fits in
// LDS (C = 1 whenever all of X fits). The 8 waves of a workgroup take T row
// tiles of 16 x KS = 8 / T reduction slices. Each lane issues the code loads
// of its slice in two halves (16 bytes per quad-piece: 128 elements of its
// row = two 64-blocks; lane group g = lane / 16 holds bytes 16 g .. 16 g + 15,
// i.e. half g % 2 of block g / 2), then decodes byte by byte through a table
// of bf16 level pairs in LDS into the B operand of v_mfma_f32_16x16x32_bf16.
// The A operand is X in block-diagonal form: MFMA rows 0-7 carry X rows
// 8 mt .. 8 mt + 7 against the lanes of block 0 (lane groups 0, 1), rows 8-15
// the same X rows against block 1 (lane groups 2, 3), zero elsewhere. An
// output lane therefore holds only its own block's contribution and scales it
// by that block's constant c_b after the four MFMAs of the quad-piece: the
// scale costs one FMA per output and block, not one multiply per weight. The
// two block halves are added across lanes once at the end, the slices in a
// fixed order through LDS.
//
// Split reduction (C > 1): a workgroup writes its fp32 partial and bumps its
// strip's arrival counter; the last of the C to arrive sums the C partials in
// chunk order, resets the counter and finishes the strip.
//
// Adapter workgroups. Unit u = (column group jg of 16 adapter columns, a
// range hk of the reduction) forms that piece of H = X A^T with the fp32 rows
// of A rounded to bf16 as MFMA operands, writes it and bumps its column
// group's arrival counter. The last of the group's HK units to arrive resets
// the counter, sums the group's pieces in range order into the final H
// columns and marks them published in one flag word per strip. A strip's
// finisher waits for its rp / 16 flags (bounded), resets them, reads H and
// adds bf16(s H) bf16(B)^T on the MFMA to its outputs before rounding Y to
// bf16.
//
// Cross-workgroup data (partials, H pieces, counters, flags) is written with
// write-through stores (agent-scope relaxed atomic stores, sc1), made
// complete with a wait on every outstanding memory access before the
// counter or flag that announces it, and read with agent-scope atomic loads
// (sc1): no L2 write-back or invalidate is issued, since those walk a whole
// XCD's L2. Counters and flags live at the start of the workspace and are
// zero between calls: every word a call raises is cleared again by the call
// (the counter by its strip's last arrival, a flag by its strip's finisher).
// Waits are bounded; a wait that runs out sets an error word and the call
// finishes (its output is then wrong). Adapter workgroups come first in the
// grid and never wait, so a waiting finisher never holds a slot an adapter
// workgroup still needs.
//
// Numerics: the base enters the MFMA as bf16(level) and c_b is applied in
// fp32 to each block's partial product; A, B and s H enter as bf16; all
// accumulation is fp32 in a fixed order, so results are deterministic.
#include <algorithm>

#include "gemm_core.h"
#include "xwg.h"

namespace qnf4 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kGvWaves = 8;
constexpr int kGvThreads = 64 * kGvWaves;
constexpr int kLutCopies = 16;                  // table copies: lanes 16 apart share one
constexpr int kLutBytes = 256 * kLutCopies * 4;  // 16 KB
constexpr int kScaleMax = 4096;                  // block constants of a workgroup's region, fp32 in LDS
constexpr int kScaleBytes = kScaleMax * 4;       // 16 KB
constexpr int kXOffset = kLutBytes + kScaleBytes;  // X slice after the table and the constants
constexpr int kZeroBytes = 8 * 512;              // zero row: the largest A-operand read offset of a slice
constexpr int kXPad = 8;                         // bf16 per X row in LDS: b128 reads of 8 rows on distinct banks
constexpr int kXLdsMax = 40 * 1024;              // X slice in LDS: two workgroups per CU (72 KB each)
constexpr int kMaxNq = 16;                       // quad-pieces per wave slice
constexpr int kHBlocks = 16;                     // reduction blocks (1024 elements) per adapter step
constexpr int kMaxUnits = 64;                    // adapter units: a unit's range grows past that
constexpr int kSpinLimit = 1 << 16;              // polls of about 1 us: a wait gives up after about 65 ms
constexpr int kStripTarget = 512;                // weight workgroups: two per CU
constexpr int kGvLdsMax = kXOffset + kXLdsMax + kZeroBytes + 1024;   // dynamic LDS bound of every plan


struct GemvParams {
  const __bf16 *X;         // [M][K]
  const uint8_t *codes;    // [N][K/2]
  const int8_t *absmax_q;  // [N*K/64] (with DQ)
  const float *dq_scale;   // [nd]
  const float *dq_mean;    // [1]
  const float *absmax;     // [N*K/64] fp32 block constants (without DQ)
  const float *A;          // [r][K] fp32 (r > 0)
  const float *B;          // [N][r] fp32 (r > 0)
  __bf16 *Y;               // [M][N]
  float *part;             // [S][C][M][16 T] split partials (C > 1)
  float *hpart;            // [HK][M][rp] pieces of H
  float *hfin;             // [M][rp] H, summed by each column group's last unit
  uint32_t *flags;         // [S][G], G = rp / 16 column groups
  uint32_t *hctr;          // [G] adapter arrival counters
  uint32_t *ctr;           // [S]
  uint32_t *err;           // [1]
  int64_t M, N, K;
  int r, rp;
  float scale;
  int T, S, C;             // row tiles per strip, strips, reduction chunks
  int cq;                  // quad-pieces per chunk (the last may be shorter)
  int U, HK, hb;           // adapter units: (rp / 16) x HK reduction ranges of hb blocks
  int hstep;               // blocks per adapter step (16, or 8 when M > 16)
  int xstride;             // bf16 per X row in LDS
  int zoff;                // byte offset in LDS of a zero row of kZeroBytes
  int rs_nw, rs_P, rs_RW;  // row-stream path: waves per row, rows per pass, rows per workgroup
  Nf4Tables tab;
};


// Raw buffer loads: a load whose offset lies past the buffer's end returns
// zero without a memory access, so every load of the row-stream kernel is
// issued unconditionally (no branch around a load, whose join would make the
// compiler wait for every load in flight) and the ones that must not happen
// get kOob.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t buf_b32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ int buf_i8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return static_cast<int>(static_cast<int8_t>(__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0)));
}

// X[0:M][k0 : k0 + len) (len a multiple of 64) staged into LDS rows of
// `stride` bf16, zero from len up to `width` (a multiple of 8): at most XP
// 16-byte pieces per thread. load() issues the reads (stripes with no piece
// are skipped as a whole, the rest read a clamped, valid address), store()
// writes LDS; in between the caller may issue loads that must not be waited
// for before X (loads complete in issue order).
template <int XP>
struct XStage {
  uint4 v[XP];
  int pieces, total, len8;
  __device__ __forceinline__ void load(const __bf16 *X, int64_t K, int M, int64_t k0, int len, int width) {
    pieces = width / 8;
    total = M * pieces;
    len8 = len / 8;
#pragma unroll
    for (int u = 0; u < XP; ++u) {
      if (u * kGvThreads >= total) break;   // uniform
      const int i = min(static_cast<int>(threadIdx.x) + u * kGvThreads, total - 1);
      const int m = i / pieces, c = min(i - m * pieces, len8 - 1);
      v[u] = *reinterpret_cast<const uint4 *>(X + static_cast<int64_t>(m) * K + k0 + 8 * c);
    }
  }
  __device__ __forceinline__ void store(int stride, __bf16 *xs) const {
#pragma unroll
    for (int u = 0; u < XP; ++u) {
      if (u * kGvThreads >= total) break;   // uniform
      const int i = threadIdx.x + u * kGvThreads;
      if (i >= total) continue;
      const int m = i / pieces, c = i - m * pieces;
      *reinterpret_cast<uint4 *>(xs + m * stride + 8 * c) = c < len8 ? v[u] : make_uint4(0, 0, 0, 0);
    }
  }
};
// pieces per thread: the weight strips' slice (<= kXLdsMax bytes) and the
// adapter units' range (M x 64 hstep, at most 32 x 512 or 16 x 1024)
constexpr int kXPieces = (kXLdsMax / 16 + kGvThreads - 1) / kGvThreads;
constexpr int kHPieces = 16 * kHBlocks * kBlock / 8 / kGvThreads;
constexpr int kScalePieces = kScaleMax / kGvThreads;

// Block constants c_b of a workgroup's region (`rows` weight rows from n0 x
// nblk blocks from blk0) for LDS, element e = row * nblk + block: with DQ
// c_b = fp32(fp32(q_b k_d) + mean), k_d = fp32(scale_d / 127); without it the
// stored fp32 constant. Consecutive threads take consecutive elements, so the
// int8 codes (and the constants) arrive in a few coalesced loads instead of
// one gather per block and lane. load() issues the reads, store() computes
// and writes LDS.
template <bool kDq>
struct ScaleStage {
  int q[kScalePieces];
  float f[kScalePieces];
  int total;
  __device__ __forceinline__ void load(const GemvParams &p, int64_t n0, int rows, int64_t kb, int64_t blk0,
                                       int nblk) {
    total = rows * nblk;
#pragma unroll
    for (int u = 0; u < kScalePieces; ++u) {
      if (u * kGvThreads >= total) break;   // uniform
      const int e = min(static_cast<int>(threadIdx.x) + u * kGvThreads, total - 1);
      const int r = e / nblk, b = e - r * nblk;
      const int64_t gb = min(n0 + r, p.N - 1) * kb + blk0 + b;
      if constexpr (kDq) {
        q[u] = p.absmax_q[gb];
        f[u] = p.dq_scale[gb / kDqBlock];
      } else {
        f[u] = p.absmax[gb];
      }
    }
  }
  __device__ __forceinline__ void store(float mu, float *cs) const {
#pragma unroll
    for (int u = 0; u < kScalePieces; ++u) {
      if (u * kGvThreads >= total) break;   // uniform
      const int e = threadIdx.x + u * kGvThreads;
      if (e >= total) continue;
      cs[e] = kDq ? __fadd_rn(__fmul_rn(static_cast<float>(q[u]), __fdiv_rn(f[u], 127.0f)), mu) : f[u];
    }
  }
};

// ---------------------------------------------------------------- adapter units
// Unit u: adapter columns 16 jg .. 16 jg + 15 over the reduction blocks
// [hk hb, (hk + 1) hb), taken kHBlocks (1024 elements) at a time: X of the
// range staged in LDS, 32-element steps round robin over the waves, A read as
// fp32 and rounded to bf16.
template <int MT16>
__device__ void adapter_unit(const GemvParams &p, char *smem) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int u = blockIdx.x, jg = u / p.HK, hk = u % p.HK;
  const int M = static_cast<int>(p.M);
  const int64_t kb = p.K / kBlock;
  const int64_t ublk0 = static_cast<int64_t>(hk) * p.hb;
  const int64_t ublk1 = min<int64_t>(kb, ublk0 + p.hb);
  __bf16 *xs = reinterpret_cast<__bf16 *>(smem + kXOffset);
  f32x4 *red = reinterpret_cast<f32x4 *>(smem);   // [8 waves][MT16][64 lanes]
  constexpr int kSteps = kHBlocks * kBlock / 32 / kGvWaves;   // 32-element steps per wave and range
  const int j = 16 * jg + (lane & 15), g = lane >> 4;
  const bool jok = j < p.r;
  const float *arow = p.A + static_cast<int64_t>(min(j, p.r - 1)) * p.K + 8 * g;

  f32x4 acc[MT16];
#pragma unroll
  for (int mt = 0; mt < MT16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t blk0 = ublk0; blk0 < ublk1; blk0 += p.hstep) {
    const int nblk = static_cast<int>(min<int64_t>(p.hstep, ublk1 - blk0));
    const int64_t k0 = blk0 * kBlock;
    const int len = nblk * kBlock, nsteps = len / 32;
    XStage<kHPieces> xst;
    xst.load(p.X, p.K, M, k0, len, len);
    float4 av[kSteps][2];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int st = min(w + kGvWaves * i, nsteps - 1);
      av[i][0] = *reinterpret_cast<const float4 *>(arow + k0 + 32 * st);
      av[i][1] = *reinterpret_cast<const float4 *>(arow + k0 + 32 * st + 4);
    }
    __syncthreads();   // the previous range's X is no longer read
    xst.store(p.xstride, xs);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int st = w + kGvWaves * i;
      if (st >= nsteps) break;   // uniform
      const float4 a0 = av[i][0], a1 = av[i][1];
      const uint4 bw = jok ? make_uint4(pack_bf16x2(a0.x, a0.y), pack_bf16x2(a0.z, a0.w), pack_bf16x2(a1.x, a1.y),
                                        pack_bf16x2(a1.z, a1.w))
                           : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < MT16; ++mt) {
        const int m = 16 * mt + (lane & 15);
        bf16x8 xv = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        if (m < M) xv = *reinterpret_cast<const bf16x8 *>(xs + m * p.xstride + 32 * st + 8 * g);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, __builtin_bit_cast(bf16x8, bw), acc[mt], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT16; ++mt) red[(w * MT16 + mt) * 64 + lane] = acc[mt];
  __syncthreads();
  if (w < MT16) {   // wave mt sums the eight waves' tiles of m-tile mt, in wave order
    const int mt = w;
    f32x4 v = red[mt * 64 + lane];
    for (int ww = 1; ww < kGvWaves; ++ww) v += red[(ww * MT16 + mt) * 64 + lane];
    // lane holds rows 16 mt + 4 (lane / 16) + e of column j
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * mt + 4 * g + e;
      if (m < M) st_wt(p.hpart + (static_cast<int64_t>(hk) * M + m) * p.rp + j, v[e]);
    }
  }
  wait_all_memory();
  __syncthreads();   // this unit's piece is complete
  uint32_t *last = reinterpret_cast<uint32_t *>(smem + kXOffset - 4);
  if (tid == 0) *last = __hip_atomic_fetch_add(p.hctr + jg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*last != static_cast<uint32_t>(p.HK - 1)) return;
  // the group's last unit: H[m][16 jg + c] = sum over the HK pieces in range order
  if (tid == 0) st_wt(p.hctr + jg, 0u);
  for (int i = tid; i < M * 16; i += kGvThreads) {   // element (m, c) = (i / 16, i % 16) of the group
    const int64_t off = static_cast<int64_t>(i >> 4) * p.rp + 16 * jg + (i & 15);
    float v[1];
    sum_wt<1>(p.hpart + off, static_cast<int64_t>(M) * p.rp, p.HK, 0, 0, 1, v);
    st_wt(p.hfin + off, v[0]);
  }
  wait_all_memory();
  __syncthreads();
  // published: one flag per strip
  for (int s = tid; s < p.S; s += kGvThreads) st_wt(p.flags + static_cast<int64_t>(s) * (p.rp / 16) + jg, 1u);
}

// ------------------------------------------------------------- weight strips

template <int MT, int NQ, bool kDq>
__global__ __launch_bounds__(kGvThreads, 2) void k_gemv(GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int MT16 = (MT + 1) / 2;
  if (static_cast<int>(blockIdx.x) < p.U) {
    adapter_unit<MT16>(p, smem);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int M = static_cast<int>(p.M);
  const int T = p.T, KS = kGvWaves / T, RN = 16 * T;
  const int b = blockIdx.x - p.U;
  const int s = b / p.C, c = b - s * p.C;
  const int t = w % T, ks = w / T;
  const int64_t kb = p.K / kBlock;                        // blocks per weight row
  const int64_t blk0 = static_cast<int64_t>(c) * 2 * p.cq;  // first block of the chunk
  const int nblk = static_cast<int>(min<int64_t>(2 * p.cq, kb - blk0));
  const int nqp = (nblk + 1) / 2;                         // quad-pieces of the chunk
  const int q0 = ks * nqp / KS, nq = (ks + 1) * nqp / KS - q0;
  const int ln = lane & 15, g = lane >> 4, half = g >> 1;
  const int64_t n_raw = static_cast<int64_t>(s) * RN + 16 * t + ln;
  const int64_t n = n_raw < p.N ? n_raw : p.N - 1;
  const int64_t rowblk = n * kb;
  uint32_t *lut = reinterpret_cast<uint32_t *>(smem);
  float *cs = reinterpret_cast<float *>(smem + kLutBytes);   // [RN][nblk] block constants
  __bf16 *xs = reinterpret_cast<__bf16 *>(smem + kXOffset);

  // ---- prologue: the X slice and the block constants are requested first:
  // they are small and mostly L2 hits, and issued behind the code stream they
  // would wait for it (vector-memory counts retire in order). The code words
  // of the slice are requested in two halves, and quad-piece jq waits for its
  // own code words only, so the decode runs while the rest of the slice
  // streams in. Quad-pieces past the slice and a second block past the end of the
  // chunk read a clamped, valid block and are scaled by 0.
  XStage<kXPieces> xst;
  xst.load(p.X, p.K, M, blk0 * kBlock, nblk * kBlock, nqp * 128);
  ScaleStage<kDq> sst;
  sst.load(p, static_cast<int64_t>(s) * RN, RN, kb, blk0, nblk);
  // a vector load: a scalar one would hold up the prologue's barrier (which
  // waits for scalar accesses too) until it came back from behind the code
  // stream
  const float mu = kDq ? __uint_as_float(buf_b32(buf(p.dq_mean, 4), 0)) : 0.0f;
  // With one row tile of X (M <= 8) the code words are requested right
  // after the table is built, before the prologue's LDS stores of X and the
  // constants: those wait only for the older loads, so the prologue finishes
  // while the code stream arrives. With two row tiles the prologue holds
  // more registers and the requests go out after it (measured faster there).
  auto blk_of = [&](int jq) { return min(2 * (q0 + min(jq, max(nq - 1, 0))) + half, nblk - 1); };
  uint4 cw[NQ];
  // quad-pieces [j0, j1) of the slice; the first half goes out in the
  // prologue, the second half once the first quad-piece is decoded (all at
  // once streamed about 5 % slower at M = 4: fewer requests in flight per CU)
  // (raw buffer loads from the strip's rows: plain loads were moved past the
  // prologue's barrier by the compiler, so the code stream started only after
  // the X slice and the constants had arrived)
  const int64_t nrow0 = static_cast<int64_t>(s) * RN;   // the strip's first row
  const __amdgpu_buffer_rsrc_t bcw =
      buf(p.codes + nrow0 * kb * (kBlock / 2), min<int64_t>(RN, p.N - nrow0) * kb * (kBlock / 2));
  const uint32_t cwoff = static_cast<uint32_t>(((n - nrow0) * kb + blk0) * (kBlock / 2)) + 16u * (g & 1);
  auto request_range = [&](int j0, int j1) {
#pragma unroll
    for (int jq = 0; jq < NQ; ++jq)
      if (jq >= j0 && jq < j1) cw[jq] = buf_b128(bcw, cwoff + static_cast<uint32_t>(blk_of(jq)) * (kBlock / 2));
  };
  auto request_codes = [&]() { request_range(0, NQ / 2); };

  // ---- the level-pair table, the X slice and the block constants into
  // LDS. Entry (byte e, copy c) at e * 16 + c holds (level[e >> 4],
  // level[e & 15]); thread tid writes entries e = tid / 16 + 32 i (copy
  // tid % 16): high nibble 2 i + tid / 256 (wave-uniform), low nibble
  // (tid / 16) % 16. The levels are kernel-argument constants picked by
  // selects: no vector load, which would have to wait behind the code words.
  {
    const int lo_i = (tid >> 4) & 15;
    float lo = p.tab.lv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) lo = lo_i == i ? p.tab.lv[i] : lo;
    const bool odd = (tid >> 8) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) lut[tid + kGvThreads * i] = pack_bf16x2(odd ? p.tab.lv[2 * i + 1] : p.tab.lv[2 * i], lo);
  }
  if constexpr (MT == 1) request_codes();
  xst.store(p.xstride, xs);
  sst.store(mu, cs);
  // the zero row the A operand reads where it is zero (inactive lanes)
  reinterpret_cast<uint2 *>(smem + p.zoff)[tid] = make_uint2(0u, 0u);
  __syncthreads();
  if constexpr (MT != 1) request_codes();

  // ---- decode + MFMA, quad-piece by quad-piece
  const float *crow = cs + (16 * t + ln) * nblk;   // this lane's weight row in the region
  const uint32_t *lt = lut + (lane & (kLutCopies - 1));
  // A operand: lane (row rho = lane % 16, group g) is X row 8 mt + rho % 8
  // when rho / 8 == g / 2 (its block), zero otherwise: those lanes read the
  // zero row, so that every read is one LDS load at an immediate offset
  const int rho = lane & 15;
  const bool blk_lane = (rho >> 3) == half;
  const __bf16 *xzero = reinterpret_cast<const __bf16 *>(smem + p.zoff);
  const __bf16 *xb[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xb[mt] = blk_lane && 8 * mt + (lane & 7) < M ? xs + (8 * mt + (lane & 7)) * p.xstride + 32 * g + 128 * q0 : xzero;
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma clang loop unroll(full)
  for (int jq = 0; jq < NQ; ++jq) {
    if (jq == 0) request_range(NQ / 2, NQ);
    if (jq >= nq) continue;   // uniform
    const int bi = 2 * (q0 + jq) + half;
    // every LDS read of the quad-piece is issued before its first MFMA, so
    // that the reads' latency is paid once per quad-piece, not once per MFMA
    const uint4 cv = cw[jq];
    uint32_t pr[16];   // level pairs of the 16 code bytes
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wq = q == 0 ? cv.x : q == 1 ? cv.y : q == 2 ? cv.z : cv.w;
#pragma unroll
      for (int b = 0; b < 4; ++b) pr[4 * q + b] = lt[((wq >> (8 * b)) & 0xFFu) * kLutCopies];
    }
    bf16x8 xv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[mt][q] = *reinterpret_cast<const bf16x8 *>(xb[mt] + 128 * jq + 8 * q);
    const float cb = bi < nblk ? crow[bi] : 0.0f;
    // two accumulator chains (MFMAs q = 0, 2 and q = 1, 3), added at the end
    f32x4 ta[MT], tb[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      ta[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      tb[mt] = ta[mt];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 bv = make_uint4(pr[4 * q], pr[4 * q + 1], pr[4 * q + 2], pr[4 * q + 3]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 &t = (q & 1) ? tb[mt] : ta[mt];
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[mt][q], __builtin_bit_cast(bf16x8, bv), t, 0, 0, 0);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[mt][e] = __builtin_fmaf(cb, ta[mt][e] + tb[mt][e], acc[mt][e]);
  }
  // ---- B rows of the adapter's up projection for the output waves (slice 0),
  // requested as soon as the main loop's registers are free, so that they
  // travel during the slice sums and the waits below (first 64 columns).
  // The adapter flags are polled by a wave that loads no B rows when there is
  // one (T < 8: the last wave), since a poll completes only after every load
  // its wave issued before (vector-memory loads retire in order); with T = 8
  // every wave is an output wave and wave 0 polls behind its B rows (asking
  // for them after the poll instead measured slower).
  float bpre[16];
  const bool out_wave = ks == 0;
  const bool poller = w == (T < kGvWaves ? kGvWaves - 1 : 0);
  if (p.r > 0 && out_wave) {
    const float *brow = p.B + n * p.r;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) bpre[8 * h + i] = brow[min(32 * h + 8 * g + i, p.r - 1)];
  }

  // the two blocks' rows: lanes l and l + 32 hold the same outputs
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[mt][e] += __shfl_xor(acc[mt][e], 32, 64);
  __syncthreads();   // every wave is done with the table and X

  // ---- slices summed in order through LDS: red[ks][m][RN], then bsum[m][RN]
  float *red = reinterpret_cast<float *>(smem);
  float *bsum = red + KS * M * RN;
  if (lane < 32) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 8 * mt + 4 * g + e;
        if (m < M) red[(ks * M + m) * RN + 16 * t + ln] = acc[mt][e];
      }
  }
  __syncthreads();
  for (int i = tid; i < M * RN; i += kGvThreads) {
    float v = red[i];
    for (int k2 = 1; k2 < KS; ++k2) v += red[k2 * M * RN + i];
    bsum[i] = v;
  }

  // ---- split reduction: the last of the strip's C workgroups finishes it
  if (p.C > 1) {
    float *mine = p.part + (static_cast<int64_t>(s) * p.C + c) * M * RN;
    for (int i = tid; i < M * RN; i += kGvThreads) st_wt(mine + i, bsum[i]);
    wait_all_memory();
    __shared__ uint32_t arrived;
    __syncthreads();
    if (tid == 0) arrived = __hip_atomic_fetch_add(p.ctr + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != static_cast<uint32_t>(p.C - 1)) return;
    if (tid == 0) st_wt(p.ctr + s, 0u);
    const float *all = p.part + static_cast<int64_t>(s) * p.C * M * RN;
    for (int i = tid; i < M * RN; i += 4 * kGvThreads) {
      float v[4];
      sum_wt<4>(all, static_cast<int64_t>(M) * RN, p.C, i, kGvThreads, M * RN, v);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i + j * kGvThreads < M * RN) bsum[i + j * kGvThreads] = v[j];
    }
  }

  // ---- adapter: wait for the column groups' flags, then bf16(s H) into LDS
  __bf16 *hs = xs;   // [MT16 * 16][rp + 8]
  const int hstride = p.rp + 8;
  if (p.r > 0) {
    const int G = p.rp / 16;   // column groups: one flag each (at most 16)
    if (poller) {
      uint32_t *fl = p.flags + static_cast<int64_t>(s) * G;
      for (int spins = 0;; ++spins) {
        const bool mine = lane >= G || ld_wt(fl + lane) != 0u;
        if (__all(mine)) break;
        if (spins >= kSpinLimit) {
          if (lane == 0) atomicOr(p.err, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (lane < G) st_wt(fl + lane, 0u);
    }
    __syncthreads();
    // H is read by the waves that load no B rows when there are such (T < 8),
    // so that its loads do not retire behind theirs
    const int nh = M * p.rp;   // H[m][j], m < M
    const int h0 = T < kGvWaves ? 64 * T : 0;
    for (int e = tid - h0; e < 16 * MT16 * p.rp; e += kGvThreads - h0) {
      if (e < 0) break;
      const int m = e / p.rp, jj = e - m * p.rp;
      const float h = e < nh ? ld_wt(p.hfin + e) : 0.0f;
      hs[m * hstride + jj] = static_cast<__bf16>(e < nh && jj < p.r ? p.scale * h : 0.0f);
    }
  }
  __syncthreads();

  // ---- outputs: waves of slice 0 take their row tile; adapter on the MFMA
  if (!out_wave) return;
  f32x4 ad[MT16];
#pragma unroll
  for (int mt = 0; mt < MT16; ++mt) ad[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // 32 adapter columns j0 .. j0 + 31: B row values bv (this lane's 8 of them)
  auto adapter_mma = [&](int j0, const float *bv) {
    uint32_t wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 8 * g + 2 * i;
      wv[i] = pack_bf16x2(j < p.r ? bv[2 * i] : 0.0f, j + 1 < p.r ? bv[2 * i + 1] : 0.0f);
    }
    const uint4 bw = make_uint4(wv[0], wv[1], wv[2], wv[3]);
#pragma unroll
    for (int mt = 0; mt < MT16; ++mt) {
      const bf16x8 hv = *reinterpret_cast<const bf16x8 *>(hs + (16 * mt + ln) * hstride + j0 + 8 * g);
      ad[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv, __builtin_bit_cast(bf16x8, bw), ad[mt], 0, 0, 0);
    }
  };
  if (p.r > 0) {
    adapter_mma(0, bpre);
    if (p.rp > 32) adapter_mma(32, bpre + 8);
    const float *brow = p.B + n * p.r;
    for (int j0 = 64; j0 < p.rp; j0 += 32) {
      float bvf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) bvf[i] = brow[min(j0 + 8 * g + i, p.r - 1)];
      adapter_mma(j0, bvf);
    }
  }
  if (n_raw >= p.N) return;
#pragma unroll
  for (int mt = 0; mt < MT16; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * mt + 4 * g + e;
      if (m < M) p.Y[static_cast<int64_t>(m) * p.N + n] = static_cast<__bf16>(bsum[m * RN + 16 * t + ln] + ad[mt][e]);
    }
}

// ------------------------------------------------------- row-stream path
// One row of X (M = 1) and K <= 16384: no matrix cores, one 1024-thread
// workgroup per CU. Workgroup b owns up to 8 P consecutive weight rows,
// whole: passes of P rows. A row is split into K / 32 chunks of 16 code bytes
// (32 elements, half a 64-block); thread (row slot rs, chunk slot j) reads
// chunk j of row rs of every pass, so the 64 lanes of a wave read 1 KB of one
// row per load instruction and each thread's 32 elements of X stay in
// registers for the whole call.
//
// Requests are few and early. At the start of a call every wave of the chip
// issues its loads at once, and each vector-memory instruction costs the
// address unit time (64 addresses), out-of-range ones too, so the kernel
// spends as few instructions as the data allow, and waves that have nothing
// to fetch skip a request by a wave-uniform branch: X is fetched once per
// workgroup (16 bytes a thread) and staged in LDS; the int8 constants of the
// workgroup's blocks arrive as one word per thread with their DQ scales and
// the mean, and become c_b in LDS; B rows come 16 bytes a thread (when
// r % 4 == 0); A rows only in the waves that form an adapter column. These
// small requests go out first, then the first D passes' code chunks, one
// instruction per pass (the int8 constant and DQ scale of every pass, read
// per lane, had cost two more). A code byte becomes its bf16 level pair
// through a table in LDS (address: one byte permute of the code word with the
// lane's copy offset), v_dot2_f32_bf16 multiplies the pair with the X pair in
// the register, and the chunk's sum is scaled by its block constant c_b from
// LDS. The passes' sums are reduce-scattered across the wave (three halving
// exchanges, then three full ones); one lane per row writes the wave's
// partial to LDS, and the waves of a row are added in wave order at the end.
//
// Adapter: column j of H = X A^T is formed in fp32 by the row slot that owns
// it (workgroup b, slot rs: columns b + Gw (rs + P t)), round t = 0 from the
// X registers and the A row loaded at the start, after the first passes,
// rounds t > 0 after all passes. A column is published as one write-through
// store of its value into every workgroup's own slot (a word that is zero
// until published: +0 is stored as -0), so it needs no wait for earlier
// stores and no counter. After its passes every workgroup waits (bounded)
// until its r words are nonzero, clears them, and adds s (X A^T) B^T in fp32
// to its rows, B rows having been loaded at the start. So every word is zero
// between calls.
constexpr int kRsEntry = 256;                  // bytes between table entries
constexpr int kRsLds = 256 * kRsEntry;         // 64 KB: 32 copies of an entry fill the first half of its stride
constexpr int kRsAux = 256 * 32;               // floats in the second halves (partials, B rows, s H)
constexpr int kRsThreads = 1024;               // one workgroup per CU: 16 waves
constexpr int kRsWaves = kRsThreads / 64;
constexpr int kRsPasses = 8;                   // passes per workgroup at most (of P rows each)
constexpr int kRsBpre = 4;                     // B values per thread loaded at the start: RW r <= 4 * 1024
constexpr int kRsMaxChunks = 64 * 8;           // K <= 16384: at most 8 waves per row
constexpr int kRsCus = 256;                    // compute units of the GPU
constexpr int kRsXBytes = 16384 * 2;           // X row in LDS (K <= 16384)
constexpr int kRsMaxBlocks = 4096;             // blocks of a workgroup's rows (c_b in LDS)
// 112 KB of LDS, declared static: the table's address is then a constant of
// the kernel, and each lookup address goes to the LDS read as it is (with the
// array declared extern, every lookup paid one more add of its base)
constexpr int kRsLdsTotal = kRsLds + kRsXBytes + kRsMaxBlocks * 4;
constexpr int kRsHword0 = 256;                 // sync word of the H slots: [Gw][r] fp32 bits, 0 = not yet published

__device__ __forceinline__ float *rs_aux(char *smem, int i) {
  return reinterpret_cast<float *>(smem + (i >> 5) * kRsEntry + 128 + 4 * (i & 31));
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }


// fp32(s / 127) for s >= 0 in three operations: the product with fp32(1/127)
// corrected once by its fused remainder. Equal to the correctly rounded
// quotient for every finite fp32 s (checked exhaustively on the host; only
// s = -0 differs, in the sign of the zero).
__device__ __forceinline__ float div127(float s) {
  const float c = 1.0f / 127.0f;
  const float q0 = s * c;
  return __builtin_fmaf(__builtin_fmaf(-q0, 127.0f, s), c, q0);
}

// D passes in flight: 3 without an adapter, 2 with one (where the adapter's
// requests and columns share the start of the call, a third pass in flight
// made the gate/up shape slower)
template <bool kDq, int D>
__global__ __launch_bounds__(kRsThreads) void k_gemv_rows(GemvParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kRsLdsTotal];
  constexpr int NP = kRsPasses;   // passes per workgroup at most
  static_assert(D >= 1 && D <= NP, "passes in flight");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nw = p.rs_nw, P = p.rs_P, RW = p.rs_RW, Gw = p.S;
  const int C = static_cast<int>(p.K / 32);
  const int64_t kb = p.K / kBlock;
  const int b = blockIdx.x;
  const int64_t n0 = static_cast<int64_t>(b) * RW;
  const int rows = static_cast<int>(min<int64_t>(RW, p.N - n0));
  const int npass = (rows + P - 1) / P;
  const int rs = w / nw, wr = w - rs * nw;
  const bool wave_on = rs < P;   // uniform per wave
  const int j = wr * 64 + lane;
  const bool jon = wave_on && j < C;
  // aux floats: row partials [nw][RW], B rows [RW][r], s H [r], H partials [16 waves], H columns [P]
  const int a_b = nw * RW, a_h = a_b + RW * p.r, a_hp = a_h + p.r;
  const int jcol = b + Gw * rs;   // this slot's first adapter column
  const bool producer = p.r > 0 && wave_on && jcol < p.r;
  char *const xs = smem + kRsLds;                                           // X, bf16 [K]
  float *const cs = reinterpret_cast<float *>(smem + kRsLds + kRsXBytes);   // c_b of the rows' blocks
  const int nblk = static_cast<int>(rows * kb);                             // <= kRsMaxBlocks
  const int64_t gblk0 = n0 * kb;

  // ---- small requests first, in as few vector-memory instructions as the
  // data allow: each instruction costs the wave's address unit time (64
  // addresses), out-of-range ones too, and at the start of the call every
  // wave of the chip issues them at once. Waves that have nothing to fetch
  // skip a request by a wave-uniform branch.
  //   X: 16 bytes per thread, staged in LDS (K / 512 instructions per
  //      workgroup instead of four per wave);
  //   block constants: four blocks per thread (int8 codes as one word, their
  //      DQ scales, the mean), made into c_b in LDS;
  //   B rows: four floats per thread (one 16-byte load when r % 4 == 0);
  //   A row: the producer waves only.
  const int xch = static_cast<int>(p.K / 8);   // 16-byte pieces of X (<= 2 per thread)
  uint4 xv[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  {
    const __amdgpu_buffer_rsrc_t bx = buf(p.X, p.K * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kRsThreads * i;
      if (w * 64 + kRsThreads * i < xch) xv[i] = buf_b128(bx, c < xch ? 16u * c : kOob);
    }
  }
  uint32_t qw = 0;   // int8 codes of blocks 4 tid .. + 3 (DQ), or unused
  int qt[3] = {0, 0, 0};   // the bytes of a last, partial word (one lane)
  float cv[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // DQ: scales of the first and last of them, mean; else c_b
  if (w * 256 < nblk) {   // wave-uniform
    if constexpr (kDq) {
      const int full = nblk >> 2;
      qw = buf_b32(buf(p.absmax_q + gblk0, nblk), tid < full ? 4u * tid : kOob);
      if (tid == full && (nblk & 3)) {   // the last, partial word: one lane of one wave
#pragma unroll
        for (int i = 0; i < 3; ++i) qt[i] = buf_i8(buf(p.absmax_q + gblk0, nblk), i < (nblk & 3) ? 4u * tid + i : kOob);
      }
      const __amdgpu_buffer_rsrc_t bs = buf(p.dq_scale, (p.N * kb + kDqBlock - 1) / kDqBlock * 4);
      const bool own = 4 * tid < nblk;
      const int64_t g0 = gblk0 + 4 * tid, g1 = gblk0 + min(4 * tid + 3, nblk - 1);
      cv[0] = __uint_as_float(buf_b32(bs, own ? static_cast<uint32_t>(g0 / kDqBlock) * 4u : kOob));
      cv[1] = __uint_as_float(buf_b32(bs, own ? static_cast<uint32_t>(g1 / kDqBlock) * 4u : kOob));
      cv[2] = __uint_as_float(buf_b32(buf(p.dq_mean, 4), 0));
    } else {
      const __amdgpu_buffer_rsrc_t ba32 = buf(p.absmax + gblk0, static_cast<int64_t>(nblk) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = 4 * tid + i;
        cv[i] = __uint_as_float(buf_b32(ba32, g < nblk ? 4u * g : kOob));
      }
    }
  }
  const int nbe = rows * p.r;
  const bool b4 = (p.r & 3) == 0;   // B rows as 16-byte loads: element 4 tid + i, else tid + 1024 i
  float bpre[kRsBpre] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (p.r > 0) {
    const __amdgpu_buffer_rsrc_t bbr = buf(p.B + n0 * p.r, static_cast<int64_t>(nbe) * 4);
    if (b4) {
      if (w * 256 < nbe) {   // wave-uniform
        const uint4 v = buf_b128(bbr, 4 * tid < nbe ? 16u * tid : kOob);
        bpre[0] = __uint_as_float(v.x);
        bpre[1] = __uint_as_float(v.y);
        bpre[2] = __uint_as_float(v.z);
        bpre[3] = __uint_as_float(v.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kRsBpre; ++i) {
        const int e = tid + kRsThreads * i;
        bpre[i] = __uint_as_float(buf_b32(bbr, e < nbe ? static_cast<uint32_t>(e) * 4u : kOob));
      }
    }
  }
  const __amdgpu_buffer_rsrc_t ba = buf(p.A, p.r > 0 ? static_cast<int64_t>(p.r) * p.K * 4 : 0);
  float4 arow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) arow[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (producer) {   // wave-uniform
    const uint32_t off = jon ? static_cast<uint32_t>((static_cast<int64_t>(jcol) * p.K + 32 * j) * 4) : kOob;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = buf_b128(ba, off + 16u * i);
      arow[i] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
    }
  }

  // ---- the passes' code chunks, D ahead (the first D before the tables are
  // built, so the code stream starts at once); one instruction per pass
  uint4 cw[D];
  const __amdgpu_buffer_rsrc_t bc = buf(p.codes + n0 * (p.K / 2), static_cast<int64_t>(rows) * (p.K / 2));
  auto issue = [&](int i) {
    const int rl = i * P + rs, slot = i % D;
    const bool ok = jon && i < npass && rl < rows;
    const uint32_t lb = static_cast<uint32_t>(rl * kb + (j >> 1));   // block within the workgroup's rows
    cw[slot] = buf_b128(bc, ok ? lb * 32u + 16u * (j & 1) : kOob);
  };
#pragma unroll
  for (int i = 0; i < D; ++i) issue(i);

  // ---- table: entry e (code byte) = (bf16 level[e >> 4], bf16 level[e & 15]),
  // copy c at byte e * 256 + 4 c. Thread tid writes copies 4 (tid % 8) .. + 3
  // of entries tid / 8 + 128 i, so that a half-wave's 16-byte stores cover all
  // banks. The levels are kernel-argument constants picked by selects.
  {
    const int e0 = tid >> 3, lo_i = e0 & 15;
    const int hi0 = __builtin_amdgcn_readfirstlane(e0 >> 4);   // wave-uniform, 0 .. 7
    float lo = p.tab.lv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) lo = lo_i == i ? p.tab.lv[i] : lo;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float hi = p.tab.lv[8 * i];
#pragma unroll
      for (int h = 1; h < 8; ++h) hi = hi0 == h ? p.tab.lv[8 * i + h] : hi;
      const uint32_t v = pack_bf16x2(hi, lo);
      *reinterpret_cast<uint4 *>(smem + (e0 + 128 * i) * kRsEntry + 16 * (tid & 7)) = make_uint4(v, v, v, v);
    }
  }
  // ---- X and the block constants c_b into LDS
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + kRsThreads * i;
    if (c < xch) *reinterpret_cast<uint4 *>(xs + 16 * c) = xv[i];
  }
  if (4 * tid < nblk) {
    float c4[4];
    if constexpr (kDq) {
      const int64_t dlo = (gblk0 + 4 * tid) / kDqBlock;
      const float klo = div127(cv[0]), khi = div127(cv[1]);
      qw |= (static_cast<uint32_t>(qt[0]) & 0xFFu) | ((static_cast<uint32_t>(qt[1]) & 0xFFu) << 8) |
            ((static_cast<uint32_t>(qt[2]) & 0xFFu) << 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float q = static_cast<float>(static_cast<int8_t>((qw >> (8 * i)) & 0xFFu));
        const float k = (gblk0 + 4 * tid + i) / kDqBlock == dlo ? klo : khi;
        c4[i] = __fadd_rn(__fmul_rn(q, k), cv[2]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) c4[i] = cv[i];
    }
    *reinterpret_cast<float4 *>(cs + 4 * tid) = make_float4(c4[0], c4[1], c4[2], c4[3]);
  }
  __syncthreads();   // table, X and c_b ready (waits for LDS and scalar accesses only)

  // this thread's 32 elements of X (zero for idle lanes)
  uint32_t xr[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = jon ? *reinterpret_cast<const uint4 *>(xs + 64 * j + 16 * q) : make_uint4(0, 0, 0, 0);
    xr[4 * q] = v.x;
    xr[4 * q + 1] = v.y;
    xr[4 * q + 2] = v.z;
    xr[4 * q + 3] = v.w;
  }

  // ---- the slot's adapter column over this wave's chunks, parked in LDS
  auto h_partial = [&]() {
    float h = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 a = arow[i];
      h = __builtin_fmaf(bf16_lo(xr[2 * i]), a.x, h);
      h = __builtin_fmaf(bf16_hi(xr[2 * i]), a.y, h);
      h = __builtin_fmaf(bf16_lo(xr[2 * i + 1]), a.z, h);
      h = __builtin_fmaf(bf16_hi(xr[2 * i + 1]), a.w, h);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) h += __shfl_xor(h, off, 64);
    if (lane == 0) *rs_aux(smem, a_hp + w) = h;
  };
  uint32_t *hw = p.err + kRsHword0;   // [Gw][r] fp32 bits, 0 until published
  // publish round t's columns: H[0][js] = the slot's waves' partials in wave
  // order, into every workgroup's slot (call after a barrier that follows
  // h_partial; ends with one)
  auto publish = [&](int t) {
    if (tid < P) {
      float hv = 0.0f;
      for (int ww = 0; ww < nw; ++ww) hv += *rs_aux(smem, a_hp + tid * nw + ww);
      *rs_aux(smem, a_hp + kRsWaves + tid) = hv;
    }
    __syncthreads();
    for (int srs = 0; srs < P; ++srs) {
      const int js = b + Gw * (srs + P * t);
      if (js >= p.r) break;
      const uint32_t hb = __float_as_uint(*rs_aux(smem, a_hp + kRsWaves + srs));
      const uint32_t word = hb == 0u ? 0x80000000u : hb;   // +0 published as -0
      for (int g = tid; g < Gw; g += kRsThreads) st_wt(hw + static_cast<int64_t>(g) * p.r + js, word);
    }
    __syncthreads();
  };

  // ---- passes: one accumulator per pass; after pass 1
  // the adapter columns (their X and A requests were issued before the
  // passes', so they have arrived); then the reduce-scatter of the 8 sums
  const uint32_t lane4 = 4u * static_cast<uint32_t>(lane & 31);
  float v[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) v[i] = 0.0f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (wave_on && i < npass) {   // uniform; no load inside
      const int slot = i % D;
      const uint4 c = cw[slot];
      const int rl = i * P + rs;
      const float cb = cs[jon && rl < rows ? rl * kb + (j >> 1) : 0];
      // one accumulator for the chunk's 16 pairs (four per code word): no
      // zeroing or combining of partial sums, and the SIMD's other waves
      // cover the chain's latency
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t wq = q == 0 ? c.x : q == 1 ? c.y : q == 2 ? c.z : c.w;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const uint32_t addr = __builtin_amdgcn_perm(wq, lane4, 0x0C0C0400u | (static_cast<uint32_t>(bb) << 8));
          const uint32_t pr = *reinterpret_cast<const uint32_t *>(smem + addr);
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr), __builtin_bit_cast(bf16x2_t, xr[4 * q + bb]),
                                              s, false);
        }
      }
      v[i] = cb * s;
    }
    issue(i + D);
    if (i == 1 && b < p.r) {   // workgroup-uniform: it owns adapter columns
      if (producer) h_partial();
      __syncthreads();
      publish(0);
    }
  }
  if (wave_on) {
#pragma unroll
    for (int st = 0; st < 3; ++st) {
      const int mask = 32 >> st, half = 4 >> st;
      const bool hi = (lane & mask) != 0;
#pragma unroll
      for (int u = 0; u < half; ++u) {
        const float keep = hi ? v[u + half] : v[u];
        const float give = hi ? v[u] : v[u + half];
        v[u] = keep + __shfl_xor(give, mask, 64);
      }
    }
    float t = v[0];
    t += __shfl_xor(t, 4, 64);
    t += __shfl_xor(t, 2, 64);
    t += __shfl_xor(t, 1, 64);
    // lanes 8 i .. 8 i + 7 hold pass i
    const int rl = (lane >> 3) * P + rs;
    if ((lane & 7) == 0 && rl < rows) *rs_aux(smem, wr * RW + rl) = t;
  }

  if (p.r > 0) {
    // ---- rounds t > 0 of this workgroup's columns (r > Gw P)
    for (int t = 1; b + Gw * P * t < p.r; ++t) {
      __syncthreads();   // round t - 1's partials have been read
      const int jt = jcol + Gw * P * t;
      if (wave_on && jt < p.r) {   // wave-uniform
        const uint32_t off = jon ? static_cast<uint32_t>((static_cast<int64_t>(jt) * p.K + 32 * j) * 4) : kOob;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 v = buf_b128(ba, off + 16u * i);
          arow[i] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
        }
        h_partial();
      }
      __syncthreads();
      publish(t);
    }
    // ---- B rows into LDS; wait until every H word is flagged, s H into LDS
#pragma unroll
    for (int i = 0; i < kRsBpre; ++i) {
      const int e = b4 ? 4 * tid + i : tid + kRsThreads * i;
      if (e < nbe) *rs_aux(smem, a_b + e) = bpre[i];
    }
    if (w == 0) {
      uint32_t *mine = hw + static_cast<int64_t>(b) * p.r;
      for (int j0 = 0; j0 < p.r; j0 += 64) {
        const int jj = j0 + lane;
        uint32_t hv = 0;
        for (int spins = 0;; ++spins) {
          if (jj < p.r) hv = ld_wt(mine + jj);
          if (__all(jj >= p.r || hv != 0u)) break;
          if (spins >= kSpinLimit) {
            if (lane == 0) atomicOr(p.err, 1u);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        if (jj < p.r) {
          *rs_aux(smem, a_h + jj) = p.scale * __uint_as_float(hv);
          st_wt(mine + jj, 0u);
        }
      }
    }
  }
  __syncthreads();

  // ---- outputs: 16 threads per row (64 rows at a time); the adapter term
  // over j = seg, seg + 16, ... then summed across the 16, added to the
  // row's wave partials in wave order
  for (int r0 = 0; r0 < rows; r0 += kRsThreads / 16) {
    const int rl = r0 + tid / 16, seg = tid & 15;
    float ad = 0.0f;
    if (rl < rows)
      for (int jj = seg; jj < p.r; jj += 16) ad = __builtin_fmaf(*rs_aux(smem, a_h + jj), *rs_aux(smem, a_b + rl * p.r + jj), ad);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) ad += __shfl_xor(ad, off, 16);
    if (seg == 0 && rl < rows) {
      float y = 0.0f;
      for (int ww = 0; ww < nw; ++ww) y += *rs_aux(smem, ww * RW + rl);
      p.Y[n0 + rl] = static_cast<__bf16>(y + ad);
    }
  }
}

// ------------------------------------------------------------------ planning

struct GemvPlan {
  int T, S, C, cq, KS, nq_max;
  int U, HK, hb, hstep, rp;
  int xstride, zoff;
  size_t lds;
  bool rows;          // row-stream path (S = its workgroups)
  int nw, P, RW;
};

// Row-stream plan (M = 1): one workgroup per CU, each with the same number
// of passes (at most 8) of P rows; fewer rows per workgroup when the B rows or
// the LDS aux space would not hold them.
bool rows_plan(int64_t M, int64_t N, int64_t K, int r, GemvPlan &pl) {
  const int64_t C = K / 32;
  if (M != 1 || C > kRsMaxChunks || r > 256) return false;
  const int nw = static_cast<int>(ceil_div(C, 64));
  const int P = std::max(1, kRsWaves / nw);
  auto fits = [&](int64_t rw) {
    return rw * r <= kRsBpre * kRsThreads && nw * rw + rw * r + r + kRsWaves + P <= kRsAux;
  };
  const int64_t npass = std::min<int64_t>(kRsPasses, ceil_div(ceil_div(N, static_cast<int64_t>(P)), static_cast<int64_t>(kRsCus)));
  int64_t RW = P * npass;
  while (RW > P && !fits(RW)) RW -= P;
  // every workgroup's H slot in the synchronization words
  if (!fits(RW) || RW * (K / kBlock) > kRsMaxBlocks ||
      (kRsHword0 + ceil_div(N, RW) * r) * 4 > static_cast<int64_t>(kLinearSyncBytes))
    return false;
  pl.rows = true;
  pl.nw = nw;
  pl.P = P;
  pl.RW = static_cast<int>(RW);
  pl.S = static_cast<int>(ceil_div(N, RW));
  pl.C = 1;
  pl.U = 0;
  pl.lds = 0;
  return true;
}

GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K, int r) {
  GemvPlan pl{};
  const int64_t kb = K / kBlock;
  const int64_t qk = (kb + 1) / 2;                 // quad-pieces per row
  const int Mi = static_cast<int>(M);
  // largest chunk (quad-pieces) whose X slice fits
  const int64_t cq_x = std::max<int64_t>(1, (kXLdsMax / (2 * Mi) - kXPad) / 128);
  pl.cq = static_cast<int>(std::min<int64_t>(qk, cq_x));
  pl.C = static_cast<int>(ceil_div(qk, pl.cq));
  pl.cq = static_cast<int>(ceil_div(qk, pl.C));   // even out the chunks
  const int64_t tiles16 = N / 16;
  pl.T = 1;
  while (pl.T < 8 && ceil_div(tiles16, pl.T) * pl.C > kStripTarget) pl.T *= 2;
  pl.KS = kGvWaves / pl.T;
  // the slices of a chunk must fit the unrolled code loads, and a
  // workgroup's block constants the LDS array
  while (ceil_div(pl.cq, pl.KS) > kMaxNq || 16 * pl.T * 2 * pl.cq > kScaleMax) {
    pl.C *= 2;
    pl.cq = static_cast<int>(ceil_div(qk, pl.C));
    pl.C = static_cast<int>(ceil_div(qk, pl.cq));
  }
  pl.S = static_cast<int>(ceil_div(tiles16, pl.T));
  const int nq = static_cast<int>(ceil_div(pl.cq, pl.KS));
  pl.nq_max = nq <= 4 ? 4 : nq <= 8 ? 8 : nq <= 12 ? 12 : 16;
  pl.rp = r > 0 ? static_cast<int>(ceil_div(r, 32) * 32) : 0;
  if (r > 0) {
    const int jgroups = pl.rp / 16;
    const int hk_max = std::max(1, kMaxUnits / jgroups);
    pl.hb = static_cast<int>(kHBlocks * ceil_div(ceil_div(kb, kHBlocks), hk_max));
    pl.HK = static_cast<int>(ceil_div(kb, pl.hb));
    pl.U = jgroups * pl.HK;
  }
  pl.hstep = M <= 16 ? kHBlocks : kHBlocks / 2;   // adapter step: X of M x 64 hstep in LDS
  const int xw = std::max<int>(pl.cq * 128, pl.hstep * kBlock);
  pl.xstride = xw + kXPad;
  const int mt16 = static_cast<int>(ceil_div(M, 16));
  const size_t xbytes = static_cast<size_t>(M) * pl.xstride * 2;
  const size_t hbytes = static_cast<size_t>(16 * mt16) * (pl.rp + 8) * 2;
  pl.zoff = static_cast<int>(align_up(kXOffset + std::max(xbytes, hbytes), 16));
  pl.lds = pl.zoff + kZeroBytes;
  rows_plan(M, N, K, r, pl);
  return pl;   // pl.lds <= kGvLdsMax: X slice <= kXLdsMax, adapter X <= 32 x 520 x 2, H <= 32 x 264 x 2
}

// Dynamic LDS above 64 KB must be allowed per kernel, once.
template <int MT, int NQ, bool kDq>
void launch_one(unsigned grid, size_t lds, hipStream_t s, const GemvParams &p) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemv<MT, NQ, kDq>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kGvLdsMax);
  (void)attr;
  hipLaunchKernelGGL((k_gemv<MT, NQ, kDq>), dim3(grid), dim3(kGvThreads), lds, s, p);
}

template <int MT, int NQ>
void launch_mt_nq(bool dq, unsigned grid, size_t lds, hipStream_t s, const GemvParams &p) {
  if (dq) launch_one<MT, NQ, true>(grid, lds, s, p);
  else launch_one<MT, NQ, false>(grid, lds, s, p);
}

template <int MT>
void launch_mt(int nq, bool dq, unsigned grid, size_t lds, hipStream_t s, const GemvParams &p) {
  if (nq <= 4) launch_mt_nq<MT, 4>(dq, grid, lds, s, p);
  else if (nq <= 8) launch_mt_nq<MT, 8>(dq, grid, lds, s, p);
  else if (nq <= 12) launch_mt_nq<MT, 12>(dq, grid, lds, s, p);
  else launch_mt_nq<MT, 16>(dq, grid, lds, s, p);
}

template <bool kDq>
void launch_rows(unsigned grid, hipStream_t s, const GemvParams &p) {
  if (p.r > 0) hipLaunchKernelGGL((k_gemv_rows<kDq, 2>), dim3(grid), dim3(kRsThreads), 0, s, p);
  else hipLaunchKernelGGL((k_gemv_rows<kDq, 3>), dim3(grid), dim3(kRsThreads), 0, s, p);
}

size_t part_bytes(const GemvPlan &pl, int64_t M) {
  return pl.C > 1 ? align_up(static_cast<size_t>(pl.S) * pl.C * M * 16 * pl.T * sizeof(float), 256) : 0;
}

}  // namespace

bool gemv_sync_fits(int64_t M, int64_t N, int64_t K, int r) {
  const GemvPlan pl = gemv_plan(M, N, K, r);
  if (pl.rows) return true;   // error word and two counters
  // error word and strip counters, flags [S][G], adapter counters [G]
  const int64_t G = pl.rp / 16;
  return (64 + static_cast<size_t>(pl.S) * (G + 1) + G) * sizeof(uint32_t) <= kLinearSyncBytes;
}

size_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K, int r) {
  const GemvPlan pl = gemv_plan(M, N, K, r);
  return kLinearSyncBytes + part_bytes(pl, M) +
         align_up(static_cast<size_t>(pl.HK) * M * pl.rp * sizeof(float), 256) +
         align_up(static_cast<size_t>(M) * pl.rp * sizeof(float), 256);
}

hipError_t launch_gemv(const LinearArgs &a, const void *X, const float *A, const float *B, void *Y, void *ws,
                       hipStream_t s) {
  const GemvPlan pl = gemv_plan(a.M, a.N, a.K, a.r);
  GemvParams p{};
  p.X = static_cast<const __bf16 *>(X);
  p.codes = a.codes;
  p.absmax_q = a.absmax_q;
  p.dq_scale = a.dq_scale;
  p.dq_mean = a.dq_mean;
  p.absmax = a.absmax;
  p.A = A;
  p.B = B;
  p.Y = static_cast<__bf16 *>(Y);
  p.M = a.M;
  p.N = a.N;
  p.K = a.K;
  p.r = a.r;
  p.rp = pl.rp;
  p.scale = a.scale;
  p.T = pl.T;
  p.S = pl.S;
  p.C = pl.C;
  p.cq = pl.cq;
  p.U = pl.U;
  p.HK = pl.HK;
  p.hb = pl.hb;
  p.hstep = pl.hstep;
  p.xstride = pl.xstride;
  p.zoff = pl.zoff;
  p.rs_nw = pl.nw;
  p.rs_P = pl.P;
  p.rs_RW = pl.RW;
  p.tab = format_tables(a.format);
  // sync words: [0] error, [64 ..) strip counters [S], flags [S][G], adapter counters [G]
  char *base = static_cast<char *>(ws);
  p.err = reinterpret_cast<uint32_t *>(base);
  p.ctr = p.err + 64;
  p.flags = p.ctr + pl.S;
  p.hctr = p.flags + static_cast<int64_t>(pl.S) * (pl.rp / 16);
  p.part = reinterpret_cast<float *>(base + kLinearSyncBytes);
  p.hpart = reinterpret_cast<float *>(base + kLinearSyncBytes + part_bytes(pl, a.M));
  p.hfin = reinterpret_cast<float *>(base + kLinearSyncBytes + part_bytes(pl, a.M) +
                                     align_up(static_cast<size_t>(pl.HK) * a.M * pl.rp * sizeof(float), 256));
  const unsigned grid = static_cast<unsigned>(pl.U + pl.S * pl.C);
  const int mt = static_cast<int>(ceil_div(a.M, 8));
  const bool dq = fmt_dq(a.format);
  prof_begin(kProfFwdGemm, s);
  if (pl.rows) {
    if (dq) launch_rows<true>(grid, s, p);
    else launch_rows<false>(grid, s, p);
  } else if (mt == 1) launch_mt<1>(pl.nq_max, dq, grid, pl.lds, s, p);
  else if (mt == 2) launch_mt<2>(pl.nq_max, dq, grid, pl.lds, s, p);
  else launch_mt<4>(pl.nq_max, dq, grid, pl.lds, s, p);
  prof_end(kProfFwdGemm, s);
  return hipGetLastError();
}

}  // namespace qnf4

