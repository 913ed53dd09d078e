// One AdamW step of the adapter parameters, with the optimizer state either
// in device memory or paged from host memory (Guanaco topic page, "Technical
// Innovations: Paged Optimizers": optimizer states go to CPU RAM under memory
// pressure; QLoRA vs ChatGPT page, capability on paged optimizers: momentum and
// variance paged between GPU and CPU memory). Per element, fp32, each
// operation rounded to nearest even, no fused multiply-add:
//   m' = b1 m + c1 g            c1 = 1 - b1
//   v' = b2 v + c2 (g g)        c2 = 1 - b2
//   u  = (m' / bc1) / (sqrt(v' / bc2) + eps)
//   p' = p - lr (u + wd p)
// The step is bound by memory traffic: 16 bytes read and 12 written per
// parameter from HBM; with paged state, m and v also cross PCIe both ways.
//
// Paging: when the state lives in pinned host memory the call streams it in
// chunks through two device staging arrays of the workspace, on the caller's
// stream: copy m and v of a chunk in, run the step on the chunk, copy them
// back. The stream orders the copies, so a chunk's staging is free again
// before the next chunk's copies start.
#include <cmath>

#include "adamw.h"
#include "internal.h"

namespace qnf4 {
namespace {

constexpr int kAwThreads = 256;
constexpr int64_t kPageElems = int64_t(4) << 20;   // 16 MB per state array and chunk

struct AdamwArgs {
  float lr, b1, b2, c1, c2, eps, wd, bc1, bc2;
};

// Correctly rounded square root of a finite x >= 0. The hardware root s is
// within one ulp of sqrt(x), so the rounded root is s or a neighbour; the
// midpoints between them have at most 25 significant bits, so their squares
// are exact in fp64, and sqrt(x) < mid  <=>  x < mid^2 picks the nearest (a
// root of an fp32 number is never exactly halfway between two fp32 numbers).
__device__ __forceinline__ float sqrt_rn(float x) {
  const float s = __builtin_sqrtf(x);
  if (!(s > 0.0f) || !(s < __builtin_huge_valf())) return s;   // 0, inf, nan
  const float lo = __uint_as_float(__float_as_uint(s) - 1u);
  const float hi = __uint_as_float(__float_as_uint(s) + 1u);
  const double xd = static_cast<double>(x);
  const double mlo = 0.5 * (static_cast<double>(lo) + static_cast<double>(s));
  const double mhi = 0.5 * (static_cast<double>(s) + static_cast<double>(hi));
  if (xd < __dmul_rn(mlo, mlo)) return lo;
  if (xd > __dmul_rn(mhi, mhi)) return hi;
  return s;
}

__device__ __forceinline__ void adamw_one(float &p, float g, float &m, float &v, const AdamwArgs &h) {
  m = __fadd_rn(__fmul_rn(h.b1, m), __fmul_rn(h.c1, g));
  v = __fadd_rn(__fmul_rn(h.b2, v), __fmul_rn(h.c2, __fmul_rn(g, g)));
  const float mh = __fdiv_rn(m, h.bc1);
  const float vh = __fdiv_rn(v, h.bc2);
  const float u = __fdiv_rn(mh, __fadd_rn(sqrt_rn(vh), h.eps));
  p = __fsub_rn(p, __fmul_rn(h.lr, __fadd_rn(u, __fmul_rn(h.wd, p))));
}

// Four elements per thread with 16-byte accesses, grid-stride; the n % 4
// tail is taken element by element by the first threads.
__global__ __launch_bounds__(kAwThreads) void k_adamw(float *__restrict__ p, const float *__restrict__ g,
                                                      float *__restrict__ m, float *__restrict__ v, int64_t n,
                                                      AdamwArgs h) {
  const int64_t n4 = n / 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kAwThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kAwThreads + threadIdx.x; i < n4; i += stride) {
    float4 pp = reinterpret_cast<float4 *>(p)[i];
    const float4 gg = reinterpret_cast<const float4 *>(g)[i];
    float4 mm = reinterpret_cast<float4 *>(m)[i];
    float4 vv = reinterpret_cast<float4 *>(v)[i];
    adamw_one(pp.x, gg.x, mm.x, vv.x, h);
    adamw_one(pp.y, gg.y, mm.y, vv.y, h);
    adamw_one(pp.z, gg.z, mm.z, vv.z, h);
    adamw_one(pp.w, gg.w, mm.w, vv.w, h);
    reinterpret_cast<float4 *>(p)[i] = pp;
    reinterpret_cast<float4 *>(m)[i] = mm;
    reinterpret_cast<float4 *>(v)[i] = vv;
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) {
    const int64_t e = 4 * n4 + threadIdx.x;
    float pp = p[e], mm = m[e], vv = v[e];
    adamw_one(pp, g[e], mm, vv, h);
    p[e] = pp;
    m[e] = mm;
    v[e] = vv;
  }
}

// One float4 per thread (a grid-stride loop of one pass): at 160 M elements
// this streams at 5.2 TB/s against 4.2 TB/s for a grid capped at 4096
// workgroups that loops 38 times.
void launch_step(float *p, const float *g, float *m, float *v, int64_t n, const AdamwArgs &h, hipStream_t s) {
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(n / 4, kAwThreads), int64_t(1) << 30));
  hipLaunchKernelGGL(k_adamw, dim3(static_cast<unsigned>(blocks)), dim3(kAwThreads), 0, s, p, g, m, v, n, h);
}

}  // namespace

float adamw_bias_correction(float beta, int64_t t) {
  return static_cast<float>(1.0 - std::pow(static_cast<double>(beta), static_cast<double>(t)));
}

// staging elements per state array, rounded up so that both arrays stay 16-byte aligned
int64_t stage_elems(int64_t n) { return ceil_div(std::min(n, kPageElems), 64) * 64; }

size_t adamw_ws_bytes(int64_t n, bool state_on_host) {
  if (!state_on_host) return 0;
  return 2 * static_cast<size_t>(stage_elems(n)) * sizeof(float);
}

hipError_t launch_adamw(float *param, const float *grad, float *m, float *v, int64_t n, const AdamwHparams &hp,
                        bool state_on_host, void *ws, hipStream_t s) {
  AdamwArgs h;
  h.lr = hp.lr;
  h.b1 = hp.beta1;
  h.b2 = hp.beta2;
  h.c1 = 1.0f - hp.beta1;   // exact (Sterbenz) for beta in [0.5, 1]; otherwise rounded once
  h.c2 = 1.0f - hp.beta2;
  h.eps = hp.eps;
  h.wd = hp.weight_decay;
  h.bc1 = adamw_bias_correction(hp.beta1, hp.step);
  h.bc2 = adamw_bias_correction(hp.beta2, hp.step);
  if (!state_on_host) {
    launch_step(param, grad, m, v, n, h, s);
    return hipGetLastError();
  }
  float *sm = static_cast<float *>(ws);
  float *sv = sm + stage_elems(n);
  for (int64_t o = 0; o < n; o += kPageElems) {
    const int64_t len = std::min(kPageElems, n - o);
    const size_t bytes = static_cast<size_t>(len) * sizeof(float);
    hipError_t e = hipMemcpyAsync(sm, m + o, bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(sv, v + o, bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return e;
    launch_step(param + o, grad + o, sm, sv, len, h, s);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(m + o, sm, bytes, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(v + o, sv, bytes, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qnf4
