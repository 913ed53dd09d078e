// Data exchanged between workgroups of one launch: written with write-through
// stores (agent-scope relaxed atomic stores, sc1), made complete with a wait
// on every outstanding memory access before the counter that announces it,
// and read with agent-scope atomic loads (sc1) or sc1 copies. No L2
// write-back or invalidate is issued: those walk a whole XCD's L2.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace qnf4 {

__device__ __forceinline__ void st_wt(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wt(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_wt(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_wt(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every memory access this wave issued is complete (stores included).
__device__ __forceinline__ void wait_all_memory() {
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// sum_{i < count} src[e_j + i stride] for the E elements e_j = e0 + j estep
// (those with e_j < elim), each added in index order i = 0, 1, ... The loads
// of eight terms of all E elements go out together (clamped indices, the
// extra terms dropped), so a sum costs ceil(count / 8) memory round trips
// instead of one per term.
template <int E>
__device__ __forceinline__ void sum_wt(const float *src, int64_t stride, int count, int e0, int estep, int elim,
                                       float (&out)[E]) {
#pragma unroll
  for (int j = 0; j < E; ++j) out[j] = 0.0f;
  for (int i0 = 0; i0 < count; i0 += 8) {
    float t[E][8];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = min(e0 + j * estep, elim - 1);
#pragma unroll
      for (int u = 0; u < 8; ++u) t[j][u] = ld_wt(src + e + static_cast<int64_t>(min(i0 + u, count - 1)) * stride);
    }
#pragma unroll
    for (int j = 0; j < E; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < count) out[j] += t[j][u];
  }
}

}  // namespace qnf4
