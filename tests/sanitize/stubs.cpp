// Host-only stand-ins for the HIP runtime and for the kernel launchers of the
// QLoRA NF4 library, so that its C ABI layer (api.cpp, with codebook.cpp and
// profile.cpp) builds with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and runs on a machine without a GPU. A launcher
// that is reached counts the call and fails; the driver checks that every
// invalid call is rejected before one is reached and every valid one reaches
// it. Workspace sizes are stand-ins too (the driver asks the library for
// them, so the checks compare like with like).
#include <cstdio>

#include "../../bit_nf4_quantized_03_amd/csrc/adamw.h"
#include "../../bit_nf4_quantized_03_amd/csrc/internal.h"

extern "C" {
int qlora_stub_launches = 0;
}

namespace {
hipError_t reached() {
  ++qlora_stub_launches;
  return hipErrorNotSupported;
}
}  // namespace

namespace qnf4 {
size_t quantize_ws_bytes(int64_t n) { return n > 0 ? static_cast<size_t>(ceil_div(n, kBlock)) * 4 + 256 : 0; }
hipError_t launch_quantize(const void *, bool, int64_t, int, uint8_t *, int8_t *, float *, float *, float *, void *,
                           hipStream_t) {
  return reached();
}
hipError_t launch_dequantize(const uint8_t *, int, const int8_t *, const float *, const float *, const float *,
                             int64_t, void *, bool, hipStream_t) {
  return reached();
}
size_t linear_ws_bytes(int64_t M, int64_t N, int64_t K, int r) {
  return static_cast<size_t>(M + N + K + r) * 16 + kLinearSyncBytes;
}
size_t linear_fwd_ws_bytes(int64_t M, int64_t N, int64_t K, int r, bool) { return linear_ws_bytes(M, N, K, r); }
hipError_t noalloc_scratch(void **ptr) {
  static unsigned char fake[256];
  *ptr = fake;
  return hipSuccess;
}
hipError_t linear_fwd(const LinearArgs &, const void *, const float *, const float *, void *, void *, hipStream_t, bool,
                      void *) {
  return reached();
}
hipError_t linear_bwd(const LinearArgs &, const void *, const void *, const float *, const float *, void *, float *,
                      float *, void *, hipStream_t, const void *) {
  return reached();
}
size_t merge_ws_bytes(int64_t N, int64_t K, int r) { return static_cast<size_t>(N + K + r) * 16; }
hipError_t launch_merge(const LinearArgs &, const float *, const float *, int, uint8_t *, int8_t *, float *, float *,
                        float *, void *, hipStream_t) {
  return reached();
}
size_t adamw_ws_bytes(int64_t n, bool on_host) { return on_host && n > 0 ? 4096 : 0; }
hipError_t launch_adamw(float *, const float *, float *, float *, int64_t, const AdamwHparams &, bool, void *,
                        hipStream_t) {
  return reached();
}
}  // namespace qnf4

// The HIP runtime calls the host layer makes (error strings, the opt-in
// profiling events).
const char *hipGetErrorString(hipError_t) { return "stub HIP runtime: no device"; }
hipError_t hipEventCreate(hipEvent_t *e) {
  *e = nullptr;
  return hipErrorNotSupported;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipErrorNotSupported; }
hipError_t hipEventElapsedTime(float *ms, hipEvent_t, hipEvent_t) {
  *ms = 0.0f;
  return hipErrorNotSupported;
}
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
