// Private interface of the AdamW step (adamw.hip), used by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstddef>

namespace qnf4 {

struct AdamwHparams {
  float lr, beta1, beta2, eps, weight_decay;
  int64_t step;   // t >= 1
};

// fp32(1 - beta^t): beta is already an fp32 value; the power and the
// difference are taken in fp64 and rounded once.
float adamw_bias_correction(float beta, int64_t t);

// Workspace: with the state on the host, two device staging arrays (m, v) of
// up to 4 Mi elements each; none otherwise.
size_t adamw_ws_bytes(int64_t n, bool state_on_host);
hipError_t launch_adamw(float *param, const float *grad, float *m, float *v, int64_t n, const AdamwHparams &hp,
                        bool state_on_host, void *ws, hipStream_t s);

}  // namespace qnf4
