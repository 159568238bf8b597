// Internal interface of the gate projection kernel (gate_proj.hip); the public one is
// include/ssw.h (ssw_gate_projection).
#pragma once

#include <hip/hip_runtime_api.h>

namespace ssw {

// gates [2, rows, Hq] = sigmoid(x [rows, Hm] * w_t^T + bias), bf16 x and w_t [2 Hq, Hm];
// Hm % 16 == 0, 1 <= Hq <= 64 (checked by the caller).
hipError_t launch_gate_projection(const void* x, const void* w_t, const float* bias,
                                  float* gates, int rows, int Hm, int Hq, hipStream_t stream);

}  // namespace ssw
