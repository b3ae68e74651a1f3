// Internal declarations shared by the host layer and the kernel launchers of libdq.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace dq {

// Per-row FP8 quantization of a bf16 [R, K] matrix (activations per token, weights per output
// channel). Arguments are already validated. Returns the launch status.
hipError_t launch_quantize_rows(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, float* scale,
                                hipStream_t stream);

// FP8 GEMM + fused epilogue. Arguments are already validated. Returns the launch status.
hipError_t launch_linear(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                         const uint8_t* qw, const float* w_scale, int64_t N, const uint16_t* bias,
                         int epilogue, const uint16_t* gate, const uint16_t* residual,
                         uint16_t* out, hipStream_t stream);

}  // namespace dq
