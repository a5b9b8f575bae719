// Internal launchers between the C ABI (abi.cpp) and the kernels (*.hip).
// Shapes and pointers are validated by the caller; each launcher enqueues on
// `stream` and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace w4 {

hipError_t launch_quantize_rtn(const float* W, int64_t N, int64_t K, uint8_t* q_packed,
                               float* d_packed, hipStream_t stream);
hipError_t launch_pack(const int8_t* q_canon, const float* d_canon, int64_t N, int64_t K,
                       uint8_t* q_packed, float* d_packed, hipStream_t stream);
hipError_t launch_unpack(const uint8_t* q_packed, const float* d_packed, int64_t N, int64_t K,
                         int8_t* q_canon, float* d_canon, hipStream_t stream);

// MFMA streaming kernel: any M (16-row slabs of x per grid row).
hipError_t launch_linear_mfma(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                              const float* d_packed, int64_t N, uint16_t* y, hipStream_t stream);
// VALU dot2 streaming kernel: any M (4-row slabs of x per grid row).
hipError_t launch_linear_gemv(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                              const float* d_packed, int64_t N, uint16_t* y, hipStream_t stream);

}  // namespace w4
