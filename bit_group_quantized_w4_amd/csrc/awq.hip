// Activation-aware channel scaling before RTN (Qwen3.5-4B quantization study,
// section 2: the AWQ row of the methods table, the 20-exponent scale search of
// the settings table, and the channel-scaling equation W'_ij = W_ij s_j,
// x'_j = x_j / s_j with W'x' = Wx).  The offline steps of the search:
//   * mean |x_j| per input channel over calibration rows,
//   * the candidate scales for one exponent (geometric mean 1),
//   * x' = bf16(fl32(x * inv_s)),
//   * the squared output error of one candidate.
// The scaled quantizer is quantize_rtn_kernel with column scales, and the
// decode linear with x' formed in its x staging is the dot2 kernel.
// Everything here runs once per matrix and candidate, so the kernels aim at
// determinism (fixed summation orders) rather than bandwidth.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {
namespace {

constexpr int kReduceThreads = 1024;

// Sum over the block in a fixed order (tree over LDS), result in lane 0 of
// thread 0.  `red` has kReduceThreads doubles.
__device__ double block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int h = kReduceThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  return red[0];
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// m[j] = (sum_t |x[t][j]|) / T, the sum taken over t in order in fp32.
__global__ __launch_bounds__(256) void channel_absmean_kernel(const uint16_t* __restrict__ x, int T, int K,
                                                              float* __restrict__ m) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= K) return;
  float s = 0.0f;
  for (int t = 0; t < T; ++t) s += fabsf(bf16_to_f32(x[(int64_t)t * K + j]));
  m[j] = s / (float)T;
}

// One block: p_j = max(m_j, 1e-30)^alpha in fp64, g = exp(mean log p),
// s_j = fl32(p_j / g), inv_j = fl32(1 / s_j).
__global__ __launch_bounds__(kReduceThreads) void awq_scales_kernel(const float* __restrict__ m, int K, double alpha,
                                                                    float* __restrict__ s, float* __restrict__ inv) {
  __shared__ double red[kReduceThreads];
  double acc = 0.0;
  for (int j = threadIdx.x; j < K; j += kReduceThreads) acc += log(pow(fmax((double)m[j], 1e-30), alpha));
  const double mean_log = block_sum(acc, red) / (double)K;
  for (int j = threadIdx.x; j < K; j += kReduceThreads) {
    const double p = pow(fmax((double)m[j], 1e-30), alpha);
    const float s32 = (float)(p / exp(mean_log));
    s[j] = s32;
    inv[j] = (float)(1.0 / (double)s32);
  }
}

// x' = bf16_rne(fl32(x * inv_s)), elementwise over [M][K].
__global__ __launch_bounds__(256) void scale_activations_kernel(const uint16_t* __restrict__ x, int64_t M, int K,
                                                                const float* __restrict__ inv,
                                                                uint16_t* __restrict__ xo) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= M * K) return;
  const int j = (int)(e % K);
  xo[e] = f32_to_bf16_rne(bf16_to_f32(x[e]) * inv[j]);
}

// out[0] = sum_e (y[e] - y_ref[e])^2 in fp64, one block, fixed order.
__global__ __launch_bounds__(kReduceThreads) void sq_error_kernel(const uint16_t* __restrict__ y,
                                                                  const float* __restrict__ yref, int64_t n,
                                                                  double* __restrict__ out) {
  __shared__ double red[kReduceThreads];
  double acc = 0.0;
  for (int64_t e = threadIdx.x; e < n; e += kReduceThreads) {
    const double d = (double)bf16_to_f32(y[e]) - (double)yref[e];
    acc += d * d;
  }
  const double total = block_sum(acc, red);
  if (threadIdx.x == 0) out[0] = total;
}

}  // namespace

hipError_t launch_channel_absmean(const uint16_t* x, int64_t T, int64_t K, float* m, hipStream_t stream) {
  channel_absmean_kernel<<<(unsigned)((K + 255) / 256), 256, 0, stream>>>(x, (int)T, (int)K, m);
  return hipGetLastError();
}

hipError_t launch_awq_scales(const float* m, int64_t K, double alpha, float* s, float* inv, hipStream_t stream) {
  awq_scales_kernel<<<1, kReduceThreads, 0, stream>>>(m, (int)K, alpha, s, inv);
  return hipGetLastError();
}

hipError_t launch_scale_activations(const uint16_t* x, int64_t M, int64_t K, const float* inv, uint16_t* xo,
                                    hipStream_t stream) {
  const int64_t n = M * K;
  scale_activations_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(x, M, (int)K, inv, xo);
  return hipGetLastError();
}

hipError_t launch_sq_error(const uint16_t* y, const float* yref, int64_t n, double* out, hipStream_t stream) {
  sq_error_kernel<<<1, kReduceThreads, 0, stream>>>(y, yref, n, out);
  return hipGetLastError();
}

}  // namespace w4
