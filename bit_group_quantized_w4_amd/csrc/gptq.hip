// GPTQ steps that are specific to the method (the dense products around them
// -- the Hessian X^T X and the factorization of its inverse, in fp64, and the
// correction of the columns after each block, in fp32 -- are plain library
// linear algebra).
//
// Qwen3.5-4B quantization study, section 2: GPTQ keeps RTN's storage
// (symmetric INT4, group 128) and quantizes one input column at a time,
// correcting the columns not yet quantized through a damped Hessian of the
// calibration inputs (damping 0.01 of the mean diagonal, 128-column blocks,
// no reordering).  The update rule is the published GPTQ algorithm: with U
// upper triangular and H'^-1 = U^T U, quantizing column j gives
// err = (w_j - w_hat_j) / U[j][j] and every later column k loses
// err * U[j][k].
//
// gptq_block_kernel runs that loop over one 128-column block, which is also
// one quantization group: one lane per weight row holds the row's 128
// current weights in registers, takes the group's scale by the RTN rule
// (d = fl32(max|w| / 7)), decides each code as RTN does (fl32(w / d), round
// half away from zero, clamp to [-8, 7]), and applies the within-block
// corrections with fused multiply-adds.  The block's row of U entries is the
// same for every lane, so it is read with uniform (scalar) loads.  The
// column errors go out column-major ([128][N], coalesced) for the product
// that corrects the later columns.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {
namespace {

constexpr int kGptqRowsPerBlock = 64;  // one wavefront, one row per lane

// S: the stored scale, float (fp32) or uint16_t (bf16 bit pattern; the codes
// and the corrections then use that stored value widened to fp32).
template <typename S>
__global__ __launch_bounds__(kGptqRowsPerBlock) void gptq_block_kernel(const float* __restrict__ W, int N,
                                                                        int K, int b0,
                                                                        const float* __restrict__ U,
                                                                        int8_t* __restrict__ qc,
                                                                        S* __restrict__ dc,
                                                                        float* __restrict__ errT) {
  const int n = blockIdx.x * kGptqRowsPerBlock + threadIdx.x;
  const bool live = n < N;
  // rows past N repeat row N-1 so the wavefront stays uniform; nothing of theirs is stored
  const float4* wr = reinterpret_cast<const float4*>(W + (int64_t)(live ? n : N - 1) * K + b0);
  float v[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup / 4; ++i) {
    const float4 a = wr[i];
    v[4 * i + 0] = a.x;
    v[4 * i + 1] = a.y;
    v[4 * i + 2] = a.z;
    v[4 * i + 3] = a.w;
  }

  // the group's scale from its current weights (RTN rule; finite inputs)
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < kGroup; ++k) amax = fmaxf(amax, fabsf(v[k]));
  const float d32 = amax / kMaxCode;  // IEEE fp32 division
  S stored;
  float d;
  if constexpr (sizeof(S) == 2) {
    stored = f32_to_bf16_rne(d32);
    d = __uint_as_float((uint32_t)stored << 16);
  } else {
    stored = d32;
    d = d32;
  }
  const bool usable = d != 0.0f;
  const float dd = usable ? d : 1.0f;

  const float* Ub = U + (int64_t)b0 * K + b0;
  uint32_t words[kGroup / 4];
#pragma unroll
  for (int i = 0; i < kGroup / 4; ++i) words[i] = 0;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    const float wj = v[j];
    const float t = wj / dd;  // IEEE fp32 quotient, as RTN
    float r = truncf(t);
    r = fabsf(t - r) >= 0.5f ? r + copysignf(1.0f, t) : r;  // ties away from zero
    r = fminf(fmaxf(r, -8.0f), 7.0f);
    const float qf = usable ? r : 0.0f;
    words[j >> 2] |= ((uint32_t)(int)qf & 0xFFu) << (8 * (j & 3));
    const float e = (wj - d * qf) / Ub[(int64_t)j * K + j];  // d * qf is exact in fp32
    if (live) errT[(int64_t)j * N + n] = e;
#pragma unroll
    for (int k = j + 1; k < kGroup; ++k) v[k] = fmaf(-e, Ub[(int64_t)j * K + k], v[k]);
  }
  if (!live) return;
  uint4* qo = reinterpret_cast<uint4*>(qc + (int64_t)n * K + b0);
#pragma unroll
  for (int i = 0; i < kGroup / 16; ++i)
    qo[i] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
  dc[(int64_t)n * (K / kGroup) + b0 / kGroup] = stored;
}

// Damping of the fp64 Hessian in place: a zero diagonal entry (a column
// whose inputs are all zero) becomes 1, then lambda = damp * mean(diag) is
// added to the diagonal.  One block; the mean is a fixed-order tree sum.
constexpr int kDampThreads = 1024;

__global__ __launch_bounds__(kDampThreads) void gptq_damp_kernel(double* __restrict__ H, int K, double damp) {
  __shared__ double part[kDampThreads];
  double s = 0.0;
  for (int i = threadIdx.x; i < K; i += kDampThreads) {
    double h = H[(int64_t)i * K + i];
    if (h == 0.0) {
      h = 1.0;
      H[(int64_t)i * K + i] = h;
    }
    s += h;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = kDampThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const double lam = damp * (part[0] / (double)K);
  for (int i = threadIdx.x; i < K; i += kDampThreads) H[(int64_t)i * K + i] += lam;
}

}  // namespace

hipError_t launch_gptq_block(const float* W, int64_t N, int64_t K, int64_t b0, const float* U, int8_t* q_canon,
                             void* d_canon, bool s16, float* errT, hipStream_t stream) {
  const unsigned blocks = (unsigned)((N + kGptqRowsPerBlock - 1) / kGptqRowsPerBlock);
  if (blocks == 0) return hipSuccess;
  if (s16)
    gptq_block_kernel<uint16_t><<<blocks, kGptqRowsPerBlock, 0, stream>>>(
        W, (int)N, (int)K, (int)b0, U, q_canon, static_cast<uint16_t*>(d_canon), errT);
  else
    gptq_block_kernel<float><<<blocks, kGptqRowsPerBlock, 0, stream>>>(W, (int)N, (int)K, (int)b0, U, q_canon,
                                                                       static_cast<float*>(d_canon), errT);
  return hipGetLastError();
}

hipError_t launch_gptq_damp(double* H, int64_t K, double damp, hipStream_t stream) {
  gptq_damp_kernel<<<1, kDampThreads, 0, stream>>>(H, (int)K, damp);
  return hipGetLastError();
}

}  // namespace w4
