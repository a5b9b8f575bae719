// Dense linear algebra of the offline quantizers (GPTQ and the channel-scaling
// search), on the GPU's vector ALUs:
//   * a tiled matrix product C = beta C + alpha op(A) op(B) in fp32 or fp64
//     (inputs bf16, fp32 or fp64, widened exactly), optionally only the lower
//     triangle of C, or the lower triangle mirrored into the upper one;
//   * the pieces of a blocked Cholesky factorization and of the inverse of a
//     lower triangular matrix (64 x 64 diagonal blocks in LDS, everything
//     else through the matrix product).
// On MI355X the fp64 and fp32 matrix-core rates equal the vector rates, and
// these products are a small, offline part of quantization, so they stay on
// the VALU with LDS-tiled operands.
//
// GPTQ (Qwen3.5-4B quantization study, section 2: the GPTQ row and settings
// table; the update rule of the published GPTQ algorithm) needs
//   H = (2/T) X^T X in fp64, its damped inverse factor U (upper triangular,
//   H^-1 = U^T U), and after each block of 128 columns the correction
//   W[:, b1:] -= E U[b0:b1, b1:] in fp32;
// the channel-scaling search needs the output of the unquantized layer, x W^T.
#include "w4_device.h"
#include "w4_launch.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace w4 {
namespace {

template <typename Acc, typename E>
__device__ __forceinline__ Acc load_elem(const E* p) {
  if constexpr (std::is_same<E, uint16_t>::value)
    return (Acc)__uint_as_float((uint32_t)*p << 16);  // bf16 -> fp32 is exact
  else
    return (Acc)*p;
}

// C[m][n] = beta * C[m][n] + alpha * sum_k opA(m, k) opB(k, n), m < M, n < N, with
// opA(m, k) = TA ? A[k lda + m] : A[m lda + k] and opB(k, n) = TB ? B[n ldb + k] : B[k ldb + n].
// A block of 256 threads computes a (16 TM) x (16 TM) tile, TM x TM per
// thread, over K in chunks of kKC staged in LDS (widened to Acc).  Modes:
// kFull; kLower (tiles entirely above the diagonal are skipped and only
// elements m >= n are stored); kSymmetric (as kLower, and C[n][m] = C[m][n]
// is stored too; beta must be 0).  Products and sums are in Acc, sums in k
// order per element (deterministic).
enum { kFull = 0, kLower = 1, kSymmetric = 2 };
constexpr int kKC = 16;

template <typename EA, typename EB, typename Acc, bool TA, bool TB, int TM, int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(int M, int N, int K, Acc alpha, const EA* __restrict__ A,
                                                   int64_t lda, const EB* __restrict__ B, int64_t ldb, Acc beta,
                                                   Acc* C, int64_t ldc) {
  constexpr int BT = 16 * TM;  // tile edge
  const int m0 = blockIdx.y * BT, n0 = blockIdx.x * BT;
  if (MODE != kFull && n0 > m0 + BT - 1) return;  // entirely above the diagonal
  // rows padded by 16 bytes: 16-byte aligned for wide LDS reads, rows on shifted banks
  constexpr int kPad = 16 / sizeof(Acc);
  __shared__ Acc as[kKC][BT + kPad];
  __shared__ Acc bs[kKC][BT + kPad];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  Acc acc[TM][TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = 0;

  for (int k0 = 0; k0 < K; k0 += kKC) {
    // stage the chunk: consecutive threads along the contiguous dimension
#pragma unroll
    for (int e = tid; e < BT * kKC; e += 256) {
      int mm, kk;
      if (TA) { kk = e / BT; mm = e % BT; } else { mm = e / kKC; kk = e % kKC; }
      const int m = m0 + mm, k = k0 + kk;
      as[kk][mm] = (m < M && k < K) ? load_elem<Acc>(TA ? A + (int64_t)k * lda + m : A + (int64_t)m * lda + k)
                                     : (Acc)0;
      int nn, kb;
      if (TB) { nn = e / kKC; kb = e % kKC; } else { kb = e / BT; nn = e % BT; }
      const int n = n0 + nn, kq = k0 + kb;
      bs[kb][nn] = (n < N && kq < K) ? load_elem<Acc>(TB ? B + (int64_t)n * ldb + kq : B + (int64_t)kq * ldb + n)
                                      : (Acc)0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKC; ++kk) {
      Acc a[TM], b[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = as[kk][ty * TM + i];
#pragma unroll
      for (int j = 0; j < TM; ++j) b[j] = bs[kk][tx * TM + j];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + ty * TM + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int n = n0 + tx * TM + j;
      if (n >= N || (MODE != kFull && n > m)) continue;
      Acc* c = C + (int64_t)m * ldc + n;
      const Acc v = beta == (Acc)0 ? alpha * acc[i][j] : fma(alpha, acc[i][j], beta * *c);
      *c = v;
      if (MODE == kSymmetric && n != m) C[(int64_t)n * ldc + m] = v;
    }
  }
}

template <typename EA, typename EB, typename Acc, bool TA, bool TB, int TM, int MODE>
hipError_t gemm(int64_t M, int64_t N, int64_t K, Acc alpha, const EA* A, int64_t lda, const EB* B, int64_t ldb,
                Acc beta, Acc* C, int64_t ldc, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  constexpr int BT = 16 * TM;
  const dim3 grid((unsigned)((N + BT - 1) / BT), (unsigned)((M + BT - 1) / BT));
  gemm_kernel<EA, EB, Acc, TA, TB, TM, MODE><<<grid, 256, 0, s>>>((int)M, (int)N, (int)K, alpha, A, lda, B, ldb,
                                                                   beta, C, ldc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 64 x 64 diagonal blocks
// ---------------------------------------------------------------------------
constexpr int kNB = 64;

// In place: the lower triangle of the 64 x 64 block at A (leading dimension
// lda) becomes its Cholesky factor L (A = L L^T), by the right-looking
// algorithm in LDS with one wavefront, lane r owning row r.  A pivot that is
// not positive gives NaN (or infinity), which spreads through everything
// computed from it.
__global__ __launch_bounds__(kNB) void potrf_diag_kernel(double* A, int64_t lda) {
  __shared__ double a[kNB][kNB + 1];
  const int r = threadIdx.x;
  for (int c = 0; c <= r; ++c) a[r][c] = A[(int64_t)r * lda + c];
  __syncthreads();
  for (int c = 0; c < kNB; ++c) {
    if (r == c) a[c][c] = sqrt(a[c][c]);
    __syncthreads();
    if (r > c) {
      const double l = a[r][c] / a[c][c];
      a[r][c] = l;
      for (int k = c + 1; k <= r; ++k) a[r][k] = fma(-l, a[k][c], a[r][k]);
    }
    __syncthreads();
  }
  for (int c = 0; c <= r; ++c) A[(int64_t)r * lda + c] = a[r][c];
}

// X = L^-1 for the lower triangular 64 x 64 blocks L at A + i (64 lda + 64)
// (block i = blockIdx.x), written to X at the same position (leading
// dimension ldx; its upper triangle becomes 0).  Column j of X by forward
// substitution, X[i][j] = -(sum_{k=j}^{i-1} L[i][k] X[k][j]) / L[i][i], with
// the sum over k split among four lanes (k = j + 4t + u, lane u) and their
// partial sums added in a fixed order.
__global__ __launch_bounds__(256) void trtri_diag_kernel(const double* A, int64_t lda, double* X, int64_t ldx) {
  __shared__ double l[kNB][kNB + 1];
  __shared__ double x[kNB][kNB + 1];
  const int64_t o = (int64_t)blockIdx.x * kNB;
  const double* Ab = A + o * lda + o;
  double* Xb = X + o * ldx + o;
  const int tid = threadIdx.x;
  for (int e = tid; e < kNB * kNB; e += 256) {
    const int r = e / kNB, c = e % kNB;
    l[r][c] = c <= r ? Ab[(int64_t)r * lda + c] : 0.0;
    x[r][c] = 0.0;
  }
  __syncthreads();
  const int j = tid >> 2, u = tid & 3;  // column, and this lane's share of the sum
  if (u == 0) x[j][j] = 1.0 / l[j][j];
  __syncthreads();
  for (int i = 1; i < kNB; ++i) {
    double s = 0.0;
    for (int k = j + u; k < i; k += 4) s = fma(l[i][k], x[k][j], s);
    // lanes 4j .. 4j+3 are adjacent: add the four shares in lane order
    const double s1 = __shfl_down(s, 1, 4), s2 = __shfl_down(s, 2, 4), s3 = __shfl_down(s, 3, 4);
    if (u == 0 && i > j) x[i][j] = -(((s + s1) + s2) + s3) / l[i][i];
    __syncthreads();
  }
  for (int e = tid; e < kNB * kNB; e += 256) {
    const int r = e / kNB, c = e % kNB;
    Xb[(int64_t)r * ldx + c] = x[r][c];
  }
}

// dst[i][j] = src[K-1-j][K-1-i] for j <= i (the lower triangle of the index
// reversal J S J of a symmetric S, read from S's lower triangle).
__global__ __launch_bounds__(256) void flip_lower_kernel(const double* src, double* dst, int64_t K) {
  const int64_t i = blockIdx.y;
  for (int64_t j = blockIdx.x * 256 + threadIdx.x; j <= i && j < K; j += (int64_t)gridDim.x * 256)
    dst[i * K + j] = src[(K - 1 - j) * K + (K - 1 - i)];
}

// U[i][j] = fl32(X[K-1-i][K-1-j]) for j >= i, 0 below the diagonal: the upper
// triangular J X J of a lower triangular X, rounded to fp32.
__global__ __launch_bounds__(256) void flip_to_upper_f32_kernel(const double* X, float* U, int64_t K) {
  const int64_t i = blockIdx.y;
  for (int64_t j = blockIdx.x * 256 + threadIdx.x; j < K; j += (int64_t)gridDim.x * 256)
    U[i * K + j] = j >= i ? (float)X[(K - 1 - i) * K + (K - 1 - j)] : 0.0f;
}

__global__ __launch_bounds__(256) void zero_f64_kernel(double* p, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) p[e] = 0.0;
}

unsigned grid_x(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 1024); }

}  // namespace

size_t gptq_factor_work_doubles(int64_t K) { return (size_t)K * K * 2 + (size_t)kNB * kNB; }

// H (fp64 [K][K], damped, lower triangle read) -> U upper triangular fp32
// [K][K] with H^-1 = U^T U.  With J the index reversal, J H J = L L^T (L
// lower) gives H = V V^T for the upper triangular V = J L J, hence
// H^-1 = (V^-1)^T V^-1 and U = V^-1 = J L^-1 J.  work: gptq_factor_work_doubles(K)
// doubles: L (the factorization in place of J H J), X = L^-1, and a 64 x 64 block.
hipError_t launch_gptq_inverse_factor(const double* H, int64_t K, double* work, float* U, hipStream_t s) {
  const int64_t nb = K / kNB;
  double* L = work;
  double* X = work + (size_t)K * K;
  double* T = X + (size_t)K * K;
  flip_lower_kernel<<<dim3(grid_x(K), (unsigned)K), 256, 0, s>>>(H, L, K);
  if (hipError_t e = hipGetLastError()) return e;
  // blocked right-looking Cholesky of J H J (lower)
  for (int64_t jb = 0; jb < nb; ++jb) {
    const int64_t j0 = jb * kNB, rest = K - j0 - kNB;
    double* Ljj = L + j0 * K + j0;
    potrf_diag_kernel<<<1, kNB, 0, s>>>(Ljj, K);
    if (hipError_t e = hipGetLastError()) return e;
    if (rest == 0) break;
    // panel P = L[j0+64:, j0:j0+64] <- P Ljj^-T (Ljj^-1 into the 64 x 64 corner of T)
    trtri_diag_kernel<<<1, 256, 0, s>>>(Ljj, K, T, kNB);
    if (hipError_t e = hipGetLastError()) return e;
    double* P = L + (j0 + kNB) * K + j0;
    // in place: one 64-wide column tile, so each block reads only the rows it writes
    if (hipError_t e = gemm<double, double, double, false, true, 4, kFull>(rest, kNB, kNB, 1.0, P, K, T, kNB, 0.0,
                                                                            P, K, s))
      return e;
    // trailing lower triangle: L[j0+64:, j0+64:] -= P P^T
    double* Ct = L + (j0 + kNB) * K + j0 + kNB;
    if (hipError_t e = rest >= 1024
                           ? gemm<double, double, double, false, true, 8, kLower>(rest, rest, kNB, -1.0, P, K, P, K,
                                                                                    1.0, Ct, K, s)
                           : gemm<double, double, double, false, true, 4, kLower>(rest, rest, kNB, -1.0, P, K, P, K,
                                                                                    1.0, Ct, K, s))
      return e;
  }
  // X = L^-1, block row by block row.  Below the finished rows, X holds the
  // running sums S[i][j] = sum over finished block rows k of L[i][k] X[k][j];
  // block row i is then X[i][j] = -X[i][i] S[i][j] (j < i), X[i][i] = L[i][i]^-1,
  // and its rows are added into S of every later block row:
  // S[i+1:, 0:i+1] += L[i+1:, i] X[i, 0:i+1] (a product with 64-wide inner dimension).
  zero_f64_kernel<<<1024, 256, 0, s>>>(X, (int64_t)K * K);
  if (hipError_t e = hipGetLastError()) return e;
  trtri_diag_kernel<<<(unsigned)nb, 256, 0, s>>>(L, K, X, K);
  if (hipError_t e = hipGetLastError()) return e;
  for (int64_t ib = 0; ib < nb; ++ib) {
    const int64_t i0 = ib * kNB;
    if (ib > 0) {
      // in place: each block reads only the 64-wide column tile of S it writes
      if (hipError_t e = gemm<double, double, double, false, false, 4, kFull>(kNB, i0, kNB, -1.0, X + i0 * K + i0, K,
                                                                               X + i0 * K, K, 0.0, X + i0 * K, K, s))
        return e;
    }
    const int64_t rest = K - i0 - kNB;
    if (rest == 0) break;
    double* Srest = X + (i0 + kNB) * K;
    if (hipError_t e = rest >= 1024 && i0 + kNB >= 1024
                           ? gemm<double, double, double, false, false, 8, kFull>(rest, i0 + kNB, kNB, 1.0,
                                                                                    L + (i0 + kNB) * K + i0, K,
                                                                                    X + i0 * K, K, 1.0, Srest, K, s)
                           : gemm<double, double, double, false, false, 4, kFull>(rest, i0 + kNB, kNB, 1.0,
                                                                                    L + (i0 + kNB) * K + i0, K,
                                                                                    X + i0 * K, K, 1.0, Srest, K, s))
      return e;
  }
  flip_to_upper_f32_kernel<<<dim3(grid_x(K), (unsigned)K), 256, 0, s>>>(X, U, K);
  return hipGetLastError();
}

// H = (2/T) x^T x in fp64 (both triangles), x bf16 [T][K].
hipError_t launch_gptq_hessian(const uint16_t* x, int64_t T, int64_t K, double* H, hipStream_t s) {
  return gemm<uint16_t, uint16_t, double, true, false, 8, kSymmetric>(K, K, T, 2.0 / (double)T, x, K, x, K, 0.0, H,
                                                                       K, s);
}

// W[:, b0+128:] -= err^T U[b0:b0+128, b0+128:] (fp32; err [128][N]).
hipError_t launch_gptq_update(float* W, int64_t N, int64_t K, int64_t b0, const float* U, const float* err,
                              hipStream_t s) {
  const int64_t b1 = b0 + kGroup;
  if (b1 >= K) return hipSuccess;
  return gemm<float, float, float, true, false, 8, kFull>(N, K - b1, kGroup, -1.0f, err, N, U + b0 * K + b1, K, 1.0f,
                                                          W + b1, K, s);
}

// y[t][n] = sum_k x[t][k] W[n][k] in fp32 (x bf16 [T][K], W fp32 [N][K]).
hipError_t launch_dense_linear_f32(const uint16_t* x, int64_t T, int64_t K, const float* W, int64_t N, float* y,
                                   hipStream_t s) {
  return gemm<uint16_t, float, float, false, true, 8, kFull>(T, N, K, 1.0f, x, K, W, K, 0.0f, y, N, s);
}

}  // namespace w4
