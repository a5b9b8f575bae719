// W4A16 linear: y[M][N] = x[M][K] * W_hat^T with W_hat = d * q (Qwen3.5-4B
// quantization study, section 1: y = W x and the group-quantization equation;
// section 2: 4-bit weights, BF16 inputs).  Decode runs it at M = 1 and
// draft verification at M = K + 1 (27B quantization-and-drafter ladder,
// stage 2), so it is bound by streaming the packed weights from HBM.
//
// Both kernels read the same native layout (one 1 KiB tile = 16 rows x one
// 128-input group, 16 bytes per lane) and the same decomposition:
//   * a workgroup owns R consecutive 16-row blocks and all K;
//   * its NW wavefronts split the groups of K into contiguous ranges;
//   * each wavefront keeps PF groups of weight tiles in flight (a register
//     ring), so the loads of later groups overlap the math of earlier ones;
//   * partial sums of the wavefronts are combined in LDS in a fixed order,
//     so results are bitwise reproducible (no atomics).
// Nibbles are widened in registers to bf16 1 + u/16 = 1.5 + q/16 (see
// unpack_word); each group's partial starts from -1.5 * (sum of the x values it
// multiplies), so after the group it holds sum(q x)/16, which is scaled by the
// group's d and accumulated in fp32.  The factor 16 is applied at the end.
#include "w4_device.h"
#include "w4_launch.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

namespace w4 {
namespace {

constexpr uint16_t kBf16NegOneHalf = 0xBFC0;  // bf16 -1.5

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return bitcast<bf16x8>(v); }

__device__ __forceinline__ bf16x8 unpack_step(uint32_t w, const UnpackConsts& uc) {
  uint32_t b[4];
  unpack_word(w, b, uc);
  return bitcast<bf16x8>(u32x4{b[0], b[1], b[2], b[3]});
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(a), bitcast<bf16x2>(b), c, false);
}

// ---------------------------------------------------------------------------
// MFMA kernel.  One v_mfma_f32_16x16x32_bf16 per 32-input step: A = 16 rows
// of x (rows >= M are zero), B = the tile's 16 rows of W^T.  Lane l holds
// A[l%16][8(l/16)..+7], B[8(l/16)..+7][l%16] and D[4(l/16)+j][l%16], j = 0..3.
// The -1.5*sum(x) start value is itself one MFMA chain with B = -1.5.
// ---------------------------------------------------------------------------
template <int R, int NW, int PF>
__global__ __launch_bounds__(NW * 64) void linear_mfma_kernel(
    const uint16_t* __restrict__ x, int M, int K, int G, const uint4* __restrict__ qp,
    const float* __restrict__ dp, int N, int Nb, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, kb = lane >> 4;
  const int rb0 = blockIdx.x * R;
  const int m0 = blockIdx.y * 16;
  const int g0 = (int)(((int64_t)G * wave) / NW);
  const int g1 = (int)(((int64_t)G * (wave + 1)) / NW);
  const int rvalid = min(R, Nb - rb0);

  const bool xok = (m0 + nl) < M;
  const uint4* xs = reinterpret_cast<const uint4*>(x + (int64_t)(xok ? m0 + nl : 0) * K) + kb;

  uint4 bq[PF][R];
  float bd[PF][R];
  auto issue = [&](int s, int g) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rvalid) {
        const int64_t t = (int64_t)(rb0 + r) * G + g;
        bq[s][r] = load_stream(qp + t * kTileLanes + lane);
        bd[s][r] = load_stream(dp + t * kTileRows + nl);
      }
    }
  };
  auto load_x = [&](int g, uint4 (&xa)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xa[i] = xok ? xs[g * 16 + i * 4] : make_uint4(0, 0, 0, 0);
  };

#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (g0 + s < g1) issue(s, g0 + s);
  uint4 xa[4], xn[4];
  if (g0 < g1) load_x(g0, xa);

  const UnpackConsts uc = unpack_consts();
  const uint32_t kneg2 = (uint32_t)kBf16NegOneHalf | ((uint32_t)kBf16NegOneHalf << 16);
  const bf16x8 kneg = bitcast<bf16x8>(u32x4{kneg2, kneg2, kneg2, kneg2});

  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int gb = g0; gb < g1; gb += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int g = gb + s;
      if (g < g1) {
        if (g + 1 < g1) load_x(g + 1, xn);
        bf16x8 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = as_bf16x8(xa[i]);
        f32x4 off = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) off = mfma16x16x32(a[i], kneg, off);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r < rvalid) {
            const uint32_t wv[4] = {bq[s][r].x, bq[s][r].y, bq[s][r].z, bq[s][r].w};
            f32x4 c = off;
#pragma unroll
            for (int i = 0; i < 4; ++i) c = mfma16x16x32(a[i], unpack_step(wv[i], uc), c);
            const float dv = bd[s][r];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[r][j] += dv * c[j];
          }
        }
        if (g + PF < g1) issue(s, g + PF);
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[i] = xn[i];
      }
    }
  }

  auto store = [&](int r, const f32x4& v) {
    const int64_t n = (int64_t)(rb0 + r) * kTileRows + nl;
    if (n >= N) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + 4 * kb + j;
      if (m < M) y[(int64_t)m * N + n] = f32_to_bf16_rne(16.0f * v[j]);
    }
  };

  if constexpr (NW == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < rvalid) store(r, acc[r]);
  } else {
    __shared__ f32x4 red[NW][R][64];
#pragma unroll
    for (int r = 0; r < R; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    for (int r = wave; r < rvalid; r += NW) {
      f32x4 v = red[0][r][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const f32x4 o = red[w][r][lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] += o[j];
      }
      store(r, v);
    }
  }
}

// ---------------------------------------------------------------------------
// VALU kernel (v_dot2_f32_bf16).  Lane (row l%16, quarter l/16) multiplies its
// 32 weights of a group by the matching 32 inputs of each of MT x rows; the
// four quarters of a row are summed with cross-lane shuffles at the end.
// ---------------------------------------------------------------------------
template <int MT, int R, int NW, int PF>
__global__ __launch_bounds__(NW * 64) void linear_gemv_kernel(
    const uint16_t* __restrict__ x, int M, int K, int G, const uint4* __restrict__ qp,
    const float* __restrict__ dp, int N, int Nb, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, kb = lane >> 4;
  const int rb0 = blockIdx.x * R;
  const int m0 = blockIdx.y * MT;
  const int g0 = (int)(((int64_t)G * wave) / NW);
  const int g1 = (int)(((int64_t)G * (wave + 1)) / NW);
  const int rvalid = min(R, Nb - rb0);

  const uint4* xs[MT];
  bool xok[MT];
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) {
    xok[mm] = (m0 + mm) < M;
    xs[mm] = reinterpret_cast<const uint4*>(x + (int64_t)(xok[mm] ? m0 + mm : 0) * K) + kb;
  }

  uint4 bq[PF][R];
  float bd[PF][R];
  auto issue = [&](int s, int g) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rvalid) {
        const int64_t t = (int64_t)(rb0 + r) * G + g;
        bq[s][r] = load_stream(qp + t * kTileLanes + lane);
        bd[s][r] = load_stream(dp + t * kTileRows + nl);
      }
    }
  };
#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (g0 + s < g1) issue(s, g0 + s);

  const UnpackConsts uc = unpack_consts();
  const uint32_t kneg2 = (uint32_t)kBf16NegOneHalf | ((uint32_t)kBf16NegOneHalf << 16);

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.f;

  for (int gb = g0; gb < g1; gb += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int g = gb + s;
      if (g < g1) {
        uint32_t xv[MT][16];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 t = xok[mm] ? xs[mm][g * 16 + i * 4] : make_uint4(0, 0, 0, 0);
            xv[mm][4 * i + 0] = t.x; xv[mm][4 * i + 1] = t.y;
            xv[mm][4 * i + 2] = t.z; xv[mm][4 * i + 3] = t.w;
          }
        }
        float c0[MT];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
          float c = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) c = dot2(xv[mm][e], kneg2, c);
          c0[mm] = c;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r < rvalid) {
            const uint32_t wv[4] = {bq[s][r].x, bq[s][r].y, bq[s][r].z, bq[s][r].w};
            uint32_t b[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) unpack_word(wv[i], &b[4 * i], uc);
            const float dv = bd[s][r];
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) {
              float c = c0[mm];
#pragma unroll
              for (int e = 0; e < 16; ++e) c = dot2(b[e], xv[mm][e], c);
              acc[r][mm] += dv * c;
            }
          }
        }
        if (g + PF < g1) issue(s, g + PF);
      }
    }
  }

  // Sum the four quarters of each row: lanes l, l^16, l^32, l^48.
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      float v = acc[r][mm];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[r][mm] = v;
    }

  auto store = [&](int r, int mm, float v) {
    const int64_t n = (int64_t)(rb0 + r) * kTileRows + nl;
    const int m = m0 + mm;
    if (n < N && m < M) y[(int64_t)m * N + n] = f32_to_bf16_rne(16.0f * v);
  };

  if constexpr (NW == 1) {
    if (kb == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (r < rvalid)
#pragma unroll
          for (int mm = 0; mm < MT; ++mm) store(r, mm, acc[r][mm]);
    }
  } else {
    __shared__ float red[NW][R][MT][16];
    if (kb == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) red[wave][r][mm][nl] = acc[r][mm];
    }
    __syncthreads();
    // thread t of the block finalizes (r, mm, row) = t / 16 ..., fixed order over waves
    for (int e = threadIdx.x; e < R * MT * 16; e += NW * 64) {
      const int row = e & 15;
      const int mm = (e >> 4) % MT;
      const int r = (e >> 4) / MT;
      if (r < rvalid) {
        float v = red[0][r][mm][row];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[w][r][mm][row];
        const int64_t n = (int64_t)(rb0 + r) * kTileRows + row;
        const int m = m0 + mm;
        if (n < N && m < M) y[(int64_t)m * N + n] = f32_to_bf16_rne(16.0f * v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launch configuration
// ---------------------------------------------------------------------------
struct Cfg {
  int R, NW, PF;
};

// Every (R, NW, PF) compiled for each kernel.  W4_MFMA_CFG / W4_GEMV_CFG
// ("R,NW,PF") may pick one of them for measurement; anything else falls back
// to the built-in choice.
constexpr Cfg kCfgs[] = {{1, 4, 4}, {1, 8, 4}, {2, 4, 4}, {2, 8, 4}, {1, 8, 8}, {1, 16, 4}, {4, 4, 2}, {2, 4, 8}};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

int cfg_from_env(const char* name) {
  const char* s = getenv(name);
  if (!s) return -1;
  int R = 0, NW = 0, PF = 0;
  if (sscanf(s, "%d,%d,%d", &R, &NW, &PF) != 3) return -1;
  for (int i = 0; i < kNumCfgs; ++i)
    if (kCfgs[i].R == R && kCfgs[i].NW == NW && kCfgs[i].PF == PF) return i;
  return -1;
}

// Built-in choice: enough wavefronts in flight for the weight stream.  The
// bytes in flight are (N/16) * NW * PF KiB whatever R is, so small N gets more
// wavefronts per block; large N keeps R = 1..2 so that there are enough blocks.
int choose_cfg(int64_t N, int64_t K) {
  (void)K;
  const int64_t Nb = (N + kTileRows - 1) / kTileRows;
  if (Nb >= 1024) return 2;  // {2, 4, 4}
  if (Nb >= 256) return 1;   // {1, 8, 4}
  return 5;                  // {1, 16, 4}
}

template <int R, int NW, int PF>
void run_mfma(dim3 grid, hipStream_t st, const uint16_t* x, int M, int K, int G, const uint4* q,
              const float* d, int N, int Nb, uint16_t* y) {
  linear_mfma_kernel<R, NW, PF><<<grid, NW * 64, 0, st>>>(x, M, K, G, q, d, N, Nb, y);
}

template <int MT, int R, int NW, int PF>
void run_gemv(dim3 grid, hipStream_t st, const uint16_t* x, int M, int K, int G, const uint4* q,
              const float* d, int N, int Nb, uint16_t* y) {
  linear_gemv_kernel<MT, R, NW, PF><<<grid, NW * 64, 0, st>>>(x, M, K, G, q, d, N, Nb, y);
}

template <int MT>
void dispatch_gemv(int ci, dim3 grid, hipStream_t st, const uint16_t* x, int M, int K, int G,
                   const uint4* q, const float* d, int N, int Nb, uint16_t* y) {
  switch (ci) {
#define W4_CASE(i)                                                                          \
  case i:                                                                                   \
    run_gemv<MT, kCfgs[i].R, kCfgs[i].NW, kCfgs[i].PF>(grid, st, x, M, K, G, q, d, N, Nb, y); \
    break;
    W4_CASE(0) W4_CASE(1) W4_CASE(2) W4_CASE(3) W4_CASE(4) W4_CASE(5) W4_CASE(6) W4_CASE(7)
#undef W4_CASE
  }
}

}  // namespace

hipError_t launch_linear_mfma(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                              const float* d_packed, int64_t N, uint16_t* y, hipStream_t stream) {
  const int env = cfg_from_env("W4_MFMA_CFG");
  const int ci = env >= 0 ? env : choose_cfg(N, K);
  const int Nb = (int)((N + kTileRows - 1) / kTileRows);
  const int G = (int)(K / kGroup);
  const Cfg c = kCfgs[ci];
  const dim3 grid((unsigned)((Nb + c.R - 1) / c.R), (unsigned)((M + 15) / 16));
  const uint4* q = reinterpret_cast<const uint4*>(q_packed);
  switch (ci) {
#define W4_CASE(i)                                                                                   \
  case i:                                                                                            \
    run_mfma<kCfgs[i].R, kCfgs[i].NW, kCfgs[i].PF>(grid, stream, x, (int)M, (int)K, G, q, d_packed, \
                                                   (int)N, Nb, y);                                   \
    break;
    W4_CASE(0) W4_CASE(1) W4_CASE(2) W4_CASE(3) W4_CASE(4) W4_CASE(5) W4_CASE(6) W4_CASE(7)
#undef W4_CASE
  }
  return hipGetLastError();
}

hipError_t launch_linear_gemv(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                              const float* d_packed, int64_t N, uint16_t* y, hipStream_t stream) {
  const int env = cfg_from_env("W4_GEMV_CFG");
  const int ci = env >= 0 ? env : choose_cfg(N, K);
  const int Nb = (int)((N + kTileRows - 1) / kTileRows);
  const int G = (int)(K / kGroup);
  const Cfg c = kCfgs[ci];
  const uint4* q = reinterpret_cast<const uint4*>(q_packed);
  const int MT = M >= 4 ? 4 : (int)M;
  const dim3 grid((unsigned)((Nb + c.R - 1) / c.R), (unsigned)((M + MT - 1) / MT));
  switch (MT) {
    case 1: dispatch_gemv<1>(ci, grid, stream, x, (int)M, (int)K, G, q, d_packed, (int)N, Nb, y); break;
    case 2: dispatch_gemv<2>(ci, grid, stream, x, (int)M, (int)K, G, q, d_packed, (int)N, Nb, y); break;
    case 3: dispatch_gemv<3>(ci, grid, stream, x, (int)M, (int)K, G, q, d_packed, (int)N, Nb, y); break;
    default: dispatch_gemv<4>(ci, grid, stream, x, (int)M, (int)K, G, q, d_packed, (int)N, Nb, y); break;
  }
  return hipGetLastError();
}

}  // namespace w4
