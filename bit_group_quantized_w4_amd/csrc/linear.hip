// W4A16 linear: y[M][N] = x[M][K] * W_hat^T with W_hat = d * q (Qwen3.5-4B
// quantization study, section 1: y = W x and the group-quantization equation;
// section 2: 4-bit weights, BF16 inputs).  Decode runs it at M = 1 and
// draft verification at M = K + 1 (27B quantization-and-drafter ladder,
// stage 2), so it is bound by streaming the packed weights from HBM.
//
// One launch serves a batch of up to kMaxBatch independent linears (a single
// w4_linear call is a batch of one).  Work decomposition, per linear:
//   * a workgroup owns R consecutive 16-row blocks, all K, and one slab of
//     x rows (16 for the MFMA kernel, MT for the dot2 kernel);
//   * its NW wavefronts split K into contiguous ranges of whole scale quads
//     (4 groups of 128 inputs);
//   * each wavefront walks its range one group at a time with a 4-deep
//     register ring of loads, issued in exactly the order they are consumed,
//     so waiting for group g never waits for loads issued after it; the
//     16-byte scale quad of each row is loaded once per 4 groups into a
//     double buffer;
//   * weight tiles and scales use non-temporal loads (each byte is read once);
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

namespace w4 {
namespace {

constexpr uint16_t kBf16NegOneHalf = 0xBFC0;  // bf16 -1.5
constexpr int kRing = 4;                      // groups in flight per wavefront = one scale quad

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 unpack_step(uint32_t w, const UnpackConsts& uc) {
  uint32_t b[4];
  unpack_word(w, b, uc);
  return bitcast<bf16x8>(u32x4{b[0], b[1], b[2], b[3]});
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(a), bitcast<bf16x2>(b), c, false);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float quad_elem(const uint4& v, int s) { return __uint_as_float(word(v, s)); }

// Which linear of the batch, and which (row panel, x slab) of it, a block runs.
struct Work {
  int di, rb0, m0;
};

__device__ __forceinline__ Work locate(const BatchArgs& a, int R, int MT) {
  const int b = blockIdx.x;
  int di = 0;
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (i < a.count && b >= a.block0[i]) di = i;
  const LinearDesc& d = a.desc[di];
  const int nb = (d.N + kTileRows - 1) / kTileRows;
  const int panels = (nb + R - 1) / R;
  const int local = b - a.block0[di];
  const int slab = local / panels;
  return Work{di, (local - slab * panels) * R, slab * MT};
}

// ---------------------------------------------------------------------------
// MFMA kernel.  One v_mfma_f32_16x16x32_bf16 per 32-input step: A = 16 rows
// of x, B = the tile's 16 rows of W^T.  Lane l holds A[l%16][8(l/16)..+7],
// B[8(l/16)..+7][l%16] and D[4(l/16)+j][l%16], j = 0..3.  Rows of A at or
// beyond M repeat row M-1 (their outputs are computed and discarded), so every
// lane loads valid memory with no branches.  The -1.5*sum(x) start value is
// itself one MFMA chain with B = -1.5.
// ---------------------------------------------------------------------------
template <int R, int NW>
__global__ __launch_bounds__(NW * 64) void linear_mfma_kernel(const BatchArgs args) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, kb = lane >> 4;
  const Work wk = locate(args, R, 16);
  const LinearDesc& D = args.desc[wk.di];
  const int M = D.M, K = D.K, N = D.N;
  const int G = K / kGroup;
  const int Q = (G + 3) >> 2;  // scale quads; the native layout pads G to 4Q groups
  const int nb = (N + kTileRows - 1) / kTileRows;
  const int rvalid = min(R, nb - wk.rb0);
  const int j0 = (int)(((int64_t)Q * wave) / NW), j1 = (int)(((int64_t)Q * (wave + 1)) / NW);

  const int xrow = min(wk.m0 + nl, M - 1);
  const uint4* xs = reinterpret_cast<const uint4*>(D.x + (int64_t)xrow * K) + kb;
  // Row blocks past the end of the matrix re-read the last one (never stored).
  const uint4* qrow[R];
  const uint4* srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rb = min(wk.rb0 + r, nb - 1);
    qrow[r] = reinterpret_cast<const uint4*>(D.q) + rb * (4 * Q) * kTileLanes + lane;
    srow[r] = reinterpret_cast<const uint4*>(D.d) + rb * Q * kTileRows + nl;
  }

  uint4 bx[kRing][4];
  uint4 bw[kRing][R];
  uint4 sc[R], sn[R];  // scale quads: current and next

  auto issue_group = [&](int s, int g) {
    const int gx = min(g, G - 1);  // padding groups: any valid x (their scale is 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) bx[s][i] = xs[gx * 16 + i * 4];
#pragma unroll
    for (int r = 0; r < R; ++r) bw[s][r] = load_stream(qrow[r] + g * kTileLanes);
  };
  auto issue_scales = [&](uint4 (&dst)[R], int j) {
#pragma unroll
    for (int r = 0; r < R; ++r) dst[r] = load_stream(srow[r] + j * kTileRows);
  };

  const UnpackConsts uc = unpack_consts();
  const uint32_t kneg2 = (uint32_t)kBf16NegOneHalf | ((uint32_t)kBf16NegOneHalf << 16);
  const bf16x8 kneg = bitcast<bf16x8>(u32x4{kneg2, kneg2, kneg2, kneg2});

  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int s) {
    bf16x8 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = bitcast<bf16x8>(bx[s][i]);
    f32x4 off = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) off = mfma16x16x32(a[i], kneg, off);
    f32x4 c[R];
#pragma unroll
    for (int r = 0; r < R; ++r) c[r] = off;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < R; ++r) c[r] = mfma16x16x32(a[i], unpack_step(word(bw[s][r], i), uc), c[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float dv = quad_elem(sc[r], s);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] += dv * c[r][e];
    }
  };

  if (j0 < j1) {
    issue_scales(sc, j0);
#pragma unroll
    for (int s = 0; s < kRing; ++s) issue_group(s, 4 * j0 + s);
    // steady state: every load unconditional, issued in consumption order
    for (int j = j0; j < j1 - 1; ++j) {
      issue_scales(sn, j + 1);
#pragma unroll
      for (int s = 0; s < kRing; ++s) {
        compute(s);
        issue_group(s, 4 * (j + 1) + s);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) sc[r] = sn[r];
    }
#pragma unroll
    for (int s = 0; s < kRing; ++s) compute(s);
  }

  auto store = [&](int r, const f32x4& v) {
    const int n = (wk.rb0 + r) * kTileRows + nl;
    if (n >= N) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = wk.m0 + 4 * kb + e;
      if (m < M) D.y[(int64_t)m * N + n] = f32_to_bf16_rne(16.0f * v[e]);
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
        for (int e = 0; e < 4; ++e) v[e] += o[e];
      }
      store(r, v);
    }
  }
}

// ---------------------------------------------------------------------------
// VALU kernel (v_dot2_f32_bf16).  Lane (row l%16, quarter l/16) multiplies its
// 32 weights of a group by the matching 32 inputs of each of the MT x rows of
// its slab; x is staged once per block in LDS (MT * K bf16).  The four
// quarters of a row are summed with cross-lane shuffles at the end.
// ---------------------------------------------------------------------------
template <int MT, int R, int NW>
__global__ __launch_bounds__(NW * 64) void linear_gemv_kernel(const BatchArgs args) {
  // LDS: x of the slab, [MT][4Q * 16] uint4 (zero past K), then the start
  // values -1.5 * sum(x) of every (row, group, quarter), [MT][4Q][4] floats.
  extern __shared__ uint4 xlds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, kb = lane >> 4;
  const Work wk = locate(args, R, MT);
  const LinearDesc& D = args.desc[wk.di];
  const int M = D.M, K = D.K, N = D.N;
  const int G = K / kGroup;
  const int Q = (G + 3) >> 2;
  const int GP = 4 * Q;
  const int nb = (N + kTileRows - 1) / kTileRows;
  const int rvalid = min(R, nb - wk.rb0);
  const int j0 = (int)(((int64_t)Q * wave) / NW), j1 = (int)(((int64_t)Q * (wave + 1)) / NW);
  const uint4* qrow[R];
  const uint4* srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rb = min(wk.rb0 + r, nb - 1);
    qrow[r] = reinterpret_cast<const uint4*>(D.q) + rb * GP * kTileLanes + lane;
    srow[r] = reinterpret_cast<const uint4*>(D.d) + rb * Q * kTileRows + nl;
  }

  uint4 bw[kRing][R];
  uint4 sc[R], sn[R];
  auto issue_group = [&](int s, int g) {
#pragma unroll
    for (int r = 0; r < R; ++r) bw[s][r] = load_stream(qrow[r] + g * kTileLanes);
  };
  auto issue_scales = [&](uint4 (&dst)[R], int j) {
#pragma unroll
    for (int r = 0; r < R; ++r) dst[r] = load_stream(srow[r] + j * kTileRows);
  };
  if (j0 < j1) {
    issue_scales(sc, j0);
#pragma unroll
    for (int s = 0; s < kRing; ++s) issue_group(s, 4 * j0 + s);
  }

  const uint32_t kneg2 = (uint32_t)kBf16NegOneHalf | ((uint32_t)kBf16NegOneHalf << 16);

  // Stage the slab's x rows (rows beyond M repeat row M-1; their outputs are
  // dropped) together with the start value of every (row, group, quarter).
  float* offs = reinterpret_cast<float*>(xlds + MT * GP * 16);
  for (int e = threadIdx.x; e < MT * GP * 4; e += NW * 64) {
    const int mm = e / (GP * 4);
    const int rem = e - mm * GP * 4;
    const int g = rem >> 2, q4 = rem & 3;
    uint4 v[4];
    if (g < G) {
      const uint4* src = reinterpret_cast<const uint4*>(D.x + (int64_t)min(wk.m0 + mm, M - 1) * K) + g * 16 + q4;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = src[i * 4];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = make_uint4(0, 0, 0, 0);
    }
    float c = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c = dot2(v[i].x, kneg2, c);
      c = dot2(v[i].y, kneg2, c);
      c = dot2(v[i].z, kneg2, c);
      c = dot2(v[i].w, kneg2, c);
      xlds[(mm * GP + g) * 16 + i * 4 + q4] = v[i];
    }
    offs[(mm * GP + g) * 4 + q4] = c;
  }
  __syncthreads();

  const UnpackConsts uc = unpack_consts();

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.f;

  auto compute = [&](int s, int g) {
    uint32_t xv[MT][16];
    float c0[MT];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 t = xlds[(mm * GP + g) * 16 + i * 4 + kb];
        xv[mm][4 * i + 0] = t.x; xv[mm][4 * i + 1] = t.y;
        xv[mm][4 * i + 2] = t.z; xv[mm][4 * i + 3] = t.w;
      }
      c0[mm] = offs[(mm * GP + g) * 4 + kb];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t b[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) unpack_word(word(bw[s][r], i), &b[4 * i], uc);
      const float dv = quad_elem(sc[r], s);
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        float c = c0[mm];
#pragma unroll
        for (int e = 0; e < 16; ++e) c = dot2(b[e], xv[mm][e], c);
        acc[r][mm] += dv * c;
      }
    }
  };

  if (j0 < j1) {
    for (int j = j0; j < j1 - 1; ++j) {
      issue_scales(sn, j + 1);
#pragma unroll
      for (int s = 0; s < kRing; ++s) {
        compute(s, 4 * j + s);
        issue_group(s, 4 * (j + 1) + s);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) sc[r] = sn[r];
    }
#pragma unroll
    for (int s = 0; s < kRing; ++s) compute(s, 4 * (j1 - 1) + s);
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

  __shared__ float red[NW][R][MT][16];
  if (kb == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) red[wave][r][mm][nl] = acc[r][mm];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < R * MT * 16; e += NW * 64) {
    const int row = e & 15;
    const int mm = (e >> 4) % MT;
    const int r = (e >> 4) / MT;
    if (r < rvalid) {
      float v = red[0][r][mm][row];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += red[w][r][mm][row];
      const int n = (wk.rb0 + r) * kTileRows + row;
      const int m = wk.m0 + mm;
      if (n < N && m < M) D.y[(int64_t)m * N + n] = f32_to_bf16_rne(16.0f * v);
    }
  }
}

// ---------------------------------------------------------------------------
// launch configuration
// ---------------------------------------------------------------------------
struct Cfg {
  int R, NW;
};

// Every (R, NW) compiled for each kernel.  W4_MFMA_CFG / W4_GEMV_CFG ("R,NW")
// may pick one of them for measurement; anything else falls back to the
// built-in choice.
constexpr Cfg kCfgs[] = {{1, 4}, {1, 8}, {2, 4}, {2, 8}, {1, 16}, {4, 4}, {4, 8}, {1, 2}};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

int cfg_from_env(const char* name) {
  const char* s = getenv(name);
  if (!s) return -1;
  int R = 0, NW = 0;
  if (sscanf(s, "%d,%d", &R, &NW) != 2) return -1;
  for (int i = 0; i < kNumCfgs; ++i)
    if (kCfgs[i].R == R && kCfgs[i].NW == NW) return i;
  return -1;
}

int find_cfg(int R, int NW) {
  for (int i = 0; i < kNumCfgs; ++i)
    if (kCfgs[i].R == R && kCfgs[i].NW == NW) return i;
  return 0;
}

// Built-in choices, from graph-replayed sweeps of every (R, NW) on MI355X over
// the 4B/27B/70B-class projection shapes: enough wavefronts in flight on all
// 256 CUs for the batch's total row blocks, more wavefronts per block when K
// is long.
int choose_cfg_mfma(const BatchArgs& a) {
  int64_t rows = 0;
  for (int i = 0; i < a.count; ++i) rows += (a.desc[i].N + kTileRows - 1) / kTileRows;
  return rows >= 384 ? find_cfg(2, 4) : find_cfg(1, 4);
}

int choose_cfg_gemv(const BatchArgs& a) {
  int64_t rows = 0;
  int kmax = 0;
  for (int i = 0; i < a.count; ++i) {
    rows += (a.desc[i].N + kTileRows - 1) / kTileRows;
    kmax = a.desc[i].K > kmax ? a.desc[i].K : kmax;
  }
  if (rows < 256) return find_cfg(1, 8);
  return find_cfg(1, kmax >= 16384 ? 8 : 4);
}

int64_t fill_blocks(BatchArgs& a, int R, int slab_rows) {
  int64_t total = 0;
  for (int i = 0; i < a.count; ++i) {
    a.block0[i] = (int)total;
    const int nb = (a.desc[i].N + kTileRows - 1) / kTileRows;
    const int panels = (nb + R - 1) / R;
    const int slabs = (a.desc[i].M + slab_rows - 1) / slab_rows;
    total += (int64_t)panels * slabs;
  }
  return total;
}

}  // namespace

hipError_t launch_linear_mfma(BatchArgs& a, hipStream_t stream) {
  const int env = cfg_from_env("W4_MFMA_CFG");
  const int ci = env >= 0 ? env : choose_cfg_mfma(a);
  const Cfg c = kCfgs[ci];
  const int64_t blocks = fill_blocks(a, c.R, 16);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  switch (ci) {
#define W4_CASE(i)                                                                               \
  case i:                                                                                        \
    linear_mfma_kernel<kCfgs[i].R, kCfgs[i].NW><<<(unsigned)blocks, kCfgs[i].NW * 64, 0, stream>>>(a); \
    break;
    W4_CASE(0) W4_CASE(1) W4_CASE(2) W4_CASE(3) W4_CASE(4) W4_CASE(5) W4_CASE(6) W4_CASE(7)
#undef W4_CASE
  }
  return hipGetLastError();
}

int gemv_rows_per_slab(int64_t M, int64_t K) {
  for (int mt = 4; mt > 1; mt >>= 1)
    if (M >= mt && gemv_lds_bytes(mt, K) <= kGemvLdsBytes) return mt;
  return 1;
}

hipError_t launch_linear_gemv(BatchArgs& a, int MT, hipStream_t stream) {
  const int env = cfg_from_env("W4_GEMV_CFG");
  int ci = env >= 0 ? env : choose_cfg_gemv(a);
  if (MT == 4 && kCfgs[ci].NW == 16) ci = find_cfg(1, 8);  // 16 wavefronts x 4 rows exceeds 128 VGPRs
  const Cfg c = kCfgs[ci];
  const int64_t blocks = fill_blocks(a, c.R, MT);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  int kmax = 0;
  for (int i = 0; i < a.count; ++i) kmax = a.desc[i].K > kmax ? a.desc[i].K : kmax;
  const size_t lds = (size_t)gemv_lds_bytes(MT, kmax);
#define W4_LAUNCH(mt, i)                                                                          \
  linear_gemv_kernel<mt, kCfgs[i].R, kCfgs[i].NW><<<(unsigned)blocks, kCfgs[i].NW * 64, lds, stream>>>(a)
#define W4_CASES(mt)                                 \
  switch (ci) {                                      \
    case 0: W4_LAUNCH(mt, 0); break;                 \
    case 1: W4_LAUNCH(mt, 1); break;                 \
    case 2: W4_LAUNCH(mt, 2); break;                 \
    case 3: W4_LAUNCH(mt, 3); break;                 \
    case 4: W4_LAUNCH(mt, 4); break;                 \
    case 5: W4_LAUNCH(mt, 5); break;                 \
    case 6: W4_LAUNCH(mt, 6); break;                 \
    default: W4_LAUNCH(mt, 7); break;                \
  }
  if (MT == 4) {
    W4_CASES(4)
  } else if (MT == 2) {
    W4_CASES(2)
  } else {
    W4_CASES(1)
  }
#undef W4_CASES
#undef W4_LAUNCH
  return hipGetLastError();
}

}  // namespace w4
