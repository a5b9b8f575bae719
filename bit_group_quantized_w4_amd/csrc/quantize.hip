// RTN INT4 group quantization and native <-> canonical layout conversion.
//
// Quantizer: Qwen3.5-4B quantization study, section 1 group-quantization
// equation q = clip(round(w/d) + z, qmin, qmax) with z = 0 (symmetric), one
// restore scale d per group of 128 consecutive inputs of a row; section 2
// settings: RTN, group 128, min/max symmetric range, no clipping search.
// Conventions (pages silent): d = fl32(max|w| / 7) by IEEE division; codes
// clamp(round_half_away(fl32(w / d)), -8, 7); a group with a NaN/Inf gets
// d = NaN (0x7FC00000) and codes 0; d == 0 gives codes 0.  Subnormals are
// kept (the build leaves fp32 denormals on and uses no fast-math).
//
// One wavefront quantizes one 16 x 128 tile: every lane reads the 32 weights
// it will own in the native layout (its row, 8 inputs in each of the four
// 32-input steps), the group max is finished across the four lanes that share
// a row, and the lane writes its 16 bytes of codes; the 16 scales of the tile
// are written by the lanes of the first quarter into their rows' scale quads.
#include "w4_device.h"
#include "w4_launch.h"

#include <float.h>

namespace w4 {
namespace {

constexpr int kTilesPerBlock = 4;  // one tile per wavefront, 4 wavefronts per block

// Native scale layout: the scales of row n for the four consecutive groups
// 4j .. 4j+3 are one 16-byte quad, quad (r, j) of row block r holding rows
// 16r .. 16r+15 in order; the group count is padded to a multiple of 4 with
// zero scales.
__device__ __forceinline__ int64_t scale_index(int64_t r, int Q, int g, int nl) {
  return ((r * Q + (g >> 2)) * kTileRows + nl) * 4 + (g & 3);
}

// Zero scales of the padding groups G .. 4Q-1 (written by the last group's tile).
__device__ __forceinline__ void zero_scale_padding(float* dp, int64_t r, int Q, int G, int g, int nl) {
  if (g == G - 1)
    for (int gp = G; gp < 4 * Q; ++gp) dp[scale_index(r, Q, gp, nl)] = 0.0f;
}

__device__ __forceinline__ uint32_t native_word(const int u[8]) {
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) v |= (uint32_t)u[j] << nibble_shift(j);
  return rotl32(v, 3);
}

__global__ __launch_bounds__(256) void quantize_rtn_kernel(const float* __restrict__ W, int N,
                                                           int K, int G, int64_t ntiles,
                                                           uint4* __restrict__ qp,
                                                           float* __restrict__ dp) {
#pragma clang fp contract(off)
  const int64_t tile = (int64_t)blockIdx.x * kTilesPerBlock + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int lane = threadIdx.x & 63;
  const int nl = lane & 15, kb = lane >> 4;
  const int64_t r = tile / G;
  const int g = (int)(tile - r * G);
  const int64_t n = r * kTileRows + nl;

  float v[32];
  if (n < N) {
    const float4* src = reinterpret_cast<const float4*>(W + n * K + (int64_t)g * kGroup + 8 * kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = src[8 * i];
      const float4 b = src[8 * i + 1];
      v[8 * i + 0] = a.x; v[8 * i + 1] = a.y; v[8 * i + 2] = a.z; v[8 * i + 3] = a.w;
      v[8 * i + 4] = b.x; v[8 * i + 5] = b.y; v[8 * i + 6] = b.z; v[8 * i + 7] = b.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = 0.0f;  // padding rows quantize as zero rows
  }

  // Group range (symmetric min/max): the largest magnitude, plus a flag for
  // non-finite members.  max is exact, so the reduction order does not matter.
  float amax = 0.0f;
  int bad = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float a = fabsf(v[j]);
    bad |= !(a <= FLT_MAX);
    amax = fmaxf(amax, a);
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  bad |= __shfl_xor(bad, 16);
  bad |= __shfl_xor(bad, 32);

  // Restore scale: +-max maps to code +-7.
  const float d = bad ? __uint_as_float(kNanBits) : amax / kMaxCode;
  const bool usable = !bad && d != 0.0f;

  uint32_t words[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int code = 0;
      if (usable) {
        const float t = v[8 * i + j] / d;  // IEEE fp32 quotient by the stored scale
        float rr = truncf(t);
        if (fabsf(t - rr) >= 0.5f) rr += copysignf(1.0f, t);  // ties away from zero
        rr = fminf(fmaxf(rr, -8.0f), 7.0f);
        code = (int)rr;
      }
      u[j] = code + 8;
    }
    words[i] = native_word(u);
  }
  qp[tile * kTileLanes + lane] = make_uint4(words[0], words[1], words[2], words[3]);
  if (kb == 0) {
    const int Q = (G + 3) >> 2;
    dp[scale_index(r, Q, g, nl)] = d;
    zero_scale_padding(dp, r, Q, G, g, nl);
  }
}

__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ qc,
                                                   const float* __restrict__ dc, int N, int K,
                                                   int G, int64_t ntiles, uint4* __restrict__ qp,
                                                   float* __restrict__ dp) {
  const int64_t tile = (int64_t)blockIdx.x * kTilesPerBlock + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int lane = threadIdx.x & 63;
  const int nl = lane & 15, kb = lane >> 4;
  const int64_t r = tile / G;
  const int g = (int)(tile - r * G);
  const int64_t n = r * kTileRows + nl;

  uint32_t words[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int u[8];
    if (n < N) {
      const uint2 raw = *reinterpret_cast<const uint2*>(qc + n * K + (int64_t)g * kGroup + 32 * i + 8 * kb);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t wv = j < 4 ? raw.x : raw.y;
        const int code = (int)(int8_t)((wv >> (8 * (j & 3))) & 0xFFu);
        u[j] = (code + 8) & 15;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = 8;
    }
    words[i] = native_word(u);
  }
  qp[tile * kTileLanes + lane] = make_uint4(words[0], words[1], words[2], words[3]);
  if (kb == 0) {
    const int Q = (G + 3) >> 2;
    dp[scale_index(r, Q, g, nl)] = n < N ? dc[n * G + g] : 0.0f;
    zero_scale_padding(dp, r, Q, G, g, nl);
  }
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint4* __restrict__ qp,
                                                     const float* __restrict__ dp, int N, int K,
                                                     int G, int64_t ntiles, int8_t* __restrict__ qc,
                                                     float* __restrict__ dc) {
  const int64_t tile = (int64_t)blockIdx.x * kTilesPerBlock + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int lane = threadIdx.x & 63;
  const int nl = lane & 15, kb = lane >> 4;
  const int64_t r = tile / G;
  const int g = (int)(tile - r * G);
  const int64_t n = r * kTileRows + nl;
  if (n >= N) return;

  const uint4 wq = qp[tile * kTileLanes + lane];
  const uint32_t w4v[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = rotr32(w4v[i], 3);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t code = (uint32_t)(int8_t)((int)((v >> nibble_shift(j)) & 15u) - 8) & 0xFFu;
      if (j < 4) lo |= code << (8 * j);
      else hi |= code << (8 * (j - 4));
    }
    *reinterpret_cast<uint2*>(qc + n * K + (int64_t)g * kGroup + 32 * i + 8 * kb) = make_uint2(lo, hi);
  }
  if (kb == 0) dc[n * G + g] = dp[scale_index(r, (G + 3) >> 2, g, nl)];
}

inline int64_t tiles_of(int64_t N, int64_t K) { return ((N + kTileRows - 1) / kTileRows) * (K / kGroup); }
inline unsigned blocks_of(int64_t ntiles) { return (unsigned)((ntiles + kTilesPerBlock - 1) / kTilesPerBlock); }

}  // namespace

hipError_t launch_quantize_rtn(const float* W, int64_t N, int64_t K, uint8_t* q_packed,
                               float* d_packed, hipStream_t stream) {
  const int64_t nt = tiles_of(N, K);
  quantize_rtn_kernel<<<blocks_of(nt), 256, 0, stream>>>(
      W, (int)N, (int)K, (int)(K / kGroup), nt, reinterpret_cast<uint4*>(q_packed), d_packed);
  return hipGetLastError();
}

hipError_t launch_pack(const int8_t* q_canon, const float* d_canon, int64_t N, int64_t K,
                       uint8_t* q_packed, float* d_packed, hipStream_t stream) {
  const int64_t nt = tiles_of(N, K);
  pack_kernel<<<blocks_of(nt), 256, 0, stream>>>(q_canon, d_canon, (int)N, (int)K,
                                                 (int)(K / kGroup), nt,
                                                 reinterpret_cast<uint4*>(q_packed), d_packed);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* q_packed, const float* d_packed, int64_t N, int64_t K,
                         int8_t* q_canon, float* d_canon, hipStream_t stream) {
  const int64_t nt = tiles_of(N, K);
  unpack_kernel<<<blocks_of(nt), 256, 0, stream>>>(reinterpret_cast<const uint4*>(q_packed),
                                                   d_packed, (int)N, (int)K, (int)(K / kGroup),
                                                   nt, q_canon, d_canon);
  return hipGetLastError();
}

}  // namespace w4
