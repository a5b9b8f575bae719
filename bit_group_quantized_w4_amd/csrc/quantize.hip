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
// Scales are stored as fp32 or, in the 16-bit variant, as the nearest bf16
// (the codes then divide by that stored value).
// Weights are read with raw buffer loads over the tile's row block: padding
// rows (N .. Np-1) and padding groups (G .. 4Q-1) read zeros, so they come out
// as code 0 with scale 0 without a branch.  Each load instruction covers two
// whole rows of the group (eight full 128-byte lines), so the loads can use
// the streaming (non-temporal) policy without fetching any line twice; the
// tile then goes through LDS (one 16 x 128 tile per wavefront, rows padded to
// 132 floats so the read-back is free of bank conflicts) to the lanes that own
// each weight in the native layout.  One tile per wavefront (rather than a
// loop over tiles) keeps the most loads in flight.
#include "w4_device.h"
#include "w4_launch.h"

#include <float.h>

namespace w4 {
namespace {

constexpr int kTilesPerBlock = 4;  // one tile per wavefront, 4 wavefronts per block

// Tile (r, g) of the native layout, g < GP = 4 * ceil(G / 4).
struct TileAt {
  int64_t tile, r;
  int g, nl, kb, lane;
  int64_t n;
};

__device__ __forceinline__ bool tile_at(int64_t ntiles, int GP, TileAt& t) {
  t.tile = (int64_t)blockIdx.x * kTilesPerBlock + (threadIdx.x >> 6);
  if (t.tile >= ntiles) return false;
  t.lane = threadIdx.x & 63;
  t.nl = t.lane & 15;
  t.kb = t.lane >> 4;
  t.r = t.tile / GP;
  t.g = (int)(t.tile - t.r * GP);
  t.n = t.r * kTileRows + t.nl;
  return true;
}

// Scales of row n for groups 4j .. 4j+3 form one 16-byte quad; quad (r, j)
// of row block r holds rows 16r .. 16r+15 in order.
__device__ __forceinline__ int64_t scale_index(int64_t r, int GP, int g, int nl) {
  return ((r * (GP >> 2) + (g >> 2)) * kTileRows + nl) * 4 + (g & 3);
}

__device__ __forceinline__ uint32_t native_word(const int u[8]) {
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) v |= (uint32_t)u[j] << nibble_shift(j);
  return rotl32(v, 3);
}

// S: the stored scale, float (fp32) or uint16_t (bf16 bit pattern).
// kColScale: the weights are first multiplied column by column by cs[k] in
// fp32 (channel scaling before RTN, the study's section 2 AWQ row).
template <typename S, bool kColScale = false>
__global__ __launch_bounds__(256) void quantize_rtn_kernel(const float* __restrict__ W, int N,
                                                           int K, int G, int GP, int64_t ntiles,
                                                           uint4* __restrict__ qp,
                                                           S* __restrict__ dp,
                                                           const float* __restrict__ cs = nullptr) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, nl = lane & 15, kb = lane >> 4;
  // the wavefront index is uniform across the wavefront: keep the tile, and
  // with it the buffer resource, in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t tile = (int64_t)blockIdx.x * kTilesPerBlock + wave;
  if (tile >= ntiles) return;
  const int64_t r = tile / GP;
  const int g = (int)(tile - r * GP);

  // The 32 weights of this lane; zeros outside the matrix.
  __shared__ float tile_lds[kTilesPerBlock][kTileRows][132];
  float(&tl)[kTileRows][132] = tile_lds[wave];
  float v[32];
  {
    const int64_t n0 = r * kTileRows;
    const int64_t rows = min((int64_t)kTileRows, (int64_t)N - n0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + n0 * K, (uint32_t)(rows * K * 4));
    // instruction p: lanes 0-31 read row 2p, lanes 32-63 row 2p+1, 16 bytes each
    const int hr = lane >> 5, c4 = lane & 31;
    const uint32_t off = g < G ? ((uint32_t)hr * K + (uint32_t)g * kGroup + 4u * c4) * 4u : 0x80000000u;
    uint4 raw[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) raw[p] = bload<kNonTemporal>(rs, off + (uint32_t)(2 * p) * (uint32_t)K * 4u);
#pragma unroll
    for (int p = 0; p < 8; ++p) *reinterpret_cast<uint4*>(&tl[2 * p + hr][4 * c4]) = raw[p];
    // the tile is private to this wavefront: order its LDS writes before the reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 a = *reinterpret_cast<const uint4*>(&tl[nl][32 * i + 8 * kb]);
      const uint4 b = *reinterpret_cast<const uint4*>(&tl[nl][32 * i + 8 * kb + 4]);
      v[8 * i + 0] = __uint_as_float(a.x); v[8 * i + 1] = __uint_as_float(a.y);
      v[8 * i + 2] = __uint_as_float(a.z); v[8 * i + 3] = __uint_as_float(a.w);
      v[8 * i + 4] = __uint_as_float(b.x); v[8 * i + 5] = __uint_as_float(b.y);
      v[8 * i + 6] = __uint_as_float(b.z); v[8 * i + 7] = __uint_as_float(b.w);
    }
    if constexpr (kColScale) {
      if (g < G) {
        const float4* c = reinterpret_cast<const float4*>(cs + (int64_t)g * kGroup + 8 * kb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 a = c[8 * i], b = c[8 * i + 1];
          v[8 * i + 0] *= a.x; v[8 * i + 1] *= a.y; v[8 * i + 2] *= a.z; v[8 * i + 3] *= a.w;
          v[8 * i + 4] *= b.x; v[8 * i + 5] *= b.y; v[8 * i + 6] *= b.z; v[8 * i + 7] *= b.w;
        }
      }
    }
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

  // Restore scale: +-max maps to code +-7.  A 16-bit scale is stored as the
  // nearest bf16, and the codes are taken against that stored value.
  const float d32 = bad ? __uint_as_float(kNanBits) : amax / kMaxCode;
  S stored;
  float d;
  if constexpr (sizeof(S) == 2) {
    stored = f32_to_bf16_rne(d32);
    d = __uint_as_float((uint32_t)stored << 16);
  } else {
    stored = d32;
    d = d32;
  }
  const bool usable = !bad && d != 0.0f;
  // Unusable groups (d = 0 or NaN) divide by 1 and are then forced to code 0,
  // which keeps the loop free of branches.
  const float dd = usable ? d : 1.0f;

  // Quotients w / d.  The code depends on the IEEE quotient only through
  // round-half-away, so w * rcp(d) gives the same code unless the quotient
  // lies near a half-integer: rcp is within 1 ulp and the product within
  // half an ulp, so for |w/d| <= 7 both values lie within 1.5e-6 of w/d.
  // When any lane of the wavefront has a product within 2^-17 (7.6e-6) of a
  // half-integer, or a scale outside [2^-120, 2^120] (where rcp may lose
  // range), the wavefront recomputes every quotient with IEEE division.
  float t[32];
  const float rd = __builtin_amdgcn_rcpf(dd);
  bool near = !(dd >= 0x1p-120f && dd <= 0x1p+120f);
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    t[j] = v[j] * rd;
    const float a = fabsf(t[j]);
    near |= fabsf((a - truncf(a)) - 0.5f) < 0x1p-17f;
  }
  if (__ballot(near)) {
#pragma unroll
    for (int j = 0; j < 32; ++j) t[j] = v[j] / dd;  // IEEE fp32 quotient by the stored scale
  }

  uint32_t words[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q = t[8 * i + j];
      float rr = truncf(q);
      rr = fabsf(q - rr) >= 0.5f ? rr + copysignf(1.0f, q) : rr;  // ties away from zero
      rr = fminf(fmaxf(rr, -8.0f), 7.0f);
      u[j] = (usable ? (int)rr : 0) + 8;
    }
    words[i] = native_word(u);
  }
  qp[tile * kTileLanes + lane] = make_uint4(words[0], words[1], words[2], words[3]);
  if (kb == 0) dp[scale_index(r, GP, g, nl)] = stored;
}

template <typename S>
__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ qc,
                                                   const S* __restrict__ dc, int N, int K,
                                                   int G, int GP, int64_t ntiles,
                                                   uint4* __restrict__ qp, S* __restrict__ dp) {
  TileAt t;
  if (!tile_at(ntiles, GP, t)) return;
  const bool real = t.n < N && t.g < G;
  uint32_t words[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int u[8];
    if (real) {
      const uint2 raw = *reinterpret_cast<const uint2*>(qc + t.n * K + (int64_t)t.g * kGroup + 32 * i + 8 * t.kb);
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
  qp[t.tile * kTileLanes + t.lane] = make_uint4(words[0], words[1], words[2], words[3]);
  if (t.kb == 0) dp[scale_index(t.r, GP, t.g, t.nl)] = real ? dc[t.n * G + t.g] : S(0);
}

template <typename S>
__global__ __launch_bounds__(256) void unpack_kernel(const uint4* __restrict__ qp,
                                                     const S* __restrict__ dp, int N, int K,
                                                     int G, int GP, int64_t ntiles,
                                                     int8_t* __restrict__ qc, S* __restrict__ dc) {
  TileAt t;
  if (!tile_at(ntiles, GP, t)) return;
  if (t.n >= N || t.g >= G) return;
  const uint4 wq = qp[t.tile * kTileLanes + t.lane];
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
    *reinterpret_cast<uint2*>(qc + t.n * K + (int64_t)t.g * kGroup + 32 * i + 8 * t.kb) = make_uint2(lo, hi);
  }
  if (t.kb == 0) dc[t.n * G + t.g] = dp[scale_index(t.r, GP, t.g, t.nl)];
}

struct Grid {
  int G, GP;
  int64_t ntiles;
  unsigned blocks;
};

inline Grid grid_of(int64_t N, int64_t K) {
  Grid g;
  g.G = (int)(K / kGroup);
  g.GP = (g.G + 3) / 4 * 4;
  g.ntiles = ((N + kTileRows - 1) / kTileRows) * g.GP;
  g.blocks = (unsigned)((g.ntiles + kTilesPerBlock - 1) / kTilesPerBlock);
  return g;
}

}  // namespace

hipError_t launch_quantize_rtn(const float* W, int64_t N, int64_t K, uint8_t* q_packed,
                               void* d_packed, bool s16, hipStream_t stream) {
  const Grid g = grid_of(N, K);
  uint4* qp = reinterpret_cast<uint4*>(q_packed);
  if (s16)
    quantize_rtn_kernel<uint16_t><<<g.blocks, 256, 0, stream>>>(W, (int)N, (int)K, g.G, g.GP, g.ntiles, qp,
                                                                 static_cast<uint16_t*>(d_packed));
  else
    quantize_rtn_kernel<float><<<g.blocks, 256, 0, stream>>>(W, (int)N, (int)K, g.G, g.GP, g.ntiles, qp,
                                                              static_cast<float*>(d_packed));
  return hipGetLastError();
}

hipError_t launch_quantize_rtn_scaled(const float* W, const float* cs, int64_t N, int64_t K, uint8_t* q_packed,
                                      void* d_packed, bool s16, hipStream_t stream) {
  const Grid g = grid_of(N, K);
  uint4* qp = reinterpret_cast<uint4*>(q_packed);
  if (s16)
    quantize_rtn_kernel<uint16_t, true><<<g.blocks, 256, 0, stream>>>(W, (int)N, (int)K, g.G, g.GP, g.ntiles, qp,
                                                                       static_cast<uint16_t*>(d_packed), cs);
  else
    quantize_rtn_kernel<float, true><<<g.blocks, 256, 0, stream>>>(W, (int)N, (int)K, g.G, g.GP, g.ntiles, qp,
                                                                    static_cast<float*>(d_packed), cs);
  return hipGetLastError();
}

hipError_t launch_pack(const int8_t* q_canon, const void* d_canon, int64_t N, int64_t K,
                       uint8_t* q_packed, void* d_packed, bool s16, hipStream_t stream) {
  const Grid g = grid_of(N, K);
  uint4* qp = reinterpret_cast<uint4*>(q_packed);
  if (s16)
    pack_kernel<uint16_t><<<g.blocks, 256, 0, stream>>>(q_canon, static_cast<const uint16_t*>(d_canon), (int)N,
                                                         (int)K, g.G, g.GP, g.ntiles, qp,
                                                         static_cast<uint16_t*>(d_packed));
  else
    pack_kernel<float><<<g.blocks, 256, 0, stream>>>(q_canon, static_cast<const float*>(d_canon), (int)N, (int)K,
                                                      g.G, g.GP, g.ntiles, qp, static_cast<float*>(d_packed));
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* q_packed, const void* d_packed, int64_t N, int64_t K,
                         int8_t* q_canon, void* d_canon, bool s16, hipStream_t stream) {
  const Grid g = grid_of(N, K);
  const uint4* qp = reinterpret_cast<const uint4*>(q_packed);
  if (s16)
    unpack_kernel<uint16_t><<<g.blocks, 256, 0, stream>>>(qp, static_cast<const uint16_t*>(d_packed), (int)N,
                                                           (int)K, g.G, g.GP, g.ntiles, q_canon,
                                                           static_cast<uint16_t*>(d_canon));
  else
    unpack_kernel<float><<<g.blocks, 256, 0, stream>>>(qp, static_cast<const float*>(d_packed), (int)N, (int)K,
                                                        g.G, g.GP, g.ntiles, q_canon, static_cast<float*>(d_canon));
  return hipGetLastError();
}

}  // namespace w4
