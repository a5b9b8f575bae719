// Device-side helpers shared by the w4 kernels (gfx950 / CDNA4 only).
//
// Native tile layout (see include/w4.h): a tile is 16 rows x 128 inputs (one
// quantization group of 128 consecutive inputs, Qwen3.5-4B quantization study
// section 1).  Lane L of a 64-wide wavefront owns row L%16 and, in each of the
// four 32-input steps i of the group, the 8 inputs 32i + 8(L/16) .. +7.  That
// is exactly the B-operand footprint of one v_mfma_f32_16x16x32_bf16 per step,
// so a whole tile is one coalesced 1 KiB wavefront load (16 bytes per lane).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

constexpr int kGroup = 128;      // inputs per quantization group
constexpr int kTileRows = 16;    // rows per tile
constexpr int kTileLanes = 64;   // 16-byte lanes per tile (1 KiB)
constexpr float kMaxCode = 7.0f; // largest magnitude maps to code +-7
constexpr uint32_t kNanBits = 0x7FC00000u;

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

__device__ __forceinline__ uint32_t rotl32(uint32_t v, int s) {
  return __builtin_amdgcn_alignbit(v, v, 32 - s);
}
__device__ __forceinline__ uint32_t rotr32(uint32_t v, int s) {
  return __builtin_amdgcn_alignbit(v, v, s);
}

// Offset-binary nibble u (0..15) of input j (0..7) inside a native word, before
// the rotate-left by 3: even j in the low half, odd j in the high half.
__device__ __forceinline__ int nibble_shift(int j) {
  return (j & 1) ? 16 + 4 * (j >> 1) : 4 * (j >> 1);
}

// Constants of the nibble widening, held in registers: gfx9 VOP3 encodings
// take no 32-bit literal, so with immediate masks the compiler would split
// every (w & mask) | magic into two instructions instead of one v_and_or_b32.
struct UnpackConsts {
  uint32_t mask;   // mantissa bits 3..6 of both bf16 halves (SGPR)
  uint32_t magic;  // bf16 1.0 in both halves (VGPR)
};

__device__ __forceinline__ UnpackConsts unpack_consts() {
  UnpackConsts c{0x00780078u, 0x3F803F80u};
  asm volatile("" : "+s"(c.mask));
  asm volatile("" : "+v"(c.magic));
  return c;
}

// Native word -> four bf16 pairs (inputs 2p, 2p+1 for p = 0..3).
// Each nibble u lands in mantissa bits 3..6 of bf16 1.0, giving 1 + u/16
// = 1.5 + q/16 exactly; the kernels remove the 1.5 through their accumulator
// start value and scale the result by 16 at the end.  Seven VALU
// instructions per word: three rotates and four v_and_or_b32.
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t out[4], const UnpackConsts& c) {
  out[0] = (w & c.mask) | c.magic;
  out[1] = (rotr32(w, 4) & c.mask) | c.magic;
  out[2] = (rotr32(w, 8) & c.mask) | c.magic;
  out[3] = (rotr32(w, 12) & c.mask) | c.magic;
}

// Raw buffer loads.  A resource covers [base, base + bytes); a load at or past
// `bytes` returns zeros without touching memory, which lets loops issue every
// load unconditionally (no branches, exact in-order vmcnt waits).
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw (untyped) buffer resource, gfx9 family
constexpr int kNonTemporal = 2;               // cache policy of streaming loads (each byte read once)

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

template <int AUX>
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T, typename S>
__device__ __forceinline__ T bitcast(const S& s) {
  static_assert(sizeof(T) == sizeof(S), "size mismatch");
  return __builtin_bit_cast(T, s);
}

}  // namespace w4
