// W4A16 linear: y[M][N] = x[M][K] * W_hat^T with W_hat = d * q (Qwen3.5-4B
// quantization study, section 1: y = W x and the group-quantization equation;
// section 2: 4-bit weights, BF16 inputs).  Decode runs it at M = 1 and
// draft verification at M = K + 1 (27B quantization-and-drafter ladder,
// stage 2), so it is bound by streaming the packed weights from HBM.
//
// One launch serves a batch of up to kMaxBatch independent linears (a single
// w4_linear call is a batch of one), laid out longest K first.  Work
// decomposition, per linear:
//   * a workgroup owns R consecutive 16-row blocks, all K, and one slab of
//     x rows (16 for the MFMA kernel, MT for the dot2 kernel);
//   * its NW wavefronts split K into contiguous ranges of whole scale quads
//     (4 groups of 128 inputs) -- or, in the MFMA kernel's shared-x form,
//     each of the NW wavefronts takes R row blocks of its own over all of K
//     and the block shares each x tile through LDS;
//   * each wavefront walks its range quad by quad with a ring of loads in
//     flight, issued in exactly the order they are consumed;
//   * weight, scale and x loads are raw buffer loads: a quad beyond the
//     wavefront's range, or an x row beyond M, gets an offset past the end of
//     its buffer and reads zeros without touching memory, so every load in
//     the loop is unconditional (exact vmcnt waits, no branches) and the ring
//     needs no peeled tail (a zero scale cancels whatever zero codes give);
//   * weights and scales use non-temporal loads (each byte is read once);
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

#include <type_traits>

namespace w4 {
namespace {

constexpr uint16_t kBf16NegOneHalf = 0xBFC0;  // bf16 -1.5
// Offsets at or past these read zeros.  Codes and scales of one matrix stay
// below 2 GiB and x below 1 GiB (the C ABI refuses larger operands), so an
// in-range offset plus kOobW or kOobX never wraps around 2^32.
constexpr uint32_t kOobW = 0x80000000u;
constexpr uint32_t kOobX = 0x40000000u;

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Output element i of a linear: fp32 as accumulated, or rounded to bf16.
__device__ __forceinline__ void store_out(const LinearDesc& D, int64_t i, float v) {
  if (D.flags & kOutF32)
    static_cast<float*>(D.y)[i] = v;
  else
    static_cast<uint16_t*>(D.y)[i] = f32_to_bf16_rne(v);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// One lane's four scales of a quad: fp32 (16 bytes) or bf16 (8 bytes).
template <bool S16>
using ScaleQuad = typename std::conditional<S16, uint2, uint4>::type;

__device__ __forceinline__ float quad_elem(const uint4& v, int s) { return __uint_as_float(word(v, s)); }
__device__ __forceinline__ float quad_elem(const uint2& v, int s) {
  const uint32_t w = s < 2 ? v.x : v.y;
  return __uint_as_float((s & 1) ? (w & 0xFFFF0000u) : (w << 16));  // bf16 -> fp32 is exact
}

template <int AUX>
__device__ __forceinline__ void bload_into(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4& dst) {
  dst = bload<AUX>(r, off);
}
template <int AUX>
__device__ __forceinline__ void bload_into(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2& dst) {
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX);
  dst = make_uint2(v.x, v.y);
}

__device__ __forceinline__ bf16x8 unpack_step(uint32_t w, const UnpackConsts& uc) {
  uint32_t b[4];
  unpack_word(w, b, uc);
  return bitcast<bf16x8>(u32x4{b[0], b[1], b[2], b[3]});
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(a), bitcast<bf16x2>(b), c, false);
}

// Which linear of the batch, and which (row panel, x slab) of it, a block runs.
struct Work {
  int di, rb0, m0;
  int ks = 0, nks = 1;  // K slice of the block and slices per (row panel, x slab) (split launches)
};

__device__ __forceinline__ Work locate(const BatchArgs& a, int R, int MT, int S = 1) {
  const int b = blockIdx.x;
  int di = 0;
  if (a.count <= 4) {  // the projections of a layer that share an input: a short scan
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (i < a.count && b >= a.block0[i]) di = i;
  } else {
#pragma unroll
    for (int i = 1; i < kMaxBatch; ++i)
      if (i < a.count && b >= a.block0[i]) di = i;
  }
  const LinearDesc& d = a.desc[di];
  const int nb = (d.N + kTileRows - 1) / kTileRows;
  const int panels = (nb + R - 1) / R;
  const int all = b - a.block0[di];
  const int local = S == 1 ? all : (int)((uint32_t)all / (uint32_t)S);  // no division when unsplit
  const int slab = local / panels;
  return Work{di, (local - slab * panels) * R, slab * MT, all - local * S, S};
}

// The same for a launch of one linear.
__device__ __forceinline__ Work locate_one(int N, int R, int MT, int S = 1) {
  const int all = blockIdx.x;
  const int b = S == 1 ? all : (int)((uint32_t)all / (uint32_t)S);
  const int nb = (N + kTileRows - 1) / kTileRows;
  const int panels = (nb + R - 1) / R;
  const int slab = b / panels;
  return Work{0, (b - slab * panels) * R, slab * MT, all - b * S, S};
}

// Geometry of one linear and the weight-side buffers of one wavefront
// (S16: the scales are bf16, 8 bytes per row and quad instead of 16).
template <int R, bool S16>
struct Weights {
  static constexpr uint32_t kScaleBytes = S16 ? 8u : 16u;  // one row's quad
  int G, Q, GP, nb, rvalid, j0, j1;
  __amdgpu_buffer_rsrc_t rq, rd;
  uint32_t qo[R], so[R];  // byte offsets of this lane's 16 bytes at group 0 / quad 0, per row block

  __device__ __forceinline__ Weights(const LinearDesc& D, const Work& wk, int lane, int wave, int nw) {
    G = D.K / kGroup;
    Q = (G + 3) >> 2;
    GP = 4 * Q;
    nb = (D.N + kTileRows - 1) / kTileRows;
    rvalid = min(R, nb - wk.rb0);
    // the wavefront's range of scale quads: part `wave` of nw of the block's
    // K slice (Q * parts < 2^22: 32-bit arithmetic; nw is a compile-time
    // constant, so the unsplit case needs no division instruction sequence)
    if (wk.nks == 1) {
      j0 = (int)(((uint32_t)Q * (uint32_t)wave) / (uint32_t)nw);
      j1 = (int)(((uint32_t)Q * (uint32_t)(wave + 1)) / (uint32_t)nw);
    } else {
      const uint32_t part = (uint32_t)(wk.ks * nw + wave), parts = (uint32_t)(wk.nks * nw);
      j0 = (int)(((uint32_t)Q * part) / parts);
      j1 = (int)(((uint32_t)Q * (part + 1)) / parts);
    }
    rq = make_rsrc(D.q, (uint32_t)nb * GP * 1024u);
    rd = make_rsrc(D.d, (uint32_t)nb * GP * 4u * kScaleBytes);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // row blocks past the end re-read the last one; they are never stored
      const uint32_t rb = (uint32_t)min(wk.rb0 + r, nb - 1);
      qo[r] = (rb * GP * kTileLanes + lane) * 16u;
      so[r] = (rb * Q * kTileRows + (lane & 15)) * kScaleBytes;
    }
  }
  // base added to qo / so: the group's (quad's) offset, or past the end
  __device__ __forceinline__ uint32_t qbase(int j, int g) const { return j < j1 ? (uint32_t)g * 1024u : kOobW; }
  __device__ __forceinline__ uint32_t sbase(int j) const {
    return j < j1 ? (uint32_t)j * kTileRows * kScaleBytes : kOobW;
  }
};

// ---------------------------------------------------------------------------
// Split launches (MFMA kernel, one slab of at most 16 x rows): the K range of
// a row panel is divided among S consecutive blocks.  Slices 0 .. S-2 write
// their fp32 partial sums to the workspace; the last slice waits for them,
// adds them in slice order and then its own, and stores the output, so the
// result does not depend on which block finishes first.  Completion is the
// data itself: a slot holds kPartUnwritten until its partial is written (a
// NaN pattern partial sums never take: it is replaced on the way out), is
// read with coherent loads, and is reset to kPartUnwritten by the last slice
// once read, so each call leaves the workspace as it found it.  The last
// slice of a panel is its highest-numbered block, and blocks are dispatched
// in order, so every block it waits for has been dispatched before it and
// waits for nothing: each wait ends.  It is bounded all the same (a timeout
// sets the workspace's error word and the output becomes NaN).  A
// workspace that was never initialised (no magic word in its header) is not
// waited on at all: the last slice sets bit 1 of the error word and stores NaN.
// ---------------------------------------------------------------------------
constexpr uint32_t kPartUnwritten = 0xFFFFFFFFu;
constexpr uint32_t kSplitMagic = 0x57345350u;  // header word 1 of an initialised workspace
constexpr uint32_t kPartNanForUnwritten = 0xFFC00000u;
constexpr uint32_t kSplitSpinLimit = 1u << 17;  // polls (each at least one memory round trip)
constexpr int kMaxSplit = 8;

// Slot of row block r of the panel of block b: 64 lanes x 16 bytes.
__device__ __forceinline__ uint32_t* split_slot(uint8_t* ws, int R, int b, int r) {
  return reinterpret_cast<uint32_t*>(ws + kSplitHeaderBytes + ((size_t)b * R + r) * 1024u) +
         4 * (threadIdx.x & 63);
}

__device__ __forceinline__ void split_publish(uint32_t* slot, const f32x4& v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t b = __float_as_uint(v[e]);
    __hip_atomic_store(slot + e, b == kPartUnwritten ? kPartNanForUnwritten : b, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Waits for the partial in `slot`, returns it and marks the slot unwritten again.
__device__ __forceinline__ f32x4 split_take(uint32_t* slot, uint32_t* error) {
  uint32_t v[4];
  for (uint32_t t = 0;; ++t) {
    bool u = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = __hip_atomic_load(slot + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      u |= v[e] == kPartUnwritten;
    }
    if (!__any(u)) break;
    if (t >= kSplitSpinLimit) {
      if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;  // the unwritten pattern is a NaN: the output shows the failure
    }
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) __hip_atomic_store(slot + e, kPartUnwritten, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
}

// One output tile (16 rows x 16 x rows, this lane's four values) of a block
// whose sum covers its K slice only.  Unsplit: v is final.  Slices before the
// last publish v and return false; the last slice turns v into
// ((p_0 + p_1) + ... + p_{S-2}) + v and returns true.  `slots` per block,
// `slot` this tile's index among them.
__device__ __forceinline__ bool split_combine(uint8_t* ws, const Work& wk, int slots, int slot, f32x4& v) {
  if (wk.nks == 1) return true;
  if (wk.ks + 1 < wk.nks) {
    split_publish(split_slot(ws, slots, blockIdx.x, slot), v);
    return false;
  }
  uint32_t* error = reinterpret_cast<uint32_t*>(ws);
  if (__hip_atomic_load(error + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != kSplitMagic) {
    // never initialised: its slots cannot be trusted, so nothing is waited for
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(error, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v = f32x4{__uint_as_float(kNanBits), __uint_as_float(kNanBits), __uint_as_float(kNanBits),
              __uint_as_float(kNanBits)};
    return true;
  }
  const int b0 = blockIdx.x - (wk.nks - 1);
  f32x4 t = split_take(split_slot(ws, slots, b0, slot), error);
  for (int k = 1; k + 1 < wk.nks; ++k) {
    const f32x4 p = split_take(split_slot(ws, slots, b0 + k, slot), error);
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] += p[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = t[e] + v[e];
  return true;
}

// ---------------------------------------------------------------------------
// Chained launches (protocol below the kernels' bodies): values that later
// stages read start as kUnwritten and are written once, through to memory;
// a reader loads them coherently and waits, boundedly, while any is unwritten.
// ---------------------------------------------------------------------------
constexpr uint16_t kUnwritten = 0xFFFF;     // a NaN pattern the chain never writes
constexpr uint16_t kNanForUnwritten = 0xFFC0;
// Polls before a wait gives up (each poll is a round trip to memory of at
// least ~0.5 us, so this is tens of milliseconds: far longer than any stage,
// far shorter than a hang).
constexpr uint32_t kChainSpinLimit = 1u << 17;
constexpr int kChainPollSleep = 4;  // s_sleep units (64 clocks) between polls

// Chained launches with per-item timestamps (w4_chain_trace): the GPU's
// 100 MHz real-time counter when the block's first wavefront had staged its
// input (dot2 items; MFMA items read their input group by group and record
// no such time: a stamp inside their wait spilled registers of the loop).
__device__ __forceinline__ uint64_t& chain_ready_stamp() {
  __shared__ uint64_t t;
  return t;
}
__device__ __forceinline__ uint64_t& chain_start_stamp() {
  __shared__ uint64_t t;
  return t;
}

// No dependency to wait for: x is read as soon as the block starts.
struct NoGate {
  static constexpr bool kActive = false;
  static constexpr int parity = 0;
};

struct ChainGate {
  static constexpr bool kActive = true;
  static constexpr int kCoherent = 16;  // buffer-load cache policy: agent-scope coherent (sc1)
  bool wait_x;                          // x is written by earlier stages of this pass
  bool reuse;                           // LDS already holds this x, staged by the block's previous item
  bool same_stage;                      // the block's previous item was in this stage
  int parity;                           // the block's item count mod 2 (reduction buffer)
  uint32_t* error;
  bool trace = false;                   // per-item timestamps are taken (chain_ready_stamp)

  __device__ __forceinline__ static void store(uint16_t* p, uint16_t v) {
    __hip_atomic_store(p, v == kUnwritten ? kNanForUnwritten : v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ static bool unwritten(const uint32_t w) {
    return (~w & 0xFFFFu) == 0u || (~w & 0xFFFF0000u) == 0u;
  }
  // (the checks of a chunk are or-ed without branches)
  __device__ __forceinline__ static bool unwritten(const uint4& v) {
    return ((int)unwritten(v.x) | (int)unwritten(v.y) | (int)unwritten(v.z) | (int)unwritten(v.w)) != 0;
  }
  __device__ __forceinline__ static bool unwritten(const uint4 (&v)[4]) {
    int u = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) u |= (int)unwritten(v[i]);
    return u != 0;
  }
  // true (and the launch's error flag set) once waiting has gone on too long,
  // or when a wait anywhere has timed out (this launch or an earlier one)
  __device__ __forceinline__ bool give_up(uint32_t t) const {
    if (t < kChainSpinLimit && ((t & 31) != 31 || __hip_atomic_load(error, __ATOMIC_RELAXED,
                                                                    __HIP_MEMORY_SCOPE_AGENT) == 0u)) {
      __builtin_amdgcn_s_sleep(kChainPollSleep);
      return false;
    }
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  // Lane 0 of the calling wavefront polls the 16 bytes of x at byte offset
  // `off` until they are written; false once waiting has gone on too long.
  __device__ __forceinline__ bool poll(__amdgpu_buffer_rsrc_t rx, uint32_t off) const {
    const uint32_t o = (threadIdx.x & 63) == 0 ? off : kOobX;
    for (uint32_t t = 0;; ++t) {
      if (!__any(unwritten(bload<kCoherent>(rx, o)))) return true;
      if (give_up(t)) return false;
    }
  }
  // The calling wavefront polls the last 16-byte chunk of bytes [b0, b1) of
  // x (a block's four wavefronts poll 64 bytes in all: polls compete with
  // the producers' last reads, so they are kept small) until it is written.
  // An empty range, or one past the end of x, reads zeros.
  __device__ __forceinline__ void wait_sample(__amdgpu_buffer_rsrc_t rx, uint32_t b0, uint32_t b1) const {
    const int lane = threadIdx.x & 63;
    const uint32_t off = (lane == 0 && b1 > b0) ? b1 - 16u : kOobX;
    for (uint32_t t = 0;; ++t) {
      const uint4 v = bload<kCoherent>(rx, off);
      if (!__any(unwritten(v))) break;
      if (t >= kChainSpinLimit || ((t & 31) == 31 && __hip_atomic_load(error, __ATOMIC_RELAXED,
                                                                       __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
        if (lane == 0) __hip_atomic_fetch_or(error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(kChainPollSleep);
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA kernel.  One v_mfma_f32_16x16x32_bf16 per 32-input step: A = 16 rows
// of x, B = the tile's 16 rows of W^T.  Lane l holds A[l%16][8(l/16)..+7],
// B[8(l/16)..+7][l%16] and D[4(l/16)+j][l%16], j = 0..3.  Rows of A at or
// beyond M read zeros (their outputs are discarded).  The -1.5*sum(x) start
// value is itself one MFMA chain with B = -1.5.  One quad is in flight: the x
// loads of a quad alone take 64 VGPRs.
//
// Two routes for x (XR = rows of x staged through LDS: 0, 8 or 16):
//   * registers (XR = 0; one-wavefront blocks at M <= 8): each lane loads its
//     A operand directly, 16 rows x 64 bytes per instruction; rows at or past
//     M are out of range, so at M <= 8 half the lanes load nothing;
//   * a slot of LDS private to the wavefront (XR = 16 at M > 8, XR = 8 at
//     M <= 8 with rows 8..15 of the slot zero): the group's XR x 256-byte
//     tile is loaded four rows per instruction, 16 lanes reading one
//     row's 256 contiguous bytes (two whole cache lines per row), written to
//     the slot and read back in the A layout one group ahead, so the LDS
//     round trip overlaps the previous group's MFMA chains.  With every row
//     of the tile carrying data, the direct loads touch sixteen half lines
//     per instruction whose lookups (rows a large power-of-two stride apart)
//     stall the vector L1 on tag conflicts: that was the limit of the split-K
//     launches at M = 16 (counters: the L1's address unit stalled by the
//     cache two thirds of its busy time).  At M <= 8 the slot also wins in
//     blocks of two or more wavefronts (half the load instructions of the
//     direct route); a block of one wavefront has nothing to hide the LDS
//     round trip behind and keeps the direct loads.  The slot needs no
//     barrier: a wavefront's LDS accesses execute in program order, so the
//     next group's writes follow this group's reads.
//
// Gate (kActive: an item of a chained launch, x through the LDS slot): x is
// loaded coherently, and when x is written by earlier stages each group's
// loads are checked before they are staged.  If a value is still unwritten,
// lane 0 polls one chunk until it is written -- the first time in an item the
// last chunk of the wavefront's range of x (its producer, the stage's
// highest-numbered item over that range, tends to finish last; waiting for
// the chunk found unwritten instead trails the producers one round trip each),
// later the unwritten chunk found -- then the x of all four groups in flight
// is loaded again (each may predate the write) and the group is checked anew.
// Outputs are written through (bf16 only).
// ---------------------------------------------------------------------------
template <int R, int NW, bool S16, int XR, class Gate = NoGate>
__device__ __forceinline__ void mfma_body(const LinearDesc& D, const Work& wk, uint8_t* ws = nullptr,
                                          const Gate& gate = Gate()) {
  constexpr bool XL = XR > 0;          // x through the LDS slot
  constexpr int NT = XL ? XR / 4 : 4;  // x load instructions per group
  static_assert(XL || !Gate::kActive, "a chained item reads x through the LDS slot");
  constexpr int kXPolicy = Gate::kActive ? ChainGate::kCoherent : 0;
  // (the wavefront index as a uniform value costs the register route ~20 VGPRs)
  const int lane = threadIdx.x & 63;
  const int wave = XL ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int nl = lane & 15, kb = lane >> 4;
  const int M = D.M, K = D.K, N = D.N;
  const Weights<R, S16> w(D, wk, lane, wave, NW);

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(D.x, (uint32_t)M * K * 2u);
  // this lane's x loads, at byte offsets xo[t] + (group base) + xi[t]:
  //   XL: rows xr + 4t of the slab, 16-byte chunk xc of the group;
  //   registers: row nl of the slab, the 16 bytes of step t for quarter kb.
  const int xr = lane >> 4, xc = lane & 15;
  uint32_t xo[4], xi[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {  // (the route through LDS uses the first NT)
    const int row = wk.m0 + (XL ? xr + 4 * t : nl);
    xo[t] = row < M ? ((uint32_t)row * K + 8u * (XL ? xc : kb)) * 2u : kOobX;
    xi[t] = XL ? 0u : 64u * t;
  }
  const int j1 = w.j1, G = w.G;
  // Groups past K (the padding of a partial last quad) read zeros, not the
  // start of the next row of x: their codes and scales are zero, but an
  // infinity or NaN there would still make the product NaN.
  auto xbase = [&](int j, int g) -> uint32_t { return j < j1 && g < G ? (uint32_t)g * 256u : kOobX; };

  __shared__ uint4 xs[XL ? NW : 1][XL ? kTileRows : 1][17];  // XL: a slot per wavefront, rows padded
  uint4 bx[4][NT];
  if constexpr (XL && XR < kTileRows) {
    // rows XR..15 of the slot hold zeros for the whole launch (x rows never loaded)
    for (int e = lane; e < (kTileRows - XR) * 16; e += 64) xs[wave][XR + e / 16][e % 16] = make_uint4(0, 0, 0, 0);
  }
  uint4 bw[4][R];
  ScaleQuad<S16> sc[R], sn[R];  // scale quads: current and next
  uint32_t xbs[4];              // (Gate) group base of each slot's x loads

  auto issue_group = [&](int s, int j) {
    const int g = 4 * j + s;
    const uint32_t xb = xbase(j, g), qb = w.qbase(j, g);
    if constexpr (Gate::kActive) xbs[s] = xb;
#pragma unroll
    for (int t = 0; t < NT; ++t) bx[s][t] = bload<kXPolicy>(rx, xo[t] + xb + xi[t]);
#pragma unroll
    for (int r = 0; r < R; ++r) bw[s][r] = bload<kNonTemporal>(w.rq, w.qo[r] + qb);
  };
  auto issue_scales = [&](ScaleQuad<S16> (&dst)[R], int j) {
    const uint32_t sb = w.sbase(j);
#pragma unroll
    for (int r = 0; r < R; ++r) bload_into<kNonTemporal>(w.rd, w.so[r] + sb, dst[r]);
  };

  const UnpackConsts uc = unpack_consts();
  const uint32_t kneg2 = (uint32_t)kBf16NegOneHalf | ((uint32_t)kBf16NegOneHalf << 16);
  const bf16x8 kneg = bitcast<bf16x8>(u32x4{kneg2, kneg2, kneg2, kneg2});

  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Group s of the current quad: the MFMA chains (which read the group's x
  // and code registers at issue), then the scaled accumulation (which waits
  // for the chains' results).  XL: A operands of the group being multiplied
  // and of the next one (a[2][4]); registers: the loads are the operands.
  bf16x8 a[2][4];
  // (Gate) wait until slot s holds no unwritten value (see above)
  bool polled_end = false;
  auto await_x = [&](int s) {
    if constexpr (Gate::kActive) {
      for (uint32_t it = 0;; ++it) {
        uint32_t mine = kOobX;  // this lane's first unwritten chunk, if any
#pragma unroll
        for (int t = NT - 1; t >= 0; --t)
          if (ChainGate::unwritten(bx[s][t])) mine = xo[t] + xbs[s] + xi[t];
        const uint64_t lanes = __ballot(mine != kOobX);
        if (lanes == 0) return;
        uint32_t off = (uint32_t)__builtin_amdgcn_readlane((int)mine, __builtin_ctzll(lanes));
        if (!polled_end) {  // the last 16 bytes of the range in the last row of x
          polled_end = true;
          off = ((uint32_t)(wk.m0 + min(M - wk.m0, kTileRows) - 1) * K + min(K, 512 * j1) - 8) * 2u;
        }
        // timed out (also after too many rounds): the error flag is set, the outputs are NaN
        if (!gate.poll(rx, off) || it >= kChainSpinLimit) {
          if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(gate.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
          for (int t = 0; t < NT; ++t) bx[s2][t] = bload<kXPolicy>(rx, xo[t] + xbs[s2] + xi[t]);
      }
    }
  };
  auto stage_x = [&](int s, bf16x8 (&dst)[4]) {
    if constexpr (XL) {
      if constexpr (Gate::kActive) {
        if (gate.wait_x) await_x(s);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) xs[wave][xr + 4 * t][xc] = bx[s][t];
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = bitcast<bf16x8>(xs[wave][nl][4 * i + kb]);
    }
  };

  auto products = [&](int s, const bf16x8 (&ax)[4], f32x4 (&c)[R]) {
    f32x4 off = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) off = mfma16x16x32(ax[i], kneg, off);
#pragma unroll
    for (int r = 0; r < R; ++r) c[r] = off;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < R; ++r) c[r] = mfma16x16x32(ax[i], unpack_step(word(bw[s][r], i), uc), c[r]);
  };
  auto accumulate = [&](int s, const f32x4 (&c)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float dv = quad_elem(sc[r], s);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(dv, c[r][e], acc[r][e]);
    }
  };

  // The prologue issues in the loop's order (scales, then groups 0..3), so that
  // the wait for each group at the loop head is the same on entry and on the
  // back edge.  A wavefront with no quads (j0 == j1) reads zeros here.
  issue_scales(sc, w.j0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    issue_group(s, w.j0);
    __builtin_amdgcn_sched_barrier(0);
  }
  stage_x(0, a[0]);
  for (int j = w.j0; j < j1; ++j) {
    issue_scales(sn, j + 1);  // past the range: zeros, no memory access
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f32x4 c[R];
      if constexpr (XL) {
        // the next group's x: group s + 1 of this quad, or group 0 of the
        // next quad (refilled three groups ago; zeros past the range)
        stage_x((s + 1) & 3, a[(s + 1) & 1]);
        products(s, a[s & 1], c);
      } else {
        bf16x8 ax[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ax[i] = bitcast<bf16x8>(bx[s][i]);
        products(s, ax, c);
      }
      // refill as soon as the chains have read the registers, not after their
      // results are in (nor sunk to the loop end)
      issue_group(s, j + 1);
      __builtin_amdgcn_sched_barrier(0);
      accumulate(s, c);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r] = sn[r];
  }

  // Row block r's sum over the block's K slice: stored, or (split launches)
  // published for the panel's last slice, which adds the slices in order.
  auto store = [&](int r, f32x4 v) {
    if (!split_combine(ws, wk, R, r, v)) return;
    const int n = (wk.rb0 + r) * kTileRows + nl;
    if (n >= N) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = wk.m0 + 4 * kb + e;
      if (m < M) {
        if constexpr (Gate::kActive)
          Gate::store(static_cast<uint16_t*>(D.y) + (int64_t)m * N + n, f32_to_bf16_rne(16.0f * v[e]));
        else
          store_out(D, (int64_t)m * N + n, 16.0f * v[e]);
      }
    }
  };

  if constexpr (NW == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < w.rvalid) store(r, acc[r]);
  } else {
    // (Gate: two copies by item parity, as in the dot2 kernel's reduction)
    __shared__ f32x4 red[Gate::kActive ? 2 : 1][NW][R][64];
    const int rp = Gate::kActive ? gate.parity : 0;
#pragma unroll
    for (int r = 0; r < R; ++r) red[rp][wave][r][lane] = acc[r];
    __syncthreads();
    for (int r = wave; r < w.rvalid; r += NW) {
      f32x4 v = red[rp][0][r][lane];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) {
        const f32x4 o = red[rp][ww][r][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += o[e];
      }
      store(r, v);
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel, shared-x form.  A block of NWN wavefronts owns NWN * R row
// blocks and all of K; wavefront w takes row blocks w*R .. w*R+R-1 and every
// wavefront walks the same groups in the same order.  The 16-row x tile of a
// group is read from memory once per block (each wavefront a 16/NWN-row
// slice), written to a double-buffered LDS tile and read from there as the
// MFMA A operand, so x costs one load per group and block instead of one per
// wavefront.  One barrier per group keeps the block in step; it also makes
// the two-slot tile safe (a slot is rewritten two groups later, after every
// wavefront has passed the barrier that follows its reads).  Per output row
// the arithmetic and its order are those of the one-wavefront-per-row-panel
// kernel with all of K (NW = 1), so the two give identical bits.
// ---------------------------------------------------------------------------
template <int R, int NWN, bool S16>
__device__ __forceinline__ void mfma_shared_body(const LinearDesc& D, const Work& wkb, uint8_t* ws = nullptr) {
  static_assert(16 % NWN == 0, "x rows split evenly over the wavefronts");
  constexpr int kRowsPerWave = 16 / NWN;
  constexpr int XL = kRowsPerWave >= 4 ? kRowsPerWave / 4 : 1;  // x loads per lane and group
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 15, kb = lane >> 4;
  const int M = D.M, K = D.K, N = D.N;
  const Work wk{wkb.di, wkb.rb0 + wave * R, wkb.m0, wkb.ks, wkb.nks};
  const Weights<R, S16> w(D, wk, lane, 0, 1);  // all of the block's K slice

  // This wavefront's slice of the x tile: rows xr[t] of the slab, 16-byte
  // chunk xc of the group's 256 bytes per row.  With fewer than four rows per
  // wavefront the lanes past the slice load nothing.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(D.x, (uint32_t)M * K * 2u);
  const bool xlane = (lane >> 4) < kRowsPerWave;
  const int xc = lane & 15;
  int xr[XL];
  uint32_t xo[XL];
#pragma unroll
  for (int t = 0; t < XL; ++t) {
    xr[t] = wave * kRowsPerWave + (lane >> 4) % kRowsPerWave + 4 * t;
    xo[t] = (xlane && wk.m0 + xr[t] < M) ? ((uint32_t)(wk.m0 + xr[t]) * K + 8u * xc) * 2u : kOobX;
  }
  const int j1 = w.j1, G = w.G;
  // Groups past K (the padding of a partial last quad) read zeros, not the
  // start of the next row of x: their codes and scales are zero, but an
  // infinity or NaN there would still make the product NaN.
  auto xbase = [&](int j, int g) -> uint32_t { return j < j1 && g < G ? (uint32_t)g * 256u : kOobX; };

  __shared__ uint4 xs[2][kTileRows][17];  // rows padded to 272 bytes: conflict-free A reads

  uint4 bx[4][XL];
  uint4 bw[4][R];
  ScaleQuad<S16> sc[R], sn[R];  // scale quads: current and next

  auto issue_group = [&](int s, int j) {
    const int g = 4 * j + s;
    const uint32_t xb = xbase(j, g), qb = w.qbase(j, g);
#pragma unroll
    for (int t = 0; t < XL; ++t) bx[s][t] = bload<0>(rx, xo[t] + xb);
#pragma unroll
    for (int r = 0; r < R; ++r) bw[s][r] = bload<kNonTemporal>(w.rq, w.qo[r] + qb);
  };
  auto issue_scales = [&](ScaleQuad<S16> (&dst)[R], int j) {
    const uint32_t sb = w.sbase(j);
#pragma unroll
    for (int r = 0; r < R; ++r) bload_into<kNonTemporal>(w.rd, w.so[r] + sb, dst[r]);
  };

  const UnpackConsts uc = unpack_consts();
  const uint32_t kneg2 = (uint32_t)kBf16NegOneHalf | ((uint32_t)kBf16NegOneHalf << 16);
  const bf16x8 kneg = bitcast<bf16x8>(u32x4{kneg2, kneg2, kneg2, kneg2});

  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto products = [&](int s, int buf, f32x4 (&c)[R]) {
    bf16x8 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = bitcast<bf16x8>(xs[buf][nl][4 * i + kb]);
    f32x4 off = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) off = mfma16x16x32(a[i], kneg, off);
#pragma unroll
    for (int r = 0; r < R; ++r) c[r] = off;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < R; ++r) c[r] = mfma16x16x32(a[i], unpack_step(word(bw[s][r], i), uc), c[r]);
  };
  auto accumulate = [&](int s, const f32x4 (&c)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float dv = quad_elem(sc[r], s);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(dv, c[r][e], acc[r][e]);
    }
  };

  // Same ring as the split-K kernel, with the x tile staged through LDS.
  // Every wavefront of the block runs the same number of iterations, so the
  // barriers line up.
  issue_scales(sc, w.j0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    issue_group(s, w.j0);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int j = w.j0; j < j1; ++j) {
    issue_scales(sn, j + 1);  // past the range: zeros, no memory access
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int buf = s & 1;
      if (xlane) {
#pragma unroll
        for (int t = 0; t < XL; ++t) xs[buf][xr[t]][xc] = bx[s][t];
      }
      __syncthreads();
      f32x4 c[R];
      products(s, buf, c);
      issue_group(s, j + 1);
      __builtin_amdgcn_sched_barrier(0);
      accumulate(s, c);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r] = sn[r];
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= w.rvalid) continue;  // row blocks past the end (a partial panel)
    f32x4 v = acc[r];
    if (!split_combine(ws, wk, R * NWN, wave * R + r, v)) continue;
    const int n = (wk.rb0 + r) * kTileRows + nl;
    if (n >= N) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = wk.m0 + 4 * kb + e;
      if (m < M) store_out(D, (int64_t)m * N + n, 16.0f * v[e]);
    }
  }
}

template <int R, int NWN, bool S16>
__global__ __launch_bounds__(NWN * 64) void linear_mfma_shared_kernel(const BatchArgs args) {
  const Work wk = locate(args, R * NWN, 16, args.ksplit);
  mfma_shared_body<R, NWN, S16>(args.desc[wk.di], wk, static_cast<uint8_t*>(args.ws));
}

template <int R, int NWN, bool S16>
__global__ __launch_bounds__(NWN * 64) void linear_mfma_shared_one(const uint16_t* x, const uint8_t* q,
                                                                   const void* d, void* y, int M, int K, int N,
                                                                   int flags, uint8_t* ws, int S) {
  const LinearDesc D{x, q, d, y, M, K, N, flags};
  mfma_shared_body<R, NWN, S16>(D, locate_one(N, R * NWN, 16, S), ws);
}

// Batched launch: the block finds its linear in the kernel arguments.
template <int R, int NW, bool S16, int XR>
__global__ __launch_bounds__(NW * 64) void linear_mfma_kernel(const BatchArgs args) {
  const Work wk = locate(args, R, 16, args.ksplit);
  mfma_body<R, NW, S16, XR>(args.desc[wk.di], wk, static_cast<uint8_t*>(args.ws));
}

// Launch of one linear.  Its arguments are plain scalars that the hardware
// preloads into SGPRs at wave launch, so the kernel does not wait for a
// kernel-argument fetch before it can issue its first loads.
template <int R, int NW, bool S16, int XR>
__global__ __launch_bounds__(NW * 64) void linear_mfma_one(const uint16_t* x, const uint8_t* q, const void* d,
                                                           void* y, int M, int K, int N, int flags, uint8_t* ws,
                                                           int S) {
  const LinearDesc D{x, q, d, y, M, K, N, flags};
  mfma_body<R, NW, S16, XR>(D, locate_one(N, R, 16, S), ws);
}

// ---------------------------------------------------------------------------
// VALU kernel (v_dot2_f32_bf16).  Lane (row l%16, quarter l/16) multiplies its
// 32 weights of a group by the matching 32 inputs of each of the MT x rows of
// its slab; x is staged once per block in LDS (MT * K bf16) together with the
// start value of every (row, group, quarter).  One quad of weights is in
// flight per wavefront, refilled group by group as each is consumed: with
// few VGPRs many wavefronts stay resident, which hides more latency than a
// deeper ring per wavefront.  The four quarters of a row are summed with
// cross-lane shuffles at the end.
// ---------------------------------------------------------------------------
// kXScale: x is divided by channel scales while it is staged,
// x'[k] = bf16(fl32(x[k] * inv_s[k])) (channel scaling before RTN, the
// study's section 2 AWQ row; inv_s holds the fp32 reciprocals of the scales).
// Gate (kActive, chained launches): the block's weight prologue is issued
// first, then x is staged once it is completely written (see ChainGate).
template <int MT, int R, int NW, bool S16, bool kXScale = false, class Gate = NoGate>
__device__ __forceinline__ void gemv_body(const LinearDesc& D, const Work& wk, const float* inv_s = nullptr,
                                          const Gate& gate = Gate()) {
  // LDS: x of the slab, [MT][GP * 16] uint4 (zero past K), then the start
  // values -1.5 * sum(x) of every (row, group, quarter), [MT][GP][4] floats.
  extern __shared__ uint4 xlds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, kb = lane >> 4;
  const int M = D.M, K = D.K, N = D.N;
  const Weights<R, S16> w(D, wk, lane, wave, NW);
  const int GP = w.GP;

  uint4 bw[4][R];
  ScaleQuad<S16> sc[R], sn[R];  // scale quads: current and next
  auto issue_group = [&](int s, int j) {
    const uint32_t qb = w.qbase(j, 4 * j + s);
#pragma unroll
    for (int r = 0; r < R; ++r) bw[s][r] = bload<kNonTemporal>(w.rq, w.qo[r] + qb);
  };
  auto issue_scales = [&](ScaleQuad<S16> (&dst)[R], int j) {
    const uint32_t sb = w.sbase(j);
#pragma unroll
    for (int r = 0; r < R; ++r) bload_into<kNonTemporal>(w.rd, w.so[r] + sb, dst[r]);
  };

  // Stage the slab's x rows (rows beyond M repeat row M-1; their outputs are
  // dropped) together with the start value of every (row, group, quarter).
  // Element e = (row, group, quarter) covers 4 x 16 bytes; groups past K read
  // zeros.  Leading elements are loaded before the weight prologue: loads
  // retire in issue order, so x queued behind the weights would wait for
  // their HBM round trip.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(D.x, (uint32_t)M * K * 2u);
  const int total = MT * GP * 4;
  auto x_off = [&](int e) -> uint32_t {
    const int mm = e / (GP * 4);
    const int rem = e - mm * GP * 4;
    const int g = rem >> 2, q4 = rem & 3;
    if (e >= total || g >= w.G) return kOobX;
    return ((uint32_t)min(wk.m0 + mm, M - 1) * K + (uint32_t)g * kGroup + 8u * q4) * 2u;
  };
  auto load_x = [&](uint32_t o, uint4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = bload<0>(rx, o + 64u * i);
  };
  const uint32_t kneg2 = (uint32_t)kBf16NegOneHalf | ((uint32_t)kBf16NegOneHalf << 16);
  float* offs = reinterpret_cast<float*>(xlds + MT * GP * 16);
  auto store_x = [&](int e, const uint4 (&vin)[4]) {
    uint4 v[4] = {vin[0], vin[1], vin[2], vin[3]};
    if constexpr (kXScale) {
      const int rg = e >> 2;
      const int g = rg - (rg / GP) * GP;
      if (g < w.G) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4* r4 = reinterpret_cast<const float4*>(inv_s + g * kGroup + 32 * i + 8 * (e & 3));
          const float4 a = r4[0], b = r4[1];
          const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          uint32_t wds[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const float lo = __uint_as_float(wds[h] << 16) * f[2 * h];
            const float hi = __uint_as_float(wds[h] & 0xFFFF0000u) * f[2 * h + 1];
            wds[h] = (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
          }
          v[i] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
        }
      }
    }
    float c = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c = dot2(v[i].x, kneg2, c);
      c = dot2(v[i].y, kneg2, c);
      c = dot2(v[i].z, kneg2, c);
      c = dot2(v[i].w, kneg2, c);
      xlds[(e >> 2) * 16 + i * 4 + (e & 3)] = v[i];
    }
    offs[e] = c;
  };

  {
    // The first kPre elements of every thread (all of x for M = 1 and K up to
    // 32 768 with 4+ wavefronts) go out before the weight prologue.
    constexpr int kPre = 2;
    uint4 v[kPre][4];
    (void)v;
    if constexpr (!Gate::kActive) {
#pragma unroll
      for (int p = 0; p < kPre; ++p) load_x(x_off(threadIdx.x + p * NW * 64), v[p]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Weight prologue in the loop's order (scales, then groups 0..3); a
    // wavefront with no quads (j0 == j1) reads zeros here.
    issue_scales(sc, w.j0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      issue_group(s, w.j0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (Gate::kActive) {
      // The weights do not depend on earlier stages; x may still be being
      // written by them.  Each wavefront stages only its own range of x (the
      // groups of its quads) and waits only for that range: at the block's
      // first item of a stage it polls a sample of the range until it is
      // written; then it stages the range (coherent loads), checking every
      // value, and polls and starts over while any is still unwritten.  No
      // block barrier follows: a wavefront reads back only what it staged.
      if (!gate.reuse) {  // else the block's previous item staged this x (and found it written)
        const int e0 = 16 * w.j0, e1 = 16 * w.j1;  // elements (group, quarter) of this wavefront's quads
        const uint32_t xb1 = min(1024u * w.j1, (uint32_t)K * 2u);  // its bytes of x: [1024 j0, xb1)
        if (gate.wait_x && !gate.same_stage) gate.wait_sample(rx, 1024u * w.j0, xb1);
        for (uint32_t t = 0;; ++t) {
          bool unwritten = false;
          for (int e = e0 + lane; e < e1; e += 64) {
            uint4 tt[4];
            if (gate.wait_x) {
#pragma unroll
              for (int i = 0; i < 4; ++i) tt[i] = bload<Gate::kCoherent>(rx, x_off(e) + 64u * i);
              unwritten |= Gate::unwritten(tt);
            } else {
              load_x(x_off(e), tt);
            }
            store_x(e, tt);
          }
          if (!__any(unwritten) || gate.give_up(t)) break;
          // poll a sample of the range before loading all of it again
          gate.wait_sample(rx, 1024u * w.j0, xb1);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wavefront's LDS writes land before its reads
        if (gate.trace && threadIdx.x == 0) chain_ready_stamp() = __builtin_amdgcn_s_memrealtime();
      }
    } else {
      // Consume x here, before the branches, so the loads are not sunk into
      // them (behind the weights).
#pragma unroll
      for (int p = 0; p < kPre; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          asm volatile("" : "+v"(v[p][i].x), "+v"(v[p][i].y), "+v"(v[p][i].z), "+v"(v[p][i].w));
#pragma unroll
      for (int p = 0; p < kPre; ++p)
        if ((int)threadIdx.x + p * NW * 64 < total) store_x(threadIdx.x + p * NW * 64, v[p]);
      for (int e = threadIdx.x + kPre * NW * 64; e < total; e += NW * 64) {
        uint4 t[4];
        load_x(x_off(e), t);
        store_x(e, t);
      }
    }
  }
  if constexpr (!Gate::kActive) __syncthreads();

  const UnpackConsts uc = unpack_consts();

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.f;

  // Group g (slot s of the current quad): its x values and start values from
  // LDS, the codes widened to bf16 pairs (this frees the slot's registers for
  // the refill), then the dot products and the scaled accumulation.
  struct Operands {
    uint32_t xv[MT][16];
    float c0[MT];
    uint32_t bb[R][16];
  };
  auto widen = [&](int s, int g, Operands& o) {
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 t = xlds[(mm * GP + g) * 16 + i * 4 + kb];
        o.xv[mm][4 * i + 0] = t.x; o.xv[mm][4 * i + 1] = t.y;
        o.xv[mm][4 * i + 2] = t.z; o.xv[mm][4 * i + 3] = t.w;
      }
      o.c0[mm] = offs[(mm * GP + g) * 4 + kb];
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) unpack_word(word(bw[s][r], i), &o.bb[r][4 * i], uc);
  };
  auto dots = [&](int s, const Operands& o) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float dv = quad_elem(sc[r], s);
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        float c = o.c0[mm];
#pragma unroll
        for (int e = 0; e < 16; ++e) c = dot2(o.bb[r][e], o.xv[mm][e], c);
        acc[r][mm] = fmaf(dv, c, acc[r][mm]);
      }
    }
  };

  for (int j = w.j0; j < w.j1; ++j) {
    issue_scales(sn, j + 1);  // past the range: zeros, no memory access
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Operands o;
      widen(s, 4 * j + s, o);
      // refill as soon as the codes are widened (not sunk to the loop end)
      issue_group(s, j + 1);
      __builtin_amdgcn_sched_barrier(0);
      dots(s, o);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) sc[r] = sn[r];
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

  // A chained block runs item after item with no barrier between them, so its
  // reduction array alternates between two copies by item parity: a wavefront
  // can write item i+1's copy while the reducing lanes still read item i's,
  // and it reaches item i+2 (the same copy) only after item i+1's barrier,
  // which those lanes pass only once they are done reading.
  __shared__ float red[Gate::kActive ? 2 : 1][NW][R][MT][16];
  const int rp = Gate::kActive ? gate.parity : 0;
  if (kb == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) red[rp][wave][r][mm][nl] = acc[r][mm];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < R * MT * 16; e += NW * 64) {
    const int row = e & 15;
    const int mm = (e >> 4) % MT;
    const int r = (e >> 4) / MT;
    if (r < w.rvalid) {
      float v = red[rp][0][r][mm][row];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) v += red[rp][ww][r][mm][row];
      const int n = (wk.rb0 + r) * kTileRows + row;
      const int m = wk.m0 + mm;
      if (n < N && m < M) {
        if constexpr (Gate::kActive)
          Gate::store(static_cast<uint16_t*>(D.y) + (int64_t)m * N + n, f32_to_bf16_rne(16.0f * v));
        else
          store_out(D, (int64_t)m * N + n, 16.0f * v);
      }
    }
  }
}

template <int MT, int R, int NW, bool S16>
__global__ __launch_bounds__(NW * 64) void linear_gemv_kernel(const BatchArgs args) {
  const Work wk = locate(args, R, MT);
  gemv_body<MT, R, NW, S16>(args.desc[wk.di], wk);
}

template <int MT, int R, int NW, bool S16>
__global__ __launch_bounds__(NW * 64) void linear_gemv_one(const uint16_t* x, const uint8_t* q, const void* d,
                                                           void* y, int M, int K, int N, int flags) {
  const LinearDesc D{x, q, d, y, M, K, N, flags};
  gemv_body<MT, R, NW, S16>(D, locate_one(N, R, MT));
}

// One linear whose x is divided by channel scales while it is staged.
template <int MT, int R, int NW>
__global__ __launch_bounds__(NW * 64) void linear_gemv_xscaled(const uint16_t* x, const uint8_t* q, const void* d,
                                                               void* y, int M, int K, int N,
                                                               const float* inv_s) {
  const LinearDesc D{x, q, d, y, M, K, N, 0};
  gemv_body<MT, R, NW, false, true>(D, locate_one(N, R, MT), inv_s);
}

// ---------------------------------------------------------------------------
// Chained launch of dependent M = 1 linears (layout and protocol in
// w4_launch.h).  Each item runs the dot2 body above with a gate: the item's
// weight prologue is issued first (weights never depend on earlier stages),
// then, when its x is produced by earlier stages, each wavefront waits until
// every value of its own range of x is written, and stages that range.  Per item the arithmetic is exactly
// the batched dot2 kernel's with the same (R, NW), so results are identical
// bits (NaN outputs aside: the unwritten marker is never written).
//
// Completion is the data itself: a fill launch marks every output that a
// later linear reads with kUnwritten before the pass; outputs are written
// through to memory (agent-scope stores), and x that may still be being
// written is read with coherent loads, so no L2 of the eight can serve a
// stale copy.  A chain writes each byte at most once and never writes a
// cache line that the pass reads earlier (the C ABI refuses such chains).
// ---------------------------------------------------------------------------
// Per-item timestamps (w4_chain_trace): the header's words 2-3 hold the
// buffer (null: none).  Thread 0 writes, per item i, stamps[3i] = start,
// [3i + 1] = when the block's first wavefront had staged its input (dot2
// items that staged one; 0 otherwise), [3i + 2] = end (after the outputs'
// stores were issued).
__device__ __forceinline__ uint64_t* chain_stamps(const uint32_t* hdr) {
  return *reinterpret_cast<uint64_t* const*>(hdr + 2);
}
// (the start is kept in LDS, not in a register live across the item's body)
__device__ __forceinline__ void chain_item_start() {
  if (threadIdx.x == 0) {
    chain_ready_stamp() = 0;
    chain_start_stamp() = __builtin_amdgcn_s_memrealtime();
  }
}
__device__ __forceinline__ void chain_item_end(uint64_t* stamps, int i) {
  if (threadIdx.x == 0) {
    stamps[3 * (size_t)i] = chain_start_stamp();
    stamps[3 * (size_t)i + 1] = chain_ready_stamp();
    stamps[3 * (size_t)i + 2] = __builtin_amdgcn_s_memrealtime();
  }
}

// lin: the table (linears + 1 entries, the last a sentinel); hdr: the
// workspace header (error word, then the timestamp buffer).  kTrace: the
// variant that takes per-item timestamps (the other has none of that code).
template <int R, int NW, bool S16, bool kTrace = false>
__global__ __launch_bounds__(NW * 64) void linear_chain_kernel(const ChainLinear* __restrict__ lin, uint32_t* hdr,
                                                               int items) {
  const int P = gridDim.x;
  int i = blockIdx.x;
  int li = 0;
  int li_end = lin[1].item0;  // first item past linear li
  while (i < items && i >= li_end) li_end = lin[++li + 1].item0;
  const uint16_t* staged = nullptr;  // x held in LDS (and its K)
  int staged_k = 0;
  int prev_stage = -1;
  int parity = 0;
  uint64_t* const stamps = kTrace ? chain_stamps(hdr) : nullptr;
  while (i < items) {
    const LinearDesc& D = lin[li].desc;
    const ChainGate gate{lin[li].wait_x != 0, D.x == staged && D.K == staged_k, lin[li].stage == prev_stage,
                         parity, hdr, kTrace && stamps != nullptr};
    prev_stage = lin[li].stage;
    parity ^= 1;
    if constexpr (kTrace) {
      if (stamps) chain_item_start();
    }
    gemv_body<1, R, NW, S16, false, ChainGate>(D, Work{0, (i - lin[li].item0) * R, 0}, nullptr, gate);
    if constexpr (kTrace) {
      if (stamps) chain_item_end(stamps, i);
    }
    staged = D.x;
    staged_k = D.K;
    i += P;
    while (i < items && i >= li_end) li_end = lin[++li + 1].item0;
  }
}

// The same walk for a chain of linears with 2..16 rows of x (verification
// widths), each item run by the MFMA body (split-K form, x through the LDS
// slot) with the gate: the item's weight and x loads are issued at once, and
// a group's x is checked for unwritten values just before it is staged.  Per
// item the arithmetic is exactly the MFMA kernel's with the same (R, NW),
// unsplit, so results are identical bits (NaN outputs aside, as above).
// At M <= 8 with up to two row blocks the item fits in 168 VGPRs without
// spilling: three wavefronts per SIMD (the batched kernel's occupancy there)
// keep more bytes in flight per CU than two.
template <int R, int NW, bool S16, int XR, bool kTrace = false>
__global__ __launch_bounds__(NW * 64, (XR == 8 && R <= 2) ? 3 : 1) void linear_chain_mfma_kernel(
    const ChainLinear* __restrict__ lin, uint32_t* hdr, int items) {
  const int P = gridDim.x;
  int i = blockIdx.x;
  int li = 0;
  int li_end = lin[1].item0;
  while (i < items && i >= li_end) li_end = lin[++li + 1].item0;
  int parity = 0;
  uint64_t* const stamps = kTrace ? chain_stamps(hdr) : nullptr;
  while (i < items) {
    const ChainGate gate{lin[li].wait_x != 0, false, false, parity, hdr, kTrace && stamps != nullptr};
    parity ^= 1;
    if constexpr (kTrace) {
      if (stamps) chain_item_start();
    }
    mfma_body<R, NW, S16, XR, ChainGate>(lin[li].desc, Work{0, (i - lin[li].item0) * R, 0}, nullptr, gate);
    if constexpr (kTrace) {
      if (stamps) chain_item_end(stamps, i);
    }
    i += P;
    while (i < items && i >= li_end) li_end = lin[++li + 1].item0;
  }
}

// Marks the outputs that later linears read as unwritten (block (i, m): row
// m of linear i's output).
__global__ __launch_bounds__(256) void chain_fill_kernel(const ChainLinear* __restrict__ lin) {
  const ChainLinear& l = lin[blockIdx.x];
  if (!l.fill || (int)blockIdx.y >= l.desc.M) return;
  uint16_t* y = static_cast<uint16_t*>(l.desc.y) + (int64_t)blockIdx.y * l.desc.N;
  for (int n = threadIdx.x; n < l.desc.N; n += 256) y[n] = kUnwritten;
}

// ---------------------------------------------------------------------------
// launch configuration
// ---------------------------------------------------------------------------
// R row blocks per wavefront and NW wavefronts per block.  Split-K
// configurations (shared = false) divide K among the block's wavefronts,
// which share one row panel; shared-x configurations (MFMA only) give each
// wavefront its own R row blocks and all of K and share the x tile.
struct Cfg {
  int R, NW;
  bool shared;
};

// Every configuration compiled for each kernel and scale format: the first
// kNumSplitCfgs (split-K) for both kernels, the shared-x forms for the MFMA
// kernel only.  (Split-K MFMA forms of eight wavefronts with two or four row
// blocks each measured slower on every projection group at M = 8 and 16.)
// W4_MFMA_CFG / W4_GEMV_CFG ("R,NW", or "R,NWs" for shared x) may pick one of
// them for measurement; a value naming no configuration compiled for that
// kernel makes the launch fail (hipErrorInvalidValue).
constexpr Cfg kCfgs[] = {{1, 4, false}, {1, 8, false}, {2, 4, false}, {4, 4, false}, {1, 2, false},
                         {2, 2, false}, {4, 1, false}, {4, 2, false}, {2, 8, true},  {2, 4, true}};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
constexpr int kNumSplitCfgs = 8;
static_assert(kNumCfgs == 10, "the launch switches below list 10 configurations");
static_assert(!kCfgs[0].shared && !kCfgs[1].shared && !kCfgs[2].shared && !kCfgs[3].shared && !kCfgs[4].shared &&
                  !kCfgs[5].shared && !kCfgs[6].shared && !kCfgs[7].shared && kCfgs[8].shared && kCfgs[9].shared,
              "configurations of both kernels first: the dot2 launch compiles only those");

// -1: not set; -2: set to something that is not compiled for this kernel
// (mfma: the MFMA kernel, which has every configuration).
int cfg_from_env(const char* name, bool mfma) {
  const char* s = getenv(name);
  if (!s) return -1;
  int R = 0, NW = 0;
  char tail[4] = {0, 0, 0, 0};
  const int got = sscanf(s, "%d,%d%3s", &R, &NW, tail);
  if (got < 2) return -2;
  const bool shared = got == 3 && tail[0] == 's' && tail[1] == 0;
  if (got == 3 && !shared) return -2;
  for (int i = 0; i < kNumCfgs; ++i)
    if (kCfgs[i].R == R && kCfgs[i].NW == NW && kCfgs[i].shared == shared)
      return i >= kNumSplitCfgs && !mfma ? -2 : i;
  return -2;
}

int find_cfg(int R, int NW, bool shared = false) {
  for (int i = 0; i < kNumCfgs; ++i)
    if (kCfgs[i].R == R && kCfgs[i].NW == NW && kCfgs[i].shared == shared) return i;
  return 0;
}

struct LaunchShape {
  int64_t rows;  // 16-row blocks over the whole batch
  int kmin, kmax, mmax;
};
LaunchShape launch_shape(const BatchArgs& a) {
  LaunchShape l{0, 1 << 30, 0, 0};
  for (int i = 0; i < a.count; ++i) {
    l.rows += (a.desc[i].N + kTileRows - 1) / kTileRows;
    l.kmin = a.desc[i].K < l.kmin ? a.desc[i].K : l.kmin;
    l.kmax = a.desc[i].K > l.kmax ? a.desc[i].K : l.kmax;
    l.mmax = a.desc[i].M > l.mmax ? a.desc[i].M : l.mmax;
  }
  return l;
}

// Built-in choices, from graph-replayed sweeps of every (R, NW) on MI355X over
// the 4B/27B/70B-class projection groups and the 2560x9216 / 9216x2560 pair
// at M = 1, 8, 13, 16.  Two effects pull against each other:
//   * enough wavefronts to keep loads in flight on all 256 CUs when the
//     launch is small (more wavefronts per block, fewer rows per wavefront);
//   * when it is large, long-lived wavefronts and small blocks: a block of one
//     wavefront leaves the moment it is done and its slot takes the next,
//     while a block of four holds its slots until the last of the four ends
//     and a new block needs four free slots on one CU.  Short K (few scale
//     quads per wavefront) makes the second effect stronger.
int choose_cfg_mfma(const BatchArgs& a, bool can_split) {
  // More row blocks per wavefront also reuse each x operand across more
  // weights (x is read through L1 once per row panel).
  const LaunchShape l = launch_shape(a);
  if (l.rows < 256) return find_cfg(1, 4);
  if (l.rows < 600) {
    // Few row panels of long rows, more than 8 rows of x (every row of the
    // x tile carries data): four row blocks per wavefront halve the x loads
    // per weight byte, and splitting K across blocks (a workspace is given)
    // wins back the wavefronts that the larger panels lose.
    if (can_split && l.mmax > 8 && l.kmin >= 16384) return find_cfg(4, 4);
    return find_cfg(2, 4);
  }
  if (l.rows < 2048) {
    if (l.kmin >= 4096) return find_cfg(4, 4);
    // short K: few quads per wavefront; with more than 8 rows of x and every
    // K short, sharing the x tile beats splitting K
    return l.mmax > 8 && l.kmax < 4096 ? find_cfg(2, 4, true) : find_cfg(2, 2);
  }
  // Large launch: each wavefront streams all of K for its row blocks, unless
  // the longest K would leave a few wavefronts streaming far longer than the
  // rest of the launch.  With more than 8 rows of x (every lane of the x
  // operand carries data), or with very many row blocks, blocks of eight such
  // wavefronts share each x tile through LDS; otherwise one wavefront per
  // block.
  const int qmax = (l.kmax / kGroup + 3) / 4;
  if (qmax > 20) return find_cfg(4, 4);
  if (l.mmax > 8 || l.rows >= 8192) return find_cfg(2, 8, true);
  // at M <= 8, four wavefronts splitting rows of 8192 inputs or more (four
  // quads each or more) with x through LDS beat one-wavefront blocks
  return l.kmin >= 8192 ? find_cfg(2, 4) : find_cfg(4, 1);
}

int choose_cfg_gemv(const BatchArgs& a) {
  const LaunchShape l = launch_shape(a);
  if (l.rows < 256) return find_cfg(1, 8);
  // long K: more wavefronts per row block, once there are enough row blocks --
  // but only when every linear of the batch is long.  One configuration
  // serves the whole batch, and an eight-way split leaves the wavefronts of a
  // short-K linear (a whole decoder layer in one launch) a quad or two each.
  if (l.kmax >= 16384 && l.rows >= 400) {
    if (l.kmin >= 16384) return find_cfg(1, 8);
    return l.kmin >= 8192 ? find_cfg(2, 4) : find_cfg(1, 4);
  }
  if (l.kmin <= 4096 && l.rows >= 8192) return find_cfg(2, 2);
  // short K and 512 row blocks or more (one 9216 x 2560 matrix: 576): two
  // wavefronts per row block, each with one quad or two, measured 8% faster
  // than four in a single call
  if (l.kmax <= 4096 && l.rows >= 512) return find_cfg(1, 2);
  // few row blocks but long rows: two row blocks per wavefront halve the x
  // staging per weight byte and still leave enough wavefronts
  if (l.rows < 400 && l.kmin >= 6144) return find_cfg(2, 4);
  return find_cfg(1, 4);
}

// K slices per row panel of a split launch (1: no split), or -1 for a
// W4_MFMA_SPLIT value that is not a slice count (1..kMaxSplit; any
// configuration may be split that way for measurement).  The count never
// needs more slots than the workspace holds.
int choose_split(const BatchArgs& a, const Cfg& c, size_t ws_bytes) {
  const LaunchShape l = launch_shape(a);
  const int pr = c.shared ? c.R * c.NW : c.R;  // row blocks per panel (and slots per block)
  const int kparts = c.shared ? 1 : c.NW;      // parts of the block's K slice
  int64_t panels = 0;
  for (int i = 0; i < a.count; ++i) {
    const int64_t nb = (a.desc[i].N + kTileRows - 1) / kTileRows;
    panels += (nb + pr - 1) / pr * ((a.desc[i].M + 15) / 16);
  }
  if (panels == 0) return 1;
  int S = 0;
  if (const char* e = getenv("W4_MFMA_SPLIT")) {
    S = atoi(e);
    if (S < 1 || S > kMaxSplit) return -1;
  } else if (!c.shared && c.R >= 4 && l.rows < 600 && l.mmax > 8) {
    // Splitting pays only where it wins back the wavefronts that four-row-
    // block panels lose on a launch of few row panels with every row of the
    // x tile carrying data (measured: splitting panels of one or two row
    // blocks, shared-x blocks, or launches at M <= 8 gained nothing on any
    // projection shape); it aims at about one wavefront per SIMD and at two
    // scale quads or more each.
    const int64_t waves = panels * c.NW;
    const int qmin = (l.kmin / kGroup + 3) / 4;
    S = (int)((1024 + waves - 1) / waves);
    S = S < qmin / (2 * kparts) ? S : qmin / (2 * kparts);
    S = S < kMaxSplit ? S : kMaxSplit;
    S = S > 1 ? S : 1;
  } else {
    S = 1;
  }
  while (S > 1 && kSplitHeaderBytes + (size_t)(panels * S * pr) * 1024u > ws_bytes) --S;
  return S;
}

// Block ranges of the batch's linears.  Blocks are dispatched roughly in index
// order, so the linears are laid out longest K first (stable for equal K):
// the blocks that run longest start first and the grid ends on short ones,
// which shortens the tail of a launch that mixes long and short rows.  Each
// linear's blocks compute the same thing wherever they sit, so the order
// changes no result.
int64_t fill_blocks(BatchArgs& a, int R, int slab_rows, int S = 1) {
  for (int i = 1; i < a.count; ++i) {
    const LinearDesc t = a.desc[i];
    int j = i;
    for (; j > 0 && a.desc[j - 1].K < t.K; --j) a.desc[j] = a.desc[j - 1];
    a.desc[j] = t;
  }
  int64_t total = 0;
  for (int i = 0; i < a.count; ++i) {
    a.block0[i] = (int)total;
    const int nb = (a.desc[i].N + kTileRows - 1) / kTileRows;
    const int panels = (nb + R - 1) / R;
    const int slabs = (a.desc[i].M + slab_rows - 1) / slab_rows;
    total += (int64_t)panels * slabs * S;
  }
  return total;
}

template <int MT, bool S16, int I>
void launch_gemv_at(unsigned blocks, size_t lds, hipStream_t st, const BatchArgs& a) {
  constexpr Cfg c = kCfgs[I];
  if (a.count == 1) {
    const LinearDesc& l = a.desc[0];
    linear_gemv_one<MT, c.R, c.NW, S16><<<blocks, c.NW * 64, lds, st>>>(l.x, l.q, l.d, l.y, l.M, l.K, l.N,
                                                                         l.flags);
  } else {
    linear_gemv_kernel<MT, c.R, c.NW, S16><<<blocks, c.NW * 64, lds, st>>>(a);
  }
}

template <int MT, bool S16>
void launch_gemv_cfg(int ci, unsigned blocks, size_t lds, hipStream_t st, const BatchArgs& a) {
  switch (ci) {
#define W4_CASE(i) \
  case i:          \
    launch_gemv_at<MT, S16, i>(blocks, lds, st, a); \
    break;
    W4_CASE(0) W4_CASE(1) W4_CASE(2) W4_CASE(3) W4_CASE(4) W4_CASE(5) W4_CASE(6) W4_CASE(7)
#undef W4_CASE
  }
}

template <bool S16, int I>
void launch_mfma_at(unsigned blocks, hipStream_t st, const BatchArgs& a) {
  constexpr Cfg c = kCfgs[I];
  const LinearDesc& l = a.desc[0];
  if constexpr (c.shared) {
    if (a.count == 1)
      linear_mfma_shared_one<c.R, c.NW, S16><<<blocks, c.NW * 64, 0, st>>>(l.x, l.q, l.d, l.y, l.M, l.K, l.N,
                                                                            l.flags, static_cast<uint8_t*>(a.ws),
                                                                            a.ksplit);
    else
      linear_mfma_shared_kernel<c.R, c.NW, S16><<<blocks, c.NW * 64, 0, st>>>(a);
  } else {
    // x route: all 16 rows through LDS when M > 8; at M <= 8 the 8 rows that
    // carry data through LDS in blocks of two or more wavefronts, registers in
    // one-wavefront blocks (whose LDS round trip nothing would hide)
    constexpr int kXrSmall = c.NW >= 2 ? 8 : 0;
    int mmax = 0;
    for (int i = 0; i < a.count; ++i) mmax = a.desc[i].M > mmax ? a.desc[i].M : mmax;
    uint8_t* wsp = static_cast<uint8_t*>(a.ws);
    if (a.count == 1) {
      if (mmax > 8)
        linear_mfma_one<c.R, c.NW, S16, 16><<<blocks, c.NW * 64, 0, st>>>(l.x, l.q, l.d, l.y, l.M, l.K, l.N,
                                                                          l.flags, wsp, a.ksplit);
      else
        linear_mfma_one<c.R, c.NW, S16, kXrSmall><<<blocks, c.NW * 64, 0, st>>>(l.x, l.q, l.d, l.y, l.M, l.K,
                                                                                l.N, l.flags, wsp, a.ksplit);
    } else {
      if (mmax > 8)
        linear_mfma_kernel<c.R, c.NW, S16, 16><<<blocks, c.NW * 64, 0, st>>>(a);
      else
        linear_mfma_kernel<c.R, c.NW, S16, kXrSmall><<<blocks, c.NW * 64, 0, st>>>(a);
    }
  }
}

template <bool S16>
void launch_mfma_cfg(int ci, unsigned blocks, hipStream_t st, const BatchArgs& a) {
  switch (ci) {
#define W4_CASE(i) \
  case i:          \
    launch_mfma_at<S16, i>(blocks, st, a); \
    break;
    W4_CASE(0) W4_CASE(1) W4_CASE(2) W4_CASE(3) W4_CASE(4) W4_CASE(5) W4_CASE(6) W4_CASE(7) W4_CASE(8) W4_CASE(9)
#undef W4_CASE
  }
}

}  // namespace

hipError_t launch_linear_mfma(BatchArgs& a, bool s16, hipStream_t stream, void* split_ws, size_t split_ws_bytes) {
  const int env = cfg_from_env("W4_MFMA_CFG", true);
  if (env == -2) return hipErrorInvalidValue;
  const int ci = env >= 0 ? env : choose_cfg_mfma(a, split_ws != nullptr);
  const Cfg c = kCfgs[ci];
  a.ksplit = 1;
  a.ws = nullptr;
  if (split_ws) {
    const int S = choose_split(a, c, split_ws_bytes);
    if (S < 0) return hipErrorInvalidValue;
    if (S > 1) {
      a.ksplit = S;
      a.ws = split_ws;
    }
  }
  const int64_t blocks = fill_blocks(a, c.shared ? c.R * c.NW : c.R, 16, a.ksplit);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (s16) launch_mfma_cfg<true>(ci, (unsigned)blocks, stream, a);
  else launch_mfma_cfg<false>(ci, (unsigned)blocks, stream, a);
  return hipGetLastError();
}

int gemv_rows_per_slab(int64_t M, int64_t K) {
  for (int mt = 4; mt > 1; mt >>= 1)
    if (M >= mt && gemv_lds_bytes(mt, K) <= kGemvLdsBytes) return mt;
  return 1;
}

hipError_t launch_linear_gemv_xscaled(const LinearDesc& l, const float* inv_s, int MT, hipStream_t stream) {
  BatchArgs a;
  a.count = 1;
  a.desc[0] = l;
  const int ci = choose_cfg_gemv(a) == find_cfg(1, 8) ? find_cfg(1, 8) : find_cfg(1, 4);
  const Cfg c = kCfgs[ci];
  const int64_t blocks = fill_blocks(a, c.R, MT);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const size_t lds = (size_t)gemv_lds_bytes(MT, l.K);
  const unsigned nb = (unsigned)blocks;
#define W4_XS(mt, nw) \
  linear_gemv_xscaled<mt, 1, nw><<<nb, nw * 64, lds, stream>>>(l.x, l.q, l.d, l.y, l.M, l.K, l.N, inv_s)
  if (c.NW == 8) {
    if (MT == 4) W4_XS(4, 8); else if (MT == 2) W4_XS(2, 8); else W4_XS(1, 8);
  } else {
    if (MT == 4) W4_XS(4, 4); else if (MT == 2) W4_XS(2, 4); else W4_XS(1, 4);
  }
#undef W4_XS
  return hipGetLastError();
}

hipError_t launch_linear_gemv(BatchArgs& a, int MT, bool s16, hipStream_t stream) {
  const int env = cfg_from_env("W4_GEMV_CFG", false);
  if (env == -2) return hipErrorInvalidValue;
  const int ci = env >= 0 ? env : choose_cfg_gemv(a);
  const Cfg c = kCfgs[ci];
  const int64_t blocks = fill_blocks(a, c.R, MT);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  int kmax = 0;
  for (int i = 0; i < a.count; ++i) kmax = a.desc[i].K > kmax ? a.desc[i].K : kmax;
  const size_t lds = (size_t)gemv_lds_bytes(MT, kmax);
  const unsigned nb = (unsigned)blocks;
  if (s16) {
    if (MT == 4) launch_gemv_cfg<4, true>(ci, nb, lds, stream, a);
    else if (MT == 2) launch_gemv_cfg<2, true>(ci, nb, lds, stream, a);
    else launch_gemv_cfg<1, true>(ci, nb, lds, stream, a);
  } else {
    if (MT == 4) launch_gemv_cfg<4, false>(ci, nb, lds, stream, a);
    else if (MT == 2) launch_gemv_cfg<2, false>(ci, nb, lds, stream, a);
    else launch_gemv_cfg<1, false>(ci, nb, lds, stream, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// chained launch
// ---------------------------------------------------------------------------
namespace {
// dot2 items (M = 1), then MFMA items (M = 2..16: split-K forms, x through the
// LDS slot); a configuration index counts through both lists.
constexpr int kChainCfgs[][2] = {{1, 4}, {1, 8}, {2, 4}, {2, 2}, {1, 2}, {4, 4}};
constexpr int kNumChainCfgs = sizeof(kChainCfgs) / sizeof(kChainCfgs[0]);
// (each also an MFMA configuration of the batched launch, whose bits it gives)
constexpr int kChainMfmaCfgs[][2] = {{2, 4}, {4, 4}, {1, 4}, {2, 2}};
constexpr int kNumChainMfmaCfgs = sizeof(kChainMfmaCfgs) / sizeof(kChainMfmaCfgs[0]);
static_assert(kNumChainCfgs == 6 && kNumChainMfmaCfgs == 4, "the switches below list these configurations");

template <int I, bool S16>
const void* chain_kernel_ptr() {
  return reinterpret_cast<const void*>(&linear_chain_kernel<kChainCfgs[I][0], kChainCfgs[I][1], S16>);
}
template <int I, bool S16, int XR>
const void* chain_mfma_kernel_ptr() {
  return reinterpret_cast<const void*>(
      &linear_chain_mfma_kernel<kChainMfmaCfgs[I][0], kChainMfmaCfgs[I][1], S16, XR>);
}
template <bool S16>
const void* chain_kernel(int ci) {
  switch (ci) {
    case 0: return chain_kernel_ptr<0, S16>();
    case 1: return chain_kernel_ptr<1, S16>();
    case 2: return chain_kernel_ptr<2, S16>();
    case 3: return chain_kernel_ptr<3, S16>();
    case 4: return chain_kernel_ptr<4, S16>();
    default: return chain_kernel_ptr<5, S16>();
  }
}
template <bool S16, int XR>
const void* chain_mfma_kernel(int mi) {
  switch (mi) {
    case 0: return chain_mfma_kernel_ptr<0, S16, XR>();
    case 1: return chain_mfma_kernel_ptr<1, S16, XR>();
    case 2: return chain_mfma_kernel_ptr<2, S16, XR>();
    default: return chain_mfma_kernel_ptr<3, S16, XR>();
  }
}
template <bool S16, bool kTrace>
void launch_chain_cfg(int ci, int blocks, size_t lds, hipStream_t stream, const ChainLinear* lin, uint32_t* hdr,
                      int items) {
  switch (ci) {
#define W4_CHAIN(i)                                                                      \
  case i:                                                                                \
    linear_chain_kernel<kChainCfgs[i][0], kChainCfgs[i][1], S16, kTrace>                 \
        <<<blocks, kChainCfgs[i][1] * 64, lds, stream>>>(lin, hdr, items);               \
    break;
    W4_CHAIN(0) W4_CHAIN(1) W4_CHAIN(2) W4_CHAIN(3) W4_CHAIN(4) W4_CHAIN(5)
#undef W4_CHAIN
  }
}
// x rows staged per group: the 8 of a slab at M <= 8, all 16 above
template <bool S16, int XR, bool kTrace>
void launch_chain_mfma_cfg(int mi, int blocks, hipStream_t stream, const ChainLinear* lin, uint32_t* hdr,
                           int items) {
  switch (mi) {
#define W4_CHAIN(i)                                                                          \
  case i:                                                                                    \
    linear_chain_mfma_kernel<kChainMfmaCfgs[i][0], kChainMfmaCfgs[i][1], S16, XR, kTrace>    \
        <<<blocks, kChainMfmaCfgs[i][1] * 64, 0, stream>>>(lin, hdr, items);                 \
    break;
    W4_CHAIN(0) W4_CHAIN(1) W4_CHAIN(2) W4_CHAIN(3)
#undef W4_CHAIN
  }
}
}  // namespace

int chain_num_cfgs() { return kNumChainCfgs + kNumChainMfmaCfgs; }

bool chain_cfg_mfma(int ci) { return ci >= kNumChainCfgs; }

void chain_cfg(int ci, int* R, int* NW) {
  const int(&c)[2] = ci < kNumChainCfgs ? kChainCfgs[ci] : kChainMfmaCfgs[ci - kNumChainCfgs];
  *R = c[0];
  *NW = c[1];
}

int chain_choose_cfg(int kmax, double stage_bytes, int M) {
  const bool mfma = M > 1;
  if (const char* e = getenv("W4_CHAIN_CFG")) {
    int R = 0, NW = 0;
    if (sscanf(e, "%d,%d", &R, &NW) != 2) return -1;
    for (int i = 0; i < chain_num_cfgs(); ++i) {
      int r = 0, nw = 0;
      chain_cfg(i, &r, &nw);
      if (chain_cfg_mfma(i) == mfma && r == R && nw == NW) return i;
    }
    return -1;
  }
  (void)kmax;
  // MFMA items (70B- and 27B-class stacks at M = 8 and 16, up to two blocks
  // per CU): two row blocks and four wavefronts were fastest of (2,4), (4,4),
  // (1,4), (2,2), (4,2) and of eight-wavefront forms (2,8) and (1,8), except
  // (2,8) by 3% on the 70B-class stack at M = 8.
  if (mfma) return kNumChainCfgs;
  // Measured on MI355X (two blocks per CU; the grid size is chosen by the C
  // ABI): with stages of tens of MB or more (27B- and 70B-class stacks, 45
  // and 110 MB of codes per stage on average) two row blocks per item and
  // four wavefronts per block; with small stages (4B-class, 12 MB) one row
  // block and eight wavefronts, so that every stage has more, shorter items.
  return stage_bytes < 24e6 ? 1 : 2;
}

hipError_t chain_blocks_per_cu(int ci, bool s16, size_t lds, int M, int* blocks) {
  if (ci < 0 || ci >= chain_num_cfgs()) return hipErrorInvalidValue;
  int R = 0, NW = 0;
  chain_cfg(ci, &R, &NW);
  const void* k = nullptr;
  if (!chain_cfg_mfma(ci))
    k = s16 ? chain_kernel<true>(ci) : chain_kernel<false>(ci);
  else if (M > 8)
    k = s16 ? chain_mfma_kernel<true, 16>(ci - kNumChainCfgs) : chain_mfma_kernel<false, 16>(ci - kNumChainCfgs);
  else
    k = s16 ? chain_mfma_kernel<true, 8>(ci - kNumChainCfgs) : chain_mfma_kernel<false, 8>(ci - kNumChainCfgs);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k, NW * 64, chain_cfg_mfma(ci) ? 0 : lds);
}

namespace {
__global__ __launch_bounds__(256) void split_init_kernel(uint32_t* ws, size_t words) {
  const size_t hdr = kSplitHeaderBytes / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256)
    ws[i] = i >= hdr ? kPartUnwritten : i == 1 ? kSplitMagic : 0u;
}
}  // namespace

hipError_t launch_split_init(void* ws, size_t bytes, hipStream_t stream) {
  const size_t words = bytes / 4;
  const unsigned blocks = (unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024);
  if (blocks == 0) return hipSuccess;
  split_init_kernel<<<blocks, 256, 0, stream>>>(static_cast<uint32_t*>(ws), words);
  return hipGetLastError();
}

namespace {
template <bool kTrace>
void launch_chain_kernels(int ci, bool s16, int blocks, size_t lds, int M, hipStream_t stream,
                          const ChainLinear* lin, uint32_t* hdr, int items) {
  if (!chain_cfg_mfma(ci)) {
    if (s16) launch_chain_cfg<true, kTrace>(ci, blocks, lds, stream, lin, hdr, items);
    else launch_chain_cfg<false, kTrace>(ci, blocks, lds, stream, lin, hdr, items);
  } else {
    const int mi = ci - kNumChainCfgs;
    if (M > 8) {
      if (s16) launch_chain_mfma_cfg<true, 16, kTrace>(mi, blocks, stream, lin, hdr, items);
      else launch_chain_mfma_cfg<false, 16, kTrace>(mi, blocks, stream, lin, hdr, items);
    } else {
      if (s16) launch_chain_mfma_cfg<true, 8, kTrace>(mi, blocks, stream, lin, hdr, items);
      else launch_chain_mfma_cfg<false, 8, kTrace>(mi, blocks, stream, lin, hdr, items);
    }
  }
}
}  // namespace

hipError_t launch_linear_chain(void* ws, int linears, int items, int ci, bool s16, int blocks, size_t lds, int M,
                               bool trace, hipStream_t stream) {
  if (ci < 0 || ci >= chain_num_cfgs() || M < 1 || M > 16 || chain_cfg_mfma(ci) != (M > 1))
    return hipErrorInvalidValue;
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint32_t* hdr = reinterpret_cast<uint32_t*>(w);
  const ChainLinear* lin = reinterpret_cast<const ChainLinear*>(w + sizeof(ChainHeader));
  chain_fill_kernel<<<dim3(linears, M), 256, 0, stream>>>(lin);
  if (trace) launch_chain_kernels<true>(ci, s16, blocks, lds, M, stream, lin, hdr, items);
  else launch_chain_kernels<false>(ci, s16, blocks, lds, M, stream, lin, hdr, items);
  return hipGetLastError();
}

}  // namespace w4
