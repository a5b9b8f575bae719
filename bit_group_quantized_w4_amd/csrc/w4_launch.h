// Internal launchers between the C ABI (abi.cpp) and the kernels (*.hip).
// Shapes and pointers are validated by the caller; each launcher enqueues on
// `stream` and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace w4 {

constexpr int kMaxBatch = 64;                // linears per launch (kernel arguments < 4 KiB)
constexpr int kGemvLdsBytes = 64 * 1024;     // x slab staged in LDS by the dot2 kernel

// LDS the dot2 kernel needs for an MT-row slab of x with K inputs: the x rows
// padded to whole scale quads (512 inputs) plus one float per (row, group,
// quarter of a group).
inline int64_t gemv_lds_bytes(int64_t MT, int64_t K) {
  const int64_t gp = (K / 128 + 3) / 4 * 4;
  return MT * gp * (128 * 2 + 4 * 4);
}

// LinearDesc::flags
constexpr int kOutF32 = 1;  // y is fp32 (the accumulated value before rounding to bf16)

// One linear of a batch, as the kernels see it (validated by the ABI layer).
struct LinearDesc {
  const uint16_t* x;  // bf16 [M][K]
  const uint8_t* q;   // native codes
  const void* d;      // native scale quads: fp32, or bf16 in the 16-bit variant
  void* y;            // [M][N]: bf16, or fp32 with kOutF32
  int M, K, N, flags;
};

// Kernel argument block: block0[i] is the first workgroup of linear i.
// Split launches (MFMA kernel): ksplit blocks share each row panel's K range
// and exchange partial sums through the workspace `ws` (see linear.hip).
struct BatchArgs {
  int count;
  int ksplit = 1;
  void* ws = nullptr;
  int block0[kMaxBatch];
  LinearDesc desc[kMaxBatch];
};

// Split workspace: a header (error word, a magic word written by the
// initialisation, then padding) and one 1 KiB slot per (block, row block of
// its panel).  Slots hold kPartUnwritten (all one bits) between calls.
constexpr size_t kSplitHeaderBytes = 256;

// ---------------------------------------------------------------------------
// Chained launch: a dependent sequence of linears with the same M (1 for a
// decode step, up to 16 for draft verification) in stages (a layer's q|k|v,
// then o, then gate|up, then down, layer after layer).  A linear whose x is
// written by earlier stages uses no value of it that is not yet written.
// One persistent grid of co-resident blocks walks the items (R-row-block
// panels) of every stage in order; block b takes items b, b+P, b+2P, ...
// Before the pass a fill launch marks every output that a later linear reads
// with an unwritten-value pattern.  A block's item issues its weight loads
// first; then (M = 1) each wavefront waits until no value of its own range of
// x is unwritten and stages that range, or (M > 1) each group's x is checked
// as it is staged and waited for while any value is unwritten.  Waits only
// ever look at outputs of earlier items, which co-resident blocks hold, so
// every wait ends; it is also bounded (a timeout sets `error` and lets the
// launch drain).
// ---------------------------------------------------------------------------
// Workspace layout (device): ChainHeader | ChainLinear[linears + 1] (the last
// is a sentinel with item0 = items).
struct ChainHeader {
  uint32_t error;      // sticky: nonzero once a wait has timed out
  uint32_t pad;
  uint64_t* stamps;    // per-item timestamps of later passes (w4_chain_trace), or null
  uint32_t pad2[4];
};
struct ChainLinear {
  LinearDesc desc;
  int item0;   // first item of this linear
  int stage;
  int wait_x;  // x is written by earlier stages of the pass
  int fill;    // y is read by later stages: marked unwritten before the pass
};
static_assert(sizeof(ChainHeader) == 32 && sizeof(ChainLinear) == 64, "workspace layout");

inline size_t chain_workspace_bytes(int64_t linears) {
  return sizeof(ChainHeader) + (size_t)(linears + 1) * sizeof(ChainLinear);
}

// Chain configurations: (R row blocks per item, NW wavefronts per block) of
// the dot2 items (chains of M = 1 linears), then of the MFMA items (chains of
// M = 2..16 linears); chain_cfg_mfma tells which list an index is in.
int chain_num_cfgs();
bool chain_cfg_mfma(int ci);
void chain_cfg(int ci, int* R, int* NW);
// Configuration for a chain of M-row linears whose longest K is kmax and
// whose stages hold stage_bytes of codes on average (W4_CHAIN_CFG "R,NW"
// overrides; -1 if it names no configuration compiled for that M).
int chain_choose_cfg(int kmax, double stage_bytes, int M);
// Co-resident blocks per CU of configuration ci (s16: bf16 scales) for
// M-row linears, with `lds` bytes of dynamic LDS (dot2 items only).
hipError_t chain_blocks_per_cu(int ci, bool s16, size_t lds, int M, int* blocks);
// The fill launch, then the chain launch (trace: the variant that writes
// per-item timestamps to the buffer named in the workspace header).
hipError_t launch_linear_chain(void* ws, int linears, int items, int ci, bool s16, int blocks, size_t lds, int M,
                               bool trace, hipStream_t stream);

// s16: scales are bf16 bit patterns (uint16_t) instead of fp32.
hipError_t launch_quantize_rtn(const float* W, int64_t N, int64_t K, uint8_t* q_packed,
                               void* d_packed, bool s16, hipStream_t stream);
// RTN of W * diag(cs) (columns scaled in fp32 first).
hipError_t launch_quantize_rtn_scaled(const float* W, const float* cs, int64_t N, int64_t K, uint8_t* q_packed,
                                      void* d_packed, bool s16, hipStream_t stream);
hipError_t launch_pack(const int8_t* q_canon, const void* d_canon, int64_t N, int64_t K,
                       uint8_t* q_packed, void* d_packed, bool s16, hipStream_t stream);
hipError_t launch_unpack(const uint8_t* q_packed, const void* d_packed, int64_t N, int64_t K,
                         int8_t* q_canon, void* d_canon, bool s16, hipStream_t stream);

// MFMA streaming kernel over a batch (16-row slabs of x).
hipError_t launch_linear_mfma(BatchArgs& a, bool s16, hipStream_t stream, void* split_ws = nullptr,
                              size_t split_ws_bytes = 0);
// Marks a split workspace ready: error word zero, every slot unwritten.
hipError_t launch_split_init(void* ws, size_t bytes, hipStream_t stream);
// dot2 streaming kernel over a batch (MT-row slabs of x staged in LDS; every
// K must satisfy gemv_lds_bytes(MT, K) <= kGemvLdsBytes).
hipError_t launch_linear_gemv(BatchArgs& a, int MT, bool s16, hipStream_t stream);
// Largest slab (4, 2 or 1 rows) the dot2 kernel can stage for M rows of K.
int gemv_rows_per_slab(int64_t M, int64_t K);
// dot2 kernel for one linear whose x is divided by channel scales while it is
// staged: x'[k] = bf16(fl32(x[k] * inv_s[k])).
hipError_t launch_linear_gemv_xscaled(const LinearDesc& l, const float* inv_s, int MT, hipStream_t stream);

// Channel-scaling search steps (awq.hip).
hipError_t launch_channel_absmean(const uint16_t* x, int64_t T, int64_t K, float* m, hipStream_t stream);
hipError_t launch_awq_scales(const float* m, int64_t K, double alpha, float* s, float* inv, hipStream_t stream);
hipError_t launch_scale_activations(const uint16_t* x, int64_t M, int64_t K, const float* inv, uint16_t* xo,
                                    hipStream_t stream);
hipError_t launch_sq_error(const uint16_t* y, const float* yref, int64_t n, double* out, hipStream_t stream);

// GPTQ steps (gptq.hip): the column loop over the 128-column block at b0, and
// the damping of the Hessian.
hipError_t launch_gptq_block(const float* W, int64_t N, int64_t K, int64_t b0, const float* U, int8_t* q_canon,
                             void* d_canon, bool s16, float* errT, hipStream_t stream);
hipError_t launch_gptq_damp(double* H, int64_t K, double damp, hipStream_t stream);

// Dense linear algebra of the offline quantizers (dense.hip).
// H = (2/T) x^T x, fp64 [K][K] (both triangles), from bf16 x [T][K].
hipError_t launch_gptq_hessian(const uint16_t* x, int64_t T, int64_t K, double* H, hipStream_t stream);
// Doubles of work launch_gptq_inverse_factor needs for a K x K Hessian.
size_t gptq_factor_work_doubles(int64_t K);
// U (fp32 [K][K], upper triangular) with H^-1 = U^T U for the damped H (fp64
// [K][K], lower triangle read, not modified); K a multiple of 64.
hipError_t launch_gptq_inverse_factor(const double* H, int64_t K, double* work, float* U, hipStream_t stream);
// W[:, b0+128:] -= err^T U[b0:b0+128, b0+128:], fp32 (err [128][N]).
hipError_t launch_gptq_update(float* W, int64_t N, int64_t K, int64_t b0, const float* U, const float* err,
                              hipStream_t stream);
// y[t][n] = sum_k x[t][k] W[n][k], fp32 (x bf16 [T][K], W fp32 [N][K], y [T][N]).
hipError_t launch_dense_linear_f32(const uint16_t* x, int64_t T, int64_t K, const float* W, int64_t N, float* y,
                                   hipStream_t stream);

}  // namespace w4
