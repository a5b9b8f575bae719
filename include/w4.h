/*
 * w4.h -- group-wise symmetric INT4 weight quantization and the W4A16 linear
 * layer for AMD Instinct MI355X (gfx950).  C ABI, C99-compatible.
 *
 * The method (Qwen3.5-4B quantization study, parksieon.github.io/
 * qwen35-4b-quantization-study):
 *   - section 1, group-quantization equation and its symbol table:
 *       q = clip(round(w/d) + z, qmin, qmax),   w_hat = d (q - z),
 *     with one restore scale d per group of 128 consecutive inputs of a row
 *     (72 groups per row of the 2560x9216 FFN example), 16 codes per 4-bit
 *     slot, and zero point z = 0 for the symmetric scheme;
 *   - section 2 settings table: RTN, group 128, min/max symmetric range, no
 *     clipping search, 4-bit weights with BF16 inputs;
 *   - section 1, y = W x with W stored N x K (N outputs, K inputs).
 * The linear layer is what memory-bound decode runs once per generated token
 * (M = 1), and what verifying K drafted tokens runs once with M = K + 1 rows
 * (27B quantization-and-drafter ladder, thakicloud.com, stage 1 "why 4-bit is
 * faster" and stage 2 "drafter").
 *
 * Conventions of this library:
 *   d        = fl32(max|w| / 7) per group (IEEE divide, no flush to zero);
 *   code     q = clamp(round_half_away_from_zero(fl32(w / d)), -8, 7);
 *   degenerate groups: a NaN or infinity in the group gives d = NaN (bits
 *   0x7FC00000) and codes 0; d == 0 gives codes 0;
 *   y[m][n]  = bf16_rne( sum_g d[n][g] * sum_{k in g} q[n][k] x[m][k] ),
 *            accumulated in fp32 per 128-group (the *_f32 entry points store
 *            the fp32 value itself, before rounding).
 *   Accuracy: the fp32 value v lies within 2e-3 * sum_k |w_hat[n][k] x[m][k]|
 *            + 1e-6 of the exact y; a bf16 output is the nearest-even bf16 of
 *            such a v, so it may differ from the exact y by that bound plus
 *            half a bf16 step (bf16 keeps 8 significant bits).
 *   Activations: a NaN or infinity anywhere in row m of x makes every
 *            y[m][n] NaN (the row is poisoned, as a non-finite weight group
 *            poisons its outputs).  The bound above is guaranteed while no
 *            fp32 intermediate can overflow: |x| <= 2^64 and |w| <= 2^38 are
 *            enough.  Past that range an output may be +-infinity or NaN
 *            where the exact y is finite, but it is never a wrong finite
 *            value.
 *
 * All data pointers are DEVICE pointers (hipMalloc'd or equivalent).  The
 * caller owns every buffer; the library allocates nothing and keeps no state
 * besides a per-thread copy of the last HIP error.  Every call is enqueued
 * asynchronously on `stream` (0 = the null stream) and performs no host
 * synchronisation (except the set-up and status calls of the chained pass,
 * which say so).  Argument errors are detected on the host before anything
 * is enqueued and leave outputs untouched.  A launch failure returns
 * W4_ERR_HIP (w4_last_hip_error() gives the hipError_t); faults during
 * execution surface at the caller's next synchronisation, as in HIP.
 * Results are bitwise reproducible run to run (no floating-point atomics).
 *
 * NATIVE LAYOUT (what w4_quantize_rtn writes and w4_linear reads)
 *   Let Np = N rounded up to a multiple of 16, G = K / 128, Q = ceil(G / 4)
 *   and GP = 4Q (the group count padded to whole scale quads).  The matrix is
 *   cut into tiles of 16 rows x 128 inputs (one group); tile (r, g) covers
 *   rows 16r .. 16r+15 and group g, for g < GP.
 *   Codes: tile (r, g) is 1024 contiguous bytes at byte offset (r*GP + g)*1024.
 *     Its 16-byte lane L (0..63) holds row n = 16r + (L % 16), and its four
 *     little-endian 32-bit words w_i (i = 0..3) hold inputs
 *     k = 128g + 32i + 8(L / 16) + j, j = 0..7, as offset-binary nibbles
 *     u_j = q_j + 8:  w_i = rotl32(v, 3) where
 *     v = sum_{p=0..3} u_{2p} << 4p  +  sum_{p=0..3} u_{2p+1} << (16 + 4p).
 *   Scales: the scales of row n for the four groups 4j .. 4j+3 form one
 *     16-byte quad at float index ((r*Q + j)*16 + n%16)*4 (r = n / 16),
 *     group 4j+t at offset t.
 *   16-bit scales (the *_s16 entry points): the same quads hold bf16 bit
 *     patterns, 8 bytes per row and quad, at uint16 index
 *     ((r*Q + j)*16 + n%16)*4 + t.
 *   Rows N .. Np-1 and groups G .. GP-1 are padding: codes 0 (u = 8), scales 0.
 *   Total sizes: w4_packed_bytes(N, K) = Np*GP*64 bytes of codes and
 *   w4_scale_count(N, K) = Np*GP floats of scales.
 *
 * CANONICAL LAYOUT (for exchange and bit-exact comparison)
 *   codes int8 [N][K] row-major, each in [-8, 7];
 *   scales float32 (or bf16 bit patterns for *_s16) [N][K/128] row-major.
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4_OK = 0,
  W4_ERR_NULL = 1,   /* a required pointer is NULL                           */
  W4_ERR_SHAPE = 2,  /* N, M < 0; K not a positive multiple of 128; too large */
  W4_ERR_ALIGN = 3,  /* a pointer is not aligned as documented                */
  W4_ERR_HIP = 4,    /* a HIP runtime call or launch failed                   */
  W4_ERR_ARG = 5,    /* another invalid argument (unknown path, aliasing ...) */
  W4_ERR_SCRATCH = 6 /* w4_chain_prepare_noalloc: the chain does not fit the static scratch */
} w4_status;

/* Which linear kernel w4_linear_ex / w4_linear_batched run. */
typedef enum {
  W4_PATH_AUTO = 0,  /* the library's choice by M and K (what w4_linear does)   */
  W4_PATH_GEMV = 1,  /* VALU dot-product kernel, x staged in LDS in slabs of up
                        to 4 rows; needs K <= 30720 (else W4_ERR_SHAPE)          */
  W4_PATH_MFMA = 2   /* bf16 MFMA kernel, any M (slabs of 16 rows)             */
} w4_path;

/* Most linears one w4_linear_batched call accepts. */
#define W4_MAX_BATCH 64

/* One linear y = W_hat x of a batch (same meaning and requirements as the
 * arguments of w4_linear). */
typedef struct w4_linear_desc {
  const uint16_t* x;       /* bf16 [M][K]                  */
  int64_t M;
  int64_t K;
  const uint8_t* q_packed; /* native codes of the N x K W  */
  const float* d_packed;   /* native scales                */
  int64_t N;
  uint16_t* y;             /* bf16 [M][N]                  */
} w4_linear_desc;

/* The same with 16-bit scales (bf16 bit patterns), for w4_linear_batched_s16. */
typedef struct w4_linear_desc_s16 {
  const uint16_t* x;        /* bf16 [M][K]                  */
  int64_t M;
  int64_t K;
  const uint8_t* q_packed;  /* native codes of the N x K W  */
  const uint16_t* d_packed; /* native bf16 scales           */
  int64_t N;
  uint16_t* y;              /* bf16 [M][N]                  */
} w4_linear_desc_s16;

/* Human-readable name of a status code (static storage, never NULL). */
const char* w4_status_str(int status);

/* The hipError_t of the last W4_ERR_HIP returned on this thread (0 if none). */
int w4_last_hip_error(void);

/* Group size along K: 128 (study, section 1). */
int w4_group_size(void);

/* Bytes of native codes for an N x K matrix: roundup(N, 16) * roundup(K, 512) / 2.
 * Returns 0 when N < 0, K <= 0 or K % 128 != 0. */
size_t w4_packed_bytes(int64_t N, int64_t K);

/* Number of native fp32 scales: roundup(N, 16) * 4 * ceil(K / 512)
 * (0 on bad shape). */
size_t w4_scale_count(int64_t N, int64_t K);

/*
 * w4_quantize_rtn -- RTN INT4 group quantization (study, section 1 equation;
 * section 2 settings: group 128, symmetric min/max, no calibration input).
 *   W        [in]  fp32 row-major [N][K] weights; 16-byte aligned.
 *   N        [in]  rows (outputs), N >= 0 (N == 0: nothing is done).
 *   K        [in]  columns (inputs), positive multiple of 128.
 *   q_packed [out] w4_packed_bytes(N, K) bytes, native layout; 16-byte aligned.
 *   d_packed [out] w4_scale_count(N, K) floats, native layout; 16-byte aligned.
 * Codes and scales are bit-exact with respect to the conventions above.
 */
w4_status w4_quantize_rtn(const float* W, int64_t N, int64_t K, uint8_t* q_packed,
                          float* d_packed, hipStream_t stream);

/*
 * w4_linear -- y = W_hat x (study, section 1: y = W x; section 2: 4-bit
 * weights, BF16 inputs), the memory-bound decode / draft-verify layer.
 *   x        [in]  bf16 bit patterns, row-major [M][K]; 16-byte aligned.
 *   M        [in]  activation rows, 0 <= M <= 262140 (M == 0: nothing is
 *                  done).  Tuned for M <= 16; larger M runs in row slabs.
 *   K        [in]  inputs, positive multiple of 128.
 *   q_packed [in]  native codes of the N x K matrix; 16-byte aligned.
 *   d_packed [in]  native scales; 16-byte aligned.
 *   N        [in]  outputs, N >= 0 (N == 0: nothing is done).
 *   y        [out] bf16 bit patterns, row-major [M][N]; 2-byte aligned; must
 *                  not overlap any input (W4_ERR_ARG).  Rounded to nearest
 *                  even from fp32.
 * Size limits (W4_ERR_SHAPE beyond them): w4_packed_bytes(N, K) < 2 GiB and
 * 2*M*K <= 1 GiB, so that every operand is addressed with 32-bit offsets.
 */
w4_status w4_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                    const float* d_packed, int64_t N, uint16_t* y, hipStream_t stream);

/* w4_linear with an explicit kernel choice (same contract; W4_ERR_ARG for an
 * unknown path). */
w4_status w4_linear_ex(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                       const float* d_packed, int64_t N, uint16_t* y, int path,
                       hipStream_t stream);

/*
 * w4_linear_batched -- up to W4_MAX_BATCH independent linears in ONE launch
 * (the projections of a decode layer that read the same input -- q/k/v,
 * gate/up -- or any set of linears with no data dependence between them).
 * Each element obeys the w4_linear contract; inputs may be shared between
 * elements, but no output may overlap any input or any other output
 * (W4_ERR_ARG).  `linears` is host memory and is read before the call
 * returns.  count == 0 does nothing.  All elements run the same kernel
 * (`path`, W4_ERR_ARG if unknown; W4_PATH_AUTO decides from the largest M
 * and K).  Results are bitwise identical to one w4_linear_ex call per element
 * with the same kernel configuration.
 */
w4_status w4_linear_batched(const w4_linear_desc* linears, int count, int path,
                            hipStream_t stream);

/*
 * fp32 outputs: the same linears storing each output as the fp32 value the
 * kernel accumulated, before it is rounded to bf16 (the bf16 entry points
 * store exactly bf16_rne of it, bitwise).  For checking the accumulation
 * against the bound above without the output rounding, and for callers that
 * sum partial outputs themselves (a K-split layer).  Same contracts as
 * w4_linear_ex / w4_linear_s16 / w4_linear_batched except that y is fp32
 * [M][N], 4-byte aligned, and occupies 4*M*N bytes for the overlap checks.
 */
typedef struct w4_linear_desc_f32 {
  const uint16_t* x;       /* bf16 [M][K]                  */
  int64_t M;
  int64_t K;
  const uint8_t* q_packed; /* native codes of the N x K W  */
  const float* d_packed;   /* native fp32 scales           */
  int64_t N;
  float* y;                /* fp32 [M][N]                  */
} w4_linear_desc_f32;

w4_status w4_linear_f32(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                        const float* d_packed, int64_t N, float* y, int path, hipStream_t stream);
w4_status w4_linear_f32_s16(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                            const uint16_t* d_packed, int64_t N, float* y, int path,
                            hipStream_t stream);
w4_status w4_linear_batched_f32(const w4_linear_desc_f32* linears, int count, int path,
                                hipStream_t stream);

/*
 * Split launches -- the same linears (study, section 1: y = W x) for the
 * draft-verification widths (M = K + 1 rows for K drafted tokens, 27B
 * quantization-and-drafter ladder, stage 2), where a launch of few, long row
 * panels leaves most compute units idle: the MFMA kernel may divide each
 * panel's inputs among up to 8 blocks that hand their fp32 partial sums to
 * the panel's last block through a caller-owned workspace.  The last block
 * adds them in a fixed order, so results are reproducible run to run (they
 * depend on the shapes, the kernel configuration and the chosen number of
 * slices, not on timing), and they obey the accuracy convention above; they
 * may differ in the last bits from the unsplit entry points.  The dot2 path
 * (W4_PATH_GEMV, and W4_PATH_AUTO at M = 1) never splits.
 *   workspace       [in/out] device memory of at least
 *                   W4_SPLIT_WORKSPACE_BYTES bytes (w4_split_workspace_bytes()),
 *                   256-byte aligned (W4_ERR_ALIGN), sharing no byte with any
 *                   operand of the call (W4_ERR_ARG); too small: W4_ERR_ARG.
 *                   Owned by the caller.  Initialise it once with
 *                   w4_split_workspace_init before its first use; every call
 *                   leaves it initialised again.  Calls that use one
 *                   workspace must not overlap in time (one stream, or
 *                   ordered by the caller): concurrent calls race on it.
 *   other arguments as w4_linear_batched / _s16 / _f32.
 * The last block's wait for the others is bounded: should it ever time out
 * (only a concurrently used workspace can cause that), the affected outputs
 * are NaN and w4_split_workspace_error reports bit 0 of its flag (it
 * synchronises `stream`).  A workspace that was never initialised is
 * detected (the initialisation writes a magic word): the split outputs are
 * NaN, nothing waits, and the flag has bit 1 set.  Re-initialise the
 * workspace after either.
 */
#define W4_SPLIT_WORKSPACE_BYTES ((size_t)4 << 20)
size_t w4_split_workspace_bytes(void);
w4_status w4_split_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);
w4_status w4_split_workspace_error(const void* workspace, uint32_t* flag, hipStream_t stream);
w4_status w4_linear_batched_split(const w4_linear_desc* linears, int count, int path,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);
w4_status w4_linear_batched_split_s16(const w4_linear_desc_s16* linears, int count, int path,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);
w4_status w4_linear_batched_split_f32(const w4_linear_desc_f32* linears, int count, int path,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * w4_pack -- canonical codes and scales -> native layout (for codes computed
 * elsewhere).  q_canon int8 [N][K] (values must lie in [-8, 7]; others are
 * reduced modulo 16), d_canon fp32 [N][K/128].  Outputs as w4_quantize_rtn.
 * q_canon and d_canon need 16- and 4-byte alignment.
 */
w4_status w4_pack(const int8_t* q_canon, const float* d_canon, int64_t N, int64_t K,
                  uint8_t* q_packed, float* d_packed, hipStream_t stream);

/*
 * w4_unpack -- native layout -> canonical codes int8 [N][K] and scales fp32
 * [N][K/128] (padding rows are dropped).  Bit-exact inverse of w4_pack.
 */
w4_status w4_unpack(const uint8_t* q_packed, const float* d_packed, int64_t N, int64_t K,
                    int8_t* q_canon, float* d_canon, hipStream_t stream);

/*
 * Chained pass -- a dependent sequence of linears with one M run as one pass
 * of two launches.  Every generated token runs each linear of every layer
 * once, one after the other (27B quantization-and-drafter ladder, stage 1:
 * decode reads all weights per token), at M = 1; verifying K drafted tokens
 * runs the same sequence at M = K + 1 (stage 2).  Within a layer q|k|v read
 * the layer input, o reads what they lead to, gate|up read o's result and
 * down reads theirs.  The linears are given in stages; a linear whose x lies
 * in outputs of earlier stages uses no value of it before that value is
 * written.  Each linear computes exactly what w4_linear computes (study,
 * section 1: y = W x with the group-quantization equation): its bits equal
 * those of one w4_linear_batched call per stage run in the chain's (R, NW)
 * configuration -- with the dot2 kernel at M = 1, with the MFMA kernel and no
 * split workspace at M = 2..16 -- except that a NaN output with bits 0xFFFF
 * is written as 0xFFC0 (0xFFFF marks unwritten values inside the pass).
 *
 * Unlike one launch per stage, the pass does not drain between stages: a
 * persistent grid walks the stages' row panels in order and issues the
 * weight loads of its next panel before that panel's input is ready; at
 * M = 1 each wavefront stages its range of the input once no value of it is
 * unwritten, at M > 1 each group of the input is checked as it is read and
 * waited for while any value is unwritten.  A first, small launch marks every
 * output that a later stage reads as unwritten.
 *
 *   w4_chain_workspace_bytes(count) -- bytes of device workspace for `count`
 *       linears (a header and a table of the linears).
 *   w4_chain_prepare(linears, count, workspace, bytes, plan, stream) --
 *       validates the chain, writes its table into `workspace` (device,
 *       16-byte aligned, >= w4_chain_workspace_bytes(count) bytes, owned by
 *       the caller and kept alive and untouched while the plan is used),
 *       fills `*plan` (host), and SYNCHRONISES `stream` once (a set-up call,
 *       not part of the pass).  `linears` is host memory, read before the
 *       call returns.  Requirements (W4_ERR_SHAPE / _NULL / _ALIGN / _ARG as
 *       for w4_linear): 1 <= count <= W4_CHAIN_MAX; one M for every linear,
 *       from 1 to 16 (x is [M][K] and y [M][N], rows contiguous); every K a
 *       multiple of 128 (up to 30720 at M = 1, as w4_linear otherwise);
 *       N >= 1; stage[0] == 0 and each stage equal to the previous one or one
 *       more.  Each byte is written at most
 *       once per pass and never after the pass has read it: no y overlaps any
 *       q or d, any other y, or the 128-byte cache lines of any x of its own
 *       or an earlier stage.  An x that overlaps outputs of earlier stages
 *       must lie entirely within them (W4_ERR_ARG otherwise).  The buffers
 *       named in `linears` must stay allocated while the plan is used.
 *   w4_chain_run(plan, stream) -- enqueues one pass (asynchronous, no
 *       allocation, capturable in a HIP graph).  Passes on one workspace must
 *       not overlap in time (one stream, or ordered streams).
 *   w4_chain_trace(plan, stamps, count, stream) -- a measuring aid: from the
 *       next pass on, thread 0 of each block writes three values of the
 *       GPU's 100 MHz real-time counter per item (the chain's panels in the
 *       order it runs them: stage by stage, within a stage longest K first,
 *       each linear's panels of rows_per_item rows in order) to the device
 *       buffer `stamps` (count >= 3 * plan->items uint64 values, 8-byte
 *       aligned, owned by the caller): [3i] the item's start, [3i + 1] at
 *       M = 1 when its block's first wavefront had staged its input (0 if it
 *       reused the previous item's, and always 0 at M > 1), [3i + 2] its end.
 *       stamps == NULL stops it.  `plan` is updated (its `trace` field).  The
 *       outputs do not change; passes run a variant of the chained kernel
 *       that takes the stamps only while it is set (the plan's `trace`), so
 *       untraced passes carry none of its cost.  Synchronises `stream`;
 *       w4_chain_prepare clears it.
 *   w4_chain_error(plan, &flag, stream) -- synchronises `stream` and reads
 *       the workspace's error flag: nonzero if a wait of some pass ran out of
 *       time (it is bounded at tens of milliseconds; it can only run out if
 *       the grid's blocks were not all resident at once, e.g. while another
 *       process held the GPU's compute units).  The results of such a pass
 *       are undefined; the flag stays set, and later passes stop waiting,
 *       until the next w4_chain_prepare.
 */
#define W4_CHAIN_MAX 8192

typedef struct w4_chain_linear {
  const uint16_t* x;       /* bf16 [M][K]                                  */
  int64_t M;               /* 1..16, the same for every linear of a chain  */
  int64_t K;
  const uint8_t* q_packed; /* native codes of the N x K W                  */
  const float* d_packed;   /* native fp32 scales                           */
  int64_t N;
  uint16_t* y;             /* bf16 [M][N]                                  */
  int64_t stage;           /* 0, 1, 2 ... non-decreasing, steps of 0 or 1  */
} w4_chain_linear;

/* The same with 16-bit scales (bf16 bit patterns, as the *_s16 entry points
 * store them), for w4_chain_prepare_s16. */
typedef struct w4_chain_linear_s16 {
  const uint16_t* x;        /* bf16 [M][K]                                  */
  int64_t M;                /* 1..16, the same for every linear of a chain  */
  int64_t K;
  const uint8_t* q_packed;  /* native codes of the N x K W                  */
  const uint16_t* d_packed; /* native bf16 scales                           */
  int64_t N;
  uint16_t* y;              /* bf16 [M][N]                                  */
  int64_t stage;
} w4_chain_linear_s16;

/* Filled by w4_chain_prepare(_s16); read by w4_chain_run (treat as opaque). */
typedef struct w4_chain_plan {
  void* workspace;
  int32_t linears, stages, items, blocks;
  int32_t config, lds_bytes, rows_per_item, waves_per_block;
  int32_t scale_bytes, rows;
  int32_t trace, reserved;  /* trace: set by w4_chain_trace */
} w4_chain_plan;

size_t w4_chain_workspace_bytes(int64_t count);
w4_status w4_chain_prepare(const w4_chain_linear* linears, int64_t count, void* workspace,
                           size_t workspace_bytes, w4_chain_plan* plan, hipStream_t stream);
/* w4_chain_prepare for linears with 16-bit scales (same contract). */
w4_status w4_chain_prepare_s16(const w4_chain_linear_s16* linears, int64_t count, void* workspace,
                               size_t workspace_bytes, w4_chain_plan* plan, hipStream_t stream);
w4_status w4_chain_run(const w4_chain_plan* plan, hipStream_t stream);
w4_status w4_chain_error(const w4_chain_plan* plan, uint32_t* flag, hipStream_t stream);
w4_status w4_chain_trace(w4_chain_plan* plan, uint64_t* stamps, size_t count, hipStream_t stream);

/*
 * w4_chain_prepare_noalloc -- w4_chain_prepare for callers that cannot
 * allocate device memory (code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc): the same checks, plan and
 * status codes, with the workspace taken from a static device array of
 * W4_CHAIN_SCRATCH_BYTES bytes that the library holds on each GPU it runs on
 * until the process ends (its device address is looked up once per device,
 * on the first call there).  No hipMalloc, hipFree or other allocation, on
 * the device or the host.  A chain whose workspace
 * (w4_chain_workspace_bytes(count): up to 1022 linears) does not fit is
 * refused with W4_ERR_SCRATCH before anything is written.  The plan is used
 * with w4_chain_run / w4_chain_error as any other.
 * Every plan prepared this way on one GPU shares that GPU's array, which
 * keeps the last call's contents: preparing a plan overwrites the table of
 * the previous one, so only the most recently prepared plan of a GPU may be
 * run, and prepares or passes of such plans that overlap in time (other
 * streams, other threads) race.
 */
#define W4_CHAIN_SCRATCH_BYTES 65536
w4_status w4_chain_prepare_noalloc(const w4_chain_linear* linears, int64_t count, w4_chain_plan* plan,
                                   hipStream_t stream);

/*
 * 16-bit scales.  The study's checkpoint sizes imply about two bytes per
 * group without naming a format; these entry points store each scale as the
 * bf16 nearest to the fp32 scale max|w| / 7 (ties to even; NaN groups get
 * 0x7FC0) and take the codes against that stored value: q = clamp(round(
 * fl32(w / d16)), -8, 7) with ties away from zero.  Scale storage halves
 * (2 instead of 4 bytes per group of 128 weights).  Each function has the
 * contract of its fp32-scale counterpart above, with scales as uint16 bf16
 * bit patterns: w4_scale_count(N, K) elements of 2 bytes natively (16-byte
 * aligned), [N][K/128] canonically (2-byte aligned).
 */
w4_status w4_quantize_rtn_s16(const float* W, int64_t N, int64_t K, uint8_t* q_packed,
                              uint16_t* d_packed, hipStream_t stream);

/* y = W_hat x with 16-bit scales; `path` as for w4_linear_ex. */
w4_status w4_linear_s16(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                        const uint16_t* d_packed, int64_t N, uint16_t* y, int path,
                        hipStream_t stream);

/* Up to W4_MAX_BATCH linears with 16-bit scales in one launch. */
w4_status w4_linear_batched_s16(const w4_linear_desc_s16* linears, int count, int path,
                                hipStream_t stream);

/* Canonical <-> native layout with 16-bit scales. */
w4_status w4_pack_s16(const int8_t* q_canon, const uint16_t* d_canon, int64_t N, int64_t K,
                      uint8_t* q_packed, uint16_t* d_packed, hipStream_t stream);
w4_status w4_unpack_s16(const uint8_t* q_packed, const uint16_t* d_packed, int64_t N, int64_t K,
                        int8_t* q_canon, uint16_t* d_canon, hipStream_t stream);

/*
 * Channel scaling before RTN (study, section 2: the AWQ row of the methods
 * table -- same storage as RTN, input channels rescaled before quantizing;
 * the settings table -- scale candidates from input statistics only, 20
 * exponents in [0, 1], chosen by the output error on calibration inputs, no
 * clipping search; and the channel-scaling equation W'_ij = W_ij s_j,
 * x'_j = x_j / s_j, W'x' = Wx).  The search runs these steps per matrix:
 *   m = w4_channel_absmean(calibration x)
 *   for alpha = k/19, k = 0..19:
 *     w4_awq_scales(m, alpha) -> s, inv_s
 *     w4_quantize_rtn_scaled(W, s) -> q, d
 *     w4_scale_activations(x, inv_s) -> x'; w4_linear(x', q, d) -> y'
 *     w4_sq_error(y', W x) -> error
 * and keeps the exponent with the smallest error.  Decoding then either
 * passes x' (1/s folded into the previous operation) to w4_linear, or x and
 * inv_s to w4_linear_awq.
 */

/* m[j] = mean over the T rows of |x[t][j]|; x bf16 [T][K] (2-byte aligned),
 * m fp32 [K] (4-byte aligned).  The sum runs over t in order, in fp32.
 * W4_ERR_SHAPE if T*K*2 > 2 GiB. */
w4_status w4_channel_absmean(const uint16_t* x, int64_t T, int64_t K, float* m, hipStream_t stream);

/* Candidate channel scales for one exponent 0 <= alpha <= 1 (else
 * W4_ERR_ARG): p_j = max(m_j, 1e-30)^alpha in fp64, s_j = fl32(p_j / g) with
 * g the geometric mean of p (so s has geometric mean 1), inv_s_j =
 * fl32(1 / s_j).  m, s, inv_s fp32 [K], 4-byte aligned, s and inv_s disjoint
 * from each other and from m.  One workgroup; fixed summation order. */
w4_status w4_awq_scales(const float* m, int64_t K, double alpha, float* s, float* inv_s,
                        hipStream_t stream);

/* w4_quantize_rtn (resp. _s16) of W' = fl32(W[n][k] * s[k]): the columns
 * are scaled in fp32 first.  s fp32 [K], 16-byte aligned; everything else
 * as w4_quantize_rtn. */
w4_status w4_quantize_rtn_scaled(const float* W, const float* s, int64_t N, int64_t K,
                                 uint8_t* q_packed, float* d_packed, hipStream_t stream);
w4_status w4_quantize_rtn_scaled_s16(const float* W, const float* s, int64_t N, int64_t K,
                                     uint8_t* q_packed, uint16_t* d_packed, hipStream_t stream);

/* x_out[m][k] = bf16_rne(fl32(x[m][k] * inv_s[k])); x, x_out bf16 [M][K]
 * (2-byte aligned, disjoint), inv_s fp32 [K].  W4_ERR_SHAPE if 2*M*K > 1 GiB. */
w4_status w4_scale_activations(const uint16_t* x, int64_t M, int64_t K, const float* inv_s,
                               uint16_t* x_out, hipStream_t stream);

/* y = W_hat' x' with x' = x * inv_s formed (as w4_scale_activations does)
 * while the dot2 kernel stages x: the decode linear of a matrix quantized by
 * w4_quantize_rtn_scaled when 1/s is not folded into the previous operation.
 * Arguments as w4_linear, plus inv_s fp32 [K] (16-byte aligned); M > 4 runs in
 * slabs of up to 4 rows; K <= 30720 (else W4_ERR_SHAPE). */
w4_status w4_linear_awq(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                        const float* d_packed, int64_t N, const float* inv_s, uint16_t* y,
                        hipStream_t stream);

/* *out = sum over e < count of (y[e] - y_ref[e])^2 in fp64 (y bf16, y_ref
 * fp32; one workgroup, fixed summation order); out is device memory,
 * 8-byte aligned.  count == 0 writes 0. */
w4_status w4_sq_error(const uint16_t* y, const float* y_ref, int64_t count, double* out,
                      hipStream_t stream);

/*
 * GPTQ (study, section 2: the GPTQ row of the methods table -- same storage
 * as RTN, one input column quantized at a time with the columns not yet
 * quantized corrected through a Hessian of calibration inputs; the settings
 * table -- damping 0.01 of the mean Hessian diagonal, blocks of 128 columns,
 * no reordering).  The update rule is the published GPTQ algorithm.  The
 * quantizer runs, per matrix W [N][K] (fp32, finite) and calibration rows
 * x [T][K]:
 *   w4_gptq_hessian(x) -> H = (2/T) x^T x           (fp64 [K][K])
 *   w4_gptq_damp(H, 0.01)
 *   w4_gptq_inverse_factor(H) -> U                  (upper triangular, fp32,
 *                                                    H^-1 = U^T U)
 *   for b0 = 0, 128, ...:
 *     w4_gptq_block(W, b0, U) -> codes and scales of columns b0..b0+127, err
 *     w4_gptq_update(W, b0, U, err): W[:, b0+128:] -= err^T U[b0:b0+128, b0+128:]
 *   w4_pack(codes, scales) -> the native layout w4_linear reads.
 * The products run in the library's LDS-tiled fp64 / fp32 kernels, each
 * element summed in a fixed order (bitwise reproducible).
 */

/* H = (2/T) x^T x, fp64 [K][K] row-major, both triangles (H[i][j] is
 * computed for i >= j and mirrored); each entry sums the exact products of
 * the bf16 inputs in fp64 over t in order.  x bf16 [T][K] (2-byte aligned),
 * H 8-byte aligned, disjoint.  T >= 1, T*K <= 2^31; K a multiple of 128 up
 * to 32768 (else W4_ERR_SHAPE). */
w4_status w4_gptq_hessian(const uint16_t* x, int64_t T, int64_t K, double* H, hipStream_t stream);

/* Bytes of device workspace w4_gptq_inverse_factor needs: (2 K^2 + 4096) * 8
 * (0 for a K it does not take). */
size_t w4_gptq_factor_workspace_bytes(int64_t K);

/* U (fp32 [K][K] row-major, upper triangular, zeros below the diagonal) with
 * H^-1 = U^T U, for a damped Hessian H (fp64 [K][K]; only its lower triangle
 * is read; not modified): with J the index reversal, J H J = L L^T (blocked
 * Cholesky, fp64), and U = J L^-1 J (blocked triangular inverse, fp64),
 * rounded to fp32.  A matrix that is not positive definite gives NaN in U.
 * workspace: device, 8-byte aligned, >= w4_gptq_factor_workspace_bytes(K)
 * (else W4_ERR_ARG); H, U and the workspace disjoint.  K as for
 * w4_gptq_hessian. */
w4_status w4_gptq_inverse_factor(const double* H, int64_t K, void* workspace, size_t workspace_bytes, float* U,
                                 hipStream_t stream);

/* The correction of the columns after block b0 (a multiple of 128):
 * W[n][k] -= sum_{j<128} err[j][n] U[b0 + j][k] for k >= b0 + 128, fp32 (each
 * element summed over j in order).  W fp32 [N][K], U fp32 [K][K], err fp32
 * [128][N] (as w4_gptq_block writes it), all 4-byte aligned; W disjoint from
 * U and err.  Nothing is done for the last block. */
w4_status w4_gptq_update(float* W, int64_t N, int64_t K, int64_t b0, const float* U, const float* err,
                         hipStream_t stream);

/* The unquantized layer's output, y[t][n] = sum_k x[t][k] W[n][k] in fp32
 * (each element summed over k in order): the reference the channel-scaling
 * search compares quantized outputs with.  x bf16 [T][K] (2-byte aligned), W
 * fp32 [N][K], y fp32 [T][N] (4-byte aligned, disjoint from x and W). */
w4_status w4_dense_linear_f32(const uint16_t* x, int64_t T, int64_t K, const float* W, int64_t N, float* y,
                              hipStream_t stream);

/* H [K][K] fp64 row-major, in place: a zero diagonal entry becomes 1, then
 * damp * mean(diag) is added to every diagonal entry (fixed summation
 * order).  K >= 1; damp finite and >= 0 (else W4_ERR_ARG); H 8-byte aligned. */
w4_status w4_gptq_damp(double* H, int64_t K, double damp, hipStream_t stream);

/* The GPTQ column loop over the block of columns b0 .. b0+127 (one group):
 * for every row n < N of W (fp32 [N][K], the current, already corrected
 * weights; only the block's columns are read), the group scale
 * d = fl32(max|w| / 7) of the block's current weights, then for each column j
 * in order the RTN code decision against d, err_j = (w_j - d q_j) / U[j][j]
 * and w_k -= err_j U[j][k] for the block's later columns k.  Writes the codes
 * to q_canon (int8 [N][K], canonical layout, the block's columns), the scale
 * to d_canon[n][b0/128] (fp32 [N][K/128]) and err_j to err[j][n] (fp32
 * [128][N], column-major).  U is fp32 [K][K] row-major (its diagonal block at
 * b0 is read).  W is not modified.  K a positive multiple of 128, b0 a
 * multiple of 128 below K, N >= 0 (else W4_ERR_SHAPE); W and q_canon 16-byte
 * aligned, U, d_canon and err 4-byte aligned (else W4_ERR_ALIGN); outputs must
 * not overlap each other or the inputs (W4_ERR_ARG).  Non-finite weights or U
 * give unspecified codes. */
w4_status w4_gptq_block(const float* W, int64_t N, int64_t K, int64_t b0, const float* U, int8_t* q_canon,
                        float* d_canon, float* err, hipStream_t stream);

/* w4_gptq_block with 16-bit scales: the group scale is stored in d_canon
 * (bf16 bit patterns [N][K/128], 2-byte aligned) as the nearest bf16 of the
 * fp32 scale, and the codes and corrections use that stored value (the rule
 * of w4_quantize_rtn_s16). */
w4_status w4_gptq_block_s16(const float* W, int64_t N, int64_t K, int64_t b0, const float* U, int8_t* q_canon,
                            uint16_t* d_canon, float* err, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
