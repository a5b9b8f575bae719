// C ABI of libw4.so (declared in include/w4.h): argument checks on the host,
// then one asynchronous launch on the caller's stream.  No allocation, no
// host synchronisation, no state beyond the thread-local last HIP error.
#include "w4.h"
#include "w4_launch.h"

#include <hip/hip_runtime.h>

#include <float.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cstddef>
#include <mutex>

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kGroup = 128;
constexpr int64_t kMaxK = int64_t(1) << 24;       // keeps every in-kernel index in range
constexpr int64_t kMaxN = (int64_t(1) << 31) - 16;
constexpr int64_t kMaxM = 65535 * 4;              // kept within 32-bit block indices

bool k_ok(int64_t K) { return K > 0 && K % kGroup == 0 && K <= kMaxK; }
bool n_ok(int64_t N) { return N >= 0 && N <= kMaxN; }
int64_t padded_rows(int64_t N) { return (N + 15) / 16 * 16; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Kernel used by w4_linear for a shape.  At M = 1 the dot2 kernel, which
// stages x in LDS and so issues no x loads through the vector memory
// pipeline, measured faster on every projection shape; from M = 2 on, the
// dot products grow with M while one MFMA serves 16 rows of x.
int auto_path(int64_t M, int64_t K) {
  if (M == 1 && w4::gemv_lds_bytes(1, K) <= w4::kGemvLdsBytes) return W4_PATH_GEMV;
  return W4_PATH_MFMA;
}

w4_status hip_status(hipError_t e) {
  if (e == hipSuccess) return W4_OK;
  g_last_hip_error = static_cast<int>(e);
  return W4_ERR_HIP;
}

// One linear of a call, whatever the scale format (fp32 or bf16 scales).
struct LinearArgs {
  const uint16_t* x;
  int64_t M, K;
  const uint8_t* q;
  const void* d;
  int64_t N;
  void* y;
  size_t ybytes;  // per output element: 2 (bf16) or 4 (fp32)
};

template <typename Desc>
LinearArgs args_of(const Desc& l) {
  return LinearArgs{l.x, l.M, l.K, l.q_packed, l.d_packed, l.N, l.y, sizeof(*l.y)};
}

// Checks one linear of a call; on success appends it to the batch.
w4_status check_linear(const LinearArgs& l, w4::BatchArgs& a) {
  if (l.M < 0 || l.M > kMaxM || !n_ok(l.N) || !k_ok(l.K)) return W4_ERR_SHAPE;
  if (l.M == 0 || l.N == 0) return W4_OK;  // empty: nothing to launch
  // The kernels address codes with 32-bit offsets below 2 GiB and x below 1 GiB.
  if (w4_packed_bytes(l.N, l.K) >= (size_t)1 << 31 || 2 * (size_t)l.M * l.K > (size_t)1 << 30) return W4_ERR_SHAPE;
  if (!l.x || !l.q || !l.d || !l.y) return W4_ERR_NULL;
  if (!aligned(l.x, 16) || !aligned(l.q, 16) || !aligned(l.d, 16) || !aligned(l.y, l.ybytes)) return W4_ERR_ALIGN;
  w4::LinearDesc& d = a.desc[a.count++];
  d.x = l.x;
  d.q = l.q;
  d.d = l.d;
  d.y = l.y;
  d.M = (int)l.M;
  d.K = (int)l.K;
  d.N = (int)l.N;
  d.flags = l.ybytes == 4 ? w4::kOutF32 : 0;
  return W4_OK;
}

// Every output must be disjoint from every input and every other output of the call.
w4_status check_aliasing(const LinearArgs* l, int count, size_t scale_elem) {
  for (int i = 0; i < count; ++i) {
    if (l[i].M <= 0 || l[i].N <= 0) continue;
    const size_t yb = l[i].ybytes * (size_t)l[i].M * l[i].N;
    for (int j = 0; j < count; ++j) {
      if (l[j].M <= 0 || l[j].N <= 0) continue;
      if (overlaps(l[i].y, yb, l[j].x, 2 * (size_t)l[j].M * l[j].K) ||
          overlaps(l[i].y, yb, l[j].q, w4_packed_bytes(l[j].N, l[j].K)) ||
          overlaps(l[i].y, yb, l[j].d, scale_elem * w4_scale_count(l[j].N, l[j].K)))
        return W4_ERR_ARG;
      if (j != i && overlaps(l[i].y, yb, l[j].y, l[j].ybytes * (size_t)l[j].M * l[j].N)) return W4_ERR_ARG;
    }
  }
  return W4_OK;
}

w4_status run_batch(w4::BatchArgs& a, int path, int64_t max_m, int64_t max_k, bool s16, hipStream_t stream,
                    void* split_ws = nullptr, size_t split_ws_bytes = 0) {
  if (a.count == 0) return W4_OK;
  if (path == W4_PATH_AUTO) path = auto_path(max_m, max_k);
  if (path == W4_PATH_GEMV) {
    if (w4::gemv_lds_bytes(1, max_k) > w4::kGemvLdsBytes) return W4_ERR_SHAPE;
    return hip_status(w4::launch_linear_gemv(a, w4::gemv_rows_per_slab(max_m, max_k), s16, stream));
  }
  return hip_status(w4::launch_linear_mfma(a, s16, stream, split_ws, split_ws_bytes));
}

bool split_workspace_ok(const void* ws, size_t bytes) {
  return ws && aligned(ws, 256) && bytes >= W4_SPLIT_WORKSPACE_BYTES;
}

// The split workspace may share no byte with any operand of the call.
bool split_workspace_disjoint(const void* ws, size_t bytes, const LinearArgs* l, int count, size_t scale_elem) {
  for (int i = 0; i < count; ++i) {
    if (l[i].M <= 0 || l[i].N <= 0) continue;
    if (overlaps(ws, bytes, l[i].x, 2 * (size_t)l[i].M * l[i].K) ||
        overlaps(ws, bytes, l[i].q, w4_packed_bytes(l[i].N, l[i].K)) ||
        overlaps(ws, bytes, l[i].d, scale_elem * w4_scale_count(l[i].N, l[i].K)) ||
        overlaps(ws, bytes, l[i].y, l[i].ybytes * (size_t)l[i].M * l[i].N))
      return false;
  }
  return true;
}

template <typename Desc>
w4_status linear_batched(const Desc* linears, int count, int path, bool s16, hipStream_t stream,
                         void* split_ws = nullptr, size_t split_ws_bytes = 0) {
  if (path != W4_PATH_AUTO && path != W4_PATH_GEMV && path != W4_PATH_MFMA) return W4_ERR_ARG;
  if (count < 0 || count > W4_MAX_BATCH) return W4_ERR_ARG;
  if (count == 0) return W4_OK;
  if (!linears) return W4_ERR_NULL;
  w4::BatchArgs a;
  a.count = 0;
  LinearArgs args[W4_MAX_BATCH];
  int64_t max_m = 0, max_k = 0;
  for (int i = 0; i < count; ++i) {
    args[i] = args_of(linears[i]);
    const w4_status st = check_linear(args[i], a);
    if (st != W4_OK) return st;
    if (args[i].M > 0 && args[i].N > 0) {
      max_m = args[i].M > max_m ? args[i].M : max_m;
      max_k = args[i].K > max_k ? args[i].K : max_k;
    }
  }
  const w4_status al = check_aliasing(args, count, s16 ? 2 : 4);
  if (al != W4_OK) return al;
  if (split_ws && !split_workspace_disjoint(split_ws, split_ws_bytes, args, count, s16 ? 2 : 4)) return W4_ERR_ARG;
  return run_batch(a, path, max_m, max_k, s16, stream, split_ws, split_ws_bytes);
}

template <typename Desc>
w4_status linear_batched_split(const Desc* linears, int count, int path, bool s16, void* ws, size_t bytes,
                               hipStream_t stream) {
  if (!ws) return W4_ERR_NULL;
  if (!split_workspace_ok(ws, bytes)) return !aligned(ws, 256) ? W4_ERR_ALIGN : W4_ERR_ARG;
  return linear_batched(linears, count, path, s16, stream, ws, bytes);
}

w4_status quantize(const float* W, int64_t N, int64_t K, uint8_t* q_packed, void* d_packed, bool s16,
                   hipStream_t stream) {
  if (!n_ok(N) || !k_ok(K)) return W4_ERR_SHAPE;
  if (N == 0) return W4_OK;
  if (!W || !q_packed || !d_packed) return W4_ERR_NULL;
  if (!aligned(W, 16) || !aligned(q_packed, 16) || !aligned(d_packed, 16)) return W4_ERR_ALIGN;
  const size_t qb = w4_packed_bytes(N, K), db = (s16 ? 2 : 4) * w4_scale_count(N, K), wb = 4 * (size_t)N * K;
  if (overlaps(q_packed, qb, d_packed, db) || overlaps(q_packed, qb, W, wb) || overlaps(d_packed, db, W, wb))
    return W4_ERR_ARG;
  return hip_status(w4::launch_quantize_rtn(W, N, K, q_packed, d_packed, s16, stream));
}

w4_status pack(const int8_t* q_canon, const void* d_canon, int64_t N, int64_t K, uint8_t* q_packed,
               void* d_packed, bool s16, hipStream_t stream) {
  if (!n_ok(N) || !k_ok(K)) return W4_ERR_SHAPE;
  if (N == 0) return W4_OK;
  if (!q_canon || !d_canon || !q_packed || !d_packed) return W4_ERR_NULL;
  const size_t e = s16 ? 2 : 4;
  if (!aligned(q_canon, 16) || !aligned(d_canon, e) || !aligned(q_packed, 16) || !aligned(d_packed, 16))
    return W4_ERR_ALIGN;
  const size_t qb = w4_packed_bytes(N, K), db = e * w4_scale_count(N, K);
  const size_t qcb = (size_t)N * K, dcb = e * (size_t)N * (K / kGroup);
  if (overlaps(q_packed, qb, d_packed, db) || overlaps(q_packed, qb, q_canon, qcb) ||
      overlaps(q_packed, qb, d_canon, dcb) || overlaps(d_packed, db, q_canon, qcb) ||
      overlaps(d_packed, db, d_canon, dcb))
    return W4_ERR_ARG;
  return hip_status(w4::launch_pack(q_canon, d_canon, N, K, q_packed, d_packed, s16, stream));
}

w4_status unpack(const uint8_t* q_packed, const void* d_packed, int64_t N, int64_t K, int8_t* q_canon,
                 void* d_canon, bool s16, hipStream_t stream) {
  if (!n_ok(N) || !k_ok(K)) return W4_ERR_SHAPE;
  if (N == 0) return W4_OK;
  if (!q_canon || !d_canon || !q_packed || !d_packed) return W4_ERR_NULL;
  const size_t e = s16 ? 2 : 4;
  if (!aligned(q_canon, 16) || !aligned(d_canon, e) || !aligned(q_packed, 16) || !aligned(d_packed, 16))
    return W4_ERR_ALIGN;
  const size_t qb = w4_packed_bytes(N, K), db = e * w4_scale_count(N, K);
  const size_t qcb = (size_t)N * K, dcb = e * (size_t)N * (K / kGroup);
  if (overlaps(q_canon, qcb, d_canon, dcb) || overlaps(q_canon, qcb, q_packed, qb) ||
      overlaps(q_canon, qcb, d_packed, db) || overlaps(d_canon, dcb, q_packed, qb) ||
      overlaps(d_canon, dcb, d_packed, db))
    return W4_ERR_ARG;
  return hip_status(w4::launch_unpack(q_packed, d_packed, N, K, q_canon, d_canon, s16, stream));
}

}  // namespace

extern "C" {

const char* w4_status_str(int status) {
  switch (status) {
    case W4_OK: return "W4_OK: success";
    case W4_ERR_NULL: return "W4_ERR_NULL: a required pointer is NULL";
    case W4_ERR_SHAPE: return "W4_ERR_SHAPE: invalid shape (K must be a positive multiple of 128; M, N >= 0; size limits)";
    case W4_ERR_ALIGN: return "W4_ERR_ALIGN: a pointer is not aligned as required";
    case W4_ERR_HIP: return "W4_ERR_HIP: a HIP runtime call or kernel launch failed";
    case W4_ERR_ARG: return "W4_ERR_ARG: invalid argument";
    case W4_ERR_SCRATCH:
      return "W4_ERR_SCRATCH: the chain's workspace exceeds the library's static scratch (W4_CHAIN_SCRATCH_BYTES)";
    default: return "unknown w4 status";
  }
}

int w4_last_hip_error(void) { return g_last_hip_error; }

int w4_group_size(void) { return (int)kGroup; }

size_t w4_packed_bytes(int64_t N, int64_t K) {
  if (!n_ok(N) || !k_ok(K)) return 0;
  return (size_t)padded_rows(N) * (size_t)((K + 511) / 512 * 512) / 2;
}

size_t w4_scale_count(int64_t N, int64_t K) {
  if (!n_ok(N) || !k_ok(K)) return 0;
  return (size_t)padded_rows(N) * (size_t)((K / kGroup + 3) / 4 * 4);
}

w4_status w4_quantize_rtn(const float* W, int64_t N, int64_t K, uint8_t* q_packed, float* d_packed,
                          hipStream_t stream) {
  return quantize(W, N, K, q_packed, d_packed, false, stream);
}

w4_status w4_quantize_rtn_s16(const float* W, int64_t N, int64_t K, uint8_t* q_packed, uint16_t* d_packed,
                              hipStream_t stream) {
  return quantize(W, N, K, q_packed, d_packed, true, stream);
}

w4_status w4_linear_batched(const w4_linear_desc* linears, int count, int path, hipStream_t stream) {
  return linear_batched(linears, count, path, false, stream);
}

w4_status w4_linear_batched_s16(const w4_linear_desc_s16* linears, int count, int path, hipStream_t stream) {
  return linear_batched(linears, count, path, true, stream);
}

w4_status w4_linear_ex(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                       const float* d_packed, int64_t N, uint16_t* y, int path, hipStream_t stream) {
  const w4_linear_desc l = {x, M, K, q_packed, d_packed, N, y};
  return w4_linear_batched(&l, 1, path, stream);
}

w4_status w4_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                    const float* d_packed, int64_t N, uint16_t* y, hipStream_t stream) {
  return w4_linear_ex(x, M, K, q_packed, d_packed, N, y, W4_PATH_AUTO, stream);
}

w4_status w4_linear_s16(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                        const uint16_t* d_packed, int64_t N, uint16_t* y, int path, hipStream_t stream) {
  const w4_linear_desc_s16 l = {x, M, K, q_packed, d_packed, N, y};
  return w4_linear_batched_s16(&l, 1, path, stream);
}

w4_status w4_linear_batched_f32(const w4_linear_desc_f32* linears, int count, int path, hipStream_t stream) {
  return linear_batched(linears, count, path, false, stream);
}

w4_status w4_linear_f32(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed, const float* d_packed,
                        int64_t N, float* y, int path, hipStream_t stream) {
  const w4_linear_desc_f32 l = {x, M, K, q_packed, d_packed, N, y};
  return w4_linear_batched_f32(&l, 1, path, stream);
}

w4_status w4_linear_f32_s16(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed,
                            const uint16_t* d_packed, int64_t N, float* y, int path, hipStream_t stream) {
  struct {
    const uint16_t* x;
    int64_t M, K;
    const uint8_t* q_packed;
    const uint16_t* d_packed;
    int64_t N;
    float* y;
  } l = {x, M, K, q_packed, d_packed, N, y};
  return linear_batched(&l, 1, path, true, stream);
}

size_t w4_split_workspace_bytes(void) { return W4_SPLIT_WORKSPACE_BYTES; }

w4_status w4_split_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return W4_ERR_NULL;
  if (!aligned(workspace, 256)) return W4_ERR_ALIGN;
  if (workspace_bytes < W4_SPLIT_WORKSPACE_BYTES) return W4_ERR_ARG;
  return hip_status(w4::launch_split_init(workspace, workspace_bytes, stream));
}

w4_status w4_split_workspace_error(const void* workspace, uint32_t* flag, hipStream_t stream) {
  if (!workspace || !flag) return W4_ERR_NULL;
  uint32_t v = 0;
  if (hipError_t e = hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, stream)) return hip_status(e);
  if (hipError_t e = hipStreamSynchronize(stream)) return hip_status(e);
  *flag = v;
  return W4_OK;
}

w4_status w4_linear_batched_split(const w4_linear_desc* linears, int count, int path, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return linear_batched_split(linears, count, path, false, workspace, workspace_bytes, stream);
}

w4_status w4_linear_batched_split_s16(const w4_linear_desc_s16* linears, int count, int path, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return linear_batched_split(linears, count, path, true, workspace, workspace_bytes, stream);
}

w4_status w4_linear_batched_split_f32(const w4_linear_desc_f32* linears, int count, int path, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return linear_batched_split(linears, count, path, false, workspace, workspace_bytes, stream);
}

w4_status w4_pack(const int8_t* q_canon, const float* d_canon, int64_t N, int64_t K,
                  uint8_t* q_packed, float* d_packed, hipStream_t stream) {
  return pack(q_canon, d_canon, N, K, q_packed, d_packed, false, stream);
}

w4_status w4_pack_s16(const int8_t* q_canon, const uint16_t* d_canon, int64_t N, int64_t K,
                      uint8_t* q_packed, uint16_t* d_packed, hipStream_t stream) {
  return pack(q_canon, d_canon, N, K, q_packed, d_packed, true, stream);
}

w4_status w4_unpack(const uint8_t* q_packed, const float* d_packed, int64_t N, int64_t K,
                    int8_t* q_canon, float* d_canon, hipStream_t stream) {
  return unpack(q_packed, d_packed, N, K, q_canon, d_canon, false, stream);
}

w4_status w4_unpack_s16(const uint8_t* q_packed, const uint16_t* d_packed, int64_t N, int64_t K,
                        int8_t* q_canon, uint16_t* d_canon, hipStream_t stream) {
  return unpack(q_packed, d_packed, N, K, q_canon, d_canon, true, stream);
}

// ---------------------------------------------------------------------------
// channel scaling before RTN (AWQ)
// ---------------------------------------------------------------------------

w4_status w4_channel_absmean(const uint16_t* x, int64_t T, int64_t K, float* m, hipStream_t stream) {
  if (T < 0 || K < 0 || K > kMaxK || T * K * 2 > ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  if (T == 0 || K == 0) return W4_OK;
  if (!x || !m) return W4_ERR_NULL;
  if (!aligned(x, 2) || !aligned(m, 4)) return W4_ERR_ALIGN;
  if (overlaps(m, 4 * (size_t)K, x, 2 * (size_t)T * K)) return W4_ERR_ARG;
  return hip_status(w4::launch_channel_absmean(x, T, K, m, stream));
}

w4_status w4_awq_scales(const float* m, int64_t K, double alpha, float* s, float* inv_s, hipStream_t stream) {
  if (K < 0 || K > kMaxK) return W4_ERR_SHAPE;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return W4_ERR_ARG;
  if (K == 0) return W4_OK;
  if (!m || !s || !inv_s) return W4_ERR_NULL;
  if (!aligned(m, 4) || !aligned(s, 4) || !aligned(inv_s, 4)) return W4_ERR_ALIGN;
  const size_t b = 4 * (size_t)K;
  if (overlaps(s, b, inv_s, b) || overlaps(s, b, m, b) || overlaps(inv_s, b, m, b)) return W4_ERR_ARG;
  return hip_status(w4::launch_awq_scales(m, K, alpha, s, inv_s, stream));
}

namespace {
w4_status quantize_scaled(const float* W, const float* s, int64_t N, int64_t K, uint8_t* q_packed, void* d_packed,
                          bool s16, hipStream_t stream) {
  if (!n_ok(N) || !k_ok(K)) return W4_ERR_SHAPE;
  if (N == 0) return W4_OK;
  if (!W || !s || !q_packed || !d_packed) return W4_ERR_NULL;
  if (!aligned(W, 16) || !aligned(s, 16) || !aligned(q_packed, 16) || !aligned(d_packed, 16)) return W4_ERR_ALIGN;
  const size_t qb = w4_packed_bytes(N, K), db = (s16 ? 2 : 4) * w4_scale_count(N, K), wb = 4 * (size_t)N * K;
  if (overlaps(q_packed, qb, d_packed, db) || overlaps(q_packed, qb, W, wb) || overlaps(d_packed, db, W, wb) ||
      overlaps(q_packed, qb, s, 4 * (size_t)K) || overlaps(d_packed, db, s, 4 * (size_t)K))
    return W4_ERR_ARG;
  return hip_status(w4::launch_quantize_rtn_scaled(W, s, N, K, q_packed, d_packed, s16, stream));
}
}  // namespace

w4_status w4_quantize_rtn_scaled(const float* W, const float* s, int64_t N, int64_t K, uint8_t* q_packed,
                                 float* d_packed, hipStream_t stream) {
  return quantize_scaled(W, s, N, K, q_packed, d_packed, false, stream);
}

w4_status w4_quantize_rtn_scaled_s16(const float* W, const float* s, int64_t N, int64_t K, uint8_t* q_packed,
                                     uint16_t* d_packed, hipStream_t stream) {
  return quantize_scaled(W, s, N, K, q_packed, d_packed, true, stream);
}

w4_status w4_scale_activations(const uint16_t* x, int64_t M, int64_t K, const float* inv_s, uint16_t* x_out,
                               hipStream_t stream) {
  if (M < 0 || K < 0 || K > kMaxK || 2 * M * K > ((int64_t)1 << 30)) return W4_ERR_SHAPE;
  if (M == 0 || K == 0) return W4_OK;
  if (!x || !inv_s || !x_out) return W4_ERR_NULL;
  if (!aligned(x, 2) || !aligned(inv_s, 4) || !aligned(x_out, 2)) return W4_ERR_ALIGN;
  const size_t xb = 2 * (size_t)M * K;
  if (overlaps(x_out, xb, x, xb) || overlaps(x_out, xb, inv_s, 4 * (size_t)K)) return W4_ERR_ARG;
  return hip_status(w4::launch_scale_activations(x, M, K, inv_s, x_out, stream));
}

w4_status w4_linear_awq(const uint16_t* x, int64_t M, int64_t K, const uint8_t* q_packed, const float* d_packed,
                        int64_t N, const float* inv_s, uint16_t* y, hipStream_t stream) {
  const LinearArgs l{x, M, K, q_packed, d_packed, N, y, 2};
  w4::BatchArgs a;
  a.count = 0;
  const w4_status st = check_linear(l, a);
  if (st != W4_OK || a.count == 0) return st;
  if (!inv_s) return W4_ERR_NULL;
  if (!aligned(inv_s, 16)) return W4_ERR_ALIGN;
  const w4_status al = check_aliasing(&l, 1, 4);
  if (al != W4_OK) return al;
  if (overlaps(y, 2 * (size_t)M * N, inv_s, 4 * (size_t)K)) return W4_ERR_ARG;
  if (w4::gemv_lds_bytes(1, K) > w4::kGemvLdsBytes) return W4_ERR_SHAPE;
  return hip_status(w4::launch_linear_gemv_xscaled(a.desc[0], inv_s, w4::gemv_rows_per_slab(M, K), stream));
}

w4_status w4_sq_error(const uint16_t* y, const float* y_ref, int64_t count, double* out, hipStream_t stream) {
  if (count < 0) return W4_ERR_SHAPE;
  if (!out) return W4_ERR_NULL;
  if (count > 0 && (!y || !y_ref)) return W4_ERR_NULL;
  if (!aligned(y, 2) || !aligned(y_ref, 4) || !aligned(out, 8)) return W4_ERR_ALIGN;
  if (overlaps(out, 8, y, 2 * (size_t)count) || overlaps(out, 8, y_ref, 4 * (size_t)count)) return W4_ERR_ARG;
  return hip_status(w4::launch_sq_error(y, y_ref, count, out, stream));
}

w4_status w4_gptq_damp(double* H, int64_t K, double damp, hipStream_t stream) {
  if (K < 1 || K > (int64_t)1 << 20) return W4_ERR_SHAPE;
  if (!(damp >= 0.0) || !(damp <= DBL_MAX)) return W4_ERR_ARG;
  if (!H) return W4_ERR_NULL;
  if (!aligned(H, 8)) return W4_ERR_ALIGN;
  return hip_status(w4::launch_gptq_damp(H, K, damp, stream));
}

namespace {
w4_status gptq_block(const float* W, int64_t N, int64_t K, int64_t b0, const float* U, int8_t* q_canon,
                     void* d_canon, bool s16, float* err, hipStream_t stream) {
  if (!n_ok(N) || !k_ok(K) || N > ((int64_t)1 << 31) - 1 || b0 < 0 || b0 >= K || b0 % kGroup) return W4_ERR_SHAPE;
  if (N == 0) return W4_OK;
  if (!W || !U || !q_canon || !d_canon || !err) return W4_ERR_NULL;
  const size_t e = s16 ? 2 : 4;
  if (!aligned(W, 16) || !aligned(U, 4) || !aligned(q_canon, 16) || !aligned(d_canon, e) || !aligned(err, 4))
    return W4_ERR_ALIGN;
  const size_t wb = 4 * (size_t)N * K, ub = 4 * (size_t)K * K, qb = (size_t)N * K,
               db = e * (size_t)N * (K / kGroup), eb = 4 * (size_t)kGroup * N;
  const void* outs[3] = {q_canon, d_canon, err};
  const size_t ob[3] = {qb, db, eb};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], ob[i], W, wb) || overlaps(outs[i], ob[i], U, ub)) return W4_ERR_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return W4_ERR_ARG;
  }
  return hip_status(w4::launch_gptq_block(W, N, K, b0, U, q_canon, d_canon, s16, err, stream));
}
}  // namespace

w4_status w4_gptq_block(const float* W, int64_t N, int64_t K, int64_t b0, const float* U, int8_t* q_canon,
                        float* d_canon, float* err, hipStream_t stream) {
  return gptq_block(W, N, K, b0, U, q_canon, d_canon, false, err, stream);
}

w4_status w4_gptq_block_s16(const float* W, int64_t N, int64_t K, int64_t b0, const float* U, int8_t* q_canon,
                            uint16_t* d_canon, float* err, hipStream_t stream) {
  return gptq_block(W, N, K, b0, U, q_canon, d_canon, true, err, stream);
}

namespace {
constexpr int64_t kMaxGptqK = 32768;  // keeps K^2 doubles of work addressable and each grid in range

bool gptq_k_ok(int64_t K) { return K >= kGroup && K % kGroup == 0 && K <= kMaxGptqK; }
}  // namespace

w4_status w4_gptq_hessian(const uint16_t* x, int64_t T, int64_t K, double* H, hipStream_t stream) {
  if (T < 1 || T > ((int64_t)1 << 31) / 2 || !gptq_k_ok(K) || T * K > ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  if (!x || !H) return W4_ERR_NULL;
  if (!aligned(x, 2) || !aligned(H, 8)) return W4_ERR_ALIGN;
  if (overlaps(H, 8 * (size_t)K * K, x, 2 * (size_t)T * K)) return W4_ERR_ARG;
  return hip_status(w4::launch_gptq_hessian(x, T, K, H, stream));
}

size_t w4_gptq_factor_workspace_bytes(int64_t K) {
  if (!gptq_k_ok(K)) return 0;
  return 8 * w4::gptq_factor_work_doubles(K);
}

w4_status w4_gptq_inverse_factor(const double* H, int64_t K, void* workspace, size_t workspace_bytes, float* U,
                                 hipStream_t stream) {
  if (!gptq_k_ok(K)) return W4_ERR_SHAPE;
  if (!H || !workspace || !U) return W4_ERR_NULL;
  if (!aligned(H, 8) || !aligned(workspace, 8) || !aligned(U, 4)) return W4_ERR_ALIGN;
  const size_t wb = w4_gptq_factor_workspace_bytes(K), hb = 8 * (size_t)K * K, ub = 4 * (size_t)K * K;
  if (workspace_bytes < wb) return W4_ERR_ARG;
  if (overlaps(workspace, wb, H, hb) || overlaps(workspace, wb, U, ub) || overlaps(U, ub, H, hb)) return W4_ERR_ARG;
  return hip_status(w4::launch_gptq_inverse_factor(H, K, static_cast<double*>(workspace), U, stream));
}

w4_status w4_gptq_update(float* W, int64_t N, int64_t K, int64_t b0, const float* U, const float* err,
                         hipStream_t stream) {
  if (!n_ok(N) || !gptq_k_ok(K) || N > ((int64_t)1 << 31) - 1 || b0 < 0 || b0 >= K || b0 % kGroup)
    return W4_ERR_SHAPE;
  if (N == 0) return W4_OK;
  if (!W || !U || !err) return W4_ERR_NULL;
  if (!aligned(W, 4) || !aligned(U, 4) || !aligned(err, 4)) return W4_ERR_ALIGN;
  const size_t wb = 4 * (size_t)N * K;
  if (overlaps(W, wb, U, 4 * (size_t)K * K) || overlaps(W, wb, err, 4 * (size_t)kGroup * N)) return W4_ERR_ARG;
  return hip_status(w4::launch_gptq_update(W, N, K, b0, U, err, stream));
}

w4_status w4_dense_linear_f32(const uint16_t* x, int64_t T, int64_t K, const float* W, int64_t N, float* y,
                              hipStream_t stream) {
  if (T < 0 || N < 0 || K < 1 || T > ((int64_t)1 << 31) - 1 || N > ((int64_t)1 << 31) - 1 ||
      K > ((int64_t)1 << 31) - 1)
    return W4_ERR_SHAPE;
  if (T == 0 || N == 0) return W4_OK;
  if (!x || !W || !y) return W4_ERR_NULL;
  if (!aligned(x, 2) || !aligned(W, 4) || !aligned(y, 4)) return W4_ERR_ALIGN;
  const size_t yb = 4 * (size_t)T * N;
  if (overlaps(y, yb, x, 2 * (size_t)T * K) || overlaps(y, yb, W, 4 * (size_t)N * K)) return W4_ERR_ARG;
  return hip_status(w4::launch_dense_linear_f32(x, T, K, W, N, y, stream));
}

// ---------------------------------------------------------------------------
// chained decode pass
// ---------------------------------------------------------------------------
extern "C++" {
namespace {
uintptr_t addr(const void* p) { return reinterpret_cast<uintptr_t>(p); }

// Is [a, a + na) covered by the outputs (M rows each) of the linears of
// stages before `stage`?  (No allocation: the covered prefix grows by any
// output that reaches past it.)
template <typename Desc>
bool covered_by_earlier(const Desc* l, int64_t count, int64_t stage, uintptr_t a, size_t na, int64_t M) {
  uintptr_t at = a;
  const uintptr_t end = a + na;
  for (bool grew = true; at < end && grew;) {
    grew = false;
    for (int64_t i = 0; i < count && l[i].stage < stage; ++i) {
      const uintptr_t y0 = addr(l[i].y), y1 = y0 + 2 * (size_t)M * l[i].N;
      if (y0 <= at && y1 > at) {
        at = y1;
        grew = true;
      }
    }
  }
  return at >= end;
}

// The chain's checks and its plan (see include/w4.h).  Allocates nothing, on
// the device or the host: flags are recomputed per linear, the table is built
// in a small buffer and uploaded in pieces, and the stream is synchronised
// before returning.  A workspace smaller than the plan needs returns
// `too_small`.
template <typename Desc>
w4_status chain_prepare(const Desc* linears, int64_t count, void* workspace, size_t workspace_bytes,
                        w4_chain_plan* plan, bool s16, w4_status too_small, hipStream_t stream) {
  if (count < 1 || count > W4_CHAIN_MAX) return W4_ERR_ARG;
  if (!linears || !workspace || !plan) return W4_ERR_NULL;
  if (!aligned(workspace, 16)) return W4_ERR_ALIGN;
  // shapes, pointers and stage numbering: one M for the whole chain, 1 (dot2
  // items, x staged whole in LDS) or 2..16 (MFMA items, one slab of x rows)
  const int64_t M = linears[0].M;
  if (M < 1 || M > 16) return W4_ERR_SHAPE;
  int64_t kmax = 0;
  for (int64_t i = 0; i < count; ++i) {
    const Desc& l = linears[i];
    if (l.M != M || l.N < 1 || !n_ok(l.N) || !k_ok(l.K)) return W4_ERR_SHAPE;
    if (M == 1 && w4::gemv_lds_bytes(1, l.K) > w4::kGemvLdsBytes) return W4_ERR_SHAPE;
    if (w4_packed_bytes(l.N, l.K) >= (size_t)1 << 31 || 2 * (size_t)M * l.K > (size_t)1 << 30)
      return W4_ERR_SHAPE;
    if (!l.x || !l.q_packed || !l.d_packed || !l.y) return W4_ERR_NULL;
    if (!aligned(l.x, 16) || !aligned(l.q_packed, 16) || !aligned(l.d_packed, 16) || !aligned(l.y, 2))
      return W4_ERR_ALIGN;
    const int64_t prev = i == 0 ? 0 : linears[i - 1].stage;
    if (i == 0 ? l.stage != 0 : (l.stage != prev && l.stage != prev + 1)) return W4_ERR_ARG;
    kmax = l.K > kmax ? l.K : kmax;
  }
  // Aliasing.  The launch keeps the eight L2s coherent only for chains that
  // write each byte once and never write a cache line (128 bytes) that the
  // pass may read before the write: no y overlaps any other y, and no line
  // of a y holds any byte of the weights, of an x of its own or an earlier
  // stage, or of an x of a later stage that does not read this y.  A y read
  // as x by a later stage is the intended use; such an x must then be
  // written entirely by earlier stages (it is read once no value of it is
  // unwritten).
  const size_t mrows = (size_t)M;  // bytes of a y: 2 * M * N; of an x: 2 * M * K
  for (int64_t i = 0; i < count; ++i) {
    const Desc& a = linears[i];
    const size_t yb = 2 * mrows * a.N;
    const uintptr_t y0 = addr(a.y) & ~(uintptr_t)127;
    const void* ylines = reinterpret_cast<const void*>(y0);
    const size_t ylb = ((addr(a.y) + yb + 127) & ~(uintptr_t)127) - y0;
    for (int64_t j = 0; j < count; ++j) {
      const Desc& b = linears[j];
      if (overlaps(ylines, ylb, b.q_packed, w4_packed_bytes(b.N, b.K)) ||
          overlaps(ylines, ylb, b.d_packed, (s16 ? 2 : 4) * w4_scale_count(b.N, b.K)))
        return W4_ERR_ARG;
      if (j != i && overlaps(a.y, yb, b.y, 2 * mrows * b.N)) return W4_ERR_ARG;
      if (!overlaps(ylines, ylb, b.x, 2 * mrows * b.K)) continue;
      // b reads a line that a writes: only as a later stage reading a's output
      if (b.stage <= a.stage || !overlaps(a.y, yb, b.x, 2 * mrows * b.K)) return W4_ERR_ARG;
    }
  }
  // an x that reads outputs of earlier stages must lie entirely within them
  auto reads_earlier = [&](int64_t j) {
    for (int64_t i = 0; i < count; ++i)
      if (linears[i].stage < linears[j].stage && overlaps(linears[i].y, 2 * mrows * linears[i].N, linears[j].x,
                                                          2 * mrows * linears[j].K))
        return true;
    return false;
  };
  auto read_later = [&](int64_t i) {
    for (int64_t j = 0; j < count; ++j)
      if (linears[j].stage > linears[i].stage && overlaps(linears[i].y, 2 * mrows * linears[i].N, linears[j].x,
                                                          2 * mrows * linears[j].K))
        return true;
    return false;
  };
  for (int64_t j = 0; j < count; ++j)
    if (reads_earlier(j) && !covered_by_earlier(linears, count, linears[j].stage, addr(linears[j].x),
                                                2 * mrows * linears[j].K, M))
      return W4_ERR_ARG;
  const int stages = (int)linears[count - 1].stage + 1;
  const size_t need = w4::chain_workspace_bytes(count);
  if (workspace_bytes < need) return too_small;
  // the workspace overlaps no buffer of the chain
  for (int64_t i = 0; i < count; ++i) {
    const Desc& l = linears[i];
    if (overlaps(workspace, need, l.x, 2 * mrows * l.K) || overlaps(workspace, need, l.y, 2 * mrows * l.N) ||
        overlaps(workspace, need, l.q_packed, w4_packed_bytes(l.N, l.K)) ||
        overlaps(workspace, need, l.d_packed, (s16 ? 2 : 4) * w4_scale_count(l.N, l.K)))
      return W4_ERR_ARG;
  }

  double code_bytes = 0;
  for (int64_t i = 0; i < count; ++i) code_bytes += (double)w4_packed_bytes(linears[i].N, linears[i].K);
  const int ci = w4::chain_choose_cfg((int)kmax, code_bytes / stages, (int)M);
  if (ci < 0) return W4_ERR_ARG;
  int R = 0, NW = 0;
  w4::chain_cfg(ci, &R, &NW);
  const size_t lds = M == 1 ? (size_t)w4::gemv_lds_bytes(1, kmax) : 0;  // the MFMA items' LDS is static

  // Grid: every block resident at once (waits look only at earlier items).
  // Dot2 items: two blocks per CU measured fastest; MFMA items: as many as are
  // resident (three per CU at M <= 8 measured 4% faster than two).
  // W4_CHAIN_BLOCKS may ask for another count, up to what is resident.
  int dev = 0, cus = 0, per_cu = 0;
  if (hipError_t e = hipGetDevice(&dev)) return hip_status(e);
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return hip_status(e);
  if (hipError_t e = w4::chain_blocks_per_cu(ci, s16, lds, (int)M, &per_cu)) return hip_status(e);
  if (per_cu < 1 || cus < 1) return hip_status(hipErrorInvalidConfiguration);
  const int64_t resident = (int64_t)per_cu * cus;
  int64_t blocks = M > 1 || resident < 2 * (int64_t)cus ? resident : 2 * (int64_t)cus;
  if (const char* e = getenv("W4_CHAIN_BLOCKS")) {
    const long v = strtol(e, nullptr, 10);
    if (v > 0) blocks = v < resident ? v : resident;
  }
  // Table: the linears of each stage laid out longest K first (stable), as a
  // batched launch does, each followed by its panels of R row blocks.  The
  // entries are built kChunk at a time and uploaded.
  constexpr int kChunk = 32;
  w4::ChainLinear buf[kChunk];
  uint8_t* const ws = static_cast<uint8_t*>(workspace);
  int nbuf = 0;
  int64_t emitted = 0;  // table entries built so far
  auto flush = [&]() -> hipError_t {
    if (nbuf == 0) return hipSuccess;
    uint8_t* dst = ws + sizeof(w4::ChainHeader) + (size_t)(emitted - nbuf) * sizeof(w4::ChainLinear);
    hipError_t err = hipMemcpyAsync(dst, buf, nbuf * sizeof(w4::ChainLinear), hipMemcpyHostToDevice, stream);
    if (err == hipSuccess) err = hipStreamSynchronize(stream);  // buf is reused
    nbuf = 0;
    return err;
  };
  int64_t items = 0;
  for (int64_t i = 0; i < count;) {
    int64_t e = i;
    while (e < count && linears[e].stage == linears[i].stage) ++e;
    // distinct K values of the stage, longest first; linears of equal K in order
    for (int64_t kcur = INT64_MAX;;) {
      int64_t knext = 0;
      for (int64_t j = i; j < e; ++j)
        if (linears[j].K < kcur) knext = std::max(knext, (int64_t)linears[j].K);
      if (knext == 0) break;
      kcur = knext;
      for (int64_t src = i; src < e; ++src) {
        const Desc& l = linears[src];
        if (l.K != kcur) continue;
        w4::ChainLinear& c = buf[nbuf++];
        memset(&c, 0, sizeof(c));
        c.desc = w4::LinearDesc{l.x, l.q_packed, l.d_packed, l.y, (int)M, (int)l.K, (int)l.N, 0};
        c.item0 = (int)items;
        c.stage = (int)l.stage;
        c.wait_x = reads_earlier(src);
        c.fill = read_later(src);
        const int64_t nb = (l.N + 15) / 16;
        items += (nb + R - 1) / R;
        if (items > 0x7FFFFFFF) return W4_ERR_SHAPE;
        ++emitted;
        if (nbuf == kChunk)
          if (hipError_t err = flush()) return hip_status(err);
      }
    }
    i = e;
  }
  {
    // the sentinel entry (the first item past the last linear), then the
    // header: the error flag starts clear
    w4::ChainLinear& c = buf[nbuf++];
    memset(&c, 0, sizeof(c));
    c.item0 = (int)items;
    c.stage = stages;
    ++emitted;
    if (hipError_t err = flush()) return hip_status(err);
    w4::ChainHeader h;
    memset(&h, 0, sizeof(h));
    if (hipError_t err = hipMemcpyAsync(ws, &h, sizeof(h), hipMemcpyHostToDevice, stream)) return hip_status(err);
    if (hipError_t err = hipStreamSynchronize(stream)) return hip_status(err);
  }

  if (blocks > items) blocks = items;

  plan->workspace = workspace;
  plan->linears = (int32_t)count;
  plan->stages = stages;
  plan->items = (int32_t)items;
  plan->blocks = (int32_t)blocks;
  plan->config = ci;
  plan->lds_bytes = (int32_t)lds;
  plan->rows_per_item = R;
  plan->waves_per_block = NW;
  plan->scale_bytes = s16 ? 2 : 4;
  plan->rows = (int32_t)M;
  plan->trace = 0;
  plan->reserved = 0;
  return W4_OK;
}
}  // namespace
}  // extern "C++"

}  // extern "C"

// ---------------------------------------------------------------------------
// chained pass set up in the library's own device memory
// ---------------------------------------------------------------------------
// The workspace of w4_chain_prepare_noalloc.  Each GPU the library runs on
// holds its own copy from the module's load until the process ends.  In host
// code `scratch` names a host-side stand-in, not a device address: the device
// address of a GPU's copy comes from hipGetSymbolAddress, looked up once per
// device (with that device current) and kept in g_scratch_addr.
static __device__ __align__(256) uint8_t scratch[W4_CHAIN_SCRATCH_BYTES];
static_assert(W4_CHAIN_SCRATCH_BYTES >= 32 + 2 * 64, "room for a chain of one linear");

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// Device address of the current device's scratch (looked up on first use).
w4_status scratch_address(void** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return W4_ERR_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return hip_status(e);
    if (!p) return hip_status(hipErrorInvalidSymbol);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return W4_OK;
}
}  // namespace

extern "C" {

w4_status w4_chain_prepare_noalloc(const w4_chain_linear* linears, int64_t count, w4_chain_plan* plan,
                                   hipStream_t stream) {
  if (count < 1 || count > W4_CHAIN_MAX) return W4_ERR_ARG;
  if (!linears || !plan) return W4_ERR_NULL;
  if (w4::chain_workspace_bytes(count) > W4_CHAIN_SCRATCH_BYTES) return W4_ERR_SCRATCH;
  void* ws = nullptr;
  if (w4_status st = scratch_address(&ws)) return st;
  return chain_prepare(linears, count, ws, W4_CHAIN_SCRATCH_BYTES, plan, false, W4_ERR_SCRATCH, stream);
}

size_t w4_chain_workspace_bytes(int64_t count) {
  if (count < 1 || count > W4_CHAIN_MAX) return 0;
  return w4::chain_workspace_bytes(count);
}

w4_status w4_chain_prepare(const w4_chain_linear* linears, int64_t count, void* workspace, size_t workspace_bytes,
                           w4_chain_plan* plan, hipStream_t stream) {
  return chain_prepare(linears, count, workspace, workspace_bytes, plan, false, W4_ERR_ARG, stream);
}

w4_status w4_chain_prepare_s16(const w4_chain_linear_s16* linears, int64_t count, void* workspace,
                               size_t workspace_bytes, w4_chain_plan* plan, hipStream_t stream) {
  return chain_prepare(linears, count, workspace, workspace_bytes, plan, true, W4_ERR_ARG, stream);
}

w4_status w4_chain_run(const w4_chain_plan* plan, hipStream_t stream) {
  if (!plan || !plan->workspace) return W4_ERR_NULL;
  if (plan->config < 0 || plan->config >= w4::chain_num_cfgs() || plan->blocks < 0) return W4_ERR_ARG;
  if (plan->scale_bytes != 2 && plan->scale_bytes != 4) return W4_ERR_ARG;
  if (plan->rows < 1 || plan->rows > 16 || w4::chain_cfg_mfma(plan->config) != (plan->rows > 1)) return W4_ERR_ARG;
  if (plan->blocks == 0) return W4_OK;
  return hip_status(w4::launch_linear_chain(plan->workspace, plan->linears, plan->items, plan->config,
                                            plan->scale_bytes == 2, plan->blocks, (size_t)plan->lds_bytes,
                                            plan->rows, plan->trace != 0, stream));
}

w4_status w4_chain_trace(w4_chain_plan* plan, uint64_t* stamps, size_t count, hipStream_t stream) {
  if (!plan || !plan->workspace) return W4_ERR_NULL;
  if (plan->items < 0) return W4_ERR_ARG;
  if (stamps && !aligned(stamps, 8)) return W4_ERR_ALIGN;
  if (stamps && count < 3 * (size_t)plan->items) return W4_ERR_ARG;
  uint8_t* field = static_cast<uint8_t*>(plan->workspace) + offsetof(w4::ChainHeader, stamps);
  if (hipError_t e = hipMemcpyAsync(field, &stamps, sizeof(stamps), hipMemcpyHostToDevice, stream)) return hip_status(e);
  if (hipError_t e = hipStreamSynchronize(stream)) return hip_status(e);
  plan->trace = stamps != nullptr;
  return W4_OK;
}

w4_status w4_chain_error(const w4_chain_plan* plan, uint32_t* flag, hipStream_t stream) {
  if (!plan || !plan->workspace || !flag) return W4_ERR_NULL;
  uint32_t v = 0;
  if (hipError_t e = hipMemcpyAsync(&v, plan->workspace, sizeof(v), hipMemcpyDeviceToHost, stream)) return hip_status(e);
  if (hipError_t e = hipStreamSynchronize(stream)) return hip_status(e);
  *flag = v;
  return W4_OK;
}

}  // extern "C"
