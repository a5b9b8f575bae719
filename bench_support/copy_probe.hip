// Measurement helpers for bench.py only (built as libw4_bench.so, not part of
// the w4 C ABI): a plain 16-byte copy kernel of known size, used to calibrate
// the HBM byte counters read by rocprofv3, and a read-only streaming kernel
// (non-temporal 16-byte loads, grid-stride) that gives the
// bandwidth a plain sequential read reaches on this GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// 16-byte load with the streaming (non-temporal) policy the linear kernels use.
__device__ __forceinline__ v4u ld_nt(const uint4* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
}

__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                        uint32_t* __restrict__ sink) {
  // consecutive wavefronts read consecutive 1 KiB pieces (one 16-byte load per
  // lane per step): the friendliest order for the DRAM pages
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    const v4u a = ld_nt(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // one value per thread keeps the loads live; the sink is tiny
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) on `stream`.
int w4bench_copy(const void* src, void* dst, int64_t bytes, int grid, hipStream_t stream) {
  if (!src || !dst || bytes < 0 || (bytes & 15) || grid <= 0) return 1;
  copy_kernel<<<grid, kThreads, 0, stream>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads `bytes` (a multiple of 16) on `stream`; `sink` needs `grid` uint32.
int w4bench_read(const void* src, int64_t bytes, uint32_t* sink, int grid, hipStream_t stream) {
  if (!src || !sink || bytes < 0 || (bytes & 15) || grid <= 0) return 1;
  read_kernel<<<grid, kThreads, 0, stream>>>(static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
