// Measurement kernels for the benchmark (libmla_roofs.so, gfx950): a cache
// flush, a streaming HBM read, a register-only bf16 matrix-core loop and an
// empty kernel.  None of them is on the attention path.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "mla_roofs.h"

namespace {

constexpr int kReadThreads = 512;
constexpr int kReadPerCU = 4;   // resident workgroups per compute unit
constexpr int kReadUnroll = 4;  // 16-byte loads in flight per thread
constexpr int kMfmaThreads = 256;
constexpr int kMfmaPerCU = 2;   // two waves per SIMD

int cus_cached() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

bool al16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

__global__ __launch_bounds__(256) void flush_kernel(uint4* __restrict__ p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const uint4 v = make_uint4(0x9e3779b9u, 0x7f4a7c15u, 0x85ebca6bu, blockIdx.x);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                            uint32_t* __restrict__ sink) {
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0;
  __syncthreads();
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = ld16<NT>(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = ld16<NT>(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  atomicXor(&red, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(int iters, uint32_t* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(1.0f + 1e-3f * (float)((threadIdx.x + k) & 7));
    b[k] = (__bf16)(1.0f - 1e-3f * (float)((threadIdx.x * 3 + k) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kMfmaThreads / 64) + (threadIdx.x >> 6)] = __float_as_uint(s);
}

__global__ void empty_kernel() {}

int hip_status(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

int mla_roofs_flush(void* buf, size_t bytes, void* stream) {
  if (!al16(buf) || bytes == 0 || bytes % 16 != 0) return -1;
  const int cus = cus_cached();
  if (cus == 0) return -4;
  hipLaunchKernelGGL(flush_kernel, dim3(cus * 8), dim3(256), 0, (hipStream_t)stream, static_cast<uint4*>(buf),
                     bytes / 16);
  return hip_status(hipGetLastError());
}

int mla_roofs_read_grid(void) { return cus_cached() * kReadPerCU; }

int mla_roofs_hbm_read(const void* buf, size_t bytes, int32_t nontemporal, uint32_t* sink, size_t sink_words,
                       void* stream) {
  if (!al16(buf) || !al16(sink) || bytes == 0 || bytes % 16 != 0) return -1;
  const int grid = mla_roofs_read_grid();
  if (grid == 0) return -4;
  if (sink_words < (size_t)grid) return -1;
  const u32x4* p = static_cast<const u32x4*>(buf);
  if (nontemporal)
    hipLaunchKernelGGL(read_kernel<true>, dim3(grid), dim3(kReadThreads), 0, (hipStream_t)stream, p, bytes / 16, sink);
  else
    hipLaunchKernelGGL(read_kernel<false>, dim3(grid), dim3(kReadThreads), 0, (hipStream_t)stream, p, bytes / 16,
                       sink);
  return hip_status(hipGetLastError());
}

int mla_roofs_mfma_grid(void) { return cus_cached() * kMfmaPerCU; }

int mla_roofs_mfma_bf16(int32_t iters, uint32_t* sink, size_t sink_words, double* flops, void* stream) {
  if (iters < 1 || !al16(sink) || flops == nullptr) return -1;
  const int grid = mla_roofs_mfma_grid();
  if (grid == 0) return -4;
  if (sink_words < (size_t)grid * (kMfmaThreads / 64)) return -1;
  *flops = (double)grid * (kMfmaThreads / 64) * (double)iters * 4.0 * 32.0 * 32.0 * 16.0 * 2.0;
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(kMfmaThreads), 0, (hipStream_t)stream, iters, sink);
  return hip_status(hipGetLastError());
}

int mla_roofs_empty(void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hip_status(hipGetLastError());
}

}  // extern "C"
