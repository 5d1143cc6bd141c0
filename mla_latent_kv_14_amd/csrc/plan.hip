// Device-side work planner for split-KV decode.
//
// One workgroup turns the per-sequence lengths into a cost-balanced
// schedule: sequences are cut into 64-token tiles, each non-empty sequence is
// preceded by ov overhead tiles (the fixed cost of a piece: its queries and
// its partial result), everything is laid end to end on one line, and
// workgroup w of the attention kernel takes line tiles [w*chunk, (w+1)*chunk).
// A workgroup's range may span several sequences and a sequence may span
// several workgroups; each (sequence, workgroup) piece with real tiles is one
// split.  chunk is the smallest value that (a) fits the whole line in the
// launched grid, (b) keeps every sequence within num_splits pieces and (c) is
// at least the kernel's minimum useful range.
#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 256;

__device__ __forceinline__ int block_reduce_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = 0;
  for (int i = 0; i < kPlanThreads / 64; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ int block_reduce_max(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = red[0];
  for (int i = 1; i < kPlanThreads / 64; ++i) t = max(t, red[i]);
  return t;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seq_lens, int B, int q_len,
                                                            int max_len, int splits, int grid, int min_chunk, int ov,
                                                            int32_t* __restrict__ ws) {
  __shared__ int red[kPlanThreads / 64];
  __shared__ int scan[kPlanThreads];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0x7fffffff;
  __syncthreads();
  int32_t* cu = ws + kWsHeader;
  int32_t* len = ws + kWsHeader + B + 1;

  int local_sum = 0, local_max = 0, local_empty = 0;
  for (int b = threadIdx.x; b < B; b += kPlanThreads) {
    int L = seq_lens[b];
    if (L < q_len || L > max_len) atomicMin(&bad, b);
    L = min(max(L, 0), max_len);
    len[b] = L;
    const int n = (L + kPlanTile - 1) / kPlanTile;
    local_sum += n + (n > 0 ? ov : 0);
    local_max = max(local_max, n);
    local_empty += (L == 0);
  }
  const int total = block_reduce_sum(local_sum, red);
  const int maxn = block_reduce_max(local_max, red);
  const int empty = block_reduce_sum(local_empty, red);

  int chunk, groups;
  if (splits == 1) {
    chunk = 0;  // one whole sequence per workgroup step
    groups = min(B, grid);
  } else {
    chunk = max((total + grid - 1) / grid, min_chunk);
    if (maxn > 1) chunk = max(chunk, (maxn - 1 + splits - 2) / (splits - 1));
    chunk = max(chunk, 1);
    groups = (total + chunk - 1) / chunk;
  }

  // exclusive prefix sum of tiles, one window of kPlanThreads sequences at a time
  int offset = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int b = base + threadIdx.x;
    int n = (b < B) ? (len[b] + kPlanTile - 1) / kPlanTile : 0;
    n += (n > 0) ? ov : 0;
    __syncthreads();
    scan[threadIdx.x] = n;
    __syncthreads();
    for (int d = 1; d < kPlanThreads; d <<= 1) {
      const int add = (threadIdx.x >= d) ? scan[threadIdx.x - d] : 0;
      __syncthreads();
      scan[threadIdx.x] += add;
      __syncthreads();
    }
    if (b < B) cu[b] = offset + scan[threadIdx.x] - n;
    offset += scan[kPlanThreads - 1];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    cu[B] = offset;
    ws[0] = chunk;
    ws[1] = groups;
    ws[2] = total;
    ws[3] = maxn;
    ws[4] = splits;
    ws[5] = (bad == 0x7fffffff) ? 0 : bad + 1;
    ws[6] = B;
    ws[7] = empty;
    ws[8] = ov;
    for (int k = 9; k < kWsHeader; ++k) ws[k] = 0;
  }
}

}  // namespace

hipError_t launch_plan(const mla_dims& d, const int32_t* seq_lens, int splits, int grid, int min_chunk, int ov,
                       int32_t* ws, hipStream_t stream) {
  const int max_len = d.max_blocks_per_seq * d.block_size;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, d.batch, d.q_len, max_len,
                     splits, grid, min_chunk, ov, ws);
  return hipGetLastError();
}

}  // namespace mla
