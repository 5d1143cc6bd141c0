// The device-side work planner of split-KV decode, as a device function: run
// by one whole 256-thread workgroup, either in its own launch (plan.hip) or as
// an extra workgroup of the absorb_q launch (absorb_mfma.hip).
//
// It turns the per-sequence lengths into a cost-balanced schedule: sequences
// are cut into 64-token tiles, each non-empty sequence is preceded by ov
// overhead tiles (the fixed cost of a piece: its queries and its partial
// result), everything is laid end to end on one line, and workgroup w of the
// attention kernel takes line tiles [w*chunk, (w+1)*chunk).  A workgroup's
// range may span several sequences and a sequence may span several
// workgroups; each (sequence, workgroup) piece with real tiles is one split.
// chunk is the smallest value that (a) fits the whole line in the launched
// grid, (b) keeps every sequence within num_splits pieces and (c) is at least
// the kernel's minimum useful range.
#pragma once
#include "common.h"

namespace mla {

constexpr int kPlanThreads = 256;

// With head groups (hg_log2 > 0), d counts groups: B = batch << hg_log2
// scheduled sequences, entry b taking the length of sequence b >> hg_log2.
struct PlanArgs {
  const int32_t* seq_lens;
  int32_t* ws;
  int B, q_len, max_len, splits, grid, min_chunk, ov, hg_log2;
};

inline PlanArgs make_plan_args(const mla_dims& d, const int32_t* seq_lens, int splits, int grid, int min_chunk,
                               int ov, int32_t* ws, int hg_log2) {
  return PlanArgs{seq_lens, ws,  d.batch, d.q_len, d.max_blocks_per_seq * d.block_size, splits, grid, min_chunk, ov,
                  hg_log2};
}

struct PlanShared {
  int red[kPlanThreads / 64];
  int scan[kPlanThreads];
  int bad;
};

__device__ __forceinline__ int plan_reduce_sum(int v, int* red) {
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

__device__ __forceinline__ int plan_reduce_max(int v, int* red) {
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

__device__ __forceinline__ void plan_body(const PlanArgs& pa, PlanShared& sh) {
  const int B = pa.B;
  int32_t* ws = pa.ws;
  if (threadIdx.x == 0) sh.bad = 0x7fffffff;
  __syncthreads();
  int32_t* cu = ws + kWsCu;
  int32_t* len = ws + kWsCu + B + 1;

  int local_sum = 0, local_max = 0, local_empty = 0;
  for (int b = threadIdx.x; b < B; b += kPlanThreads) {
    int L = pa.seq_lens[b >> pa.hg_log2];
    if (L < pa.q_len || L > pa.max_len) atomicMin(&sh.bad, b >> pa.hg_log2);
    L = min(max(L, 0), pa.max_len);
    len[b] = L;
    const int n = (L + kPlanTile - 1) / kPlanTile;
    local_sum += n + (n > 0 ? pa.ov : 0);
    local_max = max(local_max, n);
    local_empty += (L == 0);
  }
  const int total = plan_reduce_sum(local_sum, sh.red);
  const int maxn = plan_reduce_max(local_max, sh.red);
  const int empty = plan_reduce_sum(local_empty, sh.red);

  int chunk, groups;
  if (pa.splits == 1) {
    chunk = 0;  // one whole sequence per workgroup step
    groups = min(B, pa.grid);
  } else {
    chunk = max((total + pa.grid - 1) / pa.grid, pa.min_chunk);
    if (maxn > 1) chunk = max(chunk, (maxn - 1 + pa.splits - 2) / (pa.splits - 1));
    chunk = max(chunk, 1);
    groups = (total + chunk - 1) / chunk;
  }

  // exclusive prefix sum of tiles, one window of kPlanThreads sequences at a time
  int offset = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int b = base + threadIdx.x;
    int n = (b < B) ? (len[b] + kPlanTile - 1) / kPlanTile : 0;
    n += (n > 0) ? pa.ov : 0;
    __syncthreads();
    sh.scan[threadIdx.x] = n;
    __syncthreads();
    for (int d = 1; d < kPlanThreads; d <<= 1) {
      const int add = (threadIdx.x >= d) ? sh.scan[threadIdx.x - d] : 0;
      __syncthreads();
      sh.scan[threadIdx.x] += add;
      __syncthreads();
    }
    if (b < B) cu[b] = offset + sh.scan[threadIdx.x] - n;
    offset += sh.scan[kPlanThreads - 1];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    cu[B] = offset;
    ws[0] = chunk;
    ws[1] = groups;
    ws[2] = total;
    ws[3] = maxn;
    ws[4] = pa.splits;
    ws[5] = (sh.bad == 0x7fffffff) ? 0 : sh.bad + 1;
    ws[6] = B;
    ws[7] = empty;
    ws[8] = pa.ov;
    ws[9] = pa.hg_log2;
    for (int k = 10; k < kWsHeader; ++k) ws[k] = 0;
  }
  // each workgroup's first segment (chunked mode): the sequence that holds
  // line tile w * chunk, past any sequence that ends at or before it, with
  // its cu and length words
  __syncthreads();
  if (chunk > 0) {
    for (int w = threadIdx.x; w < min(groups, kFirstMax); w += kPlanThreads) {
      const int t = w * chunk;
      int b = (t < offset) ? find_sequence(cu, B, t) : B;
      while (b < B && cu[b + 1] <= t) ++b;
      int32_t* f = ws + kWsHeader + 4 * w;
      f[0] = b;
      f[1] = (b < B) ? cu[b] : 0;
      f[2] = (b < B) ? cu[b + 1] : 0;
      f[3] = (b < B) ? len[b] : 0;
    }
  }
}

}  // namespace mla
