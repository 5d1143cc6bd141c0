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
  int red[kPlanThreads / 64][3];
  int wsum[kPlanThreads / 64];
  int bad;
  // with B <= kPlanThreads: the prefix sums and lengths, so that the
  // first-segment searches read LDS instead of waiting on global memory
  int cu[kPlanThreads + 1];
  int len[kPlanThreads];
};

// Sum of a, maximum of b and sum of c over the workgroup, with one pair of
// barriers (integer arithmetic: the order does not matter).
__device__ __forceinline__ void plan_reduce3(int& a, int& b, int& c, int (*red)[3]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b = max(b, __shfl_xor(b, off, 64));
    c += __shfl_xor(c, off, 64);
  }
  __syncthreads();
  if (lane == 0) {
    red[wave][0] = a;
    red[wave][1] = b;
    red[wave][2] = c;
  }
  __syncthreads();
  a = red[0][0];
  b = red[0][1];
  c = red[0][2];
  for (int i = 1; i < kPlanThreads / 64; ++i) {
    a += red[i][0];
    b = max(b, red[i][1]);
    c += red[i][2];
  }
}

__device__ __forceinline__ void plan_body(const PlanArgs& pa, PlanShared& sh) {
  const int B = pa.B;
  int32_t* ws = pa.ws;
  if (threadIdx.x == 0) sh.bad = 0x7fffffff;
  __syncthreads();
  int32_t* cu = ws + kWsCu;
  int32_t* len = ws + kWsCu + B + 1;

  const bool small = B <= kPlanThreads;  // one sequence per thread: everything stays on chip
  int local_sum = 0, local_max = 0, local_empty = 0, mine = 0;
  for (int b = threadIdx.x; b < B; b += kPlanThreads) {
    int L = pa.seq_lens[b >> pa.hg_log2];
    if (L < pa.q_len || L > pa.max_len) atomicMin(&sh.bad, b >> pa.hg_log2);
    L = min(max(L, 0), pa.max_len);
    len[b] = L;
    mine = L;
    if (small) sh.len[b] = L;
    const int n = (L + kPlanTile - 1) / kPlanTile;
    local_sum += n + (n > 0 ? pa.ov : 0);
    local_max = max(local_max, n);
    local_empty += (L == 0);
  }
  plan_reduce3(local_sum, local_max, local_empty, sh.red);
  const int total = local_sum, maxn = local_max, empty = local_empty;

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
    int n = (b < B) ? ((small ? mine : len[b]) + kPlanTile - 1) / kPlanTile : 0;
    n += (n > 0) ? pa.ov : 0;
    // inclusive scan within the wave by shuffles, then the waves' totals
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int v = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(v, d, 64);
      if (lane >= d) v += y;
    }
    __syncthreads();  // the previous window's totals have been read
    if (lane == 63) sh.wsum[wave] = v;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) {
      before += (i < wave) ? sh.wsum[i] : 0;
      all += sh.wsum[i];
    }
    if (b < B) {
      cu[b] = offset + before + v - n;
      if (small) sh.cu[b] = offset + before + v - n;
    }
    offset += all;
  }
  if (small && threadIdx.x == 0) sh.cu[B] = offset;
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
    const int32_t* cs = small ? sh.cu : cu;
    const int32_t* ls = small ? sh.len : len;
    for (int w = threadIdx.x; w < min(groups, kFirstMax); w += kPlanThreads) {
      const int t = w * chunk;
      int b = (t < offset) ? find_sequence(cs, B, t) : B;
      while (b < B && cs[b + 1] <= t) ++b;
      int32_t* f = ws + kWsHeader + 4 * w;
      f[0] = b;
      f[1] = (b < B) ? cs[b] : 0;
      f[2] = (b < B) ? cs[b + 1] : 0;
      f[3] = (b < B) ? ls[b] : 0;
    }
  }
}

}  // namespace mla
