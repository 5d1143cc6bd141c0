// Shared definitions for the libmla HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// Planning granularity: the schedule hands out whole 64-token tiles of a
// sequence.  A workgroup's token range therefore starts at a multiple of 64
// within its sequence and ends at a multiple of 64 or at the sequence end.
constexpr int kPlanTile = 64;

// Workspace layout written by the planner (int32 words):
//   [0] chunk   tiles per workgroup (>= 1), or 0 in one-sequence-per-workgroup mode
//   [1] groups  number of workgroups that have work (<= launched grid)
//   [2] total   length of the schedule line in tiles (real plus overhead tiles)
//   [3] maxn    tiles of the longest sequence
//   [4] splits  S as passed by the caller
//   [5] error   0, or 1 + index of the first sequence whose length was out of range
//   [6] batch   B
//   [7] empty   number of sequences with no tokens
//   [8] ov      overhead tiles charged at the start of every non-empty sequence
//   [9] hg_log2 head groups (the schedule's B counts groups, see DecodeArgs)
//   [10 .. 15]  reserved (0)
//   [16 .. 16+4F)     first: for workgroup w < F = kFirstMax (chunked mode), the
//                     sequence of its first segment and that sequence's cu[b],
//                     cu[b+1] and len[b], so that a workgroup starts without
//                     searching cu (one round of loads instead of log2 B + 2)
//   [C .. C+B]        cu: start of each sequence on the schedule line (B + 1
//                     words), C = kWsCu = 16 + 4F
//   [C+B+1 .. C+2B+1) len: per-sequence length, clamped to [0, MB * block_size]
// On the schedule line sequence b occupies [cu[b], cu[b+1]): first ov
// overhead tiles that hold no tokens (they stand for the fixed cost of
// starting a piece of a sequence: loading its queries, writing its partial
// result), then its n_b real tiles.  A sequence with no tokens occupies
// nothing.  Workgroup w owns the line range [w*chunk, (w+1)*chunk), so that
// cost rather than token count is balanced across workgroups.
constexpr int kWsHeader = 16;
constexpr int kFirstMax = 1024;
constexpr int kWsCu = kWsHeader + 4 * kFirstMax;
inline size_t workspace_words(int batch) { return (size_t)kWsCu + 2 * (size_t)batch + 1; }

struct DecodeArgs {
  const void* q_cat;
  const void* cache;
  const int32_t* block_table;
  const int32_t* ws;  // planner output
  void* o_part;  // [B,Lq,H,S,d_c] in the storage type
  float* lse_part;
  float scale;
  int32_t B, Lq, H, d_c, d_rope, block_size, max_blocks, num_blocks, splits;
  float kv_scale;  // FP8 cache: a stored code stands for kv_scale * its value (1 otherwise)
  // Head groups: with q_len = 1 the heads of a sequence may be split into
  // 2^hg_log2 groups, each scheduled as a sequence of its own (B, H above
  // then count groups and heads per group; q_cat and the partial results
  // keep their layout).  Group b reads the block table of sequence
  // b >> hg_log2.
  int32_t hg_log2;
};

// ---- float <-> storage conversions -------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Storage;
template <> struct Storage<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Storage<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

// ---- wave64 reductions ---------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Log-sum-exp of one row's split values lp[0..S) (natural log; -inf entries
// are empty splits): every lane of an aligned group of 8 lanes returns the
// same value; j is the lane's index in its group.  The summation order is
// fixed (eight strided partial sums combined by a butterfly; float addition
// is commutative, so all eight lanes agree), which makes every kernel that
// merges splits produce bit-identical weights exp(lse_s - lse).
// Order of the merge o = sum_s w_s o_s, fixed so that every merge kernel
// rounds alike.  Token rows are taken in tiles of 32 (m0 = m - m % 32, rows =
// min(32, M - m0) of them); a tile of `rows` rows has P = 2^merge_groups_log2
// groups per row (32 / P >= rows).  Split s lies in block s / kMergeBlock, and
// block b in group b mod P.  Group p's sum C_p takes its splits in increasing
// s, each by one fma (w_s o_s + C_p) starting from +0; then o = C_0 + C_1 +
// ... + C_{P-1}, added left to right.  With P = 1 it is one sequential fma
// chain over all splits.
constexpr int kMergeBlock = 8;
__host__ __device__ __forceinline__ int merge_groups_log2(int rows) {
  int lg = 0;
  while (lg < 5 && (32 >> (lg + 1)) >= rows) ++lg;
  return lg;
}

// log sum_s exp(lp[s]) over the S splits of one row, by 8 lanes (lane j of
// the 8 takes s = j, j + 8, ...); `first` is the lane's lp[j] (-inf if j >= S),
// loaded by the caller, so that the first load can be issued ahead of others.
__device__ __forceinline__ float split_lse_first(float first, const float* lp, int S, int j) {
  float mx = fmaxf(-INFINITY, first);
  for (int s = j + 8; s < S; s += 8) mx = fmaxf(mx, lp[s]);
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (mx == -INFINITY) return -INFINITY;
  float z = 0.f;
  if (j < S) z += expf(first - mx);
  for (int s = j + 8; s < S; s += 8) z += expf(lp[s] - mx);
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) z += __shfl_xor(z, off, 64);
  return mx + logf(z);
}
// The same with the lane's second value lp[j + 8] (-inf if j + 8 >= S) also
// loaded by the caller: the same maximum and the same sum, in the same order.
__device__ __forceinline__ float split_lse_first2(float first, float second, const float* lp, int S, int j) {
  float mx = fmaxf(fmaxf(-INFINITY, first), second);
  for (int s = j + 16; s < S; s += 8) mx = fmaxf(mx, lp[s]);
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (mx == -INFINITY) return -INFINITY;
  float z = 0.f;
  if (j < S) z += expf(first - mx);
  if (j + 8 < S) z += expf(second - mx);
  for (int s = j + 16; s < S; s += 8) z += expf(lp[s] - mx);
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) z += __shfl_xor(z, off, 64);
  return mx + logf(z);
}
__device__ __forceinline__ float split_lse(const float* lp, int S, int j) {
  return split_lse_first(j < S ? lp[j] : -INFINITY, lp, S, j);
}

// ---- schedule lookups shared by every decode kernel ----------------------------------

// Largest b in [0, B) with cu[b] <= tile (cu is non-decreasing, cu[0] = 0).
__device__ __forceinline__ int find_sequence(const int32_t* cu, int B, int tile) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One contiguous piece of one sequence handled by one workgroup.
struct Segment {
  int b;          // sequence
  int tok_begin;  // first token (inclusive)
  int tok_end;    // last token + 1 (clamped to the sequence length)
  int split;      // index of this piece among the sequence's pieces
  int nsplits;    // pieces the sequence is divided into
};

// Iterates the segments of workgroup w under the planner's schedule.
struct SegmentWalker {
  const int32_t* ws;
  int B, w, chunk, groups, total, ov;
  int b;         // current sequence
  int t_begin;   // workgroup's first line tile, t_end its end (chunked mode)
  int t_end;
  int pre_b, pre_c0, pre_c1, pre_len;  // the planner's first segment: b, cu[b], cu[b + 1], len[b]

  __device__ __forceinline__ void init(const int32_t* ws_, int w_) {
    ws = ws_;
    w = w_;
    // the first-segment words sit at a fixed offset, so they are requested
    // together with the header words rather than after them
    const bool has_first = w < kFirstMax;
    int f0 = 0, f1 = 0, f2 = 0, f3 = 0;
    if (has_first) {
      const int32_t* f = ws + kWsHeader + 4 * w;
      f0 = f[0];
      f1 = f[1];
      f2 = f[2];
      f3 = f[3];
    }
    chunk = ws[0];
    groups = ws[1];
    total = ws[2];
    B = ws[6];
    ov = ws[8];
    pre_b = -1;
    if (chunk > 0) {
      t_begin = w * chunk;
      t_end = min(t_begin + chunk, total);
      if (has_first) {
        pre_b = f0;
        pre_c0 = f1;
        pre_c1 = f2;
        pre_len = f3;
        b = pre_b;
      } else {
        b = (t_begin < total) ? find_sequence(ws + kWsCu, B, t_begin) : B;
      }
    } else {
      b = w;  // one whole sequence per step, stride = groups
    }
  }

  // Returns false when the workgroup has no more work.
  __device__ __forceinline__ bool next(Segment& s) {
    const int32_t* cu = ws + kWsCu;
    const int32_t* len = ws + kWsCu + B + 1;
    if (chunk > 0) {
      int c0, c1, lb;
      if (b == pre_b) {
        // the planner's first segment: empty sequences already skipped
        c0 = pre_c0;
        c1 = pre_c1;
        lb = pre_len;
      } else {
        // skip sequences that end before the range (empty ones included)
        while (b < B && cu[b + 1] <= t_begin) ++b;
        c0 = (b < B) ? cu[b] : 0;
        c1 = (b < B) ? cu[b + 1] : 0;
        lb = (b < B) ? len[b] : 0;
      }
      if (b >= B || t_begin >= t_end) return false;
      const int rs = c0 + ov;  // first real tile of b (b is not empty here)
      if (rs >= t_end) return false;
      const int lo = max(t_begin, rs), hi = min(t_end, c1);
      s.b = b;
      s.tok_begin = (lo - rs) * kPlanTile;
      s.tok_end = min((hi - rs) * kPlanTile, lb);
      const int first = rs / chunk;
      s.split = w - first;
      s.nsplits = (c1 - 1) / chunk - first + 1;
      t_begin = hi;
      ++b;
      return true;
    }
    if (b >= B) return false;
    s.b = b;
    s.tok_begin = 0;
    s.tok_end = len[b];
    s.split = 0;
    s.nsplits = 1;
    b += groups;
    return true;
  }
};

// Workgroups are dispatched to the eight XCDs of the chip in turn (workgroup p
// runs on XCD p mod 8).  Neighbouring ranges of the schedule usually share a
// sequence (its queries are read by both), so the schedule index is chosen to
// keep neighbours on one XCD and its L2: XCD x takes a contiguous block of
// schedule indices.
__device__ __forceinline__ int xcd_local_index(int p, int grid) {
  const int q = grid >> 3, r = grid & 7, x = p & 7, k = p >> 3;
  return (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// A sequence with no tokens is visited by no workgroup: workgroup 0 marks all
// of its splits empty.  Only runs when the planner counted such sequences;
// the threads of the workgroup split the (sequence, row) pairs between them.
__device__ __forceinline__ void mark_empty_sequences(const DecodeArgs& a, int tid, int nthreads) {
  if (a.ws[7] == 0) return;
  const int32_t* len = a.ws + kWsCu + a.B + 1;
  const int R = a.Lq * a.H;
  for (int i = tid; i < a.B * R; i += nthreads) {
    const int b = i / R;
    if (len[b] != 0) continue;
    float* lp = a.lse_part + (size_t)i * a.splits;
    for (int s = 0; s < a.splits; ++s) lp[s] = -INFINITY;
  }
}

}  // namespace mla
