// Cache append: the cache rows of the new tokens, written into the paged cache.
//
//   c_t  = W^DKV h_t           "DeepSeek-V3 MLA: Multi-Head Latent Attention
//   k^R_t = RoPE_t(W^KR h_t)   Guide", Core Architecture sections 1 (joint KV
//                              compression) and 3 (decoupled RoPE key)
//
// RoPE turns each pair (x[2p], x[2p+1]) of the d_rope-wide key by the angle
// theta_p = t / base^(2p / d_rope), t the token's position ("Deconstructing
// DeepSeek V4 Pro", the apply_rope helper of its MLA module).  Token j of
// sequence b has position t = seq_lens[b] - q_len + j (the lengths already
// count the new tokens) and goes to block block_table[b, t / bs], slot t % bs.
//
// Matrix-core path (bf16 storage, d_model a multiple of 128, d_c + d_rope a
// multiple of 32).  Y = H [W^DKV; W^KR]^T is (B Lq) x d_model times d_model x
// (d_c + d_rope): both output sides are short and the contraction is long, so
// it is split along d_model.  Workgroup (column tile, row block, k-split)
// multiplies 32 output columns by 64 rows over its share of d_model; its four
// waves take alternate 128-wide chunks of that share and add their results
// through LDS in a fixed order, and the sum goes to a float32 partial.  A
// second kernel adds the partials in split order, rotates the RoPE columns
// and scatters the rows.  Both operands are contiguous along d_model, so
// every MFMA operand is one 16-byte load straight from memory: the weights
// stream from HBM once and h is re-read from L2 by every column tile.
//
// The portable path (any supported dims, float32 or bf16) computes one
// output pair per thread with float32 VALU arithmetic.
//
// A token whose position or block id is out of range is skipped (nothing is
// written for it); the RoPE angle and its sine and cosine are evaluated in
// float64 so that positions near 2^30 keep their accuracy.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kChunk = 128;     // contraction elements per wave and chunk
constexpr int kColsTile = 32;   // output columns per workgroup
constexpr int kRowsBlock = 64;  // rows per workgroup (two 32-row MFMA tiles)
constexpr int kMaxKSplit = 16;

// Element offset of token m's cache row (m = b * Lq + j), or -1 when its
// position or block id is out of range; *pos receives its position.
__device__ __forceinline__ int64_t append_slot(const int32_t* table, const int32_t* seq_lens, int m, int Lq, int bs,
                                               int MB, int NB, int D, int* pos) {
  const int b = m / Lq, j = m - b * Lq;
  const int t = seq_lens[b] - Lq + j;
  *pos = t;
  if (t < 0 || t >= MB * bs) return -1;
  const int blk = table[(size_t)b * MB + t / bs];
  if (blk < 0 || blk >= NB) return -1;
  return ((int64_t)blk * bs + t % bs) * D;
}

// Store of a column pair into a cache of element type C: the storage type,
// or (uint8_t) E4M3 codes of x / kv_scale, saturating at +-448 (a NaN stays
// NaN), rounded to the nearest code with ties to the even one by the
// hardware conversion.
template <typename C> struct PairStore {
  __device__ __forceinline__ static void store(C* dst, float x0, float x1, float) {
    Storage<C>::store(dst, x0);
    Storage<C>::store(dst + 1, x1);
  }
};
template <> struct PairStore<uint8_t> {
  __device__ __forceinline__ static void store(uint8_t* dst, float x0, float x1, float kv_scale) {
    auto sat = [](float v) { return v != v ? v : fminf(fmaxf(v, -448.f), 448.f); };
    const float a0 = sat(x0 / kv_scale), a1 = sat(x1 / kv_scale);
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);  // a0 in byte 0, a1 in byte 1
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(w & 0xffff);
  }
};

// Rotate (x0, x1) if column n lies in the RoPE part, then store the pair.
template <typename C>
__device__ __forceinline__ void store_pair(C* dst, int n, int d_c, int d_r, int pos, double base, float x0, float x1,
                                           float kv_scale) {
  if (n >= d_c) {
    const int p = (n - d_c) >> 1;
    const double theta = (double)pos / pow(base, 2.0 * p / d_r);
    double s, c;
    sincos(theta, &s, &c);
    const double y0 = (double)x0 * c - (double)x1 * s;
    const double y1 = (double)x1 * c + (double)x0 * s;
    x0 = (float)y0;
    x1 = (float)y1;
  }
  PairStore<C>::store(dst + n, x0, x1, kv_scale);
}

// ------------------------------------------------------------------ MFMA GEMM
// One-dimensional grid of column tiles x row blocks x k-splits, split-major
// in the XCD-local order, so that the workgroups of one split (which read the
// same slice of h) mostly share an XCD and its L2.  partial[ky][m][n] float32.
// Chunk c covers d_model elements [128 c, 128 c + 128); MFMA step s of a
// chunk takes its elements 16 s .. 16 s + 15, the lane with half hi = lane >>
// 5 supplying 16 s + 8 hi .. + 7 of its W row (A operand, output column n =
// lane & 31) and of its h row (B operand, output row m = lane & 31).
__global__ __launch_bounds__(kThreads) void append_gemm_mfma(const uint16_t* __restrict__ h,
                                                             const uint16_t* __restrict__ w_dkv,
                                                             const uint16_t* __restrict__ w_kr,
                                                             float* __restrict__ part, int M, int K, int d_c, int D,
                                                             int per) {
  __shared__ float4 red[kThreads / 64][8][64];  // [wave][4 tile + group][lane], 32 KiB
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5;
  const int ntiles = D / kColsTile, per_split = ntiles * ((M + kRowsBlock - 1) / kRowsBlock);
  const int L = xcd_local_index(blockIdx.x, gridDim.x);
  const int ky = L / per_split, rest = L - ky * per_split;
  const int n0 = (rest % ntiles) * kColsTile, mbase = (rest / ntiles) * kRowsBlock;
  const int nch = K / kChunk;
  const int c_hi = min(nch, (ky + 1) * per);

  const int n = n0 + (lane & 31);
  const uint16_t* wrow = (n < d_c ? w_dkv + (size_t)n * K : w_kr + (size_t)(n - d_c) * K) + 8 * hi;
  const uint16_t* hrow0 = h + (size_t)min(mbase + (lane & 31), M - 1) * K + 8 * hi;
  const uint16_t* hrow1 = h + (size_t)min(mbase + 32 + (lane & 31), M - 1) * K + 8 * hi;

  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
  uint4 wa[8], ha0[8], ha1[8];
  auto load = [&](int c, uint4(&w)[8], uint4(&a0)[8], uint4(&a1)[8]) {
    const size_t o = (size_t)c * kChunk;
#pragma unroll
    for (int s = 0; s < 8; ++s) w[s] = *reinterpret_cast<const uint4*>(wrow + o + 16 * s);
#pragma unroll
    for (int s = 0; s < 8; ++s) a0[s] = *reinterpret_cast<const uint4*>(hrow0 + o + 16 * s);
#pragma unroll
    for (int s = 0; s < 8; ++s) a1[s] = *reinterpret_cast<const uint4*>(hrow1 + o + 16 * s);
  };
  int c = ky * per + wave;
  if (c < c_hi) load(c, wa, ha0, ha1);
  while (c < c_hi) {
    const int cn = c + kThreads / 64;
    uint4 wb[8], hb0[8], hb1[8];
    if (cn < c_hi) load(cn, wb, hb0, hb1);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, wa[s]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, ha0[s]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, ha1[s]), acc1, 0, 0, 0);
    }
    if (cn >= c_hi) break;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      wa[s] = wb[s];
      ha0[s] = hb0[s];
      ha1[s] = hb1[s];
    }
    c = cn;
  }

  // accumulator element r of lane (m = lane & 31, hi) is output column
  // n0 + 8 (r >> 2) + 4 hi + (r & 3) of row tile 0 / 1
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    red[wave][g][lane] = make_float4(acc0[4 * g], acc0[4 * g + 1], acc0[4 * g + 2], acc0[4 * g + 3]);
    red[wave][4 + g][lane] = make_float4(acc1[4 * g], acc1[4 * g + 1], acc1[4 * g + 2], acc1[4 * g + 3]);
  }
  __syncthreads();
#pragma unroll
  for (int q = 2 * wave; q < 2 * wave + 2; ++q) {
    float4 sum = red[0][q][lane];
#pragma unroll
    for (int v = 1; v < kThreads / 64; ++v) {
      const float4 x = red[v][q][lane];
      sum.x += x.x;
      sum.y += x.y;
      sum.z += x.z;
      sum.w += x.w;
    }
    const int t = q >> 2, g = q & 3;
    const int m = mbase + 32 * t + (lane & 31);
    if (m < M) *reinterpret_cast<float4*>(part + ((size_t)ky * M + m) * D + n0 + 8 * g + 4 * hi) = sum;
  }
}

// One workgroup per token: add the k-split partials in split order, rotate,
// store.  Every partial is requested before the first addition (at most
// kMaxKSplit of them) and before the token's slot is looked up, so those
// latencies overlap.
template <typename C>
__global__ __launch_bounds__(576) void append_finalize(const float* __restrict__ part, int KS,
                                                       const int32_t* __restrict__ table,
                                                       const int32_t* __restrict__ seq_lens, C* __restrict__ cache,
                                                       int M, int Lq, int bs, int MB, int NB, int d_c, int d_r,
                                                       double base, float kv_scale) {
  const int m = blockIdx.x, D = d_c + d_r;
  const int p = threadIdx.x;  // one column pair per thread
  float2 v[kMaxKSplit];
  if (p < D / 2) {
#pragma unroll
    for (int k = 0; k < kMaxKSplit; ++k)
      if (k < KS) v[k] = *reinterpret_cast<const float2*>(part + ((size_t)k * M + m) * D + 2 * p);
  }
  int pos = 0;
  const int64_t off = append_slot(table, seq_lens, m, Lq, bs, MB, NB, D, &pos);
  if (off < 0 || p >= D / 2) return;
  float x0 = 0.f, x1 = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxKSplit; ++k)
    if (k < KS) {
      x0 += v[k].x;
      x1 += v[k].y;
    }
  store_pair(cache + off, 2 * p, d_c, d_r, pos, base, x0, x1, kv_scale);
}

// ------------------------------------------------------------------ portable
// grid (M, ceil(D / 2 / 256)): thread p of token m computes columns 2p, 2p+1.
template <typename T, typename C>
__global__ __launch_bounds__(kThreads) void append_generic(const T* __restrict__ h, const T* __restrict__ w_dkv,
                                                           const T* __restrict__ w_kr,
                                                           const int32_t* __restrict__ table,
                                                           const int32_t* __restrict__ seq_lens, C* __restrict__ cache,
                                                           int K, int Lq, int bs, int MB, int NB, int d_c, int d_r,
                                                           double base, float kv_scale) {
  const int m = blockIdx.x, D = d_c + d_r;
  const int p = blockIdx.y * blockDim.x + threadIdx.x;
  if (p >= D / 2) return;
  int pos = 0;
  const int64_t off = append_slot(table, seq_lens, m, Lq, bs, MB, NB, D, &pos);
  if (off < 0) return;
  const int n = 2 * p;  // d_c is even, so n and n + 1 lie in the same weight
  const T* w0 = n < d_c ? w_dkv + (size_t)n * K : w_kr + (size_t)(n - d_c) * K;
  const T* w1 = w0 + K;
  const T* hr = h + (size_t)m * K;
  float a0[4] = {0.f, 0.f, 0.f, 0.f}, a1[4] = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 4 <= K; k += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x = Storage<T>::load(hr + k + u);
      a0[u] = fmaf(x, Storage<T>::load(w0 + k + u), a0[u]);
      a1[u] = fmaf(x, Storage<T>::load(w1 + k + u), a1[u]);
    }
  }
  for (int u = 0; k < K; ++k, ++u) {
    const float x = Storage<T>::load(hr + k);
    a0[u] = fmaf(x, Storage<T>::load(w0 + k), a0[u]);
    a1[u] = fmaf(x, Storage<T>::load(w1 + k), a1[u]);
  }
  const float x0 = (a0[0] + a0[1]) + (a0[2] + a0[3]);
  const float x1 = (a1[0] + a1[1]) + (a1[2] + a1[3]);
  store_pair(cache + off, n, d_c, d_r, pos, base, x0, x1, kv_scale);
}

}  // namespace

bool append_mfma_supported(const mla_dims& d, int d_model) {
  return d.dtype == MLA_BF16 && d_model % kChunk == 0 && (d.d_c + d.d_rope) % kColsTile == 0;
}

int append_max_ksplit() { return kMaxKSplit; }

// Split count for the matrix-core path: about one workgroup per compute unit,
// no empty split, at most kMaxKSplit.
int append_ksplit(const mla_dims& d, int d_model, int cus, int* per_out) {
  const int M = d.batch * d.q_len, D = d.d_c + d.d_rope;
  const int64_t tiles = (int64_t)(D / kColsTile) * ((M + kRowsBlock - 1) / kRowsBlock);
  const int nch = d_model / kChunk;
  int64_t ks = (cus + tiles / 2) / tiles;
  if (ks < 1) ks = 1;
  if (ks > kMaxKSplit) ks = kMaxKSplit;
  if (ks > nch) ks = nch;
  const int per = (int)((nch + ks - 1) / ks);
  *per_out = per;
  return (nch + per - 1) / per;
}

hipError_t launch_append_mfma(const mla_dims& d, int d_model, int cus, const void* h, const void* w_dkv,
                              const void* w_kr, float rope_base, const int32_t* table, const int32_t* seq_lens,
                              void* cache, float* part, hipStream_t stream, bool fp8, float kv_scale) {
  const int M = d.batch * d.q_len, D = d.d_c + d.d_rope;
  int per = 0;
  const int ks = append_ksplit(d, d_model, cus, &per);
  const int blocks = (D / kColsTile) * ((M + kRowsBlock - 1) / kRowsBlock) * ks;
  hipLaunchKernelGGL(append_gemm_mfma, dim3(blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_dkv),
                     static_cast<const uint16_t*>(w_kr), part, M, d_model, d.d_c, D, per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int fin_threads = ((D / 2 + 63) / 64) * 64;  // D <= 1088, so at most 576
  if (fp8)
    hipLaunchKernelGGL(append_finalize<uint8_t>, dim3(M), dim3(fin_threads), 0, stream, part, ks, table, seq_lens,
                       static_cast<uint8_t*>(cache), M, d.q_len, d.block_size, d.max_blocks_per_seq, d.num_blocks,
                       d.d_c, d.d_rope, (double)rope_base, kv_scale);
  else
    hipLaunchKernelGGL(append_finalize<uint16_t>, dim3(M), dim3(fin_threads), 0, stream, part, ks, table, seq_lens,
                       static_cast<uint16_t*>(cache), M, d.q_len, d.block_size, d.max_blocks_per_seq, d.num_blocks,
                       d.d_c, d.d_rope, (double)rope_base, 1.f);
  return hipGetLastError();
}

hipError_t launch_append_generic(const mla_dims& d, int d_model, const void* h, const void* w_dkv, const void* w_kr,
                                 float rope_base, const int32_t* table, const int32_t* seq_lens, void* cache,
                                 hipStream_t stream, bool fp8, float kv_scale) {
  const int M = d.batch * d.q_len, pairs = (d.d_c + d.d_rope) / 2;
  const dim3 grid(M, (pairs + kThreads - 1) / kThreads);
  auto go = [&](auto hp, auto cp) {
    using T = std::remove_cv_t<std::remove_pointer_t<decltype(hp)>>;
    using C = std::remove_pointer_t<decltype(cp)>;
    hipLaunchKernelGGL((append_generic<T, C>), grid, dim3(kThreads), 0, stream, hp, static_cast<const T*>(w_dkv),
                       static_cast<const T*>(w_kr), table, seq_lens, cp, d_model, d.q_len, d.block_size,
                       d.max_blocks_per_seq, d.num_blocks, d.d_c, d.d_rope, (double)rope_base, kv_scale);
  };
  if (d.dtype == MLA_BF16) {
    if (fp8) go(static_cast<const uint16_t*>(h), static_cast<uint8_t*>(cache));
    else go(static_cast<const uint16_t*>(h), static_cast<uint16_t*>(cache));
  } else {
    if (fp8) go(static_cast<const float*>(h), static_cast<uint8_t*>(cache));
    else go(static_cast<const float*>(h), static_cast<float*>(cache));
  }
  return hipGetLastError();
}

}  // namespace mla
