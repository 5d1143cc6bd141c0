// Portable libmla kernels: plain float32 VALU arithmetic, any supported
// shape and either storage type.  They are the path for shapes the MFMA
// kernels do not cover (float32 storage, small widths, block sizes that are
// not a multiple of 32) and a second, independent HIP implementation of
// every step.  None of them is tuned.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerGroup = 16;  // absorb kernels: query rows per workgroup
constexpr int kMaxRow = 1088;      // d_c + d_rope upper bound
constexpr int kMaxCols = 1024;     // d_c, d_nope, d_v upper bound

// ---------------------------------------------------------------------------------------
// q_cat[m,h,:d_c] = sum_n q_nope[m,h,n] w_uk[h,n,:];  q_cat[m,h,d_c:] = q_rope[m,h,:]
// grid (H, ceil(M / 16)), M = B * Lq
template <typename T>
__global__ __launch_bounds__(kThreads) void absorb_q_generic(const T* __restrict__ q_nope,
                                                             const T* __restrict__ q_rope,
                                                             const T* __restrict__ w_uk, T* __restrict__ q_cat,
                                                             int M, int H, int d_n, int d_r, int d_c) {
  __shared__ float qs[kRowsPerGroup * kMaxCols];
  const int h = blockIdx.x, m0 = blockIdx.y * kRowsPerGroup;
  const int D = d_c + d_r;
  for (int i = threadIdx.x; i < kRowsPerGroup * d_n; i += kThreads) {
    const int r = i / d_n, n = i % d_n, m = m0 + r;
    qs[r * d_n + n] = (m < M) ? Storage<T>::load(q_nope + ((size_t)m * H + h) * d_n + n) : 0.f;
  }
  __syncthreads();
  const T* w = w_uk + (size_t)h * d_n * d_c;
  for (int c = threadIdx.x; c < d_c; c += kThreads) {
    float acc[kRowsPerGroup];
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) acc[r] = 0.f;
    for (int n = 0; n < d_n; ++n) {
      const float wv = Storage<T>::load(w + (size_t)n * d_c + c);
#pragma unroll
      for (int r = 0; r < kRowsPerGroup; ++r) acc[r] = fmaf(qs[r * d_n + n], wv, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r)
      if (m0 + r < M) Storage<T>::store(q_cat + ((size_t)(m0 + r) * H + h) * D + c, acc[r]);
  }
  for (int i = threadIdx.x; i < kRowsPerGroup * d_r; i += kThreads) {
    const int r = i / d_r, k = i % d_r, m = m0 + r;
    if (m < M) q_cat[((size_t)m * H + h) * D + d_c + k] = q_rope[((size_t)m * H + h) * d_r + k];
  }
}

// ---------------------------------------------------------------------------------------
// u[m,h,v] = sum_c w_uv[h,v,c] o[m,h,c];  grid (H, ceil(M / 16))
template <typename T>
__global__ __launch_bounds__(kThreads) void absorb_out_generic(const float* __restrict__ o,
                                                               const T* __restrict__ w_uv, T* __restrict__ out,
                                                               int M, int H, int d_c, int d_v) {
  __shared__ float os[kRowsPerGroup * kMaxCols];
  const int h = blockIdx.x, m0 = blockIdx.y * kRowsPerGroup;
  for (int i = threadIdx.x; i < kRowsPerGroup * d_c; i += kThreads) {
    const int r = i / d_c, c = i % d_c, m = m0 + r;
    os[r * d_c + c] = (m < M) ? o[((size_t)m * H + h) * d_c + c] : 0.f;
  }
  __syncthreads();
  for (int v = threadIdx.x; v < d_v; v += kThreads) {
    const T* w = w_uv + ((size_t)h * d_v + v) * d_c;
    float acc[kRowsPerGroup];
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) acc[r] = 0.f;
    for (int c = 0; c < d_c; ++c) {
      const float wv = Storage<T>::load(w + c);
#pragma unroll
      for (int r = 0; r < kRowsPerGroup; ++r) acc[r] = fmaf(os[r * d_c + c], wv, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r)
      if (m0 + r < M) Storage<T>::store(out + ((size_t)(m0 + r) * H + h) * d_v + v, acc[r]);
  }
}

// ---------------------------------------------------------------------------------------
// Cache element loads: the storage type, or (uint8_t) an E4M3 code decoded by
// the hardware conversion (exact in float32).
template <typename C> struct CacheLoad {
  __device__ __forceinline__ static float load(const C* p) { return Storage<C>::load(p); }
};
template <> struct CacheLoad<uint8_t> {
  __device__ __forceinline__ static float load(const uint8_t* p) { return __builtin_amdgcn_cvt_f32_fp8((int)*p, 0); }
};

// Split-KV decode, one wave per query row (j, h).  grid (groups launched, ceil(Lq*H / 4)).
// Scores: lane = token.  Weighted sum: lane = latent column.  T is the storage
// type of q_cat, C that of the cache (T, or uint8_t for an FP8 cache whose
// codes stand for kv_scale times their value).
template <typename T, typename C>
__global__ __launch_bounds__(kThreads) void decode_generic(DecodeArgs a) {
  constexpr bool kF8 = std::is_same<C, uint8_t>::value;
  __shared__ float qs[kThreads / 64][kMaxRow];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int R = a.Lq * a.H;
  const int row = blockIdx.y * (kThreads / 64) + wave;
  const bool active = row < R;
  const int j = active ? row / a.H : 0, h = active ? row % a.H : 0;
  const int D = a.d_c + a.d_rope;
  const int S = a.splits;
  const T* qc = (const T*)a.q_cat;
  const C* cache = (const C*)a.cache;
  const float kv = kF8 ? a.kv_scale : 1.f;
  const int32_t* len = a.ws + kWsCu + a.B + 1;
  // a schedule planned for another batch (or head grouping) is never walked
  if (a.ws[6] != a.B) return;

  if (blockIdx.x == 0 && blockIdx.y == 0) mark_empty_sequences(a, threadIdx.x, blockDim.x);
  SegmentWalker walk;
  walk.init(a.ws, blockIdx.x);
  if ((int)blockIdx.x >= walk.groups) return;  // uniform over the workgroup
  Segment seg;
  while (walk.next(seg)) {
    const int b = seg.b;
    __syncthreads();
    if (active) {
      const T* qrow = qc + ((size_t)(b * a.Lq + j) * a.H + h) * D;
      for (int k = lane; k < D; k += 64) qs[wave][k] = Storage<T>::load(qrow + k);
    }
    __syncthreads();
    if (!active) continue;

    const int last = len[b] - a.Lq + j;  // query j sees tokens <= last
    const int t_end = min(seg.tok_end, last + 1);
    float m = -INFINITY, l = 0.f;
    float acc[kMaxCols / 64];
#pragma unroll
    for (int i = 0; i < kMaxCols / 64; ++i) acc[i] = 0.f;

    for (int t0 = seg.tok_begin; t0 < t_end; t0 += 64) {
      const int t = t0 + lane;
      const bool valid = t < t_end;
      size_t off = 0;
      float s = -INFINITY;
      if (valid) {
        int blk = a.block_table[(size_t)(b >> a.hg_log2) * a.max_blocks + t / a.block_size];
        blk = min(max(blk, 0), a.num_blocks - 1);
        off = ((size_t)blk * a.block_size + t % a.block_size) * D;
        float dot = 0.f;
        for (int k = 0; k < D; ++k) dot = fmaf(qs[wave][k], CacheLoad<C>::load(cache + off + k), dot);
        s = dot * a.scale;
        if (kF8) s *= kv;
      }
      const float m_new = fmaxf(m, wave_max(s));
      const float alpha = expf(m - m_new);
      const float p = valid ? expf(s - m_new) : 0.f;
      l = l * alpha + wave_sum(p);
#pragma unroll
      for (int i = 0; i < kMaxCols / 64; ++i) acc[i] *= alpha;
      const int nvalid = min(64, t_end - t0);
      for (int u = 0; u < nvalid; ++u) {
        const float pu = __shfl(p, u, 64);
        const unsigned lo = __shfl((unsigned)(off & 0xffffffffu), u, 64);
        const unsigned hi = __shfl((unsigned)(off >> 32), u, 64);
        const C* rp = cache + (((size_t)hi << 32) | lo);
#pragma unroll
        for (int i = 0; i < kMaxCols / 64; ++i) {
          const int c = lane + 64 * i;
          if (c < a.d_c) acc[i] = fmaf(pu, CacheLoad<C>::load(rp + c), acc[i]);
        }
      }
      m = m_new;
    }

    const size_t prow = ((size_t)(b * a.Lq + j) * a.H + h) * S;
    if (t_end > seg.tok_begin) {
      const float inv = kF8 ? kv / l : 1.f / l;
      T* op = static_cast<T*>(a.o_part) + (prow + seg.split) * a.d_c;  // partials in the storage type
#pragma unroll
      for (int i = 0; i < kMaxCols / 64; ++i) {
        const int c = lane + 64 * i;
        if (c < a.d_c) Storage<T>::store(op + c, acc[i] * inv);
      }
      if (lane == 0) a.lse_part[prow + seg.split] = m + logf(l);
    } else if (lane == 0) {
      a.lse_part[prow + seg.split] = -INFINITY;
    }
    if (seg.split == 0)
      for (int s2 = seg.nsplits + lane; s2 < S; s2 += 64) a.lse_part[prow + s2] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// lse = log sum_s exp(lse_s); o = sum_s exp(lse_s - lse) o_s.  One wave per row.
// The partials o_s are in the storage type T; four consecutive columns are
// read at a time.
template <typename T> struct Four;
template <> struct Four<float> {
  __device__ __forceinline__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <> struct Four<uint16_t> {
  __device__ __forceinline__ static float4 load(const uint16_t* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                       __uint_as_float(v.y & 0xffff0000u));
  }
};

// One wave per (token row m, head h) row: lane c owns float4 columns c, c +
// 64, ...; the splits are added in the order merge_order fixes (common.h).
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(const T* __restrict__ o_part,
                                                           const float* __restrict__ lse_part, float* __restrict__ o,
                                                           float* __restrict__ lse, int M, int H, int S, int d_c) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + wave;
  if (row >= M * H) return;
  const int m = row / H;
  const int lgP = merge_groups_log2(min(32, M - (m - m % 32))), P = 1 << lgP;
  const float* lp = lse_part + (size_t)row * S;
  const float total = split_lse(lp, S, lane & 7);
  float4* o4 = reinterpret_cast<float4*>(o + (size_t)row * d_c);
  const int n4 = d_c / 4;
  const T* src = o_part + (size_t)row * S * d_c;
  for (int c = lane; c < n4; c += 64) {
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = 0; p < P; ++p) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int blk = p; blk * kMergeBlock < S; blk += P) {
        const int s_end = min(S, (blk + 1) * kMergeBlock);
        for (int s = blk * kMergeBlock; s < s_end; ++s) {
          const float ls = lp[s];
          if (ls == -INFINITY) continue;
          const float w = expf(ls - total);
          if (w == 0.f) continue;
          const float4 v = Four<T>::load(src + (size_t)s * d_c + 4 * c);
          acc.x = fmaf(w, v.x, acc.x);
          acc.y = fmaf(w, v.y, acc.y);
          acc.z = fmaf(w, v.z, acc.z);
          acc.w = fmaf(w, v.w, acc.w);
        }
      }
      if (p == 0) {
        sum = acc;
      } else {
        sum.x += acc.x;
        sum.y += acc.y;
        sum.z += acc.z;
        sum.w += acc.w;
      }
    }
    o4[c] = sum;
  }
  if (lse && lane == 0) lse[row] = total;
}

}  // namespace

int decode_generic_rows_per_group() { return kThreads / 64; }

hipError_t launch_absorb_q_generic(const mla_dims& d, const void* q_nope, const void* q_rope, const void* w_uk,
                                   void* q_cat, hipStream_t stream) {
  const int M = d.batch * d.q_len;
  dim3 grid(d.num_heads, (M + kRowsPerGroup - 1) / kRowsPerGroup);
  if (d.dtype == MLA_F32)
    hipLaunchKernelGGL(absorb_q_generic<float>, grid, dim3(kThreads), 0, stream, (const float*)q_nope,
                       (const float*)q_rope, (const float*)w_uk, (float*)q_cat, M, d.num_heads, d.d_nope, d.d_rope,
                       d.d_c);
  else
    hipLaunchKernelGGL(absorb_q_generic<uint16_t>, grid, dim3(kThreads), 0, stream, (const uint16_t*)q_nope,
                       (const uint16_t*)q_rope, (const uint16_t*)w_uk, (uint16_t*)q_cat, M, d.num_heads, d.d_nope,
                       d.d_rope, d.d_c);
  return hipGetLastError();
}

hipError_t launch_absorb_out_generic(const mla_dims& d, const float* o, const void* w_uv, void* out,
                                     hipStream_t stream) {
  const int M = d.batch * d.q_len;
  dim3 grid(d.num_heads, (M + kRowsPerGroup - 1) / kRowsPerGroup);
  if (d.dtype == MLA_F32)
    hipLaunchKernelGGL(absorb_out_generic<float>, grid, dim3(kThreads), 0, stream, o, (const float*)w_uv,
                       (float*)out, M, d.num_heads, d.d_c, d.d_v);
  else
    hipLaunchKernelGGL(absorb_out_generic<uint16_t>, grid, dim3(kThreads), 0, stream, o, (const uint16_t*)w_uv,
                       (uint16_t*)out, M, d.num_heads, d.d_c, d.d_v);
  return hipGetLastError();
}

hipError_t launch_decode_generic(const mla_dims& d, const void* q_cat, const void* cache, const int32_t* table,
                                 const int32_t* ws, float scale, int splits, int grid, void* o_part,
                                 float* lse_part, hipStream_t stream, bool fp8, float kv_scale) {
  DecodeArgs a{q_cat, cache, table, ws, o_part, lse_part, scale, d.batch, d.q_len, d.num_heads, d.d_c, d.d_rope,
               d.block_size, d.max_blocks_per_seq, d.num_blocks, splits, kv_scale, 0};
  const int R = d.q_len * d.num_heads;
  dim3 g(grid, (R + kThreads / 64 - 1) / (kThreads / 64));
  if (d.dtype == MLA_F32) {
    if (fp8) hipLaunchKernelGGL((decode_generic<float, uint8_t>), g, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((decode_generic<float, float>), g, dim3(kThreads), 0, stream, a);
  } else {
    if (fp8) hipLaunchKernelGGL((decode_generic<uint16_t, uint8_t>), g, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((decode_generic<uint16_t, uint16_t>), g, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const mla_dims& d, int splits, const void* o_part, const float* lse_part, float* o,
                          float* lse, hipStream_t stream) {
  const int rows = d.batch * d.q_len * d.num_heads;
  if (d.dtype == MLA_F32)
    hipLaunchKernelGGL(combine_kernel<float>, dim3((rows + 3) / 4), dim3(kThreads), 0, stream,
                       static_cast<const float*>(o_part), lse_part, o, lse, d.batch * d.q_len, d.num_heads, splits,
                       d.d_c);
  else
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3((rows + 3) / 4), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(o_part), lse_part, o, lse, d.batch * d.q_len, d.num_heads,
                       splits, d.d_c);
  return hipGetLastError();
}

}  // namespace mla
