// Offline weight folds, and the runtime products that use the folded weights.
//
// Fused output weight ("DeepSeek-V3 MLA: Multi-Head Latent Attention Guide",
// Matrix Absorption Trick section 3): the output projection W^O acts on the
// heads' u_h = W^UV_h o_h concatenated in head order, so it can absorb the
// per-head up-projections offline:
//   W~^O = W^O blockdiag(W^UV_1, ..., W^UV_H)        [d_out x H d_c]
//   y_m  = W~^O [o_{m,1}; ...; o_{m,H}]
// Fused query weight ("Deconstructing DeepSeek V4 Pro", Practical
// Deployment): the per-head query projection W_in[h] (d_nope x d_in) and
// W^UK_h^T multiply into one weight, so the absorbed query comes straight
// from the projection's input x:
//   W~_Q[h] = (W^UK_h)^T W_in[h]                      [d_c x d_in]
//   q_cat[m, h] = [W~_Q[h] x_m ; q^R_{m,h}]
//
// Folds (any supported dims, float32 or bf16) and the portable runtime path
// share one batched VALU GEMM with general element strides: one batch per
// head, 64 x 64 output tile per workgroup, 16-deep contraction steps staged
// through LDS as float32, every thread a 4 x 4 block, float32 accumulation in
// contraction order, one rounding to the output type.
//
// Matrix-core runtime path (bf16 weights): Y = X W^T with W [N x K]
// contiguous along K.  Workgroup (column tile, row block, k-split) multiplies
// 64 columns by 64 rows over its share of K; its four waves take alternate
// 64-element chunks of that share and add their four 32 x 32 accumulators
// through LDS in a fixed order.  Every MFMA operand is one 16-byte load (two
// for a float32 X) straight from memory: the weight streams from HBM once per
// row block, X is re-read from L2 by every column tile.  A float32 X (the
// latent attention output) enters the bf16 MFMAs as hi + lo with hi, lo in
// bf16, so its rounding error is that of about 16 mantissa bits.  With one
// split the workgroup writes the bf16 result; with several it writes a float32
// partial, and a second kernel adds the partials in split order.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ strided VALU GEMM
struct GemmView {
  int64_t g, f, k;  // element strides: batch, free index, contraction index
};

// C[g](i, j) = sum_k A[g](i, k) B[g](k, j) with
//   A[g](i, k) = A[g * a.g + i * a.f + k * a.k],  B[g](k, j) = B[g * b.g + j * b.f + k * b.k],
//   C[g](i, j) = C[g * c.g + i * c.f + j * c.k]   (for C, .k is the stride of j).
constexpr int kT = 64;   // output tile edge
constexpr int kKT = 16;  // contraction depth per LDS stage
constexpr int kThreads = 256;

template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(kThreads) void gemm_strided(const TA* __restrict__ A, GemmView a,
                                                          const TB* __restrict__ Bm, GemmView b, TC* __restrict__ C,
                                                          GemmView c, int M, int N, int K) {
  __shared__ __align__(16) float As[kKT][kT];  // As[k][i]
  __shared__ __align__(16) float Bs[kKT][kT];  // Bs[k][j]
  const int64_t g = blockIdx.z;
  const int i0 = blockIdx.y * kT, j0 = blockIdx.x * kT, tid = threadIdx.x;
  const TA* Ag = A + g * a.g;
  const TB* Bg = Bm + g * b.g;
  const int ti = 4 * (tid >> 4), tj = 4 * (tid & 15);  // this thread's rows ti..ti+3, columns tj..tj+3
  // tile loads: element e = tid + 256 q of the 16 x 64 stage, the unit-stride
  // axis fastest so that neighbouring threads read neighbouring elements
  const bool a_kfast = a.k == 1, b_kfast = b.k == 1;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kKT) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + kThreads * q;
      const int ak = a_kfast ? (e & 15) : (e >> 6), ai = a_kfast ? (e >> 4) : (e & 63);
      const int bk = b_kfast ? (e & 15) : (e >> 6), bj = b_kfast ? (e >> 4) : (e & 63);
      const int gai = i0 + ai, gak = k0 + ak, gbj = j0 + bj, gbk = k0 + bk;
      As[ak][ai] = (gai < M && gak < K) ? Storage<TA>::load(Ag + gai * a.f + gak * a.k) : 0.f;
      Bs[bk][bj] = (gbj < N && gbk < K) ? Storage<TB>::load(Bg + gbj * b.f + gbk * b.k) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKT; ++kk) {
      const float4 av = *reinterpret_cast<const float4*>(&As[kk][ti]);
      const float4 bv = *reinterpret_cast<const float4*>(&Bs[kk][tj]);
      const float ar[4] = {av.x, av.y, av.z, av.w}, br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(ar[u], br[v], acc[u][v]);
    }
    __syncthreads();
  }
  TC* Cg = C + g * c.g;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ti + u;
    if (i >= M) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + tj + v;
      if (j < N) Storage<TC>::store(Cg + i * c.f + j * c.k, acc[u][v]);
    }
  }
}

// q_cat[m, h, d_c + t] = q_rope[m, h, t]: the RoPE part of the query passes through.
template <typename T>
__global__ __launch_bounds__(kThreads) void pass_rope(const T* __restrict__ q_rope, T* __restrict__ q_cat,
                                                       int64_t rows, int d_c, int d_r) {
  const int64_t total = rows * d_r;
  for (int64_t e = blockIdx.x * (int64_t)kThreads + threadIdx.x; e < total; e += (int64_t)gridDim.x * kThreads) {
    const int64_t r = e / d_r;
    q_cat[r * (d_c + d_r) + d_c + (e - r * d_r)] = q_rope[e];
  }
}

// ------------------------------------------------------------------ matrix-core linear
constexpr int kLChunk = 64;  // contraction elements per wave and chunk (four MFMA steps)
constexpr int kLTile = 64;   // output columns and rows per workgroup
constexpr int kLMaxKSplit = 16;

// Where output (m, n) goes: Y[m * ldy + (n / gs) * gstride + n % gs].  With
// tail != nullptr the tail's d_t values of (m, group) follow each group:
// Y[m * ldy + grp * gstride + gs + t] = tail[(m * groups + grp) * d_t + t].
struct LinearOut {
  uint16_t* y;
  int64_t ldy;
  int gs, gstride;
  const uint16_t* tail;
  int d_t, groups;
};

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2((uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16),
                    (uint32_t)f32_to_bf16_bits(c) | ((uint32_t)f32_to_bf16_bits(d) << 16));
}

// hi + lo split of eight floats (two 16-byte loads) into two bf16x8 operands
__device__ __forceinline__ void split_hilo(const uint4& p, const uint4& q, bf16x8& hi, bf16x8& lo) {
  const float x[8] = {__uint_as_float(p.x), __uint_as_float(p.y), __uint_as_float(p.z), __uint_as_float(p.w),
                      __uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z), __uint_as_float(q.w)};
  uint16_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = f32_to_bf16_bits(x[e]);
    l[e] = f32_to_bf16_bits(x[e] - bf16_bits_to_f32(h[e]));
  }
  const uint4 hu = make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16, h[4] | (uint32_t)h[5] << 16,
                              h[6] | (uint32_t)h[7] << 16);
  const uint4 lu = make_uint4(l[0] | (uint32_t)l[1] << 16, l[2] | (uint32_t)l[3] << 16, l[4] | (uint32_t)l[5] << 16,
                              l[6] | (uint32_t)l[7] << 16);
  hi = __builtin_bit_cast(bf16x8, hu);
  lo = __builtin_bit_cast(bf16x8, lu);
}

// One-dimensional grid of column tiles x row blocks x k-splits, split-major
// in the XCD-local order, so that the workgroups reading one split's slice of
// X mostly share an XCD and its L2.  MFMA step s of chunk c takes K elements
// 64 c + 16 s .. + 15; the lane with half hi = lane >> 5 supplies 8 hi .. 8 hi
// + 7 of them from its W row (A operand, output column n = lane & 31 of the
// column tile) and of its X row (B operand, output row m = lane & 31 of the
// row tile).
template <bool XF32>
__global__ __launch_bounds__(kThreads) void linear_mfma(const void* __restrict__ Xv, const uint16_t* __restrict__ W,
                                                        float* __restrict__ part, LinearOut out, int M, int N, int K,
                                                        int per, int ks) {
  __shared__ float4 red[kThreads / 64][16][64];  // [wave][4 tile + group][lane], 64 KiB
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5;
  const int ntiles = N / kLTile, per_split = ntiles * ((M + kLTile - 1) / kLTile);
  const int L = xcd_local_index(blockIdx.x, gridDim.x);
  const int ky = L / per_split, rest = L - ky * per_split;
  const int n0 = (rest % ntiles) * kLTile, mbase = (rest / ntiles) * kLTile;
  const int nch = K / kLChunk;
  const int c_hi = min(nch, (ky + 1) * per);

  const uint16_t* w0 = W + (size_t)(n0 + (lane & 31)) * K + 8 * hi;
  const uint16_t* w1 = w0 + (size_t)32 * K;
  const size_t xr0 = (size_t)min(mbase + (lane & 31), M - 1) * K + 8 * hi;
  const size_t xr1 = (size_t)min(mbase + 32 + (lane & 31), M - 1) * K + 8 * hi;
  constexpr int kXLoads = XF32 ? 2 : 1;  // 16-byte loads per X operand

  f32x16 acc[2][2] = {};  // [row tile][column tile]
  uint4 wa[2][4], xa[2][4 * kXLoads];
  auto load = [&](int c, uint4(&w)[2][4], uint4(&x)[2][4 * kXLoads]) {
    const size_t o = (size_t)c * kLChunk;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      w[0][s] = *reinterpret_cast<const uint4*>(w0 + o + 16 * s);
      w[1][s] = *reinterpret_cast<const uint4*>(w1 + o + 16 * s);
    }
    if constexpr (XF32) {
      const float* X = static_cast<const float*>(Xv);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        x[0][2 * s] = *reinterpret_cast<const uint4*>(X + xr0 + o + 16 * s);
        x[0][2 * s + 1] = *reinterpret_cast<const uint4*>(X + xr0 + o + 16 * s + 4);
        x[1][2 * s] = *reinterpret_cast<const uint4*>(X + xr1 + o + 16 * s);
        x[1][2 * s + 1] = *reinterpret_cast<const uint4*>(X + xr1 + o + 16 * s + 4);
      }
    } else {
      const uint16_t* X = static_cast<const uint16_t*>(Xv);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        x[0][s] = *reinterpret_cast<const uint4*>(X + xr0 + o + 16 * s);
        x[1][s] = *reinterpret_cast<const uint4*>(X + xr1 + o + 16 * s);
      }
    }
  };
  int c = ky * per + wave;
  if (c < c_hi) load(c, wa, xa);
  while (c < c_hi) {
    const int cn = c + kThreads / 64;
    uint4 wb[2][4], xb[2][4 * kXLoads];
    if (cn < c_hi) load(cn, wb, xb);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if constexpr (XF32) {
          bf16x8 xh, xl;
          split_hilo(xa[t][2 * s], xa[t][2 * s + 1], xh, xl);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bf16x8 wv = __builtin_bit_cast(bf16x8, wa[u][s]);
            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv, xh, acc[t][u], 0, 0, 0);
            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv, xl, acc[t][u], 0, 0, 0);
          }
        } else {
          const bf16x8 xv = __builtin_bit_cast(bf16x8, xa[t][s]);
#pragma unroll
          for (int u = 0; u < 2; ++u)
            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wa[u][s]), xv, acc[t][u],
                                                                0, 0, 0);
        }
      }
    }
    if (cn >= c_hi) break;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int s = 0; s < 4; ++s) wa[u][s] = wb[u][s];
#pragma unroll
      for (int s = 0; s < 4 * kXLoads; ++s) xa[u][s] = xb[u][s];
    }
    c = cn;
  }

  // accumulator element r of lane (m = lane & 31, hi) is output column
  // 8 (r >> 2) + 4 hi + (r & 3) of its column tile
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        red[wave][(2 * t + u) * 4 + g][lane] =
            make_float4(acc[t][u][4 * g], acc[t][u][4 * g + 1], acc[t][u][4 * g + 2], acc[t][u][4 * g + 3]);
  __syncthreads();
  // wave w adds up tile w: row tile w >> 1, column tile w & 1
  const int m = mbase + 32 * (wave >> 1) + (lane & 31);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int q = 4 * wave + g;
    float4 sum = red[0][q][lane];
#pragma unroll
    for (int v = 1; v < kThreads / 64; ++v) {
      const float4 x = red[v][q][lane];
      sum.x += x.x;
      sum.y += x.y;
      sum.z += x.z;
      sum.w += x.w;
    }
    const int n = n0 + 32 * (wave & 1) + 8 * g + 4 * hi;
    if (m >= M) continue;
    if (ks == 1) {
      const int grp = n / out.gs;
      *reinterpret_cast<uint2*>(out.y + m * out.ldy + (int64_t)grp * out.gstride + (n - grp * out.gs)) =
          pack_bf16x4(sum.x, sum.y, sum.z, sum.w);
    } else {
      *reinterpret_cast<float4*>(part + ((size_t)ky * M + m) * N + n) = sum;
    }
  }

  // the tail of each group starting in this column tile (split 0 only)
  if (out.tail != nullptr && ky == 0 && n0 % out.gs == 0) {
    const int grp = n0 / out.gs;
    for (int e = tid; e < kLTile * out.d_t; e += kThreads) {
      const int mm = mbase + e / out.d_t, t = e % out.d_t;
      if (mm < M) out.y[mm * out.ldy + (int64_t)grp * out.gstride + out.gs + t] =
          out.tail[((int64_t)mm * out.groups + grp) * out.d_t + t];
    }
  }
}

// grid (M, ceil(N / 4 / 256)): thread p of row m adds columns 4p..4p+3 over the splits in order.
__global__ __launch_bounds__(kThreads) void linear_finalize(const float* __restrict__ part, int ks, LinearOut out,
                                                            int M, int N) {
  const int m = blockIdx.x, p = blockIdx.y * kThreads + threadIdx.x;
  if (4 * p >= N) return;
  float4 v[kLMaxKSplit];
#pragma unroll
  for (int k = 0; k < kLMaxKSplit; ++k)
    if (k < ks) v[k] = *reinterpret_cast<const float4*>(part + ((size_t)k * M + m) * N + 4 * p);
  float4 s = v[0];
#pragma unroll
  for (int k = 1; k < kLMaxKSplit; ++k)
    if (k < ks) {
      s.x += v[k].x;
      s.y += v[k].y;
      s.z += v[k].z;
      s.w += v[k].w;
    }
  const int n = 4 * p, grp = n / out.gs;
  *reinterpret_cast<uint2*>(out.y + m * out.ldy + (int64_t)grp * out.gstride + (n - grp * out.gs)) =
      pack_bf16x4(s.x, s.y, s.z, s.w);
}

template <typename TA, typename TB, typename TC>
hipError_t gemm(const TA* A, GemmView a, const TB* Bm, GemmView b, TC* C, GemmView c, int M, int N, int K, int batch,
                hipStream_t stream) {
  const dim3 grid((N + kT - 1) / kT, (M + kT - 1) / kT, batch);
  hipLaunchKernelGGL((gemm_strided<TA, TB, TC>), grid, dim3(kThreads), 0, stream, A, a, Bm, b, C, c, M, N, K);
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ host side

int linear_max_ksplit() { return kLMaxKSplit; }

// Split count for the matrix-core linear: as many splits as keep the grid
// within two workgroups per compute unit (at least one, at most
// kLMaxKSplit and max_ks, no empty split).
int linear_ksplit(int M, int N, int K, int cus, int max_ks, int* per_out) {
  const int64_t tiles = (int64_t)(N / kLTile) * ((M + kLTile - 1) / kLTile);
  const int nch = K / kLChunk;
  int64_t ks = (2 * (int64_t)cus) / tiles;
  if (ks < 1) ks = 1;
  if (ks > kLMaxKSplit) ks = kLMaxKSplit;
  if (ks > max_ks) ks = max_ks;
  if (ks > nch) ks = nch;
  const int per = (int)((nch + ks - 1) / ks);
  *per_out = per;
  return (nch + per - 1) / per;
}

bool fused_query_mfma_supported(const mla_dims& d, int d_in) {
  return d.dtype == MLA_BF16 && d_in % kLChunk == 0 && d.d_c % kLTile == 0;
}

bool fused_output_mfma_supported(const mla_dims& d, int d_out) {
  return d.dtype == MLA_BF16 && ((int64_t)d.num_heads * d.d_c) % kLChunk == 0 && d_out % kLTile == 0;
}

hipError_t launch_fold_query(const mla_dims& d, int d_in, const void* w_in, const void* w_uk, void* w_fused,
                             hipStream_t stream) {
  // C[h](c, i) = sum_n w_uk[h, n, c] w_in[h, n, i]
  const GemmView a{(int64_t)d.d_nope * d.d_c, 1, d.d_c};
  const GemmView b{(int64_t)d.d_nope * d_in, 1, d_in};
  const GemmView c{(int64_t)d.d_c * d_in, d_in, 1};
  if (d.dtype == MLA_BF16)
    return gemm(static_cast<const uint16_t*>(w_uk), a, static_cast<const uint16_t*>(w_in), b,
                static_cast<uint16_t*>(w_fused), c, d.d_c, d_in, d.d_nope, d.num_heads, stream);
  return gemm(static_cast<const float*>(w_uk), a, static_cast<const float*>(w_in), b, static_cast<float*>(w_fused), c,
              d.d_c, d_in, d.d_nope, d.num_heads, stream);
}

hipError_t launch_fold_output(const mla_dims& d, int d_out, const void* w_o, const void* w_uv, void* w_fused,
                              hipStream_t stream) {
  // C[h](r, c) = sum_v w_o[r, h d_v + v] w_uv[h, v, c], stored at w_fused[r, h d_c + c]
  const int64_t Hdv = (int64_t)d.num_heads * d.d_v, Hdc = (int64_t)d.num_heads * d.d_c;
  const GemmView a{d.d_v, Hdv, 1};
  const GemmView b{(int64_t)d.d_v * d.d_c, 1, d.d_c};
  const GemmView c{d.d_c, Hdc, 1};
  if (d.dtype == MLA_BF16)
    return gemm(static_cast<const uint16_t*>(w_o), a, static_cast<const uint16_t*>(w_uv), b,
                static_cast<uint16_t*>(w_fused), c, d_out, d.d_c, d.d_v, d.num_heads, stream);
  return gemm(static_cast<const float*>(w_o), a, static_cast<const float*>(w_uv), b, static_cast<float*>(w_fused), c,
              d_out, d.d_c, d.d_v, d.num_heads, stream);
}

hipError_t launch_fused_query(const mla_dims& d, int d_in, int cus, const void* x, const void* q_rope,
                              const void* w_fused, void* q_cat, bool mfma, hipStream_t stream) {
  const int M = d.batch * d.q_len, D = d.d_c + d.d_rope;
  if (mfma) {
    const int N = d.num_heads * d.d_c;
    int per = 0;
    const int ks = linear_ksplit(M, N, d_in, cus, 1, &per);
    const LinearOut out{static_cast<uint16_t*>(q_cat), (int64_t)d.num_heads * D, d.d_c, D,
                        d.d_rope > 0 ? static_cast<const uint16_t*>(q_rope) : nullptr, d.d_rope, d.num_heads};
    const int blocks = (N / kLTile) * ((M + kLTile - 1) / kLTile) * ks;
    hipLaunchKernelGGL(linear_mfma<false>, dim3(blocks), dim3(kThreads), 0, stream, x,
                       static_cast<const uint16_t*>(w_fused), nullptr, out, M, N, d_in, per, ks);
    return hipGetLastError();
  }
  // C[h](m, c) = sum_i x[m, i] w_fused[h, c, i], stored at q_cat[m, h, c]
  const GemmView a{0, d_in, 1};
  const GemmView b{(int64_t)d.d_c * d_in, d_in, 1};
  const GemmView c{D, (int64_t)d.num_heads * D, 1};
  hipError_t e;
  const int64_t rows = (int64_t)M * d.num_heads;
  if (d.dtype == MLA_BF16) {
    e = gemm(static_cast<const uint16_t*>(x), a, static_cast<const uint16_t*>(w_fused), b,
             static_cast<uint16_t*>(q_cat), c, M, d.d_c, d_in, d.num_heads, stream);
    if (e == hipSuccess && d.d_rope > 0)
      hipLaunchKernelGGL(pass_rope<uint16_t>, dim3(256), dim3(kThreads), 0, stream,
                         static_cast<const uint16_t*>(q_rope), static_cast<uint16_t*>(q_cat), rows, d.d_c, d.d_rope);
  } else {
    e = gemm(static_cast<const float*>(x), a, static_cast<const float*>(w_fused), b, static_cast<float*>(q_cat), c, M,
             d.d_c, d_in, d.num_heads, stream);
    if (e == hipSuccess && d.d_rope > 0)
      hipLaunchKernelGGL(pass_rope<float>, dim3(256), dim3(kThreads), 0, stream, static_cast<const float*>(q_rope),
                         static_cast<float*>(q_cat), rows, d.d_c, d.d_rope);
  }
  return e == hipSuccess ? hipGetLastError() : e;
}

hipError_t launch_fused_output(const mla_dims& d, int d_out, int cus, const float* o, const void* w_fused, void* y,
                               float* ws, bool mfma, hipStream_t stream) {
  const int M = d.batch * d.q_len, K = d.num_heads * d.d_c;
  if (mfma) {
    int per = 0;
    const int ks = linear_ksplit(M, d_out, K, cus, kLMaxKSplit, &per);
    const LinearOut out{static_cast<uint16_t*>(y), d_out, d_out, 0, nullptr, 0, 1};
    const int blocks = (d_out / kLTile) * ((M + kLTile - 1) / kLTile) * ks;
    hipLaunchKernelGGL(linear_mfma<true>, dim3(blocks), dim3(kThreads), 0, stream, o,
                       static_cast<const uint16_t*>(w_fused), ws, out, M, d_out, K, per, ks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ks == 1) return e;
    hipLaunchKernelGGL(linear_finalize, dim3(M, (d_out / 4 + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                       ws, ks, out, M, d_out);
    return hipGetLastError();
  }
  // y(m, r) = sum_k o[m, k] w_fused[r, k]
  const GemmView a{0, K, 1};
  const GemmView b{0, K, 1};
  const GemmView c{0, d_out, 1};
  if (d.dtype == MLA_BF16)
    return gemm(o, a, static_cast<const uint16_t*>(w_fused), b, static_cast<uint16_t*>(y), c, M, d_out, K, 1, stream);
  return gemm(o, a, static_cast<const float*>(w_fused), b, static_cast<float*>(y), c, M, d_out, K, 1, stream);
}

}  // namespace mla
