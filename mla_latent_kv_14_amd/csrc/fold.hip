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
// contiguous along K and at most a few dozen rows of X, so the product is
// bound by streaming W from HBM.  Workgroup (column block, row block,
// k-split) owns 128 (query) or 256 (output) columns and 64 rows over its
// share of K; its four waves own disjoint columns.  X passes through LDS once
// per workgroup; W, stored in MFMA fragment order (below), goes straight from
// memory into the MFMA operands through a register ring of three (query) or
// four (output) chunks.  A float32 X (the latent attention output) enters
// the bf16 MFMAs as hi + lo with hi, lo in bf16, so its rounding error is that
// of about 16 mantissa bits.  With one split the workgroup writes the bf16
// result; with several it writes a float32 partial, and a second kernel adds
// the partials in split order.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ packed weight order
// A fused weight viewed as W [N x K] (N output columns, K the contraction) is
// stored, when the matrix-core path serves its shape, in MFMA fragment order:
// a [N/32][K/64][4][2][32][8] array over (32-row tile, 64-element chunk, MFMA
// step, half, row in tile, element), so that element (n, k) sits at
//   ((n/32) (K/64) + k/64) 2048 + (k%64)/16 512 + ((k%16)/8 32 + n%32) 8 + k%8
// and each operand load of a wave reads 1 KiB of contiguous memory.
__device__ __forceinline__ int64_t packed_offset(int64_t n, int64_t k, int64_t K) {
  return ((n >> 5) * (K >> 6) + (k >> 6)) * 2048 + ((k >> 4) & 3) * 512 + ((((k >> 3) & 1) << 5) + (n & 31)) * 8 +
         (k & 7);
}

// ------------------------------------------------------------------ strided VALU GEMM
struct GemmView {
  int64_t g, f, k;  // element strides: batch, free index, contraction index
};

// Packed addressing of an operand: its (n, k) in the packed weight are
// n = g ng + f nf + k nk and k = g kg + f kf + k kk (f the free index, k the
// contraction index of the operand, or for C the index j), K the packed
// weight's contraction length.
struct PackMap {
  int64_t ng, nf, nk, kg, kf, kk, K;
};

// C[g](i, j) = sum_k A[g](i, k) B[g](k, j) with
//   A[g](i, k) = A[g * a.g + i * a.f + k * a.k],  B[g](k, j) = B[g * b.g + j * b.f + k * b.k],
//   C[g](i, j) = C[g * c.g + i * c.f + j * c.k]   (for C, .k is the stride of j).
constexpr int kT = 64;   // output tile edge
constexpr int kKT = 16;  // contraction depth per LDS stage
constexpr int kThreads = 256;

template <typename TA, typename TB, typename TC, bool PB, bool PC>
__global__ __launch_bounds__(kThreads) void gemm_strided(const TA* __restrict__ A, GemmView a,
                                                          const TB* __restrict__ Bm, GemmView b, TC* __restrict__ C,
                                                          GemmView c, PackMap pb, PackMap pc, int M, int N, int K) {
  __shared__ __align__(16) float As[kKT][kT];  // As[k][i]
  __shared__ __align__(16) float Bs[kKT][kT];  // Bs[k][j]
  const int64_t g = blockIdx.z;
  const int i0 = blockIdx.y * kT, j0 = blockIdx.x * kT, tid = threadIdx.x;
  const TA* Ag = A + g * a.g;
  const TB* Bg = Bm + (PB ? 0 : g * b.g);
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
      int64_t bo;
      if constexpr (PB)
        bo = packed_offset(g * pb.ng + gbj * pb.nf + gbk * pb.nk, g * pb.kg + gbj * pb.kf + gbk * pb.kk, pb.K);
      else
        bo = gbj * b.f + gbk * b.k;
      Bs[bk][bj] = (gbj < N && gbk < K) ? Storage<TB>::load(Bg + bo) : 0.f;
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
  TC* Cg = C + (PC ? 0 : g * c.g);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ti + u;
    if (i >= M) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + tj + v;
      if (j >= N) continue;
      int64_t co;
      if constexpr (PC)
        co = packed_offset(g * pc.ng + i * pc.nf + j * pc.nk, g * pc.kg + i * pc.kf + j * pc.kk, pc.K);
      else
        co = i * c.f + j * c.k;
      Storage<TC>::store(Cg + co, acc[u][v]);
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
constexpr int kLChunk = 64;  // contraction elements per chunk (four MFMA steps)
constexpr int kLRows = 64;   // rows per workgroup (two 32-row MFMA tiles)
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

// Two floats to a pair of bf16 (low half: a), by the hardware conversion
// (round to nearest even).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2 w = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(w, bf16x2));
}

// hi + lo split of eight floats into two 16-byte groups of bf16:
// hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split_hilo(const uint4& p, const uint4& q, uint4& hi, uint4& lo) {
  const uint32_t in[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x0 = __uint_as_float(in[2 * e]), x1 = __uint_as_float(in[2 * e + 1]);
    h[e] = pk_bf16(x0, x1);
    l[e] = pk_bf16(x0 - __uint_as_float(h[e] << 16), x1 - __uint_as_float(h[e] & 0xffff0000u));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Columns per workgroup: four waves, each owning CT 32-column MFMA tiles.
template <int CT> constexpr int linear_block() { return 4 * 32 * CT; }

// step(R, c + R) for R = 0, 1, ... while R < RING and c + R < c_hi, with R a
// compile-time constant (so that register-ring slots are static).
template <int R, int RING, typename F>
__device__ __forceinline__ void ring_steps(F& step, int c, int c_hi) {
  if constexpr (R < RING) {
    if (c + R < c_hi) {
      step(std::integral_constant<int, R>{}, c + R);
      ring_steps<R + 1, RING>(step, c, c_hi);
    }
  }
}

// step(R, c + R) for every R < RING, unconditionally.
template <int R, int RING, typename F>
__device__ __forceinline__ void ring_steps_all(F& step, int c) {
  if constexpr (R < RING) {
    step(std::integral_constant<int, R>{}, c + R);
    ring_steps_all<R + 1, RING>(step, c);
  }
}

// One-dimensional grid of column blocks x row blocks x k-splits, split-major
// in the XCD-local order.  Each wave owns CT column tiles and both row tiles
// of its workgroup over the workgroup's whole share of K, so no partial sums
// cross waves.  Per 64-element chunk the workgroup stages X (64 rows) in LDS
// once, as bf16 (hi and lo planes for a float32 X), and every wave reads its
// B operands there; the W operands (A: output column n = lane & 31 of a
// tile, K elements 16 s + 8 hi .. + 7 of step s, hi = lane >> 5) stream
// straight from memory into a ring of RING chunks, RING - 1 chunks ahead of
// the MFMAs.  X for the next chunk is requested before the ring's newest W chunk,
// so writing it to LDS never waits for that W chunk.
//
// LDS row of a plane: 64 bf16 = eight 16-byte groups, group j of row m kept
// at slot j ^ (m & 7) so that the 32 rows read by one MFMA operand load fall
// on distinct banks.
template <bool XF32, int CT, int RING>
__global__ __launch_bounds__(kThreads) void linear_mfma(const void* __restrict__ Xv, const uint16_t* __restrict__ W,
                                                        float* __restrict__ part, LinearOut out, int M, int N, int K,
                                                        int per, int ks) {
  constexpr int kPlanes = XF32 ? 2 : 1;
  constexpr int kBlock = linear_block<CT>();
  constexpr int kXLoads = XF32 ? 4 : 2;  // 16-byte X loads per thread and chunk
  __shared__ __align__(16) uint8_t xs[2][kPlanes][kLRows * 128];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5;
  const int nblocks = N / kBlock, per_split = nblocks * ((M + kLRows - 1) / kLRows);
  const int L = xcd_local_index(blockIdx.x, gridDim.x);
  const int ky = L / per_split, rest = L - ky * per_split;
  const int n0 = (rest % nblocks) * kBlock, mbase = (rest / nblocks) * kLRows;
  const int nch = K / kLChunk;
  const int c_lo = ky * per, c_hi = min(nch, c_lo + per);
  const int nw = n0 + wave * 32 * CT;  // this wave's first column

  // this wave's column tiles in the packed weight: chunk c of tile u starts
  // at wtile[u] + 2048 c, step s of it 512 further per step, lane l at 8 l
  const uint16_t* wtile[CT];
#pragma unroll
  for (int u = 0; u < CT; ++u) wtile[u] = W + (size_t)((nw >> 5) + u) * nch * 2048 + 8 * lane;

  // X staging: thread tid covers 8-element groups g = tid and tid + 256 of
  // the chunk (row g >> 3, group g & 7)
  auto x_src = [&](int q) -> size_t {
    const int g = tid + kThreads * q;
    return (size_t)min(mbase + (g >> 3), M - 1) * K + 8 * (g & 7);
  };
  const size_t xo0 = x_src(0), xo1 = x_src(1);
  auto lds_slot = [](int m, int j) { return m * 128 + ((j ^ (m & 7)) << 4); };
  const int st0 = lds_slot(tid >> 3, tid & 7), st1 = lds_slot((tid + kThreads) >> 3, tid & 7);

  struct XStage {
    uint4 v[kXLoads];
  };
  auto load_x = [&](int c) {
    XStage xs_;
    uint4* xg = xs_.v;
    const size_t o = (size_t)c * kLChunk;
    if constexpr (XF32) {
      const float* X = static_cast<const float*>(Xv);
      xg[0] = *reinterpret_cast<const uint4*>(X + xo0 + o);
      xg[1] = *reinterpret_cast<const uint4*>(X + xo0 + o + 4);
      xg[2] = *reinterpret_cast<const uint4*>(X + xo1 + o);
      xg[3] = *reinterpret_cast<const uint4*>(X + xo1 + o + 4);
    } else {
      const uint16_t* X = static_cast<const uint16_t*>(Xv);
      xg[0] = *reinterpret_cast<const uint4*>(X + xo0 + o);
      xg[1] = *reinterpret_cast<const uint4*>(X + xo1 + o);
    }
    return xs_;
  };
  auto store_x = [&](int buf, const XStage& st) {
    const uint4* xg = st.v;
    if constexpr (XF32) {
      uint4 h0, l0, h1, l1;
      split_hilo(xg[0], xg[1], h0, l0);
      split_hilo(xg[2], xg[3], h1, l1);
      *reinterpret_cast<uint4*>(&xs[buf][0][st0]) = h0;
      *reinterpret_cast<uint4*>(&xs[buf][1][st0]) = l0;
      *reinterpret_cast<uint4*>(&xs[buf][0][st1]) = h1;
      *reinterpret_cast<uint4*>(&xs[buf][1][st1]) = l1;
    } else {
      *reinterpret_cast<uint4*>(&xs[buf][0][st0]) = xg[0];
      *reinterpret_cast<uint4*>(&xs[buf][0][st1]) = xg[1];
    }
  };
  auto load_w = [&](int c, uint4(&w)[CT][4]) {
    const size_t o = (size_t)c * 2048;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int u = 0; u < CT; ++u) w[u][s] = *reinterpret_cast<const uint4*>(wtile[u] + o + 512 * s);
  };

  f32x16 acc[2][CT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < CT; ++u) acc[t][u] = f32x16{};
  auto compute = [&](int buf, const uint4(&w)[CT][4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int slot = lds_slot(32 * t + (lane & 31), 2 * s + hi);
        const bf16x8 xh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&xs[buf][0][slot]));
#pragma unroll
        for (int u = 0; u < CT; ++u)
          acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w[u][s]), xh, acc[t][u], 0,
                                                              0, 0);
        if constexpr (XF32) {
          const bf16x8 xl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&xs[buf][1][slot]));
#pragma unroll
          for (int u = 0; u < CT; ++u)
            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w[u][s]), xl, acc[t][u],
                                                                0, 0, 0);
        }
      }
    }
  };

  // Loads past the workgroup's last chunk re-read that chunk (an L2 hit), so
  // that no load sits under a branch and the compiler's wait counts stay
  // exact across the loop.
  uint4 wr[RING][CT][4];
  if (c_lo < c_hi) {
    const XStage x0 = load_x(c_lo);
#pragma unroll
    for (int r = 0; r + 1 < RING; ++r) load_w(min(c_lo + r, c_hi - 1), wr[r]);
    store_x(0, x0);
  }
  __syncthreads();
  auto step = [&](auto R, int cc) {
    constexpr int r = decltype(R)::value;
    const XStage xn = load_x(min(cc + 1, c_hi - 1));
    load_w(min(cc + RING - 1, c_hi - 1), wr[(r + RING - 1) % RING]);
    compute((cc - c_lo) & 1, wr[r]);
    store_x((cc + 1 - c_lo) & 1, xn);  // that buffer was last read before the previous barrier
    __syncthreads();
  };
  int c = c_lo;
  for (; c + RING <= c_hi; c += RING) ring_steps_all<0, RING>(step, c);
  ring_steps<0, RING>(step, c, c_hi);

  // accumulator element r of lane (m = lane & 31, hi) is column
  // 8 (r >> 2) + 4 hi + (r & 3) of its tile
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = mbase + 32 * t + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int u = 0; u < CT; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nw + 32 * u + 8 * g + 4 * hi;
        const f32x16& a = acc[t][u];
        if (ks == 1) {
          const int grp = n / out.gs;
          *reinterpret_cast<uint2*>(out.y + m * out.ldy + (int64_t)grp * out.gstride + (n - grp * out.gs)) =
              pack_bf16x4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        } else {
          *reinterpret_cast<float4*>(part + ((size_t)ky * M + m) * N + n) =
              make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
      }
  }

  // the tails of the groups starting in this column block (split 0 only)
  if (out.tail != nullptr && ky == 0) {
    for (int grp = (n0 + out.gs - 1) / out.gs; grp < out.groups && grp * out.gs < n0 + kBlock; ++grp)
      for (int e = tid; e < kLRows * out.d_t; e += kThreads) {
        const int mm = mbase + e / out.d_t, t = e % out.d_t;
        if (mm < M)
          out.y[mm * out.ldy + (int64_t)grp * out.gstride + out.gs + t] =
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

template <bool PB, bool PC, typename TA, typename TB, typename TC>
hipError_t gemm(const TA* A, GemmView a, const TB* Bm, GemmView b, TC* C, GemmView c, PackMap pb, PackMap pc, int M,
                int N, int K, int batch, hipStream_t stream) {
  const dim3 grid((N + kT - 1) / kT, (M + kT - 1) / kT, batch);
  hipLaunchKernelGGL((gemm_strided<TA, TB, TC, PB, PC>), grid, dim3(kThreads), 0, stream, A, a, Bm, b, C, c, pb, pc,
                     M, N, K);
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ host side

int linear_max_ksplit() { return kLMaxKSplit; }

// Split count for the matrix-core linear with column blocks of `block`:
// as many splits as keep the grid within `slots` workgroups per compute unit
// (at least one, at most kLMaxKSplit and max_ks, no empty split).
int linear_ksplit(int M, int N, int K, int block, int slots, int cus, int max_ks, int* per_out) {
  const int64_t tiles = (int64_t)(N / block) * ((M + kLRows - 1) / kLRows);
  const int nch = K / kLChunk;
  int64_t ks = ((int64_t)slots * cus) / tiles;
  if (ks < 1) ks = 1;
  if (ks > kLMaxKSplit) ks = kLMaxKSplit;
  if (ks > max_ks) ks = max_ks;
  if (ks > nch) ks = nch;
  const int per = (int)((nch + ks - 1) / ks);
  *per_out = per;
  return (nch + per - 1) / per;
}

// query: one 32-column tile per wave and a three-chunk ring (ks = 1 keeps the
// grid full); output: two tiles per wave (fewer re-reads of the float32
// latent output) and a four-chunk ring, two workgroups per compute unit.
constexpr int kQueryCT = 1, kQueryRing = 3, kOutputCT = 2, kOutputRing = 4, kOutputSlots = 2;

bool fused_query_mfma_supported(const mla_dims& d, int d_in) {
  return d.dtype == MLA_BF16 && d_in % kLChunk == 0 &&
         ((int64_t)d.num_heads * d.d_c) % linear_block<kQueryCT>() == 0;
}

bool fused_output_mfma_supported(const mla_dims& d, int d_out) {
  return d.dtype == MLA_BF16 && ((int64_t)d.num_heads * d.d_c) % kLChunk == 0 &&
         d_out % linear_block<kOutputCT>() == 0;
}

hipError_t launch_fold_query(const mla_dims& d, int d_in, const void* w_in, const void* w_uk, void* w_fused,
                             bool packed, hipStream_t stream) {
  // C[h](c, i) = sum_n w_uk[h, n, c] w_in[h, n, i], stored at w_fused[h, c, i]
  // (packed: row h d_c + c, column i of W~_Q viewed as [H d_c x d_in])
  const GemmView a{(int64_t)d.d_nope * d.d_c, 1, d.d_c};
  const GemmView b{(int64_t)d.d_nope * d_in, 1, d_in};
  const GemmView c{(int64_t)d.d_c * d_in, d_in, 1};
  const PackMap none{}, pc{d.d_c, 1, 0, 0, 0, 1, d_in};
  const int M = d.d_c, N = d_in, K = d.d_nope, G = d.num_heads;
  if (d.dtype == MLA_BF16) {
    const auto* A = static_cast<const uint16_t*>(w_uk);
    const auto* B = static_cast<const uint16_t*>(w_in);
    auto* C = static_cast<uint16_t*>(w_fused);
    return packed ? gemm<false, true>(A, a, B, b, C, c, none, pc, M, N, K, G, stream)
                  : gemm<false, false>(A, a, B, b, C, c, none, none, M, N, K, G, stream);
  }
  return gemm<false, false>(static_cast<const float*>(w_uk), a, static_cast<const float*>(w_in), b,
                            static_cast<float*>(w_fused), c, none, none, M, N, K, G, stream);
}

hipError_t launch_fold_output(const mla_dims& d, int d_out, const void* w_o, const void* w_uv, void* w_fused,
                              bool packed, hipStream_t stream) {
  // C[h](r, c) = sum_v w_o[r, h d_v + v] w_uv[h, v, c], stored at w_fused[r, h d_c + c]
  const int64_t Hdv = (int64_t)d.num_heads * d.d_v, Hdc = (int64_t)d.num_heads * d.d_c;
  const GemmView a{d.d_v, Hdv, 1};
  const GemmView b{(int64_t)d.d_v * d.d_c, 1, d.d_c};
  const GemmView c{d.d_c, Hdc, 1};
  const PackMap none{}, pc{0, 1, 0, d.d_c, 0, 1, Hdc};
  const int M = d_out, N = d.d_c, K = d.d_v, G = d.num_heads;
  if (d.dtype == MLA_BF16) {
    const auto* A = static_cast<const uint16_t*>(w_o);
    const auto* B = static_cast<const uint16_t*>(w_uv);
    auto* C = static_cast<uint16_t*>(w_fused);
    return packed ? gemm<false, true>(A, a, B, b, C, c, none, pc, M, N, K, G, stream)
                  : gemm<false, false>(A, a, B, b, C, c, none, none, M, N, K, G, stream);
  }
  return gemm<false, false>(static_cast<const float*>(w_o), a, static_cast<const float*>(w_uv), b,
                            static_cast<float*>(w_fused), c, none, none, M, N, K, G, stream);
}

hipError_t launch_fused_query(const mla_dims& d, int d_in, int cus, const void* x, const void* q_rope,
                              const void* w_fused, void* q_cat, bool mfma, bool packed, hipStream_t stream) {
  const int M = d.batch * d.q_len, D = d.d_c + d.d_rope;
  if (mfma) {  // the matrix-core path always reads the packed order
    const int N = d.num_heads * d.d_c;
    int per = 0;
    const int ks = linear_ksplit(M, N, d_in, linear_block<kQueryCT>(), 2, cus, 1, &per);
    const LinearOut out{static_cast<uint16_t*>(q_cat), (int64_t)d.num_heads * D, d.d_c, D,
                        d.d_rope > 0 ? static_cast<const uint16_t*>(q_rope) : nullptr, d.d_rope, d.num_heads};
    const int64_t blocks = (int64_t)(N / linear_block<kQueryCT>()) * ((M + kLRows - 1) / kLRows) * ks;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((linear_mfma<false, kQueryCT, kQueryRing>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, x,
                       static_cast<const uint16_t*>(w_fused), nullptr, out, M, N, d_in, per, ks);
    return hipGetLastError();
  }
  // C[h](m, c) = sum_i x[m, i] w_fused[h, c, i], stored at q_cat[m, h, c]
  const GemmView a{0, d_in, 1};
  const GemmView b{(int64_t)d.d_c * d_in, d_in, 1};
  const GemmView c{D, (int64_t)d.num_heads * D, 1};
  const PackMap none{}, pb{d.d_c, 1, 0, 0, 0, 1, d_in};
  const int64_t rows = (int64_t)M * d.num_heads;
  hipError_t e;
  if (d.dtype == MLA_BF16) {
    const auto* A = static_cast<const uint16_t*>(x);
    const auto* B = static_cast<const uint16_t*>(w_fused);
    auto* C = static_cast<uint16_t*>(q_cat);
    e = packed ? gemm<true, false>(A, a, B, b, C, c, pb, none, M, d.d_c, d_in, d.num_heads, stream)
               : gemm<false, false>(A, a, B, b, C, c, none, none, M, d.d_c, d_in, d.num_heads, stream);
    if (e == hipSuccess && d.d_rope > 0)
      hipLaunchKernelGGL(pass_rope<uint16_t>, dim3(256), dim3(kThreads), 0, stream,
                         static_cast<const uint16_t*>(q_rope), C, rows, d.d_c, d.d_rope);
  } else {
    e = gemm<false, false>(static_cast<const float*>(x), a, static_cast<const float*>(w_fused), b,
                           static_cast<float*>(q_cat), c, none, none, M, d.d_c, d_in, d.num_heads, stream);
    if (e == hipSuccess && d.d_rope > 0)
      hipLaunchKernelGGL(pass_rope<float>, dim3(256), dim3(kThreads), 0, stream, static_cast<const float*>(q_rope),
                         static_cast<float*>(q_cat), rows, d.d_c, d.d_rope);
  }
  return e == hipSuccess ? hipGetLastError() : e;
}

hipError_t launch_fused_output(const mla_dims& d, int d_out, int cus, const float* o, const void* w_fused, void* y,
                               float* ws, bool mfma, bool packed, hipStream_t stream) {
  const int M = d.batch * d.q_len, K = d.num_heads * d.d_c;
  if (mfma) {  // the matrix-core path always reads the packed order
    int per = 0;
    const int ks = linear_ksplit(M, d_out, K, linear_block<kOutputCT>(), kOutputSlots, cus, kLMaxKSplit, &per);
    const LinearOut out{static_cast<uint16_t*>(y), d_out, d_out, 0, nullptr, 0, 1};
    const int64_t blocks = (int64_t)(d_out / linear_block<kOutputCT>()) * ((M + kLRows - 1) / kLRows) * ks;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((linear_mfma<true, kOutputCT, kOutputRing>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, o,
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
  const PackMap none{}, pb{0, 1, 0, 0, 0, 1, K};
  if (d.dtype == MLA_BF16) {
    const auto* B = static_cast<const uint16_t*>(w_fused);
    auto* C = static_cast<uint16_t*>(y);
    return packed ? gemm<true, false>(o, a, B, b, C, c, pb, none, M, d_out, K, 1, stream)
                  : gemm<false, false>(o, a, B, b, C, c, none, none, M, d_out, K, 1, stream);
  }
  return gemm<false, false>(o, a, static_cast<const float*>(w_fused), b, static_cast<float*>(y), c, none, none, M,
                            d_out, K, 1, stream);
}

}  // namespace mla
