// Matrix-core absorption GEMMs for bf16 storage (d_nope = d_v = 128, d_c = 512).
//
// absorb_q:   q~[m,h,:] = q_nope[m,h,:] . W_UK[h]         (M x 128) x (128 x 512)
//   "DeepSeek-V3 MLA: Multi-Head Latent Attention Guide", Matrix Absorption
//   Trick section 2 (Folding W^UK into Query Projection).  W_UK[h] is stored
//   [d_nope][d_c], so its contraction index is the strided one: a 128 x 128
//   quarter is staged in LDS and the MFMA operand is built with the LDS
//   transpose read.  q_rope is copied into the tail of each q_cat row.
// absorb_out: u[m,h,:] = o[m,h,:] . W_UV[h]^T               (M x 512) x (512 x 128)
//   Same guide, section 3 (Absorbing W^UV).  W_UV[h] is [d_v][d_c], already
//   contiguous along the contraction, so it feeds the MFMA straight from
//   memory.  o is float32: it is split as o = hi + lo with hi, lo in bf16 and
//   both halves are multiplied, which keeps about 16 mantissa bits of o.
#include "common.h"
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kThreads = 256;
constexpr int kDN = 128;   // d_nope
constexpr int kDV = 128;   // d_v
constexpr int kDC = 512;   // d_c
constexpr int kNQ = 128;   // absorb_q: columns of q~ per workgroup

// ------------------------------------------------------------------ absorb_q
// grid (H, d_c / 128, ceil(M / 64)): workgroup (h, nq, mt) computes columns
// 128 nq .. 128 nq + 127 of q~ for rows 64 mt .. 64 mt + 63; wave w takes the
// 32 columns 32 w .. 32 w + 31 of that quarter.  The W quarter and the 64
// q_nope rows are both staged in LDS once per workgroup.  The MFMA computes q~^T =
// W_UK[h]^T . q_nope^T (A = W_UK^T from the LDS transpose read, B = q_nope
// rows), so each lane ends up with four consecutive latent columns of one row
// and stores them as one 8-byte write.
constexpr int kRowsQ = 64;  // rows of q_nope per workgroup (two 32-row MFMA tiles)

__global__ __launch_bounds__(kThreads) void absorb_q_mfma(const uint16_t* __restrict__ q_nope,
                                                          const uint16_t* __restrict__ q_rope,
                                                          const uint16_t* __restrict__ w_uk,
                                                          uint16_t* __restrict__ q_cat, int M, int H, int d_r) {
  // W quarter: row k (0..127) holds 16 chunks of 16 B; chunk c sits at c ^ (4 * (k & 3))
  __shared__ __attribute__((aligned(16))) uint8_t wt[kDN * kNQ * 2];
  const int h = blockIdx.x, nq = blockIdx.y, mbase = blockIdx.z * kRowsQ;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5;
  const int D = kDC + d_r;

  // the workgroup's q_nope rows (64 x 256 B) are staged once in LDS, row m's
  // chunk c at slot c ^ (m & 15); rows past M read row M - 1
  __shared__ __attribute__((aligned(16))) uint8_t qs[kRowsQ * kDN * 2];
  uint4 qv[(kRowsQ * kDN / 8) / kThreads];
#pragma unroll
  for (int i = 0; i < (kRowsQ * kDN / 8) / kThreads; ++i) {
    const int q = i * kThreads + tid, r = q >> 4, c = q & 15;
    const int m = min(mbase + r, M - 1);
    qv[i] = *reinterpret_cast<const uint4*>(q_nope + ((size_t)m * H + h) * kDN + 8 * c);
  }
  const uint16_t* w = w_uk + (size_t)h * kDN * kDC + nq * kNQ;
  uint4 wv[(kDN * kNQ / 8) / kThreads];
#pragma unroll
  for (int i = 0; i < (kDN * kNQ / 8) / kThreads; ++i) {  // 8 x 16 B per thread
    const int q = i * kThreads + tid;
    wv[i] = *reinterpret_cast<const uint4*>(w + (size_t)(q >> 4) * kDC + 8 * (q & 15));
  }

  // the RoPE part of each row is copied unchanged, 16 B per thread, spread
  // over the d_c / 128 workgroups of the row block (d_r is a multiple of 8)
  {
    const int per_row = d_r / 8, rows = min(kRowsQ, M - mbase), nchunk = rows * per_row;
    for (int i = nq * kThreads + tid; i < nchunk; i += kThreads * (kDC / kNQ)) {
      const int m = mbase + i / per_row, k = i % per_row;
      *reinterpret_cast<uint4*>(q_cat + ((size_t)m * H + h) * D + kDC + 8 * k) =
          *reinterpret_cast<const uint4*>(q_rope + ((size_t)m * H + h) * d_r + 8 * k);
    }
  }

#pragma unroll
  for (int i = 0; i < (kDN * kNQ / 8) / kThreads; ++i) {
    const int q = i * kThreads + tid;
    const int k = q >> 4, c = q & 15;
    *reinterpret_cast<uint4*>(wt + k * 256 + ((c ^ (4 * (k & 3))) * 16)) = wv[i];
  }
#pragma unroll
  for (int i = 0; i < (kRowsQ * kDN / 8) / kThreads; ++i) {
    const int q = i * kThreads + tid, r = q >> 4, c = q & 15;
    *reinterpret_cast<uint4*>(qs + r * 256 + ((c ^ (r & 15)) * 16)) = qv[i];
  }
  __syncthreads();
  uint4 a[2][kDN / 16];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 32 * t + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < kDN / 16; ++ks)
      a[t][ks] = *reinterpret_cast<const uint4*>(qs + r * 256 + (((2 * ks + hi) ^ (r & 15)) * 16));
  }

  // transpose-read supplier mapping (see the decode kernel): lane supplies row
  // 16 ks + 8 (g16 >> 1) + 4 h + (j16 >> 2), columns 32 w + 16 (g16 & 1) + 4 (j16 & 3)
  const int g16 = lane >> 4, j16 = lane & 15;
  const int col = 32 * wave + 16 * (g16 & 1) + 4 * (j16 & 3);
  const int row0 = 8 * (g16 >> 1) + (j16 >> 2);

  bf16x8 wop[kDN / 16];
#pragma unroll
  for (int ks = 0; ks < kDN / 16; ++ks) {
    bf16x4 v[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = 16 * ks + row0 + 4 * hh;
      const int off = k * 256 + (((col >> 3) ^ (4 * (k & 3))) * 16) + (col & 7) * 2;
      v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wt + off));
    }
    wop[ks] = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
  }

  // accumulator element r of lane (row j = lane & 31, hi) is column
  // 32 wave + 8 (r >> 2) + 4 hi + (r & 3) of the quarter
  const int c0 = nq * kNQ + 32 * wave + 4 * hi;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = mbase + 32 * t + (lane & 31);
    if (mbase + 32 * t >= M) break;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kDN / 16; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop[ks], __builtin_bit_cast(bf16x8, a[t][ks]), acc, 0, 0, 0);
    if (m < M) {
      uint16_t* dst = q_cat + ((size_t)m * H + h) * D + c0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t lo = (uint32_t)f32_to_bf16_bits(acc[4 * g]) | ((uint32_t)f32_to_bf16_bits(acc[4 * g + 1]) << 16);
        const uint32_t up = (uint32_t)f32_to_bf16_bits(acc[4 * g + 2]) | ((uint32_t)f32_to_bf16_bits(acc[4 * g + 3]) << 16);
        *reinterpret_cast<uint2*>(dst + 8 * g) = make_uint2(lo, up);
      }
    }
  }
}

// ------------------------------------------------------------ W_UV product
// u tile (32 rows x 128 outputs) = o tile (32 x 512, LDS bf16 hi + lo, row r's
// 16-B chunk c at c ^ (r & 15)) . W_UV[h]^T, by 8 waves: wave w computes
// outputs 32 (w & 3) .. + 31 over d_c half (w >> 2) with the W_UV rows it
// requested into bw; the second half adds into the first through LDS.  Both
// kernels that apply W_UV use this, so they round identically.
constexpr int kThreadsC = 512;

struct WuvOperands {
  uint4 bw[kDC / 32];
};

__device__ __forceinline__ void wuv_request(const uint16_t* __restrict__ w_uv, int h, int wave, int lane,
                                            WuvOperands& op) {
  const int v = 32 * (wave & 3) + (lane & 31), hi = lane >> 5;
  const uint16_t* wrow = w_uv + ((size_t)h * kDV + v) * kDC + (wave >> 2) * (kDC / 2) + 8 * hi;
#pragma unroll
  for (int ks = 0; ks < kDC / 32; ++ks) op.bw[ks] = *reinterpret_cast<const uint4*>(wrow + 16 * ks);
}

__device__ __forceinline__ void wuv_product(const uint8_t (*ot)[32 * kDC * 2], float (*red)[16][64],
                                            const WuvOperands& op, int wave, int lane, int m0, int M, int H, int h,
                                            uint16_t* __restrict__ out) {
  const int vblk = wave & 3, chalf = wave >> 2, hi = lane >> 5, r = lane & 31;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int kq = 0; kq < kDC / 32; ++kq) {
    const int ks = chalf * (kDC / 32) + kq;
    const bf16x8 b = __builtin_bit_cast(bf16x8, op.bw[kq]);
    const int off = r * 1024 + (((2 * ks + hi) ^ (r & 15)) * 16);
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&ot[0][off]);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&ot[1][off]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b, acc, 0, 0, 0);
  }
  if (chalf == 1) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) red[vblk][rr][lane] = acc[rr];
  }
  __syncthreads();
  if (chalf == 0) {
    const int v = 32 * vblk + r;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float x = acc[rr] + red[vblk][rr][lane];
      const int m = m0 + 8 * (rr >> 2) + 4 * hi + (rr & 3);
      if (m < M) out[((size_t)m * H + h) * kDV + v] = f32_to_bf16_bits(x);
    }
  }
}

// o row r (fp32, 8 consecutive values starting at column 8 c + 4 half) into
// the hi/lo tile: writes the 8-byte half 'half' of 16-B chunk c
__device__ __forceinline__ void stage_hilo(uint8_t (*ot)[32 * kDC * 2], int r, int c, int half, const float4& x) {
  const float e[4] = {x.x, x.y, x.z, x.w};
  uint32_t hw[2], lw[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint16_t h0 = f32_to_bf16_bits(e[2 * q]), h1 = f32_to_bf16_bits(e[2 * q + 1]);
    const uint16_t l0 = f32_to_bf16_bits(e[2 * q] - bf16_bits_to_f32(h0));
    const uint16_t l1 = f32_to_bf16_bits(e[2 * q + 1] - bf16_bits_to_f32(h1));
    hw[q] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lw[q] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  const int off = r * 1024 + ((c ^ (r & 15)) * 16) + 8 * half;
  *reinterpret_cast<uint2*>(&ot[0][off]) = make_uint2(hw[0], hw[1]);
  *reinterpret_cast<uint2*>(&ot[1][off]) = make_uint2(lw[0], lw[1]);
}

// ------------------------------------------------------------------ absorb_out
// grid (H, ceil(M / 32)), 8 waves: the o tile is staged as bf16 hi + lo, then
// multiplied by W_UV[h] (requested first, so its latency overlaps the staging).
__global__ __launch_bounds__(kThreadsC) void absorb_out_mfma(const float* __restrict__ o,
                                                             const uint16_t* __restrict__ w_uv,
                                                             uint16_t* __restrict__ out, int M, int H) {
  __shared__ __attribute__((aligned(16))) uint8_t ot[2][32 * kDC * 2];
  __shared__ __attribute__((aligned(16))) float red[4][16][64];
  const int h = blockIdx.x, m0 = blockIdx.y * 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  WuvOperands op;
  wuv_request(w_uv, h, wave, lane, op);
  // thread (row r, lane j of 16) stages float4 columns j + 16 k, k < 8
  {
    const int r = tid >> 4, j = tid & 15, m = m0 + r;
    float4 x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      x[k] = (m < M) ? reinterpret_cast<const float4*>(o + ((size_t)m * H + h) * kDC)[j + 16 * k]
                     : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 8; ++k) stage_hilo(ot, r, (j + 16 * k) >> 1, (j + 16 * k) & 1, x[k]);
  }
  __syncthreads();
  wuv_product(ot, red, op, wave, lane, m0, M, H, h, out);
}

// ------------------------------------------------------------ combine + absorb_out
// The log-sum-exp merge of the split partials fused with the W_UV product, so
// that the merged latent output never leaves the chip:
//   lse = log sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) o_s,  u = W_UV[h] o.
// grid (H, ceil(M / 32)), 8 waves.  The 32 rows of a workgroup are merged
// straight into the bf16 hi/lo LDS tile of absorb_out_mfma; each thread owns
// 32 columns of one row and keeps two splits' loads in flight.  Splits with
// lse_s = -inf are skipped (their o_s is never read).  o_latent and lse are
// written when given.
constexpr int kMaxFusedSplits = 64;

__global__ __launch_bounds__(kThreadsC) void combine_out_mfma(const float* __restrict__ o_part,
                                                              const float* __restrict__ lse_part,
                                                              const uint16_t* __restrict__ w_uv,
                                                              uint16_t* __restrict__ out, float* __restrict__ o_latent,
                                                              float* __restrict__ lse_out, int M, int H, int S) {
  __shared__ __attribute__((aligned(16))) uint8_t ot[2][32 * kDC * 2];
  __shared__ float wts[32][kMaxFusedSplits];
  __shared__ __attribute__((aligned(16))) float red[4][16][64];
  const int h = blockIdx.x, m0 = blockIdx.y * 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  WuvOperands op;
  wuv_request(w_uv, h, wave, lane, op);

  // split weights: 16 lanes per row (two groups of 8 compute the same total)
  {
    const int r = tid >> 4, j = tid & 15, m = m0 + r;
    const float* lp = lse_part + ((size_t)min(m, M - 1) * H + h) * S;
    const float total = split_lse(lp, S, j & 7);
    for (int s2 = j; s2 < S; s2 += 16) {
      const float ls = lp[s2];
      wts[r][s2] = (ls == -INFINITY || m >= M) ? 0.f : expf(ls - total);
    }
    if (lse_out != nullptr && j == 0 && m < M) lse_out[(size_t)m * H + h] = total;
  }
  __syncthreads();

  // merge: thread (row r, lane j of 16) owns float4 columns j + 16 k, k < 8
  {
    const int r = tid >> 4, j = tid & 15, m = m0 + r;
    float4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m < M) {
      const float4* src = reinterpret_cast<const float4*>(o_part + ((size_t)m * H + h) * S * kDC) + j;
      auto fma4 = [&](float wgt, const float4* x) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          acc[k].x = fmaf(wgt, x[k].x, acc[k].x);
          acc[k].y = fmaf(wgt, x[k].y, acc[k].y);
          acc[k].z = fmaf(wgt, x[k].z, acc[k].z);
          acc[k].w = fmaf(wgt, x[k].w, acc[k].w);
        }
      };
      for (int s2 = 0; s2 < S; s2 += 2) {
        const float w0 = wts[r][s2];
        const float w1 = (s2 + 1 < S) ? wts[r][s2 + 1] : 0.f;
        float4 x0[8], x1[8];
        if (w0 != 0.f) {
#pragma unroll
          for (int k = 0; k < 8; ++k) x0[k] = src[(size_t)s2 * (kDC / 4) + 16 * k];
        }
        if (w1 != 0.f) {
#pragma unroll
          for (int k = 0; k < 8; ++k) x1[k] = src[(size_t)(s2 + 1) * (kDC / 4) + 16 * k];
        }
        if (w0 != 0.f) fma4(w0, x0);
        if (w1 != 0.f) fma4(w1, x1);
      }
      if (o_latent != nullptr) {
        float4* dst = reinterpret_cast<float4*>(o_latent + ((size_t)m * H + h) * kDC) + j;
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[16 * k] = acc[k];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) stage_hilo(ot, r, (j + 16 * k) >> 1, (j + 16 * k) & 1, acc[k]);
  }
  __syncthreads();
  wuv_product(ot, red, op, wave, lane, m0, M, H, h, out);
}

}  // namespace

bool absorb_mfma_supported(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_c == kDC && d.d_nope == kDN && d.d_v == kDV && d.d_rope <= 1024 - kDC;
}

hipError_t launch_absorb_q_mfma(const mla_dims& d, const void* q_nope, const void* q_rope, const void* w_uk,
                                void* q_cat, hipStream_t stream) {
  const int M = d.batch * d.q_len;
  hipLaunchKernelGGL(absorb_q_mfma, dim3(d.num_heads, kDC / kNQ, (M + kRowsQ - 1) / kRowsQ), dim3(kThreads), 0, stream,
                     (const uint16_t*)q_nope, (const uint16_t*)q_rope, (const uint16_t*)w_uk, (uint16_t*)q_cat, M,
                     d.num_heads, d.d_rope);
  return hipGetLastError();
}

int combine_out_max_splits() { return kMaxFusedSplits; }

hipError_t launch_combine_out_mfma(const mla_dims& d, int splits, const float* o_part, const float* lse_part,
                                   const void* w_uv, void* out, float* o_latent, float* lse, hipStream_t stream) {
  const int M = d.batch * d.q_len;
  hipLaunchKernelGGL(combine_out_mfma, dim3(d.num_heads, (M + 31) / 32), dim3(kThreadsC), 0, stream, o_part, lse_part,
                     (const uint16_t*)w_uv, (uint16_t*)out, o_latent, lse, M, d.num_heads, splits);
  return hipGetLastError();
}

hipError_t launch_absorb_out_mfma(const mla_dims& d, const float* o, const void* w_uv, void* out,
                                  hipStream_t stream) {
  const int M = d.batch * d.q_len;
  hipLaunchKernelGGL(absorb_out_mfma, dim3(d.num_heads, (M + 31) / 32), dim3(kThreadsC), 0, stream, o,
                     (const uint16_t*)w_uv, (uint16_t*)out, M, d.num_heads);
  return hipGetLastError();
}

}  // namespace mla
