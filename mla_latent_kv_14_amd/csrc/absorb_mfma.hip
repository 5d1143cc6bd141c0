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
// grid (H, d_c / 128); wave w computes columns 32 w .. 32 w + 31 of the quarter
// for every 32-row tile of M.
__global__ __launch_bounds__(kThreads) void absorb_q_mfma(const uint16_t* __restrict__ q_nope,
                                                          const uint16_t* __restrict__ q_rope,
                                                          const uint16_t* __restrict__ w_uk,
                                                          uint16_t* __restrict__ q_cat, int M, int H, int d_r) {
  // W quarter: row k (0..127) holds 16 chunks of 16 B; chunk c sits at c ^ (4 * (k & 3))
  __shared__ __attribute__((aligned(16))) uint8_t wt[kDN * kNQ * 2];
  const int h = blockIdx.x, nq = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5;
  const int D = kDC + d_r;

  // A operands (q_nope rows) of the first 32-row tile are requested before the
  // weight staging so that both memory round trips overlap
  auto load_a = [&](int m0, uint4* a) {
    const int m = m0 + (lane & 31);
    const uint16_t* src = q_nope + ((size_t)min(m, M - 1) * H + h) * kDN + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kDN / 16; ++ks) a[ks] = *reinterpret_cast<const uint4*>(src + 16 * ks);
  };
  uint4 a_cur[kDN / 16];
  load_a(0, a_cur);

  // the RoPE part of each row is copied unchanged, 16 B per thread, spread
  // over the d_c / 128 workgroups of head h (d_r is a multiple of 8)
  {
    const int per_row = d_r / 8, nchunk = M * per_row;
    for (int i = nq * kThreads + tid; i < nchunk; i += kThreads * (kDC / kNQ)) {
      const int m = i / per_row, k = i - m * per_row;
      *reinterpret_cast<uint4*>(q_cat + ((size_t)m * H + h) * D + kDC + 8 * k) =
          *reinterpret_cast<const uint4*>(q_rope + ((size_t)m * H + h) * d_r + 8 * k);
    }
  }

  const uint16_t* w = w_uk + (size_t)h * kDN * kDC + nq * kNQ;
  uint4 wv[(kDN * kNQ / 8) / kThreads];
#pragma unroll
  for (int i = 0; i < (kDN * kNQ / 8) / kThreads; ++i) {  // 8 x 16 B per thread
    const int q = i * kThreads + tid;
    wv[i] = *reinterpret_cast<const uint4*>(w + (size_t)(q >> 4) * kDC + 8 * (q & 15));
  }
#pragma unroll
  for (int i = 0; i < (kDN * kNQ / 8) / kThreads; ++i) {
    const int q = i * kThreads + tid;
    const int k = q >> 4, c = q & 15;
    *reinterpret_cast<uint4*>(wt + k * 256 + ((c ^ (4 * (k & 3))) * 16)) = wv[i];
  }
  __syncthreads();

  // transpose-read supplier mapping (see the decode kernel): lane supplies row
  // 16 ks + 8 (g16 >> 1) + 4 h + (j16 >> 2), columns 32 w + 16 (g16 & 1) + 4 (j16 & 3)
  const int g16 = lane >> 4, j16 = lane & 15;
  const int col = 32 * wave + 16 * (g16 & 1) + 4 * (j16 & 3);
  const int row0 = 8 * (g16 >> 1) + (j16 >> 2);

  bf16x8 bop[kDN / 16];
#pragma unroll
  for (int ks = 0; ks < kDN / 16; ++ks) {
    bf16x4 v[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = 16 * ks + row0 + 4 * hh;
      const int off = k * 256 + (((col >> 3) ^ (4 * (k & 3))) * 16) + (col & 7) * 2;
      v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wt + off));
    }
    bop[ks] = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
  }

  const int n = nq * kNQ + 32 * wave + (lane & 31);
  for (int m0 = 0; m0 < M; m0 += 32) {
    uint4 a_next[kDN / 16];
    if (m0 + 32 < M) load_a(m0 + 32, a_next);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kDN / 16; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a_cur[ks]), bop[ks], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mr = m0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (mr < M) q_cat[((size_t)mr * H + h) * D + n] = f32_to_bf16_bits(acc[r]);
    }
    if (m0 + 32 < M) {
#pragma unroll
      for (int ks = 0; ks < kDN / 16; ++ks) a_cur[ks] = a_next[ks];
    }
  }

}

// ------------------------------------------------------------------ absorb_out
// grid (H, ceil(M / 32)); wave w computes outputs 32 w .. 32 w + 31 of d_v.
__global__ __launch_bounds__(kThreads) void absorb_out_mfma(const float* __restrict__ o,
                                                            const uint16_t* __restrict__ w_uv,
                                                            uint16_t* __restrict__ out, int M, int H) {
  // o tile as bf16 hi and lo: row m (0..31) holds 64 chunks of 16 B; chunk c
  // sits at c ^ (m & 15)
  __shared__ __attribute__((aligned(16))) uint8_t ot[2][32 * kDC * 2];
  const int h = blockIdx.x, m0 = blockIdx.y * 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5;

  // every B operand (W_UV rows) of this wave is requested first; its latency
  // overlaps the staging of o
  const int v = 32 * wave + (lane & 31);
  const uint16_t* wrow = w_uv + ((size_t)h * kDV + v) * kDC + 8 * hi;
  uint4 bw[kDC / 16];
#pragma unroll
  for (int ks = 0; ks < kDC / 16; ++ks) bw[ks] = *reinterpret_cast<const uint4*>(wrow + 16 * ks);

#pragma unroll
  for (int i = 0; i < (32 * kDC / 8) / kThreads; ++i) {  // 8 chunks of 8 floats per thread
    const int q = i * kThreads + tid;
    const int r = q >> 6, c = q & 63, m = m0 + r;
    float f[8];
    if (m < M) {
      const float4* src = reinterpret_cast<const float4*>(o + ((size_t)m * H + h) * kDC + 8 * c);
      const float4 x0 = src[0], x1 = src[1];
      f[0] = x0.x; f[1] = x0.y; f[2] = x0.z; f[3] = x0.w;
      f[4] = x1.x; f[5] = x1.y; f[6] = x1.z; f[7] = x1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = 0.f;
    }
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t h0 = f32_to_bf16_bits(f[2 * e]), h1 = f32_to_bf16_bits(f[2 * e + 1]);
      const uint16_t l0 = f32_to_bf16_bits(f[2 * e] - bf16_bits_to_f32(h0));
      const uint16_t l1 = f32_to_bf16_bits(f[2 * e + 1] - bf16_bits_to_f32(h1));
      hw[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lw[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    const int off = r * 1024 + ((c ^ (r & 15)) * 16);
    *reinterpret_cast<uint4*>(&ot[0][off]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4*>(&ot[1][off]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  __syncthreads();

  const int r = lane & 31;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int ks = 0; ks < kDC / 16; ++ks) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, bw[ks]);
    const int off = r * 1024 + (((2 * ks + hi) ^ (r & 15)) * 16);
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&ot[0][off]);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&ot[1][off]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b, acc, 0, 0, 0);
  }
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int m = m0 + 8 * (rr >> 2) + 4 * hi + (rr & 3);
    if (m < M) out[((size_t)m * H + h) * kDV + v] = f32_to_bf16_bits(acc[rr]);
  }
}


// ------------------------------------------------------------ combine + absorb_out
// The log-sum-exp merge of the split partials fused with the W_UV product, so
// that the merged latent output never leaves the chip:
//   lse = log sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) o_s,  u = W_UV[h] o.
// grid (H, ceil(M / 32)); the 32 rows of a workgroup are merged straight into
// the bf16 hi/lo LDS tile of absorb_out_mfma.  Splits with lse_s = -inf are
// skipped (their o_s is never read).  o_latent and lse are written when given.
constexpr int kMaxFusedSplits = 64;

__global__ __launch_bounds__(kThreads) void combine_out_mfma(const float* __restrict__ o_part,
                                                             const float* __restrict__ lse_part,
                                                             const uint16_t* __restrict__ w_uv,
                                                             uint16_t* __restrict__ out, float* __restrict__ o_latent,
                                                             float* __restrict__ lse_out, int M, int H, int S) {
  __shared__ __attribute__((aligned(16))) uint8_t ot[2][32 * kDC * 2];
  __shared__ float wts[32][kMaxFusedSplits];
  const int h = blockIdx.x, m0 = blockIdx.y * 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5;

  // every B operand (W_UV rows) of this wave is requested first
  const int v = 32 * wave + (lane & 31);
  const uint16_t* wrow = w_uv + ((size_t)h * kDV + v) * kDC + 8 * hi;
  uint4 bw[kDC / 16];
#pragma unroll
  for (int ks = 0; ks < kDC / 16; ++ks) bw[ks] = *reinterpret_cast<const uint4*>(wrow + 16 * ks);

  // split weights: 8 lanes per row
  {
    const int r = tid >> 3, j = tid & 7, m = m0 + r;
    const float* lp = lse_part + ((size_t)min(m, M - 1) * H + h) * S;
    const float total = split_lse(lp, S, j);
    for (int s2 = j; s2 < S; s2 += 8) {
      const float ls = lp[s2];
      wts[r][s2] = (ls == -INFINITY || m >= M) ? 0.f : expf(ls - total);
    }
    if (lse_out != nullptr && j == 0 && m < M) lse_out[(size_t)m * H + h] = total;
  }
  __syncthreads();

  // merge: thread (row r, lane j of 8) owns float4 columns j + 8 k, k < 16
  {
    const int r = tid >> 3, j = tid & 7, m = m0 + r;
    float4 acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m < M) {
      const float4* src = reinterpret_cast<const float4*>(o_part + ((size_t)m * H + h) * S * kDC);
      for (int s2 = 0; s2 < S; ++s2) {
        const float wgt = wts[r][s2];
        if (wgt == 0.f) continue;
        float4 x[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) x[k] = src[(size_t)s2 * (kDC / 4) + j + 8 * k];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          acc[k].x = fmaf(wgt, x[k].x, acc[k].x);
          acc[k].y = fmaf(wgt, x[k].y, acc[k].y);
          acc[k].z = fmaf(wgt, x[k].z, acc[k].z);
          acc[k].w = fmaf(wgt, x[k].w, acc[k].w);
        }
      }
      if (o_latent != nullptr) {
        float4* dst = reinterpret_cast<float4*>(o_latent + ((size_t)m * H + h) * kDC);
#pragma unroll
        for (int k = 0; k < 16; ++k) dst[j + 8 * k] = acc[k];
      }
    }
    // float4 column f = j + 8 k covers half of 16-B chunk c = f / 2 (8 bytes of bf16)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int f = j + 8 * k, c = f >> 1;
      const float e[4] = {acc[k].x, acc[k].y, acc[k].z, acc[k].w};
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint16_t h0 = f32_to_bf16_bits(e[2 * q]), h1 = f32_to_bf16_bits(e[2 * q + 1]);
        const uint16_t l0 = f32_to_bf16_bits(e[2 * q] - bf16_bits_to_f32(h0));
        const uint16_t l1 = f32_to_bf16_bits(e[2 * q + 1] - bf16_bits_to_f32(h1));
        hw[q] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lw[q] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
      const int off = r * 1024 + ((c ^ (r & 15)) * 16) + 8 * (f & 1);
      *reinterpret_cast<uint2*>(&ot[0][off]) = make_uint2(hw[0], hw[1]);
      *reinterpret_cast<uint2*>(&ot[1][off]) = make_uint2(lw[0], lw[1]);
    }
  }
  __syncthreads();

  const int r = lane & 31;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int ks = 0; ks < kDC / 16; ++ks) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, bw[ks]);
    const int off = r * 1024 + (((2 * ks + hi) ^ (r & 15)) * 16);
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&ot[0][off]);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&ot[1][off]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b, acc, 0, 0, 0);
  }
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int m = m0 + 8 * (rr >> 2) + 4 * hi + (rr & 3);
    if (m < M) out[((size_t)m * H + h) * kDV + v] = f32_to_bf16_bits(acc[rr]);
  }
}

}  // namespace

bool absorb_mfma_supported(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_c == kDC && d.d_nope == kDN && d.d_v == kDV && d.d_rope <= 1024 - kDC;
}

hipError_t launch_absorb_q_mfma(const mla_dims& d, const void* q_nope, const void* q_rope, const void* w_uk,
                                void* q_cat, hipStream_t stream) {
  const int M = d.batch * d.q_len;
  hipLaunchKernelGGL(absorb_q_mfma, dim3(d.num_heads, kDC / kNQ), dim3(kThreads), 0, stream,
                     (const uint16_t*)q_nope, (const uint16_t*)q_rope, (const uint16_t*)w_uk, (uint16_t*)q_cat, M,
                     d.num_heads, d.d_rope);
  return hipGetLastError();
}

int combine_out_max_splits() { return kMaxFusedSplits; }

hipError_t launch_combine_out_mfma(const mla_dims& d, int splits, const float* o_part, const float* lse_part,
                                   const void* w_uv, void* out, float* o_latent, float* lse, hipStream_t stream) {
  const int M = d.batch * d.q_len;
  hipLaunchKernelGGL(combine_out_mfma, dim3(d.num_heads, (M + 31) / 32), dim3(kThreads), 0, stream, o_part, lse_part,
                     (const uint16_t*)w_uv, (uint16_t*)out, o_latent, lse, M, d.num_heads, splits);
  return hipGetLastError();
}

hipError_t launch_absorb_out_mfma(const mla_dims& d, const float* o, const void* w_uv, void* out,
                                  hipStream_t stream) {
  const int M = d.batch * d.q_len;
  hipLaunchKernelGGL(absorb_out_mfma, dim3(d.num_heads, (M + 31) / 32), dim3(kThreads), 0, stream, o,
                     (const uint16_t*)w_uv, (uint16_t*)out, M, d.num_heads);
  return hipGetLastError();
}

}  // namespace mla
