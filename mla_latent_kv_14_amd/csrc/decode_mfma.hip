// Split-KV absorbed-MLA attention on gfx950 matrix cores (bf16 storage,
// d_c = 512, d_rope = 64, block_size a multiple of 32).
//
// One workgroup = 4 waves = one token range of the planner's schedule, with
// every query row of the sequence (all heads x all new tokens).  Each 32-token
// sub-tile of latent rows [c^KV | k^R] (32 x 1152 B) is copied HBM -> LDS once
// by the LDS-DMA path (global_load_lds, 16 B per lane) and then read by every
// wave, so all heads share one staging of the cache ("DeepSeek-V3 MLA:
// Multi-Head Latent Attention Guide", section 4: latents and RoPE keys loaded
// once into on-chip memory, scores and latent-weighted sums in one pass).
// Four sub-tile buffers (144 KiB) keep three sub-tiles in flight while one is
// computed.
//
// Per sub-tile and wave (32 query rows):
//   S^T[token, row] = K[token, 0:576] . q_cat[row, 0:576]   36 MFMA 32x32x16
//       A = LDS rows (ds_read_b128), B = q_cat held in registers for the
//       whole range: one shared-latent score q~.c + q^R.k^R per pair.
//   softmax in base 2, per lane = per query row (max/sum need only the lane
//       and lane^32).  Each row's reference max is fixed at its first
//       sub-tile, so the accumulator is never rescaled (see the pass loop).
//   O^T[col, row] += V^T[col, token] . P^T[token, row]     32 MFMA per 512 cols
//       A = V^T built with ds_read_b64_tr_b16 (LDS transpose read) from the
//       same row-major tile, B = the lane's own probabilities: the token order
//       inside each 16-token k-step is permuted so that the accumulator layout
//       of the score MFMA is directly the operand layout of this one.
//
// LDS layout of a sub-tile: row r (token) holds 72 chunks of 16 B; logical
// chunk c sits at physical chunk c ^ g(r), g(r) = ((r>>1)&1)<<2 | (r>>2)&3,
// which spreads both the score reads (16 rows, same chunk) and the transpose
// reads (4 rows x 4 chunks) over all 64 banks.
#include <cstdlib>

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kD = kDC + kDR;            // 576 elements per row
constexpr int kRowBytes = kD * 2;        // 1152
constexpr int kChunks = kRowBytes / 16;  // 72
constexpr int kSub = 32;                 // tokens per sub-tile
constexpr int kSubBytes = kSub * kRowBytes;   // 36864
constexpr int kSubChunks = kSub * kChunks;    // 2304
constexpr int kStages = 4;
constexpr int kThreads = 256;
constexpr int kDmaPerWave = kSubChunks / 64 / 4;  // 9 DMA instructions per wave per sub-tile
constexpr int kKSteps = kD / 16;         // 36
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kHeadroom = 64.0f;  // log2 units a score may exceed the reference max

__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// byte offset of (row, logical 16-B chunk) inside a sub-tile buffer
__device__ __forceinline__ int tile_off(int r, int c) { return (r * kChunks + (c ^ swz(r))) * 16; }

__device__ __forceinline__ void vm_wait(int n) {
  // s_waitcnt vmcnt(n) with expcnt/lgkmcnt left at their maxima (no wait)
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8) | ((0 >> 4) << 14)); break;
    case 9: __builtin_amdgcn_s_waitcnt((9 & 15) | (7 << 4) | (15 << 8) | ((9 >> 4) << 14)); break;
    default: __builtin_amdgcn_s_waitcnt((18 & 15) | (7 << 4) | (15 << 8) | ((18 >> 4) << 14)); break;
  }
}

__device__ __forceinline__ void block_sync() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// The read-only inputs come as separate __restrict__ arguments so that the
// compiler may read the schedule and the block table through the scalar cache
// (a vector load there would make it wait for every outstanding copy).
template <int RG>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(DecodeArgs a, const int32_t* __restrict__ ws,
                                                                   const int32_t* __restrict__ table,
                                                                   const uint16_t* __restrict__ qc,
                                                                   const uint8_t* __restrict__ cache) {
  constexpr int CG = 4 / RG;   // waves sharing one group of 32 rows (split over O columns)
  constexpr int MB = 16 / CG;  // 32-column blocks of O per wave
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kSubBytes];
  __shared__ int red_flag;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rg = wave / CG, cg = wave % CG;
  const int R = a.Lq * a.H;
  const int n = rg * 32 + (lane & 31);  // query row of this lane's accumulator column
  const bool row_ok = n < R;
  const int jq = row_ok ? n / a.H : 0;  // which new token this row belongs to
  const int hi = lane >> 5;
  const int S = a.splits;
  const int32_t* len = ws + kWsHeader + a.B + 1;

  if (blockIdx.x == 0) mark_empty_sequences(a, tid, blockDim.x);

  SegmentWalker walk;
  walk.init(ws, blockIdx.x);
  if ((int)blockIdx.x >= walk.groups) return;

  // ---- per-lane LDS byte offsets, split so that every per-step term is an
  // immediate: (base register) + (compile-time constant).
  // score operand (A of S^T): row = lane & 31, logical chunk 2*ks + hi.  Since
  // the swizzle only touches the low 3 chunk bits,
  //   chunk(ks) ^ g = 8*(ks >> 2) + ((2*(ks & 3) + hi) ^ g)
  int kbase[4];
  {
    const int r = lane & 31, g = swz(r);
#pragma unroll
    for (int v = 0; v < 4; ++v) kbase[v] = r * kRowBytes + 16 * ((2 * v + hi) ^ g);
  }
  // transpose operand (A of O^T): this lane supplies row 16*kk + 8*h + tr_row,
  // columns 32*mb + tr_col .. +3 (8 bytes).  With sw = g(tr_row) ^ (h << 1):
  //   chunk ^ sw = 4*(mb ^ (sw >> 2)) + (y ^ (sw & 3)),  y = tr_col >> 3
  // and the mb ^ bit swap is folded into one base per (h, mb parity).
  int vbase[2][2];
  {
    const int g16 = lane >> 4, j16 = lane & 15;
    const int tr_row = 4 * (g16 >> 1) + (j16 >> 2);
    const int y = 2 * (g16 & 1) + ((j16 & 3) >> 1);
    const int s2 = (swz(tr_row) >> 2) & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sw = swz(tr_row) ^ (h << 1);
      const int b0 = tr_row * kRowBytes + 16 * (y ^ (sw & 3)) + 8 * (j16 & 1) + 64 * (cg * MB);
#pragma unroll
      for (int par = 0; par < 2; ++par) vbase[h][par] = b0 + (s2 ? (par ? -64 : 64) : 0);
    }
  }
  // DMA source offsets inside a sub-tile for this lane's 9 instructions
  int dma_src[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int q = (wave + 4 * i) * 64 + lane;  // destination 16-B slot
    const int r = q / kChunks, pc = q - r * kChunks;
    dma_src[i] = r * kRowBytes + (pc ^ swz(r)) * 16;
  }

  Segment seg;
  while (walk.next(seg)) {
    const int b = seg.b;
    const int L = len[b];
    const int n_sub = (seg.tok_end - seg.tok_begin + kSub - 1) / kSub;
    const int32_t* trow = table + (size_t)b * a.max_blocks;

    // Copy sub-tile `sub` of this range into its stage buffer.  The LDS-DMA
    // load is written as inline asm so that the compiler does not treat every
    // later LDS read as a possible alias of the in-flight copy (it would then
    // wait for all outstanding copies before each sub-tile); the explicit
    // vmcnt waits and barriers in the main loop order every buffer access.
    auto issue = [&](int sub) {
      const int t = seg.tok_begin + sub * kSub;
      int blk = trow[t / a.block_size];
      blk = min(max(blk, 0), a.num_blocks - 1);
      const uint8_t* base = cache + ((size_t)blk * a.block_size + (t % a.block_size)) * kRowBytes;
      const uint32_t dst = (uint32_t)(uintptr_t)smem + (sub & (kStages - 1)) * kSubBytes + wave * 1024;
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) {
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst + 4096 * i);
        __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(dma_src[i]), "s"(base), "{m0}"(m0)
                         : "memory");
      }
    };

    // queries of this sequence as the B operand of the score MFMA: lane holds
    // q_cat[row n][16 ks + 8 hi .. +7].  Lanes past the last row read row 0;
    // their results are never stored.
    bf16x8 q[kKSteps];
    {
      const uint16_t* qrow = qc + ((size_t)b * R + (row_ok ? n : 0)) * kD + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        q[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 16 * ks));
    }

    const float qk_scale = a.scale * kLog2e;
    const int lim_row = row_ok ? min(seg.tok_end, L - a.Lq + jq + 1) : 0;  // exclusive token bound
    const int lim_all = min(seg.tok_end, L - a.Lq + 1);  // bound every row satisfies

    f32x16 o[MB];
    float m = -INFINITY, l = 0.f;
    float m_seen = -INFINITY;  // largest scaled score of this row in the range
    // The reference max m of each row is fixed at the first sub-tile where the
    // row has a visible key, so the accumulator is never rescaled.  Scores up to
    // 2^kHeadroom above m keep every sum finite in float32; if any row exceeds
    // that, the whole range is processed again with m = m_seen.
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) o[mb] = f32x16{};
      l = 0.f;
      m = pass ? m_seen : -INFINITY;
      bool overflow = false;
      for (int s = 0; s < min(3, n_sub); ++s) issue(s);

      for (int i = 0; i < n_sub; ++i) {
        const int t0 = seg.tok_begin + i * kSub;
        const int left = n_sub - 1 - i;
        vm_wait(left >= 2 ? 18 : left * 9);
        block_sync();
        uint8_t* buf = smem + (i & (kStages - 1)) * kSubBytes;
        if (t0 + kSub > seg.tok_end) {
          // rows past the sequence end hold unspecified data (possibly NaN): zero them
          const int first = seg.tok_end - t0;
          for (int q2 = first * kChunks + tid; q2 < kSubChunks; q2 += kThreads)
            *reinterpret_cast<uint4*>(buf + q2 * 16) = make_uint4(0, 0, 0, 0);
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
          block_sync();
        }
        if (i + 3 < n_sub) issue(i + 3);

        // per-iteration operand bases, made opaque so the compiler keeps one
        // register per base and folds every per-step term into the immediate
        // offset of the LDS read instead of precomputing one address per step
        const int stage_off = (i & (kStages - 1)) * kSubBytes;
        int kb[4], vb[2][2];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          kb[v] = stage_off + kbase[v];
          __asm__ volatile("" : "+v"(kb[v]));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int par = 0; par < 2; ++par) {
            vb[h][par] = stage_off + vbase[h][par];
            __asm__ volatile("" : "+v"(vb[h][par]));
          }

        // ---- scores S^T = K . Q^T (32 tokens x 32 rows); operands fetched two
        // steps ahead, order pinned with scheduling barriers
        f32x16 sacc = f32x16{};
        {
          constexpr int kAhead = 4;
          bf16x8 kop[kAhead];
          auto kload = [&](int ks) {
            return *reinterpret_cast<const bf16x8*>(smem + kb[ks & 3] + 128 * (ks >> 2));
          };
#pragma unroll
          for (int ks = 0; ks < kAhead - 1; ++ks) kop[ks] = kload(ks);
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) {
            if (ks + kAhead - 1 < kKSteps) kop[(ks + kAhead - 1) % kAhead] = kload(ks + kAhead - 1);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks % kAhead], q[ks], sacc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // ---- softmax weights (base 2); lane holds tokens 8*(r/4) + 4*hi + r%4 of
        // row n.  Only a sub-tile that reaches past some row's last visible
        // token needs masking; that test is uniform over the workgroup.
        if (t0 + kSub > lim_all) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tok = t0 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (tok >= lim_row) sacc[r] = -INFINITY;
          }
        }
        float tmax = __builtin_fmaxf(__builtin_fmaxf(sacc[0], sacc[1]), __builtin_fmaxf(sacc[2], sacc[3]));
#pragma unroll
        for (int r = 4; r < 16; r += 2) tmax = __builtin_fmaxf(tmax, __builtin_fmaxf(sacc[r], sacc[r + 1]));
        tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * qk_scale;  // scale > 0 keeps the order
        m_seen = __builtin_fmaxf(m_seen, tmax);
        if (m == -INFINITY) m = tmax;  // nothing accumulated yet for this row
        overflow |= tmax > m + kHeadroom;
        const float neg_m = (m == -INFINITY) ? 0.f : -m;
        float psum = 0.f;
        bf16x8 pb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // 2^(s * scale * log2 e - m); the hardware exp2 flushes tiny results to 0
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], qk_scale, neg_m));
          psum += p;
          pb[r >> 3][r & 7] = (__bf16)p;
        }
        l += psum + __shfl_xor(psum, 32, 64);

        // ---- O^T += V^T . P^T over this wave's columns; step st = (mb, kk)
        {
          constexpr int kSteps = 2 * MB;
          constexpr int kAhead = 4;
          bf16x8 vop[kAhead];
          auto vload = [&](int st) {
            const int mb = st >> 1, kk = st & 1;
            const int imm = 16 * kk * kRowBytes + 64 * mb;
            const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + vb[0][mb & 1] + imm));
            const bf16x4 v1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + vb[1][mb & 1] + imm + 8 * kRowBytes));
            return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          };
#pragma unroll
          for (int st = 0; st < kAhead - 1; ++st) vop[st] = vload(st);
#pragma unroll
          for (int st = 0; st < kSteps; ++st) {
            if (st + kAhead - 1 < kSteps) vop[(st + kAhead - 1) % kAhead] = vload(st + kAhead - 1);
            o[st >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[st % kAhead], pb[st & 1], o[st >> 1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // every wave must be done with the buffers before they are refilled, and
      // the workgroup agrees on whether a second pass is needed
      if (tid == 0) red_flag = 0;
      block_sync();
      if (overflow && row_ok) red_flag = 1;
      __builtin_amdgcn_s_waitcnt(0xc07f);
      block_sync();
      if (red_flag == 0) break;
      block_sync();
    }

    // ---- epilogue: o_s = O / l, lse_s = (m + log2 l) ln 2
    if (row_ok) {
      const size_t prow = ((size_t)b * R + n) * S;
      if (l > 0.f) {
        const float inv = 1.f / l;
        float* op = a.o_part + (prow + seg.split) * kDC;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int c0 = (cg * MB + mb) * 32 + 4 * hi;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float4 v = make_float4(o[mb][4 * g] * inv, o[mb][4 * g + 1] * inv, o[mb][4 * g + 2] * inv,
                                   o[mb][4 * g + 3] * inv);
            *reinterpret_cast<float4*>(op + c0 + 8 * g) = v;
          }
        }
        if (cg == 0 && hi == 0) a.lse_part[prow + seg.split] = (m + log2f(l)) * kLn2;
      } else if (cg == 0 && hi == 0) {
        a.lse_part[prow + seg.split] = -INFINITY;
      }
      if (seg.split == 0 && cg == 0 && hi == 0)
        for (int s2 = seg.nsplits; s2 < S; ++s2) a.lse_part[prow + s2] = -INFINITY;
    }
  }
}

// ===================================================================================
// Eight-wave variant: 16 query rows per wave, MFMA 16x16x32, two waves per SIMD.
// Same stage buffers and DMA as above; O (16 rows x 512) and the queries (16 x
// 576) take 200 of a wave's 256 registers, and the second wave on each SIMD
// hides the other's softmax and LDS latency.  LDS swizzle for this access
// pattern: logical chunk c of row r sits at c ^ f(r), f(r) = ((r>>1)&3)<<1 |
// (r>>3)&1, conflict-free for 16-row score reads and 8-row x 2-chunk transpose
// reads.
constexpr int kThreads16 = 512;
constexpr int kKSteps16 = kD / 32;  // 18

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz16(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }

template <int RG>
__global__ __launch_bounds__(kThreads16, 1) void decode_mfma16_kernel(DecodeArgs a, const int32_t* __restrict__ ws,
                                                                       const int32_t* __restrict__ table,
                                                                       const uint16_t* __restrict__ qc,
                                                                       const uint8_t* __restrict__ cache) {
  constexpr int CG = 8 / RG;   // waves sharing one group of 16 rows (split over O columns)
  constexpr int MB = 32 / CG;  // 16-column blocks of O per wave
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kSubBytes];
  __shared__ int red_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lives in a scalar register
  const int rg = wave / CG, cg = wave % CG;
  const int R = a.Lq * a.H;
  const int g = lane >> 4, j16 = lane & 15;
  const int n = rg * 16 + j16;  // query row of this lane's accumulator column
  const bool row_ok = n < R;
  const int jq = row_ok ? n / a.H : 0;
  const int S = a.splits;
  const int32_t* len = ws + kWsHeader + a.B + 1;

  if (blockIdx.x == 0) mark_empty_sequences(a, tid, blockDim.x);

  SegmentWalker walk;
  walk.init(ws, blockIdx.x);
  if ((int)blockIdx.x >= walk.groups) return;

  // score operand: row j16 (+16 for the second token block), logical chunk 4 ks + g
  //   (4 ks + g) ^ f = 8 (ks >> 1) + ((4 (ks & 1) + g) ^ f)
  int kbase[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) kbase[par] = j16 * kRowBytes + 16 * ((4 * par + g) ^ swz16(j16));
  // transpose operand supplier: row 16 h + 4 g + (j16 >> 2), columns 16 cb + 4 (j16 & 3)
  //   chunk 2 cb + y, y = (j16 & 3) >> 1:  (2 cb + y) ^ f = 8 (cb >> 2) + ((2 (cb & 3) + y) ^ f)
  int vbase[4];
  {
    const int rr = 4 * g + (j16 >> 2), y = (j16 & 3) >> 1, f = swz16(rr);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) vbase[c4] = rr * kRowBytes + 16 * ((2 * c4 + y) ^ f) + 8 * (j16 & 1);
  }
  // DMA: 36 instructions per sub-tile, instruction k = wave + 8 i
  constexpr int kDma16 = (kSubChunks / 64 + 7) / 8;  // 5
  int dma_src[kDma16];
#pragma unroll
  for (int i = 0; i < kDma16; ++i) {
    const int q = min((wave + 8 * i) * 64 + lane, kSubChunks - 1);
    const int r = q / kChunks, pc = q - r * kChunks;
    dma_src[i] = r * kRowBytes + (pc ^ swz16(r)) * 16;
  }
  const int n_dma = (wave + 8 * (kDma16 - 1) < kSubChunks / 64) ? kDma16 : kDma16 - 1;  // 5 for waves 0-3

  Segment seg;
  while (walk.next(seg)) {
    const int b = seg.b;
    const int L = len[b];
    const int n_sub = (seg.tok_end - seg.tok_begin + kSub - 1) / kSub;
    const int32_t* trow = table + (size_t)b * a.max_blocks;

    auto issue = [&](int sub) {
      const int t = seg.tok_begin + sub * kSub;
      int blk = trow[t / a.block_size];
      blk = min(max(blk, 0), a.num_blocks - 1);
      const uint8_t* base = cache + ((size_t)blk * a.block_size + (t % a.block_size)) * kRowBytes;
      const uint32_t dst = (uint32_t)(uintptr_t)smem + (sub & (kStages - 1)) * kSubBytes + wave * 1024;
#pragma unroll
      for (int i = 0; i < kDma16; ++i) {
        if (i < n_dma) {
          const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst + 8192 * i);
          __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(dma_src[i]), "s"(base), "{m0}"(m0)
                           : "memory");
        }
      }
    };

    bf16x8 q[kKSteps16];
    {
      const uint16_t* qrow = qc + ((size_t)b * R + (row_ok ? n : 0)) * kD + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKSteps16; ++ks)
        q[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 32 * ks));
    }

    const float qk_scale = a.scale * kLog2e;
    const int lim_row = row_ok ? min(seg.tok_end, L - a.Lq + jq + 1) : 0;
    const int lim_all = min(seg.tok_end, L - a.Lq + 1);

    f32x4 o[MB];
    float m = -INFINITY, l = 0.f, m_seen = -INFINITY;
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int cb = 0; cb < MB; ++cb) o[cb] = f32x4{};
      l = 0.f;
      m = pass ? m_seen : -INFINITY;
      bool overflow = false;
      for (int s2 = 0; s2 < min(3, n_sub); ++s2) issue(s2);

      for (int i = 0; i < n_sub; ++i) {
        const int t0 = seg.tok_begin + i * kSub;
        const int left = n_sub - 1 - i;
        // this wave's outstanding copies: n_dma per later sub-tile already issued
        if (n_dma == kDma16) {
          if (left >= 2) __builtin_amdgcn_s_waitcnt((10 & 15) | (7 << 4) | (15 << 8));
          else if (left == 1) __builtin_amdgcn_s_waitcnt((5 & 15) | (7 << 4) | (15 << 8));
          else __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
        } else {
          if (left >= 2) __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));
          else if (left == 1) __builtin_amdgcn_s_waitcnt((4 & 15) | (7 << 4) | (15 << 8));
          else __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
        }
        block_sync();
        uint8_t* buf = smem + (i & (kStages - 1)) * kSubBytes;
        if (t0 + kSub > seg.tok_end) {
          const int first = seg.tok_end - t0;
          for (int q2 = first * kChunks + tid; q2 < kSubChunks; q2 += kThreads16)
            *reinterpret_cast<uint4*>(buf + q2 * 16) = make_uint4(0, 0, 0, 0);
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
          block_sync();
        }
        if (i + 3 < n_sub) issue(i + 3);

        // kbase/vbase track the current stage buffer (advanced at the end of the
        // iteration); the empty asm keeps each one a single register
        int* kb = kbase;
        int* vb = vbase;
#pragma unroll
        for (int v = 0; v < 2; ++v) __asm__ volatile("" : "+v"(kb[v]));
#pragma unroll
        for (int v = 0; v < 4; ++v) __asm__ volatile("" : "+v"(vb[v]));

        // ---- scores: two 16-token blocks, 18 k-steps each
        f32x4 s0 = f32x4{}, s1 = f32x4{};
        {
          constexpr int kAhead = 2;
          bf16x8 k0[kAhead], k1[kAhead];
          auto kload = [&](int ks, int blk) {
            return *reinterpret_cast<const bf16x8*>(smem + kb[ks & 1] + 128 * (ks >> 1) + blk * 16 * kRowBytes);
          };
#pragma unroll
          for (int ks = 0; ks < kAhead - 1; ++ks) {
            k0[ks] = kload(ks, 0);
            k1[ks] = kload(ks, 1);
          }
#pragma unroll
          for (int ks = 0; ks < kKSteps16; ++ks) {
            if (ks + kAhead - 1 < kKSteps16) {
              k0[(ks + kAhead - 1) % kAhead] = kload(ks + kAhead - 1, 0);
              k1[(ks + kAhead - 1) % kAhead] = kload(ks + kAhead - 1, 1);
            }
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[ks % kAhead], q[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[ks % kAhead], q[ks], s1, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // ---- softmax weights; lane holds tokens 4 g + e (s0) and 16 + 4 g + e (s1) of row n
        if (t0 + kSub > lim_all) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (t0 + 4 * g + e >= lim_row) s0[e] = -INFINITY;
            if (t0 + 16 + 4 * g + e >= lim_row) s1[e] = -INFINITY;
          }
        }
        float tmax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(s0[0], s0[1]), __builtin_fmaxf(s0[2], s0[3])),
                                     __builtin_fmaxf(__builtin_fmaxf(s1[0], s1[1]), __builtin_fmaxf(s1[2], s1[3])));
        tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * qk_scale;
        m_seen = __builtin_fmaxf(m_seen, tmax);
        if (m == -INFINITY) m = tmax;
        overflow |= tmax > m + kHeadroom;
        const float neg_m = (m == -INFINITY) ? 0.f : -m;
        float psum = 0.f;
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[e], qk_scale, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[e], qk_scale, neg_m));
          psum += p0 + p1;
          pb[e] = (__bf16)p0;
          pb[4 + e] = (__bf16)p1;
        }
        psum += __shfl_xor(psum, 16, 64);
        l += psum + __shfl_xor(psum, 32, 64);

        // ---- O^T += V^T . P^T, one 32-token k-step per 16-column block
        {
          constexpr int kAhead = 3;
          bf16x8 vop[kAhead];
          auto vload = [&](int cb) {
            const int c = cg * MB + cb;
            const int off = vb[c & 3] + 128 * (c >> 2);
            const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + off));
            const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + off + 16 * kRowBytes));
            return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          };
#pragma unroll
          for (int cb = 0; cb < kAhead - 1; ++cb) vop[cb] = vload(cb);
#pragma unroll
          for (int cb = 0; cb < MB; ++cb) {
            if (cb + kAhead - 1 < MB) vop[(cb + kAhead - 1) % kAhead] = vload(cb + kAhead - 1);
            o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[cb % kAhead], pb, o[cb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // next stage buffer: +1 stage, wrapping after the last one
        const int step = ((i & (kStages - 1)) == kStages - 1) ? -(kStages - 1) * kSubBytes : kSubBytes;
#pragma unroll
        for (int v = 0; v < 2; ++v) kbase[v] += step;
#pragma unroll
        for (int v = 0; v < 4; ++v) vbase[v] += step;
      }
      // back to stage 0 for a second pass or the next range
      const int back = ((n_sub - 1) & (kStages - 1)) + 1;
      const int rewind = (back == kStages) ? 0 : back * kSubBytes;
#pragma unroll
      for (int v = 0; v < 2; ++v) kbase[v] -= rewind;
#pragma unroll
      for (int v = 0; v < 4; ++v) vbase[v] -= rewind;
      if (tid == 0) red_flag = 0;
      block_sync();
      if (overflow && row_ok) red_flag = 1;
      __builtin_amdgcn_s_waitcnt(0xc07f);
      block_sync();
      if (red_flag == 0) break;
      block_sync();
    }

    if (row_ok) {
      const size_t prow = ((size_t)b * R + n) * S;
      if (l > 0.f) {
        const float inv = 1.f / l;
        float* op = a.o_part + (prow + seg.split) * kDC;
#pragma unroll
        for (int cb = 0; cb < MB; ++cb) {
          const int c0 = (cg * MB + cb) * 16 + 4 * g;
          *reinterpret_cast<float4*>(op + c0) =
              make_float4(o[cb][0] * inv, o[cb][1] * inv, o[cb][2] * inv, o[cb][3] * inv);
        }
        if (cg == 0 && g == 0) a.lse_part[prow + seg.split] = (m + log2f(l)) * kLn2;
      } else if (cg == 0 && g == 0) {
        a.lse_part[prow + seg.split] = -INFINITY;
      }
      if (seg.split == 0 && cg == 0 && g == 0)
        for (int s2 = seg.nsplits; s2 < S; ++s2) a.lse_part[prow + s2] = -INFINITY;
    }
  }
}

// ===================================================================================
// Software-pipelined four-wave kernel (the default).  Per sub-tile i, the
// softmax of sub-tile i (VALU) is interleaved with the score MFMAs of
// sub-tile i+1, then the latent-sum MFMAs of sub-tile i run.  The matrix
// instructions are written as inline asm so that their register classes are
// fixed: the output accumulators stay in AGPRs for the whole range and the
// score accumulators in VGPRs, which leaves room for the two score tiles in
// flight.  The compiler does not see these as MFMAs, so the wait states a
// VALU read of an MFMA result needs are inserted explicitly (pad_mfma) where
// such a read can follow closely.

__device__ __forceinline__ void mfma_v0(f32x16& d, const bf16x8& a, const bf16x8& b) {
  __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& d, const bf16x8& a, const bf16x8& b) {
  __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a(f32x16& d, const bf16x8& a, const bf16x8& b) {
  __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// 64 wait states: more than any MFMA result latency on this part
__device__ __forceinline__ void pad_mfma() {
  __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
// value of lane l ^ 32 combined with this lane's value (v_permlane32_swap, no LDS)
__device__ __forceinline__ float xmax32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int RG>
__global__ __launch_bounds__(kThreads, 1) void decode_pipe_kernel(DecodeArgs a, const int32_t* __restrict__ ws,
                                                                   const int32_t* __restrict__ table,
                                                                   const uint16_t* __restrict__ qc,
                                                                   const uint8_t* __restrict__ cache) {
  constexpr int CG = 4 / RG;   // waves sharing one group of 32 rows (split over O columns)
  constexpr int MB = 16 / CG;  // 32-column blocks of O per wave
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kSubBytes];
  __shared__ int red_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave / CG, cg = wave % CG;
  const int R = a.Lq * a.H;
  const int n = rg * 32 + (lane & 31);
  const bool row_ok = n < R;
  const int jq = row_ok ? n / a.H : 0;
  const int hi = lane >> 5;
  const int S = a.splits;
  const int32_t* len = ws + kWsHeader + a.B + 1;

  if (blockIdx.x == 0) mark_empty_sequences(a, tid, blockDim.x);

  SegmentWalker walk;
  walk.init(ws, blockIdx.x);
  if ((int)blockIdx.x >= walk.groups) return;

  int kbase[4];
  {
    const int r = lane & 31, g = swz(r);
#pragma unroll
    for (int v = 0; v < 4; ++v) kbase[v] = r * kRowBytes + 16 * ((2 * v + hi) ^ g);
  }
  int vbase[2][2];
  {
    const int g16 = lane >> 4, j16 = lane & 15;
    const int tr_row = 4 * (g16 >> 1) + (j16 >> 2);
    const int y = 2 * (g16 & 1) + ((j16 & 3) >> 1);
    const int s2 = (swz(tr_row) >> 2) & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sw = swz(tr_row) ^ (h << 1);
      const int b0 = tr_row * kRowBytes + 16 * (y ^ (sw & 3)) + 8 * (j16 & 1) + 64 * (cg * MB);
#pragma unroll
      for (int par = 0; par < 2; ++par) vbase[h][par] = b0 + (s2 ? (par ? -64 : 64) : 0);
    }
  }
  int dma_src[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int q = (wave + 4 * i) * 64 + lane;
    const int r = q / kChunks, pc = q - r * kChunks;
    dma_src[i] = r * kRowBytes + (pc ^ swz(r)) * 16;
  }

  Segment seg;
  while (walk.next(seg)) {
    const int b = seg.b;
    const int L = len[b];
    const int n_sub = (seg.tok_end - seg.tok_begin + kSub - 1) / kSub;
    const int32_t* trow = table + (size_t)b * a.max_blocks;

    auto issue = [&](int sub) {
      const int t = seg.tok_begin + sub * kSub;
      int blk = trow[t / a.block_size];
      blk = min(max(blk, 0), a.num_blocks - 1);
      const uint8_t* base = cache + ((size_t)blk * a.block_size + (t % a.block_size)) * kRowBytes;
      const uint32_t dst = (uint32_t)(uintptr_t)smem + (sub & (kStages - 1)) * kSubBytes + wave * 1024;
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) {
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst + 4096 * i);
        __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(dma_src[i]), "s"(base), "{m0}"(m0)
                         : "memory");
      }
    };
    // rows of a sub-tile past the sequence end hold unspecified data: zero them
    auto fix_partial = [&](int sub) {
      const int t0 = seg.tok_begin + sub * kSub;
      if (t0 + kSub > seg.tok_end) {
        uint8_t* buf = smem + (sub & (kStages - 1)) * kSubBytes;
        for (int q2 = (seg.tok_end - t0) * kChunks + tid; q2 < kSubChunks; q2 += kThreads)
          *reinterpret_cast<uint4*>(buf + q2 * 16) = make_uint4(0, 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        block_sync();
      }
    };

    bf16x8 q[kKSteps];
    {
      const uint16_t* qrow = qc + ((size_t)b * R + (row_ok ? n : 0)) * kD + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        q[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 16 * ks));
    }

    const float qk_scale = a.scale * kLog2e;
    const int lim_row = row_ok ? min(seg.tok_end, L - a.Lq + jq + 1) : 0;
    const int lim_all = min(seg.tok_end, L - a.Lq + 1);

    f32x16 o[MB];
    float m = -INFINITY, l = 0.f, m_seen = -INFINITY;

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) o[mb] = f32x16{};
      l = 0.f;
      m = pass ? m_seen : -INFINITY;
      bool overflow = false;
      for (int s2 = 0; s2 < min(3, n_sub); ++s2) issue(s2);

      // score operand bases for a stage
      auto kbases = [&](int stage, int* kb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          kb[v] = stage * kSubBytes + kbase[v];
          __asm__ volatile("" : "+v"(kb[v]));
        }
      };
      auto kload = [&](const int* kb, int ks) {
        return *reinterpret_cast<const bf16x8*>(smem + kb[ks & 3] + 128 * (ks >> 2));
      };

      // ---- prologue: sub-tile 0 ready, its scores computed
      vm_wait(min(2, n_sub - 1) * 9);
      block_sync();
      fix_partial(0);
      f32x16 sc;
      {
        int kb[4];
        kbases(0, kb);
        constexpr int kAhead = 4;
        bf16x8 kop[kAhead];
#pragma unroll
        for (int ks = 0; ks < kAhead - 1; ++ks) kop[ks] = kload(kb, ks);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          if (ks + kAhead - 1 < kKSteps) kop[(ks + kAhead - 1) % kAhead] = kload(kb, ks + kAhead - 1);
          if (ks == 0) mfma_v0(sc, kop[0], q[0]);
          else mfma_v(sc, kop[ks % kAhead], q[ks]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      pad_mfma();
      __asm__ volatile("" : "+v"(sc));  // no read of sc may move above the padding

      for (int i = 0; i < n_sub; ++i) {
        const int t0 = seg.tok_begin + i * kSub;
        const bool nxt = i + 1 < n_sub;
        if (nxt) {
          vm_wait(i + 2 < n_sub ? 9 : 0);
          block_sync();  // sub-tile i+1 landed; every wave is past PV(i-1)
          fix_partial(i + 1);
        }
        if (i + 3 < n_sub) issue(i + 3);

        // masking of sub-tile i (rare: only where some row's last visible token falls inside)
        if (t0 + kSub > lim_all) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tok = t0 + 8 * (r >> 2) + 4 * hi + (r & 3);
            sc[r] = tok < lim_row ? sc[r] : -INFINITY;
          }
        }

        // ---- softmax(i) in pieces, interleaved with the scores of sub-tile i+1
        float tm = 0.f, neg_m = 0.f, psum = 0.f;
        bf16x8 pb[2];
        auto piece = [&](int k) {
          if (k == 0) tm = __builtin_fmaxf(__builtin_fmaxf(sc[0], sc[1]), __builtin_fmaxf(sc[2], sc[3]));
          if (k >= 1 && k <= 3) {
            tm = __builtin_fmaxf(tm, __builtin_fmaxf(sc[4 * k], sc[4 * k + 1]));
            tm = __builtin_fmaxf(tm, __builtin_fmaxf(sc[4 * k + 2], sc[4 * k + 3]));
          }
          if (k == 4) {
            tm = xmax32(tm) * qk_scale;  // scale > 0 keeps the order
            m_seen = __builtin_fmaxf(m_seen, tm);
            if (m == -INFINITY) m = tm;  // nothing accumulated yet for this row
            overflow |= tm > m + kHeadroom;
            neg_m = (m == -INFINITY) ? 0.f : -m;
          }
          if (k >= 5 && k < 21) {
            const int r = k - 5;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], qk_scale, neg_m));
            psum += p;
            pb[r >> 3][r & 7] = (__bf16)p;
          }
          if (k == 21) l += xsum32(psum);
        };
        constexpr int kPieces = 22;

        f32x16 sn;
        if (nxt) {
          int kb[4];
          kbases((i + 1) & (kStages - 1), kb);
          constexpr int kAhead = 4;
          bf16x8 kop[kAhead];
#pragma unroll
          for (int ks = 0; ks < kAhead - 1; ++ks) kop[ks] = kload(kb, ks);
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) {
            if (ks + kAhead - 1 < kKSteps) kop[(ks + kAhead - 1) % kAhead] = kload(kb, ks + kAhead - 1);
            if (ks == 0) mfma_v0(sn, kop[0], q[0]);
            else mfma_v(sn, kop[ks % kAhead], q[ks]);
            if (ks < kPieces) piece(ks);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int k = 0; k < kPieces; ++k) piece(k);
        }
        __asm__ volatile("s_nop 4" ::: "memory");  // VALU-written pb before its MFMA reads

        // ---- O^T += V^T . P^T for sub-tile i over this wave's columns
        {
          int vb[2][2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int par = 0; par < 2; ++par) {
              vb[h][par] = (i & (kStages - 1)) * kSubBytes + vbase[h][par];
              __asm__ volatile("" : "+v"(vb[h][par]));
            }
          constexpr int kSteps = 2 * MB;
          constexpr int kAhead = 4;
          bf16x8 vop[kAhead];
          auto vload = [&](int st) {
            const int mb = st >> 1, kk = st & 1;
            const int imm = 16 * kk * kRowBytes + 64 * mb;
            const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + vb[0][mb & 1] + imm));
            const bf16x4 v1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + vb[1][mb & 1] + imm + 8 * kRowBytes));
            return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          };
#pragma unroll
          for (int st = 0; st < kAhead - 1; ++st) vop[st] = vload(st);
#pragma unroll
          for (int st = 0; st < kSteps; ++st) {
            if (st + kAhead - 1 < kSteps) vop[(st + kAhead - 1) % kAhead] = vload(st + kAhead - 1);
            mfma_a(o[st >> 1], vop[st % kAhead], pb[st & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (nxt) {
          // sn was last written by an MFMA before the PV block; this empty asm
          // (ordered after the PV asm) keeps the copy from being hoisted into
          // the MFMA's shadow
          __asm__ volatile("" : "+v"(sn));
          sc = sn;
        }
      }
      pad_mfma();  // the output accumulators are read by VALU below
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) __asm__ volatile("" : "+a"(o[mb]));

      if (tid == 0) red_flag = 0;
      block_sync();
      if (overflow && row_ok) red_flag = 1;
      __builtin_amdgcn_s_waitcnt(0xc07f);
      block_sync();
      if (red_flag == 0) break;
      block_sync();
    }

    if (row_ok) {
      const size_t prow = ((size_t)b * R + n) * S;
      if (l > 0.f) {
        const float inv = 1.f / l;
        float* op = a.o_part + (prow + seg.split) * kDC;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int c0 = (cg * MB + mb) * 32 + 4 * hi;
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            float4 v = make_float4(o[mb][4 * gg] * inv, o[mb][4 * gg + 1] * inv, o[mb][4 * gg + 2] * inv,
                                   o[mb][4 * gg + 3] * inv);
            *reinterpret_cast<float4*>(op + c0 + 8 * gg) = v;
          }
        }
        if (cg == 0 && hi == 0) a.lse_part[prow + seg.split] = (m + log2f(l)) * kLn2;
      } else if (cg == 0 && hi == 0) {
        a.lse_part[prow + seg.split] = -INFINITY;
      }
      if (seg.split == 0 && cg == 0 && hi == 0)
        for (int s2 = seg.nsplits; s2 < S; ++s2) a.lse_part[prow + s2] = -INFINITY;
    }
  }
}

}  // namespace

bool decode_mfma_supported(const mla_dims& d) {
  const int R = d.q_len * d.num_heads;
  return d.dtype == MLA_BF16 && d.d_c == kDC && d.d_rope == kDR && d.block_size % kSub == 0 &&
         (R == 128 || R == 64 || R <= 32);
}

hipError_t launch_decode_mfma(const mla_dims& d, const void* q_cat, const void* cache, const int32_t* table,
                              const int32_t* ws, float scale, int splits, int grid, float* o_part, float* lse_part,
                              hipStream_t stream) {
  DecodeArgs a{q_cat, cache, table, ws, o_part, lse_part, scale, d.batch, d.q_len, d.num_heads, d.d_c, d.d_rope,
               d.block_size, d.max_blocks_per_seq, d.num_blocks, splits};
  const int R = d.q_len * d.num_heads;
  const uint16_t* qc = static_cast<const uint16_t*>(q_cat);
  const uint8_t* kv = static_cast<const uint8_t*>(cache);
  const char* v = std::getenv("MLA_DECODE_VARIANT");
  const int variant = v ? v[0] - '0' : 0;
  if (variant == 0) {
    if (R == 128)
      hipLaunchKernelGGL(decode_pipe_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, a, ws, table, qc, kv);
    else if (R == 64)
      hipLaunchKernelGGL(decode_pipe_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, a, ws, table, qc, kv);
    else
      hipLaunchKernelGGL(decode_pipe_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, a, ws, table, qc, kv);
  } else if (variant == 4) {
    if (R == 128)
      hipLaunchKernelGGL(decode_mfma_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, a, ws, table, qc, kv);
    else if (R == 64)
      hipLaunchKernelGGL(decode_mfma_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, a, ws, table, qc, kv);
    else
      hipLaunchKernelGGL(decode_mfma_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, a, ws, table, qc, kv);
  } else {
    if (R == 128)
      hipLaunchKernelGGL(decode_mfma16_kernel<8>, dim3(grid), dim3(kThreads16), 0, stream, a, ws, table, qc, kv);
    else if (R == 64)
      hipLaunchKernelGGL(decode_mfma16_kernel<4>, dim3(grid), dim3(kThreads16), 0, stream, a, ws, table, qc, kv);
    else if (R > 16)
      hipLaunchKernelGGL(decode_mfma16_kernel<2>, dim3(grid), dim3(kThreads16), 0, stream, a, ws, table, qc, kv);
    else
      hipLaunchKernelGGL(decode_mfma16_kernel<1>, dim3(grid), dim3(kThreads16), 0, stream, a, ws, table, qc, kv);
  }
  return hipGetLastError();
}

}  // namespace mla
