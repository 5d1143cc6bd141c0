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
// computed.  With 32 query rows or fewer the four waves share the rows and
// split the output columns; their common query block is then copied once per
// piece into the fourth buffer (free until sub-tile 3) and read from there.
// With head groups (DecodeArgs::hg_log2) a scheduled "sequence" is one group
// of heads of a real sequence, whose block-table row it reads.
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
// The softmax of sub-tile i is interleaved with the score MFMAs of sub-tile
// i+1, then the latent-sum MFMAs of sub-tile i run.  The matrix instructions
// are inline asm so that their register classes are fixed: the output
// accumulators stay in AGPRs for the whole range and the score accumulators in
// VGPRs, which leaves room for two score tiles in flight.  The compiler does
// not see these as MFMAs, so the wait states a VALU read of an MFMA result
// needs are inserted explicitly (pad_mfma) where such a read can follow.
//
// LDS layout of a sub-tile: row r (token) holds 72 chunks of 16 B; logical
// chunk c sits at physical chunk c ^ g(r), g(r) = ((r>>1)&1)<<2 | (r>>2)&3,
// which spreads both the score reads (16 rows, same chunk) and the transpose
// reads (4 rows x 4 chunks) over all 64 banks.
//
// FP8 cache (E4M3 codes, one scale per cache; "Deconstructing DeepSeek V4
// Pro", Practical Deployment: the latent tolerates FP8): a 32-token sub-tile
// is 18 KiB of contiguous codes, copied HBM -> LDS by the same copy engine
// into a ring of eight FP8 stages (seven sub-tiles ahead, as many bytes in
// flight as the bf16 path).  A stage is 18 blocks of 1 KiB, each 16 token
// rows x 64 bytes of codes with the 16-byte chunks of a row XOR-permuted by
// the row, so every 1 KiB copy reads 16 contiguous 64-byte row segments and
// neither operand read has LDS bank conflicts: the score operand (8 codes of
// one row) is a ds_read_b64, and the latent-sum operand (8 tokens of one
// column) a ds_read_b64_tr_b8, the 8-bit transpose read.  Each operand is
// converted to bf16 in registers right before its
// MFMA (E4M3 values are exact in bf16, so the matrix products see exactly
// the cached values and run in the same order as on a bf16 cache), and
// nothing but the codes ever goes through LDS.  Rows past the range are
// zeroed in the stage.  The scale multiplies the softmax scale and the
// partial result.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace mla {
namespace {

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
// LDS operand ring depth of the score and latent-sum loops (reads issued this
// many steps ahead of their MFMA; deeper rings measured slower)
constexpr int kOperandAhead = 4;
// FP8 cache: 576-byte rows, an 18 KiB sub-tile copied in 18 pieces of 1 KiB
// (five per wave; the last two pieces of waves 2 and 3 go to the sink)
constexpr int kF8Row = kD;                       // 576
constexpr int kF8Sub = kSub * kF8Row;            // 18432
constexpr int kF8Pieces = kF8Sub / 1024;         // 18
constexpr int kF8DmaPerWave = 5;
constexpr int kF8Chunks = kF8Sub / 16;           // 1152 16-byte chunks per sub-tile
constexpr int kF8Stages = 8;                     // FP8 ring (144 KiB)
constexpr int kF8Ahead = 7;                      // sub-tile i + 7 is copied while sub-tile i + 1 is scored

// byte offset of (row, logical 16-B chunk) inside a sub-tile buffer
__device__ __forceinline__ int tile_off(int r, int c) { return (r * kChunks + (c ^ swz(r))) * 16; }

// wait until at most `tiles` sub-tiles of N copies each are still in flight
template <int N>
__device__ __forceinline__ void vm_wait_tiles(int tiles) {  // tiles in {0, 1, 2}
  switch (tiles) {
    case 0: vm_wait<0>(); break;
    case 1: vm_wait<N>(); break;
    default: vm_wait<2 * N>(); break;
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

// The read-only inputs come as separate __restrict__ arguments so that the
// compiler may read the schedule through the scalar cache.
template <int RG, bool F8>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(DecodeArgs a, const int32_t* __restrict__ ws,
                                                                   const int32_t* __restrict__ table,
                                                                   const uint16_t* __restrict__ qc,
                                                                   const uint8_t* __restrict__ cache) {
  constexpr int CG = 4 / RG;   // waves sharing one group of 32 rows (split over O columns)
  constexpr int MB = 16 / CG;  // 32-column blocks of O per wave
  // the copy ring: four bf16 sub-tiles, or eight FP8 ones
  constexpr int kDmaN = F8 ? kF8DmaPerWave : kDmaPerWave;  // copies per wave per sub-tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[F8 ? kF8Stages * kF8Sub : kStages * kSubBytes];
  // sink for the copies issued when there is no sub-tile left to fetch (so
  // that the score loop carries no per-step condition); never read
  __shared__ __attribute__((aligned(1024))) uint8_t sink[kThreads / 64 * 1024];
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
  const int32_t* len = ws + kWsCu + a.B + 1;
  // a schedule planned for another batch (or head grouping) is never walked
  if (ws[6] != a.B) return;

  if (blockIdx.x == 0) mark_empty_sequences(a, tid, blockDim.x);

  const int w = xcd_local_index(blockIdx.x, gridDim.x);
  SegmentWalker walk;
  walk.init(ws, w);
  if (w >= walk.groups) return;

  // Per-lane LDS byte offsets inside a sub-tile (held in registers):
  //   score operand v (logical chunk 2 v + hi of row r = lane & 31):
  //     r * 1152 + 16 ((2 v + hi) ^ g(r))
  //   transpose operand (h, mb parity par): this lane supplies row
  //     16 kk + 8 h + tr_row, columns 32 mb + tr_col .. +3; with
  //     sw = g(tr_row) ^ (h << 1) the swizzled chunk is
  //     4 (mb ^ (sw >> 2)) + (y ^ (sw & 3)), y = tr_col >> 3, and the mb ^ bit
  //     swap is folded into one base per (h, mb parity).
  int kbase_r[4];
  {
    const int r = lane & 31;
#pragma unroll
    for (int v = 0; v < 4; ++v) kbase_r[v] = r * kRowBytes + 16 * ((2 * v + hi) ^ swz(r));
  }
  int vbase_r[2][2];
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
      for (int par = 0; par < 2; ++par) vbase_r[h][par] = b0 + (s2 ? (par ? -64 : 64) : 0);
    }
  }
  auto kbase = [&](int v) { return kbase_r[v]; };
  auto vbase = [&](int h, int par) { return vbase_r[h][par]; };
  // FP8 stage offsets: 16-code chunk c of row r lies in 1 KiB block
  // 9 (r >> 4) + (c >> 2) (16 rows x 4 chunks), at slot 4 (r & 15) + ((c & 3)
  // ^ ((r >> 2) & 3)) of 16 bytes (f8_off).
  //   score operand: codes 16 ks + 8 hi .. + 7 of row lane & 31 at
  //     f8_kbase[ks & 3] + 1024 (ks >> 2);
  //   latent-sum operand (8-bit transpose read): in each group of 16 lanes,
  //     lane j reads 8 codes of token row tau(hi, j >> 1), columns 16 (g & 1)
  //     + 8 (j & 1) .. + 7 of 32-column block cb, and after the transpose
  //     holds column (lane & 31) of the block for the 8 tokens tau(hi, 0..7),
  //     tau(hi, t) = 4 hi + t + 4 (t >> 2): exactly the token order of the
  //     lane's probabilities.  Block cb (parity par) of tokens 16 kk .. is
  //     at f8_vbase[par] + 1024 (9 kk + (cb >> 1)).
  // A wave's 16-lane quarter of either read covers 16 distinct slot columns
  // of 4 bytes x 2, so no two of its lanes share an LDS bank.
  int f8_kbase[4];
  {
    const int r = lane & 31, rl = r & 15;
#pragma unroll
    for (int v = 0; v < 4; ++v) f8_kbase[v] = 1024 * 9 * (r >> 4) + 16 * (4 * rl + (v ^ ((rl >> 2) & 3))) + 8 * hi;
  }
  int f8_vbase[2];
  {
    const int g16 = lane >> 4, j16 = lane & 15, t = j16 >> 1, half = g16 & 1;
    const int tau = 4 * (g16 >> 1) + t + 4 * (t >> 2);
#pragma unroll
    for (int par = 0; par < 2; ++par)
      f8_vbase[par] = 16 * (4 * tau + ((2 * par + half) ^ ((tau >> 2) & 3))) + 8 * (j16 & 1) + 1024 * (cg * MB / 2);
  }
  // Source offset inside a sub-tile of this lane's part of copy piece i:
  // the piece fills physical chunk q = 64 (wave + 4 i) + lane, which holds
  // logical chunk (q mod 72) ^ g(r) of row r = q / 72.  Recomputed per copy
  // (a few integer ops) rather than kept in nine registers.
  const int q_lane = wave * 64 + lane;
  auto dma_src = [&](int i) {
    const int q = q_lane + 256 * i;
    if constexpr (F8) {
      // FP8 piece k = q >> 6 fills block k (rows 16 (k / 9) .., chunks
      // 4 (k % 9) ..): slot lane = 4 rl + s holds chunk s ^ ((rl >> 2) & 3) of
      // row rl, so each piece reads 16 contiguous 64-byte row segments.
      // Pieces past the 18th re-read the first blocks (into the sink).
      const int k0 = q >> 6, k = k0 < kF8Pieces ? k0 : k0 - kF8Pieces;
      const int rb = k >= 9 ? 1 : 0, cgk = k - 9 * rb;
      const int rl = lane >> 2, c = 4 * cgk + ((lane & 3) ^ ((rl >> 2) & 3));
      return (16 * rb + rl) * kF8Row + 16 * c;
    } else {
      const int r = (q * 1821) >> 17;  // q / 72 for 0 <= q < 2304
      const int pc = q - r * kChunks;
      return r * kRowBytes + ((pc ^ swz(r)) << 4);
    }
  };

  // Block-table window of a segment: lane j holds the physical block of the
  // segment's j-th block (j < 64).  The next segment's window is requested
  // while the current one starts, so the copies never wait on a table read.
  auto table_window = [&](const Segment& s) -> int {
    const int j0 = s.tok_begin / a.block_size;
    const int nblk = (s.tok_end - 1) / a.block_size - j0 + 1;
    return table[(size_t)(s.b >> a.hg_log2) * a.max_blocks + j0 + min(lane, nblk - 1)];
  };
  Segment seg, nseg;
  bool have = walk.next(seg);
  int tv = have ? table_window(seg) : 0;
  bool first_seg = true;
  while (have) {
    const bool have_next = walk.next(nseg);
    const int b = seg.b;
    const int L = len[b];
    const int n_sub = (seg.tok_end - seg.tok_begin + kSub - 1) / kSub;
    const int32_t* trow = table + (size_t)(b >> a.hg_log2) * a.max_blocks;
    const int j0 = seg.tok_begin / a.block_size;

    // Copy of one sub-tile: the source row address (uniform) and this wave's
    // nine 1 KiB pieces of it.  The pieces of a sub-tile copied during the
    // score loop are spread over its MFMAs so that the address unit works in
    // the background instead of stalling the wave.
    auto tile_src = [&](int sub) -> const uint8_t* {
      const int t = seg.tok_begin + sub * kSub;
      const int j = t / a.block_size - j0;
      int blk = (j < 64) ? __builtin_amdgcn_readlane(tv, j) : trow[t / a.block_size];
      blk = min(max(blk, 0), a.num_blocks - 1);
      return cache + ((size_t)blk * a.block_size + (t % a.block_size)) * (F8 ? kF8Row : kRowBytes);
    };
    // The cache rows are read exactly once, so the copies are marked
    // non-temporal (measured 1-5 % faster from a cold cache, more when the
    // caches hold dirty lines).  src is the lane's source offset (dma_src).
    auto dma_at = [&](const uint8_t* base, uint32_t dst, uint32_t stride, int i, int src) {
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst + stride * i);
      __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(src), "s"(base), "{m0}"(m0)
                       : "memory");
    };
    auto dma_to = [&](const uint8_t* base, uint32_t dst, uint32_t stride, int i) {
      dma_at(base, dst, stride, i, dma_src(i));
    };
    // LDS byte address of the copy destination of sub-tile sub: its ring stage
    auto stage_addr = [&](int sub) -> uint32_t {
      if constexpr (F8) return (uint32_t)(uintptr_t)smem + (sub & (kF8Stages - 1)) * kF8Sub;
      else return (uint32_t)(uintptr_t)smem + (sub & (kStages - 1)) * kSubBytes;
    };
    // byte offset of sub-tile t's stage in smem
    auto stage_off = [&](int t) -> int {
      if constexpr (F8) return (t & (kF8Stages - 1)) * kF8Sub;
      else return (t & (kStages - 1)) * kSubBytes;
    };
    // piece i of this wave lands at stage + 1 KiB * (wave + 4 i), except the
    // FP8 pieces past the 18th, which go to the sink
    auto dma = [&](const uint8_t* base, int sub, int i) {
      const bool to_sink = F8 && wave + 4 * i >= kF8Pieces;  // uniform: a select, not a branch
      dma_to(base, to_sink ? (uint32_t)(uintptr_t)sink + wave * 1024 : stage_addr(sub) + wave * 1024,
             to_sink ? 0u : 4096u, i);
    };
    auto issue = [&](int sub) {
      const uint8_t* base = tile_src(sub);
#pragma unroll
      for (int i = 0; i < kDmaN; ++i) dma(base, sub, i);
    };
    // E4M3 codes -> bf16 (exact): word x's codes 0, 1 or 2, 3 -> two bf16, the first in the low half
    auto cv_lo = [](uint32_t x) {
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
    };
    auto cv_hi = [](uint32_t x) {
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
    };
    auto cvt8 = [&](const uint2& x) -> bf16x8 {
      return __builtin_bit_cast(bf16x8, make_uint4(cv_lo(x.x), cv_hi(x.x), cv_lo(x.y), cv_hi(x.y)));
    };
    // rows of a sub-tile past the sequence end hold unspecified data: zero them
    auto fix_partial = [&](int sub) {
      const int t0 = seg.tok_begin + sub * kSub;
      if (t0 + kSub > seg.tok_end) {
        uint8_t* buf = smem + stage_off(sub);
        const int nv = seg.tok_end - t0;  // rows kept
        if constexpr (F8) {
          // rows nv .. 31 of every chunk column, at their slots
          for (int z = tid; z < (kSub - nv) * (kF8Row / 16); z += kThreads) {
            const int c = z / (kSub - nv), r = nv + z % (kSub - nv), rl = r & 15;
            const int off = 1024 * (9 * (r >> 4) + (c >> 2)) + 16 * (4 * rl + ((c & 3) ^ ((rl >> 2) & 3)));
            *reinterpret_cast<uint4*>(buf + off) = make_uint4(0, 0, 0, 0);
          }
        } else {
          for (int q2 = nv * kChunks + tid; q2 < kSubChunks; q2 += kThreads)
            *reinterpret_cast<uint4*>(buf + q2 * 16) = make_uint4(0, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        block_sync();
      }
    };

    // With 32 rows or fewer (RG = 1) all four waves need the same query rows:
    // instead of four loads of the same 37 KB, the block is copied once into
    // the fourth ring stage (free until sub-tile 3 is copied, after the first
    // loop barrier) with the sub-tile layout, and every wave reads its
    // operands from there, as it reads cache rows.
    constexpr bool kQLds = !F8 && RG == 1;
    bf16x8 q[kKSteps];
    if constexpr (!kQLds) {
      const uint16_t* qrow = qc + ((size_t)b * R + (row_ok ? n : 0)) * kD + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        q[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 16 * ks));
    }
    // in issue order: [this window (first segment only)] [36 query loads]
    // [next window]; the first copy needs this window
    const int tv_next = have_next ? table_window(nseg) : 0;
    if (first_seg) {
      constexpr int kQLoads = kQLds ? 0 : kKSteps;
      if (have_next) vm_wait<kQLoads + 1>();
      else vm_wait<kQLoads>();
      first_seg = false;
    }
    // source offset of this lane's part of query-block copy piece i: the
    // sub-tile layout over rows 0 .. 31 of the sequence, rows past R
    // repeating row R - 1 (never read past the sequence's rows)
    auto q_src = [&](int i) {
      const int qq = q_lane + 256 * i;
      const int r = (qq * 1821) >> 17;  // qq / 72
      const int pc = qq - r * kChunks;
      return min(r, R - 1) * kRowBytes + ((pc ^ swz(r)) << 4);
    };

    const float qk_scale = a.scale * (F8 ? a.kv_scale : 1.f) * kLog2e;
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
      // copies of the last real sub-tile into the sink keep every wait count
      // below a constant when there is no sub-tile left to fetch
      auto issue_or_sink = [&](int sub) {
        if (sub < n_sub) {
          issue(sub);
        } else {
          const uint8_t* base = tile_src(n_sub - 1);
#pragma unroll
          for (int i2 = 0; i2 < kDmaN; ++i2) dma_to(base, (uint32_t)(uintptr_t)sink + wave * 1024, 0, i2);
        }
      };
      if constexpr (F8) {
        // sub-tiles 0 .. 6, the missing ones as sink copies: the number of
        // copies issued after any sub-tile is then the same constant
#pragma unroll
        for (int s2 = 0; s2 < kF8Ahead; ++s2) issue_or_sink(s2);
      } else if (kQLds && pass == 0) {
        // sub-tile 0, the query block, then sub-tiles 1 and 2: the wait for
        // sub-tile 0 below also covers the query block
        issue(0);
        const uint8_t* qbase = reinterpret_cast<const uint8_t*>(qc + (size_t)b * R * kD);
#pragma unroll
        for (int i = 0; i < kDmaN; ++i) dma_at(qbase, stage_addr(3) + wave * 1024, 4096u, i, q_src(i));
        for (int s2 = 1; s2 < min(3, n_sub); ++s2) issue(s2);
      } else {
        for (int s2 = 0; s2 < min(3, n_sub); ++s2) issue(s2);
      }

      // score operand bases for a stage
      auto kbases = [&](int stage, int* kb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          kb[v] = stage * kSubBytes + kbase(v);
          __asm__ volatile("" : "+v"(kb[v]));
        }
      };
      auto kload = [&](const int* kb, int ks) {
        return *reinterpret_cast<const bf16x8*>(smem + kb[ks & 3] + 128 * (ks >> 2));
      };
      // FP8: the 8 codes of score step ks, and the stage base they are read from
      auto kload8 = [&](const int* kb8, int ks) {
        return *reinterpret_cast<const uint2*>(smem + kb8[ks & 3] + 1024 * (ks >> 2));
      };
      auto kbase8 = [&](int t, int* kb8) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          kb8[v] = stage_off(t) + f8_kbase[v];
          __asm__ volatile("" : "+v"(kb8[v]));
        }
      };

      // ---- prologue: sub-tile 0 ready, its scores computed
      if constexpr (F8) {
        vm_wait<(kF8Ahead - 1) * kDmaN>();  // this wave's copies of sub-tile 0 landed
        block_sync();
        fix_partial(0);
      } else {
        vm_wait_tiles<kDmaN>(min(2, n_sub - 1));
        block_sync();
        fix_partial(0);
        if constexpr (kQLds) {
          if (pass == 0) {
            int kq[4];
            kbases(3, kq);
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) q[ks] = kload(kq, ks);
          }
        }
      }
      f32x16 sc;
      if constexpr (F8) {
        int kb8[4];
        kbase8(0, kb8);
        constexpr int kAhead = 4;
        uint2 kop[kAhead];
#pragma unroll
        for (int ks = 0; ks < kAhead - 1; ++ks) kop[ks] = kload8(kb8, ks);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          if (ks + kAhead - 1 < kKSteps) kop[(ks + kAhead - 1) % kAhead] = kload8(kb8, ks + kAhead - 1);
          if (ks == 0) mfma_v0(sc, cvt8(kop[0]), q[0]);
          else mfma_v(sc, cvt8(kop[ks % kAhead]), q[ks]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
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
          if constexpr (F8) {
            // sub-tiles i+2 .. i+6 (real or sink copies) may still be in flight
            vm_wait<(kF8Ahead - 2) * kDmaN>();
            block_sync();  // sub-tile i+1 landed; every wave is past PV(i-1)
            fix_partial(i + 1);
          } else {
            vm_wait_tiles<kDmaN>(i + 2 < n_sub ? 1 : 0);
            block_sync();  // sub-tile i+1 landed; every wave is past PV(i-1)
            fix_partial(i + 1);
          }
        }
        // Sub-tile i+3 (FP8: i+7) is copied during the score loop below, one
        // 1 KiB piece every fourth (FP8: seventh) MFMA: a wave can queue only a
        // few copies, and a burst of nine would stall it for their whole
        // transfer.  When there is no such sub-tile the copies re-read the
        // last sub-tile (an L2 hit) into the sink, so every step issues the
        // same code and every wait count (vmcnt) is the same constant, the
        // sink's copies included.  The FP8 stage of sub-tile i+7 is that of
        // sub-tile i-1, free once every wave is past PV(i-1).
        constexpr int kAheadCopy = F8 ? kF8Ahead : 3;  // sub-tile copied during this score loop
        const bool copy_on = i + kAheadCopy < n_sub;
        const uint8_t* copy_src = tile_src(copy_on ? i + kAheadCopy : n_sub - 1);
        const uint32_t copy_dst =
            copy_on ? stage_addr(i + kAheadCopy) + wave * 1024 : (uint32_t)(uintptr_t)sink + wave * 1024;
        const uint32_t copy_stride = copy_on ? 4096u : 0u;
        int src_next = 0;

        // masking of sub-tile i (rare: only where some row's last visible token falls inside)
        if (t0 + kSub > lim_all) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tok = t0 + 8 * (r >> 2) + 4 * hi + (r & 3);
            sc[r] = tok < lim_row ? sc[r] : -INFINITY;
          }
        }

        // ---- softmax(i) in pieces, interleaved with the scores of sub-tile i+1.
        // The wave issues in order, so a piece must not wait on a result it
        // produced itself in front of the next MFMA: every instruction of a
        // piece reads only values made at least one piece (one MFMA) earlier.
        // The row maximum is a tree of independent max3s; score r is scaled
        // and shifted in piece 13 + r, exponentiated in the next piece and
        // summed and packed to bf16 in the one after.
        float tm = 0.f, neg_m = 0.f, psum = 0.f, mn = 0.f, hr = 0.f;
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, a4 = 0.f, b0 = 0.f, b1 = 0.f;
        uint32_t sw0 = 0u, sw1 = 0u;
        float xs[16], pv[16];
        uint32_t pw[8];  // P as bf16 pairs: word w holds scores 2w (low) and 2w + 1
        bf16x8 pb[2];
        auto piece = [&](int k) {
          if (k == 0) a0 = max3f(sc[0], sc[1], sc[2]);
          if (k == 1) a1 = max3f(sc[3], sc[4], sc[5]);
          if (k == 2) a2 = max3f(sc[6], sc[7], sc[8]);
          if (k == 3) a3 = max3f(sc[9], sc[10], sc[11]);
          if (k == 4) a4 = max3f(sc[12], sc[13], sc[14]);
          if (k == 5) b0 = max3f(a0, a1, a2);
          if (k == 6) b1 = max3f(a3, a4, sc[15]);
          if (k == 7) tm = max3f(b0, b1, b1);
          if (k == 8 || k == 31) {  // exchange with the lane holding the other half of the row
            const uint32_t x = __float_as_uint(k == 8 ? tm : psum);
            auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
            sw0 = r[0];
            sw1 = r[1];
          }
          if (k == 9) tm = max3f(__uint_as_float(sw0), __uint_as_float(sw1), __uint_as_float(sw1));
          if (k == 10) tm *= qk_scale;  // scale > 0 keeps the order
          if (k == 11) {
            m_seen = max3f(m_seen, tm, tm);
            mn = (m == -INFINITY) ? tm : m;  // nothing accumulated yet for this row
          }
          if (k == 12) {
            hr = mn + kHeadroom;
            neg_m = (mn == -INFINITY) ? 0.f : -mn;
            m = mn;
          }
          if (k == 13) overflow |= tm > hr;
          if (k >= 13 && k < 31) {
            const int j = k - 13;
            if (j < 16) {
              xs[j] = __builtin_fmaf(sc[j], qk_scale, neg_m);
              pin(xs[j]);
            }
            if (j >= 1 && j <= 16) {
              pv[j - 1] = __builtin_amdgcn_exp2f(xs[j - 1]);
              pin(pv[j - 1]);
            }
            if (j >= 2) {
              const int r = j - 2;
              psum += pv[r];
              if (r & 1) {
                pw[r >> 1] = pack_bf16(pv[r - 1], pv[r]);
                pin(pw[r >> 1]);
              }
            }
          }
          if (k == 32) l += __uint_as_float(sw0) + __uint_as_float(sw1);
        };
        constexpr int kPieces = 33;

        f32x16 sn;
        if (nxt) {
          constexpr int kAhead = kOperandAhead;
          int kb[4];
          if constexpr (F8) kbase8(i + 1, kb);
          else kbases((i + 1) & (kStages - 1), kb);
          using KOp = std::conditional_t<F8, uint2, bf16x8>;
          KOp kop[kAhead];
          auto kld = [&](int ks) -> KOp {
            if constexpr (F8) return kload8(kb, ks);
            else return kload(kb, ks);
          };
          auto kcv = [&](const KOp& x) -> bf16x8 {
            if constexpr (F8) return cvt8(x);
            else return x;
          };
#pragma unroll
          for (int ks = 0; ks < kAhead - 1; ++ks) kop[ks] = kld(ks);
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) {
            if (ks + kAhead - 1 < kKSteps) kop[(ks + kAhead - 1) % kAhead] = kld(ks + kAhead - 1);
            if (ks == 0) mfma_v0(sn, kcv(kop[0]), q[0]);
            else mfma_v(sn, kcv(kop[ks % kAhead]), q[ks]);
            if (ks < kPieces) piece(ks);
            if constexpr (F8) {
              // five 1 KiB pieces, the source offset one MFMA ahead of its copy
              if (ks % 7 == 1 && ks / 7 < kDmaN) {
                src_next = dma_src(ks / 7);
                pin(src_next);
              }
              if (ks % 7 == 2 && ks / 7 < kDmaN) {
                const int pc = ks / 7;
                const bool to_sink = wave + 4 * pc >= kF8Pieces;  // uniform: a select, not a branch
                dma_at(copy_src, to_sink ? (uint32_t)(uintptr_t)sink + wave * 1024 : copy_dst,
                       to_sink ? 0u : copy_stride, pc, src_next);
              }
            } else {
              // the source offset of a copy is computed one MFMA earlier, so
              // that the copy never waits on its own address arithmetic
              if (ks % 4 == 1) {
                src_next = dma_src(ks / 4);
                pin(src_next);
              }
              if (ks % 4 == 2) dma_at(copy_src, copy_dst, copy_stride, ks / 4, src_next);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int k = 0; k < kPieces; ++k) piece(k);
        }
        pb[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        pb[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
        __asm__ volatile("s_nop 4" ::: "memory");  // VALU-written pb before its MFMA reads

        // ---- O^T += V^T . P^T for sub-tile i over this wave's columns
        if constexpr (F8) {
          int vb8[2];
#pragma unroll
          for (int par = 0; par < 2; ++par) {
            vb8[par] = stage_off(i) + f8_vbase[par];
            __asm__ volatile("" : "+v"(vb8[par]));
          }
          constexpr int kSteps = 2 * MB;
          constexpr int kAhead = kOperandAhead;
          uint2 vop[kAhead];
          auto vload = [&](int st) {
            const int mb = st >> 1, kk = st & 1;
            const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2*)(smem + vb8[mb & 1] + 1024 * (9 * kk + (mb >> 1))));
            return make_uint2((uint32_t)v.x, (uint32_t)v.y);
          };
#pragma unroll
          for (int st = 0; st < kAhead - 1; ++st) vop[st] = vload(st);
#pragma unroll
          for (int st = 0; st < kSteps; ++st) {
            if (st + kAhead - 1 < kSteps) vop[(st + kAhead - 1) % kAhead] = vload(st + kAhead - 1);
            mfma_a(o[st >> 1], cvt8(vop[st % kAhead]), pb[st & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          int vb[2][2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int par = 0; par < 2; ++par) {
              vb[h][par] = stage_off(i) + vbase(h, par);
              __asm__ volatile("" : "+v"(vb[h][par]));
            }
          constexpr int kSteps = 2 * MB;
          constexpr int kAhead = kOperandAhead;
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
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the clear lands before any wave sets the flag
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
        // o_s rounded once to bf16 (the storage type of the partials)
        const float inv = (F8 ? a.kv_scale : 1.f) / l;
        uint16_t* op = static_cast<uint16_t*>(a.o_part) + (prow + seg.split) * kDC;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int c0 = (cg * MB + mb) * 32 + 4 * hi;
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const uint2 v = make_uint2(pack_bf16(o[mb][4 * gg] * inv, o[mb][4 * gg + 1] * inv),
                                       pack_bf16(o[mb][4 * gg + 2] * inv, o[mb][4 * gg + 3] * inv));
            *reinterpret_cast<uint2*>(op + c0 + 8 * gg) = v;
          }
        }
        if (cg == 0 && hi == 0) a.lse_part[prow + seg.split] = (m + log2f(l)) * kLn2;
      } else if (cg == 0 && hi == 0) {
        a.lse_part[prow + seg.split] = -INFINITY;
      }
      if (seg.split == 0 && cg == 0 && hi == 0)
        for (int s2 = seg.nsplits; s2 < S; ++s2) a.lse_part[prow + s2] = -INFINITY;
    }
    seg = nseg;
    tv = tv_next;
    have = have_next;
  }
  // The last sub-tiles' copies into the sink may still be in flight: let them
  // land before the workgroup's LDS is handed to another workgroup.
  vm_wait<0>();
}

}  // namespace

bool decode_mfma_supported(const mla_dims& d) {
  const int R = d.q_len * d.num_heads;
  return d.dtype == MLA_BF16 && d.d_c == kDC && d.d_rope == kDR && d.block_size % kSub == 0 &&
         (R == 128 || R == 64 || R <= 32);
}

hipError_t launch_decode_mfma(const mla_dims& d, const void* q_cat, const void* cache, const int32_t* table,
                              const int32_t* ws, float scale, int splits, int grid, void* o_part, float* lse_part,
                              hipStream_t stream, bool fp8, float kv_scale, int hg_log2) {
  DecodeArgs a{q_cat, cache, table, ws, o_part, lse_part, scale, d.batch, d.q_len, d.num_heads, d.d_c, d.d_rope,
               d.block_size, d.max_blocks_per_seq, d.num_blocks, splits, kv_scale, hg_log2};
  const int R = d.q_len * d.num_heads;
  const uint16_t* qc = static_cast<const uint16_t*>(q_cat);
  const uint8_t* kv = static_cast<const uint8_t*>(cache);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, stream, a, ws, table, qc, kv);
  };
  if (fp8) {
    if (R == 128) go(decode_mfma_kernel<4, true>);
    else if (R == 64) go(decode_mfma_kernel<2, true>);
    else go(decode_mfma_kernel<1, true>);
  } else {
    if (R == 128) go(decode_mfma_kernel<4, false>);
    else if (R == 64) go(decode_mfma_kernel<2, false>);
    else go(decode_mfma_kernel<1, false>);
  }
  return hipGetLastError();
}

}  // namespace mla
