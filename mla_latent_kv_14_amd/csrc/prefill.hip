// Prefill (training forward) of MLA attention over whole packed sequences.
//
// Non-absorbed form ("Deconstructing DeepSeek V4 Pro", the forward pass of
// its MLA module; "DeepSeek-V3 MLA: Multi-Head Latent Attention Guide",
// forward_train): every token's latent is up-projected per head,
//   K_{t,h} = [W^UK_h c_t ; k^R_t],   V_{t,h} = W^UV_h c_t,
// and u_{j,h} = softmax_t(scale q_{j,h} . K_{t,h}) V_{t,h} over the tokens t
// of j's sequence (t <= j when causal).  With as many queries as keys this
// costs d_nope + d_rope + d_v = 320 multiply-adds per (query, key, head)
// against the absorbed form's 2 d_c + d_rope = 1088, so prefill up-projects.
//
// Workspace (bf16 storage): Kn [T][H][d_nope] | V [T][H][d_v] | R [T][d_rope]
// (R a copy of k^R, so that every byte of a key row lies at a 32-bit offset
// from the workspace base, which the LDS-DMA copies address from).
//
// Matrix-core path (bf16, d_c = 512, d_rope = 64, d_nope = d_v = 128):
//   upproject_mfma  Kn = c_kv . W_UK^T and V = c_kv . W_UV^T as NT GEMMs
//                   (T x 512 times 512 x 128 H), 128 x 128 output tiles, both
//                   operands staged in LDS by the LDS-DMA path, 2 x 2 MFMA
//                   tiles per wave, the output tile written out through LDS
//                   in 256-B row segments; it also copies k^R into R.
//   attn_mfma       one workgroup per (sequence, head, 256-query block),
//                   eight waves of 32 queries.  32-key tiles [Kn | V | k^R]
//                   (640 B per key) go HBM -> LDS once per workgroup in a
//                   ring of four; scores S^T = K Q^T (12 MFMA 32x32x16 per
//                   tile and wave), softmax in base 2 against a reference max
//                   fixed at the first tile (exact two-pass fallback, as in
//                   decode), O^T += V^T P^T (8 MFMA).
// Portable path (float32 or other widths): one thread per output element of
// the up-projection, one workgroup per (query, head) for the attention.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma_util.h"

namespace mla {
namespace {

// ------------------------------------------------------------------ up-projection
// D[m][n] = sum_k A[m][k] B[n][k] with A = c_kv [M x 512] and B = a per-head
// weight viewed as [N x 512] (N = H * 128, row n = h * 128 + d); D is Kn or V
// viewed as [M x N].  The LDS tile of each operand holds 128 rows x 64 k (8
// chunks of 16 B per row); chunk c of row r sits at c ^ ((r >> 1) & 7), which
// puts the 16 rows that one operand read touches on 16 distinct 16-B bank
// groups.  The MFMA computes D^T tiles (A operand = B rows, B operand = A
// rows) so that each lane holds four consecutive n of one row m.
constexpr int kGT = 128;        // tile edge
constexpr int kGK = 64;         // k per stage
constexpr int kGThreads = 256;  // 4 waves: 2 (m halves) x 2 (n halves), 64 x 64 each
constexpr int kGStage = 2 * kGT * kGK * 2;  // A + B stage bytes (32 KiB)
constexpr int kDcP = 512;
constexpr int kDrP = 64;
constexpr int kDnP = 128;

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(kGThreads, 2) void upproject_mfma(const uint16_t* __restrict__ c_kv,
                                                               const uint16_t* __restrict__ w_uk,
                                                               const uint16_t* __restrict__ w_uv,
                                                               const uint16_t* __restrict__ k_rope,
                                                               uint16_t* __restrict__ ws, int M, int N,
                                                               size_t v_off, size_t r_off) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kGStage];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hi = lane >> 5, mh = wave >> 1, nh = wave & 1;
  const int n0 = blockIdx.x * kGT, m0 = blockIdx.y * kGT, which = blockIdx.z;
  const uint16_t* bmat = which ? w_uv : w_uk;
  uint16_t* dmat = which ? ws + v_off : ws;

  // the k^R copy: rows m0 .. m0 + 127, 128 B each, by the first column tile of the Kn GEMM
  if (which == 0 && blockIdx.x == 0) {
    for (int q = tid; q < kGT * (kDrP / 8); q += kGThreads) {
      const int m = m0 + q / (kDrP / 8), c = q % (kDrP / 8);
      if (m < M)
        *reinterpret_cast<uint4*>(ws + r_off + (size_t)m * kDrP + 8 * c) =
            *reinterpret_cast<const uint4*>(k_rope + (size_t)m * kDrP + 8 * c);
    }
  }

  // Stage copy: piece i (0..3) of this wave for operand X fills physical chunks
  // q = 256 i + 64 wave + lane of the 128 x 8-chunk tile: row q >> 3, physical
  // chunk q & 7, logical chunk (q & 7) ^ gswz(row).
  auto copy_stage = [&](int stage, int kc) {
    const uint32_t base = (uint32_t)(uintptr_t)smem + stage * kGStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 256 * i + 64 * wave + lane;
      const int r = q >> 3, lc = (q & 7) ^ gswz(r);
      const int ma = min(m0 + r, M - 1);
      const uint32_t off_a = (uint32_t)(((size_t)ma * kDcP + kc * kGK + 8 * lc) * 2);
      const uint32_t off_b = (uint32_t)(((size_t)(n0 + r) * kDcP + kc * kGK + 8 * lc) * 2);
      const uint32_t da = __builtin_amdgcn_readfirstlane(base + 1024 * (4 * i + wave));
      const uint32_t db = __builtin_amdgcn_readfirstlane(base + kGT * kGK * 2 + 1024 * (4 * i + wave));
      __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off_a), "s"(c_kv), "{m0}"(da) : "memory");
      __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off_b), "s"(bmat), "{m0}"(db) : "memory");
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  // operand read offsets inside a stage: lane row r = lane & 31 of the
  // 32-row MFMA tile; k-step ks reads logical chunk 2 ks + hi
  const int r32 = lane & 31;
  int aoff[2], boff[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int ra = 64 * mh + 32 * t + r32, rb = 64 * nh + 32 * t + r32;
    aoff[t] = ra * kGK * 2;
    boff[t] = kGT * kGK * 2 + rb * kGK * 2;
  }
  auto opnd = [&](int stage, int rowoff, int row, int ks) {
    const int c = (2 * ks + hi) ^ gswz(row);
    return *reinterpret_cast<const bf16x8*>(smem + stage * kGStage + rowoff + 16 * c);
  };

  constexpr int kChunksK = kDcP / kGK;  // 8
  copy_stage(0, 0);
  for (int kc = 0; kc < kChunksK; ++kc) {
    vm_wait<0>();
    block_sync();  // stage kc & 1 landed everywhere; stage (kc + 1) & 1 no longer read
    if (kc + 1 < kChunksK) copy_stage((kc + 1) & 1, kc + 1);
    const int st = kc & 1;
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = opnd(st, aoff[t], 64 * mh + 32 * t + r32, ks);
        bv[t] = opnd(st, boff[t], 64 * nh + 32 * t + r32, ks);
      }
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[tn], av[tm], acc[tn][tm], 0, 0, 0);
    }
  }

  // the output tile goes through LDS so that every store writes 16 B of a
  // 256-B row segment: lane (m = lane & 31, hi) holds, in acc[tn][tm],
  // columns 8 (r >> 2) + 4 hi + (r & 3) of the 32-column tile tn
  block_sync();  // every wave is done with the operand stages
  uint8_t* ot = smem;  // [128 rows][256 B], 16-B chunk c of row r at c ^ (r & 15)
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int r = 64 * mh + 32 * tm + r32;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 64 * nh + 32 * tn + 8 * g + 4 * hi;  // 4 columns = 8 B
        const int c = col >> 3, half = (col >> 2) & 1;
        *reinterpret_cast<uint2*>(ot + r * 256 + ((c ^ (r & 15)) << 4) + 8 * half) =
            make_uint2(pack_bf16(acc[tn][tm][4 * g], acc[tn][tm][4 * g + 1]),
                       pack_bf16(acc[tn][tm][4 * g + 2], acc[tn][tm][4 * g + 3]));
      }
  }
  // the staged tile is read by other waves: this wave's LDS writes must have
  // landed before the barrier (block_sync itself does not wait for them)
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  block_sync();
#pragma unroll
  for (int i = 0; i < (kGT * 16) / kGThreads; ++i) {  // 8 chunks of 16 B per thread
    const int q = i * kGThreads + tid, r = q >> 4, c = q & 15, m = m0 + r;
    if (m < M)
      *reinterpret_cast<uint4*>(dmat + (size_t)m * N + n0 + 8 * c) =
          *reinterpret_cast<const uint4*>(ot + r * 256 + ((c ^ (r & 15)) << 4));
  }
}


// The same product on 256 x 256 output tiles: eight waves, 2 (m halves) x 4
// (n quarters), each 128 x 64 (4 x 2 MFMA tiles of 32 x 32), one workgroup per
// CU.  A tile's operands are 512 KiB for 67 MFLOP, half the bytes per flop of
// the 128 x 128 tile, which is what the operand stream from L2 and the
// last-level cache bounds.  Stage layout as above (256 rows x 64 k per
// operand, chunk c of row r at c ^ ((r >> 1) & 7)); the output tile leaves
// through LDS in 512-B row segments, chunk c of row r at c ^ (r & 31).
constexpr int kHT = 256;
constexpr int kHThreads = 512;
constexpr int kHStage = 2 * kHT * kGK * 2;  // A + B stage bytes (64 KiB)

__global__ __launch_bounds__(kHThreads, 1) void upproject_mfma256(const uint16_t* __restrict__ c_kv,
                                                                  const uint16_t* __restrict__ w_uk,
                                                                  const uint16_t* __restrict__ w_uv,
                                                                  const uint16_t* __restrict__ k_rope,
                                                                  uint16_t* __restrict__ ws, int M, int N,
                                                                  size_t v_off, size_t r_off) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kHStage];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hi = lane >> 5, mh = wave >> 2, nq = wave & 3;
  const int n0 = blockIdx.x * kHT, m0 = blockIdx.y * kHT, which = blockIdx.z;
  const uint16_t* bmat = which ? w_uv : w_uk;
  uint16_t* dmat = which ? ws + v_off : ws;

  // the k^R copy: rows m0 .. m0 + 255, 128 B each, by the first column tile of the Kn GEMM
  if (which == 0 && blockIdx.x == 0) {
    for (int q = tid; q < kHT * (kDrP / 8); q += kHThreads) {
      const int m = m0 + q / (kDrP / 8), c = q % (kDrP / 8);
      if (m < M)
        *reinterpret_cast<uint4*>(ws + r_off + (size_t)m * kDrP + 8 * c) =
            *reinterpret_cast<const uint4*>(k_rope + (size_t)m * kDrP + 8 * c);
    }
  }

  // Stage copy: piece i (0..3) of this wave for operand X fills physical
  // chunks q = 512 i + 64 wave + lane of the 256 x 8-chunk tile: row q >> 3,
  // physical chunk q & 7, logical chunk (q & 7) ^ gswz(row).
  auto copy_stage = [&](int stage, int kc) {
    const uint32_t base = (uint32_t)(uintptr_t)smem + stage * kHStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 512 * i + 64 * wave + lane;
      const int r = q >> 3, lc = (q & 7) ^ gswz(r);
      const int ma = min(m0 + r, M - 1);
      const uint32_t off_a = (uint32_t)(((size_t)ma * kDcP + kc * kGK + 8 * lc) * 2);
      const uint32_t off_b = (uint32_t)(((size_t)(n0 + r) * kDcP + kc * kGK + 8 * lc) * 2);
      const uint32_t da = __builtin_amdgcn_readfirstlane(base + 1024 * (8 * i + wave));
      const uint32_t db = __builtin_amdgcn_readfirstlane(base + kHT * kGK * 2 + 1024 * (8 * i + wave));
      __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off_a), "s"(c_kv), "{m0}"(da) : "memory");
      __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off_b), "s"(bmat), "{m0}"(db) : "memory");
    }
  };

  f32x16 acc[2][4];  // [n tile][m tile]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

  const int r32 = lane & 31;
  auto opnd = [&](int stage, int rowoff, int row, int ks) {
    const int c = (2 * ks + hi) ^ gswz(row);
    return *reinterpret_cast<const bf16x8*>(smem + stage * kHStage + rowoff + 16 * c);
  };

  constexpr int kChunksK = kDcP / kGK;  // 8
  copy_stage(0, 0);
  for (int kc = 0; kc < kChunksK; ++kc) {
    vm_wait<0>();
    block_sync();  // stage kc & 1 landed everywhere; stage (kc + 1) & 1 no longer read
    if (kc + 1 < kChunksK) copy_stage((kc + 1) & 1, kc + 1);
    const int st = kc & 1;
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      bf16x8 av[4], bv[2];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ra = 128 * mh + 32 * t + r32;
        av[t] = opnd(st, ra * kGK * 2, ra, ks);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int rb = 64 * nq + 32 * t + r32;
        bv[t] = opnd(st, kHT * kGK * 2 + rb * kGK * 2, rb, ks);
      }
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[tn], av[tm], acc[tn][tm], 0, 0, 0);
    }
  }

  // lane (m = lane & 31, hi) holds, in acc[tn][tm], columns 8 (r >> 2) + 4 hi
  // + (r & 3) of the 32-column tile tn of its wave
  block_sync();  // every wave is done with the operand stages
  uint8_t* ot = smem;  // [256 rows][512 B]
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
    const int r = 128 * mh + 32 * tm + r32;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 64 * nq + 32 * tn + 8 * g + 4 * hi;  // 4 columns = 8 B
        const int c = col >> 3, half = (col >> 2) & 1;
        *reinterpret_cast<uint2*>(ot + r * 512 + ((c ^ (r & 31)) << 4) + 8 * half) =
            make_uint2(pack_bf16(acc[tn][tm][4 * g], acc[tn][tm][4 * g + 1]),
                       pack_bf16(acc[tn][tm][4 * g + 2], acc[tn][tm][4 * g + 3]));
      }
  }
  // the staged tile is read by other waves: this wave's LDS writes must have
  // landed before the barrier (block_sync itself does not wait for them)
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  block_sync();
#pragma unroll
  for (int i = 0; i < (kHT * 32) / kHThreads; ++i) {  // 16 chunks of 16 B per thread
    const int q = i * kHThreads + tid, r = q >> 5, c = q & 31, m = m0 + r;
    if (m < M)
      *reinterpret_cast<uint4*>(dmat + (size_t)m * N + n0 + 8 * c) =
          *reinterpret_cast<const uint4*>(ot + r * 512 + ((c ^ (r & 31)) << 4));
  }
}

// ------------------------------------------------------------------ attention
// LDS key row (640 B = 40 chunks): Kn (chunks 0-15) | V (16-31) | k^R (32-39),
// chunk c at c ^ swz(row) as in the decode kernel (same row stride modulo
// 256 B, so the same operand and transpose reads are conflict-free).
constexpr int kAThreads = 512;            // 8 waves x 32 queries
constexpr int kAWaves = kAThreads / 64;
constexpr int kQB = 32 * kAWaves;         // queries per workgroup
constexpr int kKT = 32;                   // keys per tile
constexpr int kARow = 640;
constexpr int kAChunks = kARow / 16;      // 40
constexpr int kATile = kKT * kARow;       // 20480
constexpr int kAStages = 4;
constexpr int kACopyWaves = 4;            // waves 0..3 issue the copies
constexpr int kADma = kKT * kAChunks / 64 / kACopyWaves;  // 5 pieces of 1 KiB per copying wave
constexpr int kAKSteps = (kDnP + kDrP) / 16;               // 12
constexpr int kAMB = kDnP / 32;                            // 4 output column blocks
constexpr float kALog2e = 1.4426950408889634f;
constexpr float kALn2 = 0.6931471805599453f;
constexpr float kAHeadroom = 64.0f;

struct PrefillArgs {
  const uint16_t* q_nope;  // [T][H][128]
  const uint16_t* q_rope;  // [T][H][64]
  const uint8_t* ws;       // workspace base
  const int32_t* cu;       // [B + 1]
  uint16_t* out;           // [T][H][128]
  float* lse;              // [T][H] or null
  float scale;
  int T, H, B, nqb, causal;
  uint32_t v_off, r_off;   // byte offsets of V and R in the workspace
};

__device__ __forceinline__ void vm_wait_a(int n) {  // n in {0, 5, 10}
  switch (n) {
    case 0: vm_wait<0>(); break;
    case 5: vm_wait<5>(); break;
    default: vm_wait<10>(); break;
  }
}

__global__ __launch_bounds__(kAThreads, 1) void attn_mfma(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kAStages * kATile];
  __shared__ __attribute__((aligned(1024))) uint8_t sink[kACopyWaves * 1024];  // never read
  __shared__ int red_flag;
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool copier = wave < kACopyWaves;

  // workgroup -> (sequence, head, query block): the query blocks of one
  // (head, sequence) pair are neighbours in the XCD-local order, heaviest
  // first, so their keys share an L2; pairs run head-major, so that each
  // XCD's contiguous share holds a few heads of every sequence and the
  // shares carry equal work whatever the lengths
  const int L = xcd_local_index(blockIdx.x, gridDim.x);
  const int hb = L / a.nqb, qb = a.nqb - 1 - (L - hb * a.nqb);
  const int h = hb / a.B, b = hb - h * a.B;
  const int s0 = min(max(a.cu[b], 0), a.T);
  const int s1 = min(max(a.cu[b + 1], s0), a.T);
  const int Lb = s1 - s0, q0 = qb * kQB;
  if (q0 >= Lb) return;
  const int n_keys = a.causal ? min(q0 + kQB, Lb) : Lb;
  const int n_sub = (n_keys + kKT - 1) / kKT;

  const int r32 = lane & 31;
  const int qrow = q0 + 32 * wave + r32;  // this lane's query, inside the sequence
  const bool row_ok = qrow < Lb;
  const int lim_row = row_ok ? (a.causal ? qrow + 1 : Lb) : 0;  // keys [0, lim_row) are visible
  const int lim_all = a.causal ? min(q0 + 32 * wave + 1, Lb) : Lb;  // smallest limit of the wave's rows
  const float qk_scale = a.scale * kALog2e;

  // query operands: k-step ks < 8 from q_nope, 8..11 from q_rope
  bf16x8 q[kAKSteps];
  {
    const size_t tq = (size_t)(s0 + min(qrow, Lb - 1)) * a.H + h;
    const uint16_t* qn = a.q_nope + tq * kDnP + 8 * hi;
    const uint16_t* qr = a.q_rope + tq * kDrP + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kAKSteps; ++ks)
      q[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ks < 8 ? qn + 16 * ks : qr + 16 * (ks - 8)));
  }

  // copies: piece i of copying wave w fills physical chunk p = 256 i + 64 w + lane of a
  // tile: key row p / 40, physical chunk p % 40, logical chunk (p % 40) ^ swz(row)
  // Per lane and piece (fixed for the workgroup): the source as base + token *
  // stride.  One register packs, for each piece, the key row inside the tile
  // (5 bits) and whether the chunk lies in k^R (1 bit); the token is below
  // 2^24 (the workspace is below 4 GiB), so the product is a 24-bit multiply.
  uint32_t cp_meta = 0u, cp_base[kADma];
#pragma unroll
  for (int i = 0; i < kADma; ++i) {
    const int p = 256 * i + 64 * min(wave, kACopyWaves - 1) + lane;
    const int r = p / kAChunks, pc = p - r * kAChunks;
    const int lc = pc ^ swz(r);
    const bool isr = lc >= 32;
    cp_meta |= (uint32_t)(r | (isr ? 32 : 0)) << (6 * i);
    cp_base[i] = isr ? a.r_off + 16 * (lc - 32)
                     : (lc >= 16 ? a.v_off : 0u) + (uint32_t)h * (kDnP * 2) + 16 * (lc & 15);
  }
  const uint32_t kv_stride = (uint32_t)a.H * (kDnP * 2);
  auto dma_src = [&](int t0, int i) -> uint32_t {
    const uint32_t mi = cp_meta >> (6 * i);
    const int tok = min(s0 + t0 + (int)(mi & 31), s0 + Lb - 1);
    return cp_base[i] + __umul24((uint32_t)tok, (mi & 32) ? (uint32_t)(kDrP * 2) : kv_stride);
  };
  auto dma_to = [&](int t0, uint32_t dst, uint32_t stride, int i) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst + stride * i);
    __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(dma_src(t0, i)), "s"(a.ws), "{m0}"(m0)
                     : "memory");
  };
  auto issue = [&](int sub, auto copy_tag) {
    if constexpr (!decltype(copy_tag)::value) return;
#pragma unroll
    for (int i = 0; i < kADma; ++i)
      dma_to(sub * kKT, (uint32_t)(uintptr_t)smem + (sub & (kAStages - 1)) * kATile + wave * 1024, 4096, i);
  };

  // score operand bases: logical chunk 2 v + hi of row r32, k-step ks reads
  // base[ks & 3] + 128 (ks >> 2), plus 256 B for the k^R part (ks >= 8)
  int kbase_r[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) kbase_r[v] = r32 * kARow + 16 * ((2 * v + hi) ^ swz(r32));
  // transpose-read bases of the V part (chunk 16 on): as in decode, the lane
  // supplies key 16 kk + 8 hh + tr_row, columns 32 mb + tr_col .. + 3
  int vbase_r[2][2];
  {
    const int g16 = lane >> 4, j16 = lane & 15;
    const int tr_row = 4 * (g16 >> 1) + (j16 >> 2);
    const int y = 2 * (g16 & 1) + ((j16 & 3) >> 1);
    const int s2 = (swz(tr_row) >> 2) & 1;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int sw = swz(tr_row) ^ (hh << 1);
      const int b0 = tr_row * kARow + 16 * (y ^ (sw & 3)) + 8 * (j16 & 1) + 256;
#pragma unroll
      for (int par = 0; par < 2; ++par) vbase_r[hh][par] = b0 + (s2 ? (par ? -64 : 64) : 0);
    }
  }
  auto kload = [&](const int* kb, int ks) {
    return *reinterpret_cast<const bf16x8*>(smem + kb[ks & 3] + 128 * (ks >> 2) + (ks >= 8 ? 256 : 0));
  };
  auto kbases = [&](int stage, int* kb) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      kb[v] = stage * kATile + kbase_r[v];
      __asm__ volatile("" : "+v"(kb[v]));
    }
  };

  f32x16 o[kAMB];
  float m = -INFINITY, l = 0.f, m_seen = -INFINITY;
  // The whole pass loop is instantiated twice, for the waves that issue the
  // copies and for those that do not, so that neither carries a per-copy
  // branch; both run the same sequence of barriers.
  auto passes = [&](auto copy_tag) {
  constexpr bool kCopy = decltype(copy_tag)::value;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int mb = 0; mb < kAMB; ++mb) o[mb] = f32x16{};
    l = 0.f;
    m = pass ? m_seen : -INFINITY;
    bool overflow = false;
    for (int s2 = 0; s2 < min(3, n_sub); ++s2) issue(s2, copy_tag);

    // ---- prologue: tile 0 landed, its scores computed
    if constexpr (kCopy) vm_wait_a(min(2, n_sub - 1) * kADma);
    block_sync();
    f32x16 sc;
    {
      int kb[4];
      kbases(0, kb);
      bf16x8 kop[4];
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) kop[ks] = kload(kb, ks);
#pragma unroll
      for (int ks = 0; ks < kAKSteps; ++ks) {
        if (ks + 3 < kAKSteps) kop[(ks + 3) % 4] = kload(kb, ks + 3);
        if (ks == 0) mfma_v0(sc, kop[0], q[0]);
        else mfma_v(sc, kop[ks % 4], q[ks]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    pad_mfma();
    __asm__ volatile("" : "+v"(sc));

    for (int i = 0; i < n_sub; ++i) {
      const int t0 = i * kKT;
      const bool nxt = i + 1 < n_sub;
      if (nxt) {
        if constexpr (kCopy) vm_wait_a(i + 2 < n_sub ? kADma : 0);
        block_sync();  // tile i+1 landed; every wave is past PV(i-1)
      }
      // tile i+3 is copied during the score loop below (a re-read of the
      // last tile into the sink when there is none, so the wait counts stay fixed)
      const bool copy_on = i + 3 < n_sub;
      const int copy_t0 = (copy_on ? i + 3 : n_sub - 1) * kKT;
      const uint32_t copy_dst = copy_on ? (uint32_t)(uintptr_t)smem + ((i + 3) & (kAStages - 1)) * kATile + wave * 1024
                                        : (uint32_t)(uintptr_t)sink + wave * 1024;
      const uint32_t copy_stride = copy_on ? 4096u : 0u;

      // masking of tile i: causal diagonal or the sequence end
      if (t0 + kKT > lim_all) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = t0 + 8 * (r >> 2) + 4 * hi + (r & 3);
          sc[r] = tok < lim_row ? sc[r] : -INFINITY;
        }
      }

      // ---- softmax(i), pipelined as in decode: max tree, then score r is
      // shifted, exponentiated and summed/packed in three consecutive pieces
      float tm = 0.f, neg_m = 0.f, psum = 0.f, mn = 0.f, hr = 0.f;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, a4 = 0.f, b0 = 0.f, b1 = 0.f;
      uint32_t sw0 = 0u, sw1 = 0u;
      float xs[16], pv[16];
      uint32_t pw[8];
      auto piece = [&](int k) {
        if (k == 0) a0 = max3f(sc[0], sc[1], sc[2]);
        if (k == 1) a1 = max3f(sc[3], sc[4], sc[5]);
        if (k == 2) a2 = max3f(sc[6], sc[7], sc[8]);
        if (k == 3) a3 = max3f(sc[9], sc[10], sc[11]);
        if (k == 4) a4 = max3f(sc[12], sc[13], sc[14]);
        if (k == 5) b0 = max3f(a0, a1, a2);
        if (k == 6) b1 = max3f(a3, a4, sc[15]);
        if (k == 7) tm = max3f(b0, b1, b1);
        if (k == 8 || k == 31) {
          const uint32_t x = __float_as_uint(k == 8 ? tm : psum);
          auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
          sw0 = r[0];
          sw1 = r[1];
        }
        if (k == 9) tm = max3f(__uint_as_float(sw0), __uint_as_float(sw1), __uint_as_float(sw1));
        if (k == 10) tm *= qk_scale;
        if (k == 11) {
          m_seen = max3f(m_seen, tm, tm);
          mn = (m == -INFINITY) ? tm : m;
        }
        if (k == 12) {
          hr = mn + kAHeadroom;
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
        int kb[4];
        kbases((i + 1) & (kAStages - 1), kb);
        bf16x8 kop[4];
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) kop[ks] = kload(kb, ks);
#pragma unroll
        for (int ks = 0; ks < kAKSteps; ++ks) {
          if (ks + 3 < kAKSteps) kop[(ks + 3) % 4] = kload(kb, ks + 3);
          if (ks == 0) mfma_v0(sn, kop[0], q[0]);
          else mfma_v(sn, kop[ks % 4], q[ks]);
          piece(ks);
          if constexpr (kCopy) {
            if ((ks & 1) && (ks >> 1) < kADma) dma_to(copy_t0, copy_dst, copy_stride, ks >> 1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = kAKSteps; k < kPieces; ++k) piece(k);
      } else {
#pragma unroll
        for (int k = 0; k < kPieces; ++k) piece(k);
      }
      bf16x8 pb[2];
      pb[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      pb[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
      __asm__ volatile("s_nop 4" ::: "memory");  // VALU-written pb before its MFMA reads

      // ---- O^T += V^T . P^T for tile i (all 128 columns of this wave's rows)
      {
        int vb[2][2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int par = 0; par < 2; ++par) {
            vb[hh][par] = (i & (kAStages - 1)) * kATile + vbase_r[hh][par];
            __asm__ volatile("" : "+v"(vb[hh][par]));
          }
        constexpr int kSteps = 2 * kAMB;
        auto vload = [&](int st) {
          const int mb = st >> 1, kk = st & 1;
          const int imm = 16 * kk * kARow + 64 * mb;
          const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + vb[0][mb & 1] + imm));
          const bf16x4 v1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + vb[1][mb & 1] + imm + 8 * kARow));
          return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 vop[4];
#pragma unroll
        for (int st = 0; st < 3; ++st) vop[st] = vload(st);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          if (st + 3 < kSteps) vop[(st + 3) % 4] = vload(st + 3);
          mfma_a(o[st >> 1], vop[st % 4], pb[st & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (nxt) {
        __asm__ volatile("" : "+v"(sn));
        sc = sn;
      }
    }
    pad_mfma();
#pragma unroll
    for (int mb = 0; mb < kAMB; ++mb) __asm__ volatile("" : "+a"(o[mb]));

    if (tid == 0) red_flag = 0;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the clear lands before any wave sets the flag
    block_sync();
    if (overflow && row_ok) red_flag = 1;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    block_sync();
    if (red_flag == 0) break;
    block_sync();
  }
  if constexpr (kCopy) vm_wait<0>();  // the sink copies of the last tiles
  };
  if (copier) passes(std::true_type{});
  else passes(std::false_type{});

  if (row_ok) {
    const size_t tq = (size_t)(s0 + qrow) * a.H + h;
    uint16_t* op = a.out + tq * kDnP;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int mb = 0; mb < kAMB; ++mb) {
      const int c0 = mb * 32 + 4 * hi;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *reinterpret_cast<uint2*>(op + c0 + 8 * gg) =
            make_uint2(pack_bf16(o[mb][4 * gg] * inv, o[mb][4 * gg + 1] * inv),
                       pack_bf16(o[mb][4 * gg + 2] * inv, o[mb][4 * gg + 3] * inv));
    }
    if (a.lse != nullptr && hi == 0) a.lse[tq] = l > 0.f ? (m + log2f(l)) * kALn2 : -INFINITY;
  }
}

// ------------------------------------------------------------------ portable
// Up-projection: one thread per element of Kn [T][H][d_n], V [T][H][d_v] and
// R [T][d_r] (float32 accumulation, rounded once to the storage type).
template <typename T>
__global__ __launch_bounds__(256) void upproject_generic(const T* __restrict__ c_kv, const T* __restrict__ w_uk,
                                                         const T* __restrict__ w_uv, const T* __restrict__ k_rope,
                                                         T* __restrict__ ws, int Tn, int H, int d_c, int d_n,
                                                         int d_v, int d_r, size_t v_off, size_t r_off) {
  const size_t nk = (size_t)Tn * H * d_n, nv = (size_t)Tn * H * d_v, nr = (size_t)Tn * d_r;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < nk + nv + nr; e += (size_t)gridDim.x * blockDim.x) {
    if (e >= nk + nv) {
      ws[r_off + (e - nk - nv)] = k_rope[e - nk - nv];
      continue;
    }
    const bool isv = e >= nk;
    const size_t f = isv ? e - nk : e;
    const int dw = isv ? d_v : d_n;
    const size_t t = f / ((size_t)H * dw);
    const int hd = (int)(f - t * H * dw), hh = hd / dw, d = hd - hh * dw;
    const T* w = (isv ? w_uv : w_uk) + ((size_t)hh * dw + d) * d_c;
    const T* c = c_kv + t * d_c;
    float acc = 0.f;
    for (int k = 0; k < d_c; ++k) acc = fmaf(Storage<T>::load(c + k), Storage<T>::load(w + k), acc);
    Storage<T>::store(ws + (isv ? v_off : 0) + f, acc);
  }
}

// Attention: one 64-thread workgroup per (query token, head); the threads
// split the score dot products and the output columns; online softmax with
// rescaling in float32.
template <typename T>
__global__ __launch_bounds__(64) void attn_generic(const T* __restrict__ q_nope, const T* __restrict__ q_rope,
                                                   const T* __restrict__ ws, const int32_t* __restrict__ cu,
                                                   T* __restrict__ out, float* __restrict__ lse, float scale,
                                                   int Tn, int H, int B, int d_n, int d_v, int d_r, int causal,
                                                   size_t v_off, size_t r_off) {
  const int tq = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  // the query's sequence: largest b with cu[b] <= tq (cu clamped into [0, T])
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (min(max(cu[mid], 0), Tn) <= tq) lo = mid;
    else hi = mid;
  }
  const int s0 = min(max(cu[lo], 0), Tn), s1 = min(max(cu[lo + 1], s0), Tn);
  if (tq < s0 || tq >= s1) return;  // not in any sequence
  const int kend = causal ? tq + 1 : s1;
  constexpr int kMaxCols = 16;  // d_v <= 1024
  float acc[kMaxCols];
#pragma unroll
  for (int i = 0; i < kMaxCols; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const T* qn = q_nope + ((size_t)tq * H + h) * d_n;
  const T* qr = q_rope + ((size_t)tq * H + h) * d_r;
  for (int t = s0; t < kend; ++t) {
    const T* kn = ws + ((size_t)t * H + h) * d_n;
    const T* kr = ws + r_off + (size_t)t * d_r;
    float part = 0.f;
    for (int k = lane; k < d_n; k += 64) part = fmaf(Storage<T>::load(qn + k), Storage<T>::load(kn + k), part);
    for (int k = lane; k < d_r; k += 64) part = fmaf(Storage<T>::load(qr + k), Storage<T>::load(kr + k), part);
    const float sc = wave_sum(part) * scale;
    const float mn = fmaxf(m, sc);
    const float alpha = expf(m - mn), p = expf(sc - mn);
    l = l * alpha + p;
    const T* v = ws + v_off + ((size_t)t * H + h) * d_v;
#pragma unroll
    for (int i = 0; i < kMaxCols; ++i) {
      const int d = lane + 64 * i;
      if (d < d_v) acc[i] = acc[i] * alpha + p * Storage<T>::load(v + d);
    }
    m = mn;
  }
  T* op = out + ((size_t)tq * H + h) * d_v;
#pragma unroll
  for (int i = 0; i < kMaxCols; ++i) {
    const int d = lane + 64 * i;
    if (d < d_v) Storage<T>::store(op + d, acc[i] / l);
  }
  if (lse != nullptr && lane == 0) lse[(size_t)tq * H + h] = m + logf(l);
}

}  // namespace

bool prefill_mfma_supported(const mla_dims& d) {
  return d.dtype == MLA_BF16 && d.d_c == kDcP && d.d_rope == kDrP && d.d_nope == kDnP && d.d_v == kDnP;
}

bool prefill_grid_fits(const mla_dims& d, int max_seqlen) {
  const int64_t blocks = (int64_t)d.batch * d.num_heads * ((max_seqlen + kQB - 1) / kQB);
  return blocks * kAThreads <= (int64_t)0xffffffffu;
}

// Workspace regions in elements of the storage type (each 256-B aligned).
PrefillLayout prefill_layout(const mla_dims& d, int64_t tokens) {
  const int64_t esz = d.dtype == MLA_F32 ? 4 : 2;
  auto al = [&](int64_t n) { return (n * esz + 255) / 256 * 256 / esz; };
  PrefillLayout L;
  L.v_off = al(tokens * d.num_heads * d.d_nope);
  L.r_off = L.v_off + al(tokens * d.num_heads * d.d_v);
  L.total_bytes = (L.r_off + al(tokens * d.d_rope)) * esz;
  return L;
}

hipError_t launch_prefill(const mla_dims& d, int tokens, int max_seqlen, const int32_t* cu, const void* q_nope,
                          const void* q_rope, const void* c_kv, const void* k_rope, const void* w_uk,
                          const void* w_uv, float scale, int causal, void* out, float* lse, void* ws, bool mfma,
                          hipStream_t stream) {
  const PrefillLayout Lw = prefill_layout(d, tokens);
  if (mfma) {
    const int N = d.num_heads * kDnP;
    if (N % kHT == 0)  // an even head count: the 256 x 256 tiles
      hipLaunchKernelGGL(upproject_mfma256, dim3(N / kHT, (tokens + kHT - 1) / kHT, 2), dim3(kHThreads), 0, stream,
                         static_cast<const uint16_t*>(c_kv), static_cast<const uint16_t*>(w_uk),
                         static_cast<const uint16_t*>(w_uv), static_cast<const uint16_t*>(k_rope),
                         static_cast<uint16_t*>(ws), tokens, N, (size_t)Lw.v_off, (size_t)Lw.r_off);
    else
      hipLaunchKernelGGL(upproject_mfma, dim3(N / kGT, (tokens + kGT - 1) / kGT, 2), dim3(kGThreads), 0, stream,
                         static_cast<const uint16_t*>(c_kv), static_cast<const uint16_t*>(w_uk),
                         static_cast<const uint16_t*>(w_uv), static_cast<const uint16_t*>(k_rope),
                         static_cast<uint16_t*>(ws), tokens, N, (size_t)Lw.v_off, (size_t)Lw.r_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PrefillArgs a{static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope),
                  static_cast<const uint8_t*>(ws), cu, static_cast<uint16_t*>(out), lse, scale, tokens,
                  d.num_heads, d.batch, (max_seqlen + kQB - 1) / kQB, causal ? 1 : 0,
                  (uint32_t)(Lw.v_off * 2), (uint32_t)(Lw.r_off * 2)};
    const int64_t blocks = (int64_t)d.batch * d.num_heads * a.nqb;
    hipLaunchKernelGGL(attn_mfma, dim3((unsigned)blocks), dim3(kAThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t elems = (int64_t)tokens * (d.num_heads * (int64_t)(d.d_nope + d.d_v) + d.d_rope);
  const int grid = (int)std::min<int64_t>((elems + 255) / 256, 65536);
  if (d.dtype == MLA_BF16) {
    hipLaunchKernelGGL(upproject_generic<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(c_kv), static_cast<const uint16_t*>(w_uk),
                       static_cast<const uint16_t*>(w_uv), static_cast<const uint16_t*>(k_rope),
                       static_cast<uint16_t*>(ws), tokens, d.num_heads, d.d_c, d.d_nope, d.d_v, d.d_rope,
                       (size_t)Lw.v_off, (size_t)Lw.r_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_generic<uint16_t>, dim3(tokens, d.num_heads), dim3(64), 0, stream,
                       static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope),
                       static_cast<const uint16_t*>(ws), cu, static_cast<uint16_t*>(out), lse, scale, tokens,
                       d.num_heads, d.batch, d.d_nope, d.d_v, d.d_rope, causal ? 1 : 0, (size_t)Lw.v_off,
                       (size_t)Lw.r_off);
  } else {
    hipLaunchKernelGGL(upproject_generic<float>, dim3(grid), dim3(256), 0, stream, static_cast<const float*>(c_kv),
                       static_cast<const float*>(w_uk), static_cast<const float*>(w_uv),
                       static_cast<const float*>(k_rope), static_cast<float*>(ws), tokens, d.num_heads, d.d_c,
                       d.d_nope, d.d_v, d.d_rope, (size_t)Lw.v_off, (size_t)Lw.r_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_generic<float>, dim3(tokens, d.num_heads), dim3(64), 0, stream,
                       static_cast<const float*>(q_nope), static_cast<const float*>(q_rope),
                       static_cast<const float*>(ws), cu, static_cast<float*>(out), lse, scale, tokens, d.num_heads,
                       d.batch, d.d_nope, d.d_v, d.d_rope, causal ? 1 : 0, (size_t)Lw.v_off, (size_t)Lw.r_off);
  }
  return hipGetLastError();
}

}  // namespace mla
