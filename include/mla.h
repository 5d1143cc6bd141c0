/*
 * libmla -- absorbed Multi-Head Latent Attention (MLA) decode over a paged
 * latent cache, for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For each sequence b, new token j < q_len and head h the
 * library evaluates decode attention in the "absorbed" form of
 * "DeepSeek-V3 MLA: Multi-Head Latent Attention Guide" (section Inference
 * Optimization: The Matrix Absorption Trick):
 *
 *   q~      = (W^UK_h)^T q^C                        (section 2, Folding W^UK)
 *   s_t     = scale * ( q~ . c_t  +  q^R . k^R_t )  (section 2, score on latents)
 *   p       = softmax_t(s) over the visible t       (textbook softmax)
 *   o       = sum_t p_t c_t                         (section 3, o_{t,i})
 *   u       = W^UV_h o                              (section 3, u_{t,i})
 *
 * so the per-head keys W^UK c_t and values W^UV c_t are never formed.  The
 * cache holds, per token, only the joint latent c^KV (d_c) and the decoupled,
 * already-rotated RoPE key k^R (d_rope) shared by all heads ("DeepSeek-V2
 * Multi-Head Latent Attention" knowledge note, cache rule and Decoupled RoPE).
 *
 * Pipeline (four calls, all asynchronous on the caller's stream):
 *   mla_absorb_q   q_nope, q_rope, W_UK        -> q_cat  [B,Lq,H,d_c+d_rope]
 *   mla_decode     q_cat, paged cache          -> per-split (o_s, lse_s)
 *   mla_combine    (o_s, lse_s)                -> o [B,Lq,H,d_c], lse [B,Lq,H]
 *   mla_absorb_out o, W_UV                     -> u [B,Lq,H,d_v]
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to row-major, contiguous arrays with
 *     the shapes given per call; every base pointer must be 16-byte aligned.
 *   - "storage type" is dims->dtype: MLA_F32 (float) or MLA_BF16 (bfloat16,
 *     raw 16-bit patterns).  Accumulation is always float32.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     retains a pointer, and keeps no state besides a per-device properties
 *     cache filled once.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Each
 *     call only enqueues work; it never synchronises.  Inputs must stay valid
 *     until the stream reaches the call; outputs are ready once it has.
 *   - The return value is an mla_status.  Arguments are validated on the host
 *     before anything is enqueued; on failure nothing is launched or written.
 *     A launch failure returns MLA_ERR_HIP.  Values that live only on the
 *     device (seq_lens, block ids) cannot be checked on the host: a sequence
 *     length outside [q_len, max_blocks_per_seq * block_size] or a block id
 *     outside [0, num_blocks) is undefined behaviour.
 *   - No exception crosses this interface.
 */
#ifndef LIBMLA_MLA_H
#define LIBMLA_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, misaligned pointer, bad split count */
  MLA_ERR_UNSUPPORTED = -2, /* valid but not implemented: dtype, widths or q_len outside the supported set */
  MLA_ERR_WORKSPACE = -3,   /* the workspace is smaller than the matching *_workspace_bytes() call says */
  MLA_ERR_HIP = -4          /* the HIP runtime reported an error (launch or device query) */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Problem dimensions.  Widths follow DeepSeek-V2/V3 notation: d_c is the KV
 * latent width (512), d_rope the decoupled RoPE width (64), d_nope the per-head
 * content query/key width d_h (128), d_v the per-head value width (128). */
typedef struct {
  int32_t batch;              /* B: number of sequences */
  int32_t q_len;              /* Lq: new tokens per sequence, 1 or 2 */
  int32_t num_heads;          /* H */
  int32_t d_c;                /* latent width, multiple of 16, <= 1024 */
  int32_t d_rope;             /* RoPE key width, multiple of 8, d_c + d_rope <= 1088 */
  int32_t d_nope;             /* content query width, <= 1024 */
  int32_t d_v;                /* value width, <= 1024 */
  int32_t block_size;         /* tokens per physical cache block */
  int32_t max_blocks_per_seq; /* MB: row length of block_table */
  int32_t num_blocks;         /* NB: blocks in the cache pool */
  int32_t dtype;              /* mla_dtype: storage type of q, cache and weights */
} mla_dims;

/* Absorb W^UK into the query ("DeepSeek-V3 MLA: Multi-Head Latent Attention
 * Guide", Matrix Absorption Trick section 2, Folding W^UK into Query
 * Projection):
 *   q_cat[b,j,h, 0:d_c]        = sum_n q_nope[b,j,h,n] * w_uk[h,n,:]
 *   q_cat[b,j,h, d_c:d_c+d_r]  = q_rope[b,j,h,:]
 * q_nope [B,Lq,H,d_nope], q_rope [B,Lq,H,d_rope], w_uk [H,d_nope,d_c] (a
 * Linear weight of shape (H*d_nope) x d_c viewed per head), q_cat
 * [B,Lq,H,d_c+d_rope]; all in the storage type (q~ is rounded once to it). */
int mla_absorb_q(const mla_dims* dims, const void* q_nope, const void* q_rope, const void* w_uk,
                 void* q_cat, void* stream);

/* Number of splits S that mla_decode needs so that the device's full grid
 * shares the work evenly, given the longest sequence and the total token
 * count (host-side values the caller knows).  Result in [1, 4096].  Passing a
 * smaller S to mla_decode is allowed: the library then gives each workgroup a
 * longer token range and launches fewer of them.  MLA_ERR_INVALID_ARG when
 * max_seq_len < 1, total_tokens < max_seq_len or num_splits is NULL. */
int mla_decode_num_splits(const mla_dims* dims, int32_t max_seq_len, int64_t total_tokens,
                          int32_t* num_splits);

/* The same choice from the lengths themselves, for callers that hold them
 * on the host.  seq_lens_host [B] int32 is a HOST array (read during the
 * call, not retained) or NULL; with it, max_seq_len and the total are taken
 * from the lengths (each clamped to [0, max_blocks_per_seq * block_size];
 * max_seq_len is then ignored and may be 0).  With NULL every sequence is
 * taken to be max_seq_len long (a batch of equal lengths; a batch of very
 * unequal lengths is balanced better when its lengths are given).  The result
 * equals mla_decode_num_splits(dims, max, total).  The _fp8 form sizes the
 * FP8-cache decode (mla_decode_fp8).  MLA_ERR_INVALID_ARG when num_splits is
 * NULL, or when seq_lens_host is NULL and max_seq_len < 1, or when every
 * given length is 0. */
int mla_choose_splits(const mla_dims* dims, const int32_t* seq_lens_host, int32_t max_seq_len,
                      int32_t* num_splits);
int mla_choose_splits_fp8(const mla_dims* dims, const int32_t* seq_lens_host, int32_t max_seq_len,
                          int32_t* num_splits);

/* Bytes of device workspace mla_decode needs (the work schedule it computes
 * on the device: a header, four int32 per workgroup for up to 1024
 * workgroups (16 KiB), and two int32 per scheduled sequence, counting the
 * head groups described at mla_decode, so up to four per sequence). */
int mla_decode_workspace_bytes(const mla_dims* dims, int32_t num_splits, size_t* bytes);

/* Split-KV attention over the paged latent cache (the guide's section 4,
 * End-to-End Latent Attention Computation: scores and latent-weighted sums
 * in one fused pass over rows loaded once into on-chip memory).
 *   q_cat       [B,Lq,H,d_c+d_rope]   storage type, from mla_absorb_q
 *   kv_cache    [NB,block_size,d_c+d_rope] storage type; row = [c^KV | k^R]
 *   block_table [B,MB] int32: token t of sequence b is at
 *               kv_cache[block_table[b, t / block_size], t % block_size, :]
 *   seq_lens    [B] int32: tokens of sequence b INCLUDING its q_len new
 *               ones; query j sees tokens t <= seq_lens[b] - q_len + j
 *   softmax_scale  multiplies every score (1/sqrt(d_nope + d_rope) for MLA);
 *               must be finite and > 0
 *   num_splits  S >= 1, the split dimension of the two outputs
 *   workspace   device scratch of at least mla_decode_workspace_bytes()
 *               (MLA_ERR_WORKSPACE if workspace_bytes is smaller), 16-byte
 *               aligned; overwritten by every call, so calls sharing one
 *               workspace must be ordered on one stream
 *   o_partial   [B,Lq,H,S,d_c] in the storage type (float32 or bf16): o_s =
 *               sum_{t in split} p_t c_t with p normalised within the split,
 *               rounded once to the storage type (these partials are the
 *               largest write of the step; bf16 halves it, at a relative
 *               error of 2^-9 per element, well inside the bf16 tolerances)
 *   lse_partial [B,Lq,H,S] float32: natural-log log-sum-exp of the split's
 *               scaled scores; -inf marks an unused or empty split, whose
 *               o_partial entry is left unwritten.
 * Equivalent to mla_decode_plan followed by mla_decode_planned (two kernels:
 * a one-workgroup planner that turns seq_lens into a token-balanced schedule
 * in the workspace, then the attention kernel).  Each sequence's tokens are
 * divided into at most S contiguous ranges.  Head groups: with q_len = 1 and
 * 64 or 128 heads, when B * ceil(MB * block_size / 64) 64-token tiles at most
 * would leave most CUs idle, the heads of each sequence are split into 2 or 4
 * groups of 32 (the largest count whose grouped tile total still fits the
 * CUs), and each group is scheduled as a sequence of its own, divided into
 * at most S ranges; the outputs' layout and meaning do not change.  The
 * grouping depends only on dims and the device, so mla_decode_plan and
 * mla_decode_planned always agree on it.  Unused cache slots may hold
 * anything (NaN included): they never reach a result.  A length outside
 * [0, MB * block_size] is clamped into it for memory safety (the result for
 * that sequence is then meaningless). */
int mla_decode(const mla_dims* dims, const void* q_cat, const void* kv_cache, const int32_t* block_table,
               const int32_t* seq_lens, float softmax_scale, int32_t num_splits, void* workspace,
               size_t workspace_bytes, void* o_partial, float* lse_partial, void* stream);

/* mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same planner and attention kernels, with the work schedule kept in a
 * library-owned device array instead of a caller workspace.  The array holds
 * the schedule of up to 65536 sequences (about 528 KiB; with head groups,
 * see mla_decode, each group counts as a sequence); each GPU the library
 * runs on keeps its own copy until the process ends.  Arguments and results
 * are those of mla_decode without workspace/workspace_bytes.  The call
 * allocates nothing.  MLA_ERR_WORKSPACE when dims->batch > 65536; the other
 * statuses as for mla_decode.  Every call on one GPU shares that GPU's array:
 * calls that may overlap on one GPU (several streams, several threads) race
 * and must be ordered by the caller, e.g. issued on one stream. */
int mla_decode_noalloc(const mla_dims* dims, const void* q_cat, const void* kv_cache, const int32_t* block_table,
                       const int32_t* seq_lens, float softmax_scale, int32_t num_splits, void* o_partial,
                       float* lse_partial, void* stream);

/* First half of mla_decode: enqueue only the planner, which writes the work
 * schedule for seq_lens [B] int32 (device) and num_splits into the workspace.
 * One plan serves every later mla_decode_planned call with the same dims,
 * lengths and num_splits, e.g. all layers of one decode step. */
int mla_decode_plan(const mla_dims* dims, const int32_t* seq_lens, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, void* stream);

/* mla_absorb_q and mla_decode_plan in one launch: the same q_cat and the same
 * schedule in the workspace, bit for bit, with the planner running as one
 * more workgroup of the absorb_q kernel (both depend only on their own
 * inputs), so a decode step is three launches: this, mla_decode_planned and
 * mla_combine_absorb_out.  Arguments and errors as for the two calls; every
 * argument of both is validated before anything is enqueued.  Where the
 * absorb_q matrix-core kernel does not serve the dims, the two kernels are
 * enqueued one after the other.  The _fp8 form plans for mla_decode_fp8's
 * kernels (mla_decode_planned_fp8). */
int mla_absorb_q_plan(const mla_dims* dims, const void* q_nope, const void* q_rope, const void* w_uk, void* q_cat,
                      const int32_t* seq_lens, int32_t num_splits, void* workspace, size_t workspace_bytes,
                      void* stream);
int mla_absorb_q_plan_fp8(const mla_dims* dims, const void* q_nope, const void* q_rope, const void* w_uk,
                          void* q_cat, const int32_t* seq_lens, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Second half of mla_decode: enqueue only the attention kernel, reading the
 * schedule (and the lengths) that mla_decode_plan left in the workspace.
 * Arguments as for mla_decode; num_splits must equal the planned value. */
int mla_decode_planned(const mla_dims* dims, const void* q_cat, const void* kv_cache, const int32_t* block_table,
                       float softmax_scale, int32_t num_splits, const void* workspace, size_t workspace_bytes,
                       void* o_partial, float* lse_partial, void* stream);

/* ---- FP8 latent cache ---------------------------------------------------
 * The latent cache in FP8 ("Deconstructing DeepSeek V4 Pro", Practical
 * Deployment: the compressed latent tolerates FP8 E4M3 quantization and the
 * cached row drops below a kilobyte; "DeepSeek-V3 MLA: Multi-Head Latent
 * Attention Guide", Core Architecture: the 576 cached values per token in
 * fp8 or bf16).  kv_cache is [NB, block_size, d_c + d_rope] uint8: every
 * element of the row [c^KV | k^R] is an OCP E4M3 code (bit 7 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; no infinities; all six low bits set is
 * NaN; largest magnitude 448), and a code stands for kv_scale times its value
 * (one float scale for the whole cache, finite and > 0).  The result is that
 * of mla_decode on the cache of those values: E4M3 values are exact in bf16
 * and float32, so the products see exactly the cached values (bf16 q_cat
 * storage uses the matrix-core kernel when mla_decode would, the portable
 * kernel otherwise).  o_partial/lse_partial are as for mla_decode (o_s in
 * value units, the scale applied).  Rows a sequence never reaches may hold
 * any code, NaN included.  The planner weighs a piece's fixed cost against
 * the halved row bytes, so plan FP8 calls with mla_decode_plan_fp8 and size
 * them with mla_decode_num_splits_fp8 (the schedule format is the same, so a
 * schedule from either planner serves either attention call with the same
 * num_splits); the workspace is as for mla_decode. */
int mla_decode_num_splits_fp8(const mla_dims* dims, int32_t max_seq_len, int64_t total_tokens,
                              int32_t* num_splits);
int mla_decode_plan_fp8(const mla_dims* dims, const int32_t* seq_lens, int32_t num_splits, void* workspace,
                        size_t workspace_bytes, void* stream);
int mla_decode_planned_fp8(const mla_dims* dims, const void* q_cat, const uint8_t* kv_cache, float kv_scale,
                           const int32_t* block_table, float softmax_scale, int32_t num_splits,
                           const void* workspace, size_t workspace_bytes, void* o_partial, float* lse_partial,
                           void* stream);
int mla_decode_fp8(const mla_dims* dims, const void* q_cat, const uint8_t* kv_cache, float kv_scale,
                   const int32_t* block_table, const int32_t* seq_lens, float softmax_scale, int32_t num_splits,
                   void* workspace, size_t workspace_bytes, void* o_partial, float* lse_partial, void* stream);

/* Log-sum-exp merge of the splits (exact rewrite of one softmax over the
 * union of the splits' keys):
 *   lse = log sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) * o_s
 * skipping splits with lse_s = -inf.  o_partial/lse_partial as written by
 * mla_decode; o_latent [B,Lq,H,d_c] float32; lse [B,Lq,H] float32 or NULL.
 * The float32 additions follow one fixed order (blocks of eight consecutive
 * splits, and for batches under 32 token rows several block groups summed
 * separately and then added in group order), which mla_combine_absorb_out
 * follows too, so the two routes give identical bits. */
int mla_combine(const mla_dims* dims, int32_t num_splits, const void* o_partial, const float* lse_partial,
                float* o_latent, float* lse, void* stream);

/* Apply W^UV after the latent-weighted sum ("DeepSeek-V3 MLA: Multi-Head
 * Latent Attention Guide", Matrix Absorption Trick section 3, Absorbing
 * W^UV):  u[b,j,h,v] = sum_c w_uv[h,v,c] * o_latent[b,j,h,c].
 * o_latent [B,Lq,H,d_c] float32, w_uv [H,d_v,d_c] storage type, out
 * [B,Lq,H,d_v] storage type. */
int mla_absorb_out(const mla_dims* dims, const float* o_latent, const void* w_uv, void* out, void* stream);

/* mla_combine and mla_absorb_out in one call (the guide's section 3,
 * Absorbing W^UV, applied to the merged latent output):
 *   lse = log sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) * o_s,
 *   u[b,j,h,v] = sum_c w_uv[h,v,c] * o[b,j,h,c]
 * Arguments as for the two calls: o_partial/lse_partial as written by
 * mla_decode, w_uv [H,d_v,d_c] storage type, out [B,Lq,H,d_v] storage type.
 * o_latent [B,Lq,H,d_c] float32 and lse [B,Lq,H] float32 are optional
 * outputs (NULL to skip).  When mla_combine_absorb_out_fused() returns 1 for
 * these dims and split count, one kernel merges each tile of rows on chip and
 * the merged latent output is only written if o_latent is given; otherwise the
 * call runs the two kernels and needs o_latent as their intermediate
 * (MLA_ERR_UNSUPPORTED if it is NULL). */
int mla_combine_absorb_out(const mla_dims* dims, int32_t num_splits, const void* o_partial, const float* lse_partial,
                           const void* w_uv, void* out, float* o_latent, float* lse, void* stream);

/* 1 if mla_combine_absorb_out runs as one fused kernel for these dims and
 * split count (bf16 storage, d_c = 512, d_nope = d_v = 128, any split
 * count), else 0 (also for invalid arguments).  Host only. */
int mla_combine_absorb_out_fused(const mla_dims* dims, int32_t num_splits);

/* ---- cache append: the step just before attention ---------------------- */

/* Bytes of device workspace mla_cache_append needs for these dims and model
 * width d_model (0 when the portable kernel serves them; the workspace may
 * then be NULL).  Host only; MLA_ERR_INVALID_ARG for d_model outside
 * [1, 65536] or a NULL bytes. */
int mla_cache_append_workspace_bytes(const mla_dims* dims, int32_t d_model, size_t* bytes);

/* Write the cache rows of the q_len new tokens of every sequence
 * ("DeepSeek-V3 MLA: Multi-Head Latent Attention Guide", Core Architecture
 * section 1, joint KV compression, and section 3, decoupled RoPE key):
 *   c_t   = W^DKV h_t                          (d_c values)
 *   k^R_t = RoPE_t(W^KR h_t)                   (d_rope values)
 *   kv_cache[block_table[b, t / bs], t % bs, :] = [c_t | k^R_t]
 * for token j of sequence b at position t = seq_lens[b] - q_len + j (the
 * lengths count the new tokens, as mla_decode expects).  RoPE rotates each
 * pair (x[2p], x[2p+1]) by theta_p = t / rope_base^(2p / d_rope), as the
 * apply_rope helper of the MLA module in "Deconstructing DeepSeek V4 Pro"
 * does; rope_base is 10000 there.
 *   h       [B,Lq,d_model]  hidden states of the new tokens, storage type
 *   w_dkv   [d_c,d_model]   W^DKV (a Linear weight), storage type
 *   w_kr    [d_rope,d_model] W^KR, storage type (may be NULL if d_rope = 0)
 *   kv_cache [num_blocks,block_size,d_c+d_rope] storage type, updated in place
 *   workspace  at least mla_cache_append_workspace_bytes() bytes
 *              (MLA_ERR_WORKSPACE if workspace_bytes is smaller), contents
 *              on entry irrelevant (float32 split-K partials)
 * Products accumulate in float32; the RoPE angle, its sine and cosine and
 * the rotation are evaluated in float64; each value is rounded once to the
 * storage type.  Only the slots of the new tokens are written.  A token whose
 * position falls outside [0, max_blocks_per_seq * block_size) or whose block
 * id falls outside [0, num_blocks) is skipped.  How d_model is split, and
 * so the order of the float32 additions, follows the device's compute-unit
 * count: the result is reproducible on one device type. */
int mla_cache_append(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv, const void* w_kr,
                     float rope_base, const int32_t* block_table, const int32_t* seq_lens, void* kv_cache,
                     void* workspace, size_t workspace_bytes, void* stream);

/* mla_cache_append into an FP8 (E4M3) cache (the FP8 latent cache of
 * mla_decode_fp8): each value of the row [c_t | k^R_t], computed as above in
 * float32, is divided by kv_scale (float32), saturated to +-448 (a NaN stays
 * NaN) and rounded to the nearest E4M3 code, ties to the code with an even
 * mantissa.  kv_cache is [num_blocks,block_size,d_c+d_rope] uint8; kv_scale
 * finite and > 0.  Workspace and every other argument as for
 * mla_cache_append. */
int mla_cache_append_fp8(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv, const void* w_kr,
                         float rope_base, float kv_scale, const int32_t* block_table, const int32_t* seq_lens,
                         uint8_t* kv_cache, void* workspace, size_t workspace_bytes, void* stream);

/* ---- prefill: the non-absorbed forward over whole sequences ------------ */

/* Bytes of device workspace mla_prefill needs for these dims and
 * total_tokens: the per-head up-projected keys and values and a copy of the
 * RoPE keys, T * (H * (d_nope + d_v) + d_rope) elements of the storage type.
 * Host only. */
int mla_prefill_workspace_bytes(const mla_dims* dims, int32_t total_tokens, size_t* bytes);

/* Attention of every token of every sequence over its own sequence, in the
 * non-absorbed form ("Deconstructing DeepSeek V4 Pro", the forward pass of
 * its MLA module; "DeepSeek-V3 MLA: Multi-Head Latent Attention Guide",
 * forward_train):
 *   K_{t,h} = [W^UK_h c_t ; k^R_t],  V_{t,h} = W^UV_h c_t,
 *   u_{j,h} = softmax_t(scale * [q^C_{j,h}; q^R_{j,h}] . K_{t,h}) V_{t,h}
 * over the tokens t of j's sequence, t <= j when causal = 1 (a decoder's
 * prefill), all of them when causal = 0 (the pages' code as printed).
 * Tokens of the dims->batch sequences are packed: sequence b is tokens
 * cu_seqlens[b] .. cu_seqlens[b+1]-1.
 *   cu_seqlens [B+1] int32 (device), non-decreasing, cu_seqlens[0] = 0,
 *              cu_seqlens[B] = total_tokens; no sequence longer than max_seqlen
 *   q_nope [T,H,d_nope], q_rope [T,H,d_rope]  queries, storage type
 *   c_kv   [T,d_c], k_rope [T,d_rope]         the tokens' cache rows
 *                                             (latent and rotated RoPE key)
 *   w_uk [H,d_nope,d_c], w_uv [H,d_v,d_c]     storage type
 *   out    [T,H,d_v] storage type;  lse [T,H] float32 (natural log), or NULL
 *   workspace  at least mla_prefill_workspace_bytes() (MLA_ERR_WORKSPACE if
 *              workspace_bytes is smaller); overwritten
 * Only dims->batch, num_heads, d_c, d_rope, d_nope, d_v and dtype are used
 * (the other fields must still be valid, e.g. 1).  Products accumulate in
 * float32; the up-projected K and V are rounded once to the storage type, and
 * for bf16 the softmax weights are rounded to bf16 before the weighted sum.
 * A sequence longer than max_seqlen or a cu_seqlens outside [0, T] is
 * undefined behaviour (reads stay inside the buffers).  MLA_ERR_UNSUPPORTED
 * when the bf16 workspace would reach 4 GiB, or when the matrix-core
 * attention grid (batch * num_heads * ceil(max_seqlen / 256) workgroups of
 * 512 threads) would exceed 2^32 - 1 threads (split the batch); nothing is
 * enqueued then. */
int mla_prefill(const mla_dims* dims, int32_t total_tokens, int32_t max_seqlen, const int32_t* cu_seqlens,
                const void* q_nope, const void* q_rope, const void* c_kv, const void* k_rope, const void* w_uk,
                const void* w_uv, float softmax_scale, int32_t causal, void* out, float* lse, void* workspace,
                size_t workspace_bytes, void* stream);

/* ---- offline weight folds: the steps on either side of the path -------- */

/* Fused weight storage.  A fused weight viewed as a matrix W [N x K] (N its
 * output columns, K the contraction: W~_Q as [H*d_c x d_in], W~^O as
 * [d_out x H*d_c]) is stored row-major, except where the matrix-core
 * products serve its shape (mla_fused_query_weight_packed() /
 * mla_fused_output_weight_packed() return 1): there it is stored in MFMA
 * fragment order, an array [N/32][K/64][4][2][32][8] over (32-row tile,
 * 64-element chunk, step, half, row in tile, element), element (n, k) at
 *   ((n/32)*(K/64) + k/64)*2048 + ((k%64)/16)*512 + (((k%16)/8)*32 + n%32)*8 + k%8
 * so that the products stream it in contiguous 1 KiB pieces.  The folds
 * write, and both products read, whichever order applies; the element count
 * is the same either way.  A weight made elsewhere must be put in that order
 * before it is passed to a product. */

/* 1 if the fused query weight for these dims and d_in is stored in fragment
 * order (bf16, d_in % 64 == 0, H*d_c % 128 == 0), else 0 (also for invalid
 * arguments).  Host only. */
int mla_fused_query_weight_packed(const mla_dims* dims, int32_t d_in);

/* 1 if the fused output weight for these dims and d_out is stored in
 * fragment order (bf16, H*d_c % 64 == 0, d_out % 256 == 0), else 0.  Host
 * only. */
int mla_fused_output_weight_packed(const mla_dims* dims, int32_t d_out);

/* Fold W^UK into the query projection ("Deconstructing DeepSeek V4 Pro",
 * Practical Deployment, the fused query weight; "DeepSeek-V3 MLA: Multi-Head
 * Latent Attention Guide", Matrix Absorption Trick section 2):
 *   w_fused[h,c,i] = sum_n w_uk[h,n,c] * w_in[h,n,i]
 * where w_in [H,d_nope,d_in] is the per-head content query projection (a
 * Linear weight of shape (H*d_nope) x d_in, e.g. the query up-projection of a
 * d_in = 1536 query latent), w_uk [H,d_nope,d_c] and w_fused [H,d_c,d_in]
 * (in the fused weight storage order above), all in the storage type.  Float32 accumulation in order of n, one rounding.
 * Offline: run once per weight set.  Uses num_heads, d_c, d_nope and dtype of
 * dims (the other fields must still be valid).  d_in in [1, 65536]. */
int mla_fold_query_weight(const mla_dims* dims, int32_t d_in, const void* w_in, const void* w_uk, void* w_fused,
                          void* stream);

/* The absorbed query straight from the projection's input, with the weight
 * of mla_fold_query_weight:
 *   q_cat[b,j,h, 0:d_c]       = sum_i w_fused[h,:,i] * x[b,j,i]
 *   q_cat[b,j,h, d_c:d_c+d_r] = q_rope[b,j,h,:]
 * which equals mla_absorb_q of q_nope[b,j,h] = w_in[h] x[b,j] up to rounding.
 * x [B,Lq,d_in], q_rope [B,Lq,H,d_rope] (NULL if d_rope = 0), w_fused
 * [H,d_c,d_in] in the fused weight storage order, q_cat [B,Lq,H,d_c+d_rope],
 * all in the storage type.  Float32 accumulation, one rounding.  Where the
 * weight is in fragment order the product runs on the matrix cores; other
 * supported shapes run on a portable kernel.  MLA_ERR_UNSUPPORTED when
 * B*Lq > 4194240. */
int mla_fused_query(const mla_dims* dims, int32_t d_in, const void* x, const void* q_rope, const void* w_fused,
                    void* q_cat, void* stream);

/* Fold the per-head value up-projections into the output projection
 * ("DeepSeek-V3 MLA: Multi-Head Latent Attention Guide", Matrix Absorption
 * Trick section 3, W~^O):
 *   w_fused[r, h*d_c + c] = sum_v w_o[r, h*d_v + v] * w_uv[h,v,c]
 * w_o [d_out, H*d_v] (W^O acting on the heads' outputs concatenated in head
 * order), w_uv [H,d_v,d_c], w_fused [d_out, H*d_c] (in the fused weight
 * storage order above), all in the storage type.
 * Float32 accumulation in order of v, one rounding.  Offline.  Uses
 * num_heads, d_c, d_v and dtype of dims.  d_out in [1, 65536]. */
int mla_fold_output_weight(const mla_dims* dims, int32_t d_out, const void* w_o, const void* w_uv, void* w_fused,
                           void* stream);

/* Bytes of device workspace mla_fused_output needs (float32 split-K
 * partials; 0 when none is needed and the workspace may be NULL).  Host
 * only; d_out in [1, 65536]. */
int mla_fused_output_workspace_bytes(const mla_dims* dims, int32_t d_out, size_t* bytes);

/* The attention output projected by the fused weight of
 * mla_fold_output_weight, straight from the merged latent output:
 *   y[b,j,r] = sum_{h,c} w_fused[r, h*d_c + c] * o_latent[b,j,h,c]
 * which equals W^O applied to the concatenated mla_absorb_out result up to
 * rounding.  o_latent [B,Lq,H,d_c] float32 (as mla_combine writes it),
 * w_fused [d_out, H*d_c] storage type in the fused weight storage order, y
 * [B,Lq,d_out] storage type; workspace at least
 * mla_fused_output_workspace_bytes() bytes (MLA_ERR_WORKSPACE if
 * workspace_bytes is smaller), contents on entry irrelevant.
 * Float32 accumulation; on the matrix cores (where the weight is in fragment
 * order) o_latent enters as a bf16 hi + lo pair and the split of H*d_c, and
 * so the order of the float32 additions, follows the device's compute-unit
 * count: reproducible on one device type.  MLA_ERR_UNSUPPORTED when B*Lq >
 * 4194240. */
int mla_fused_output(const mla_dims* dims, int32_t d_out, const float* o_latent, const void* w_fused, void* y,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* mla_status_str(int status);

/* Library version as major*10000 + minor*100 + patch. */
int mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_MLA_H */
