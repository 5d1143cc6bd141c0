// Launchers shared between the C-ABI front end (api.cpp) and the kernel files.
// Every launcher assumes its arguments were validated by the front end.
#pragma once

#include <hip/hip_runtime.h>

#include "mla.h"

namespace mla {

// planner (plan.hip)
// d counts head groups as sequences when hg_log2 > 0 (plan_body.h)
hipError_t launch_plan(const mla_dims& d, const int32_t* seq_lens, int splits, int grid, int min_chunk, int ov,
                       int32_t* ws, hipStream_t stream, int hg_log2);

// portable kernels for any supported shape (generic.hip)
hipError_t launch_absorb_q_generic(const mla_dims& d, const void* q_nope, const void* q_rope, const void* w_uk,
                                   void* q_cat, hipStream_t stream);
hipError_t launch_decode_generic(const mla_dims& d, const void* q_cat, const void* cache, const int32_t* table,
                                 const int32_t* ws, float scale, int splits, int grid, void* o_part,
                                 float* lse_part, hipStream_t stream, bool fp8, float kv_scale);
int decode_generic_rows_per_group();
hipError_t launch_combine(const mla_dims& d, int splits, const void* o_part, const float* lse_part, float* o,
                          float* lse, hipStream_t stream);
hipError_t launch_absorb_out_generic(const mla_dims& d, const float* o, const void* w_uv, void* out,
                                     hipStream_t stream);

// matrix-core decode for bf16, d_c = 512, d_rope = 64 (decode_mfma.hip)
bool decode_mfma_supported(const mla_dims& d);
// fp8: the cache holds E4M3 codes standing for kv_scale times their value
// hg_log2 > 0: d counts head groups as sequences (DecodeArgs::hg_log2)
hipError_t launch_decode_mfma(const mla_dims& d, const void* q_cat, const void* cache, const int32_t* table,
                              const int32_t* ws, float scale, int splits, int grid, void* o_part, float* lse_part,
                              hipStream_t stream, bool fp8, float kv_scale, int hg_log2);

// matrix-core absorption GEMMs for bf16, d_nope = d_v = 128, d_c = 512 (absorb_mfma.hip)
bool absorb_mfma_supported(const mla_dims& d);
struct PlanArgs;  // plan_body.h
// plan: when given, one extra workgroup of the same launch runs the decode planner
hipError_t launch_absorb_q_mfma(const mla_dims& d, const void* q_nope, const void* q_rope, const void* w_uk,
                                void* q_cat, hipStream_t stream, const PlanArgs* plan = nullptr);
hipError_t launch_absorb_out_mfma(const mla_dims& d, const float* o, const void* w_uv, void* out,
                                  hipStream_t stream);
// fused log-sum-exp merge + W_UV product (same support as the MFMA absorb
// kernels, any split count)
// cus: the device's CU count (a grid of at most half of it splits the outputs over two workgroups)
hipError_t launch_combine_out_mfma(const mla_dims& d, int splits, const void* o_part, const float* lse_part,
                                   const void* w_uv, void* out, float* o_latent, float* lse, hipStream_t stream,
                                   int cus);

// cache append (append.hip): matrix-core split-K path for bf16 storage with
// d_model % 128 == 0 and (d_c + d_rope) % 32 == 0, portable path otherwise
bool append_mfma_supported(const mla_dims& d, int d_model);
int append_max_ksplit();
int append_ksplit(const mla_dims& d, int d_model, int cus, int* per_out);
hipError_t launch_append_mfma(const mla_dims& d, int d_model, int cus, const void* h, const void* w_dkv,
                              const void* w_kr, float rope_base, const int32_t* table, const int32_t* seq_lens,
                              void* cache, float* part, hipStream_t stream, bool fp8, float kv_scale);
// fp8: the cache holds E4M3 codes of value / kv_scale
hipError_t launch_append_generic(const mla_dims& d, int d_model, const void* h, const void* w_dkv, const void* w_kr,
                                 float rope_base, const int32_t* table, const int32_t* seq_lens, void* cache,
                                 hipStream_t stream, bool fp8, float kv_scale);

// prefill (prefill.hip): matrix-core path for bf16 with d_c = 512, d_rope = 64,
// d_nope = d_v = 128; portable path otherwise
struct PrefillLayout {
  int64_t v_off, r_off;  // element offsets of V and R in the workspace (Kn at 0)
  int64_t total_bytes;
};
bool prefill_mfma_supported(const mla_dims& d);
PrefillLayout prefill_layout(const mla_dims& d, int64_t tokens);
// whether the matrix-core attention grid for this batch and longest sequence
// stays within 2^32 - 1 threads
bool prefill_grid_fits(const mla_dims& d, int max_seqlen);
hipError_t launch_prefill(const mla_dims& d, int tokens, int max_seqlen, const int32_t* cu, const void* q_nope,
                          const void* q_rope, const void* c_kv, const void* k_rope, const void* w_uk,
                          const void* w_uv, float scale, int causal, void* out, float* lse, void* ws, bool mfma,
                          hipStream_t stream);

// offline weight folds and the fused runtime products (fold.hip).  The
// support tests say where the matrix-core path serves a shape; there the
// fused weights are stored in the packed fragment order (packed = true),
// which the folds write and both kernel families of the products read.
bool fused_query_mfma_supported(const mla_dims& d, int d_in);
bool fused_output_mfma_supported(const mla_dims& d, int d_out);
hipError_t launch_fold_query(const mla_dims& d, int d_in, const void* w_in, const void* w_uk, void* w_fused,
                             bool packed, hipStream_t stream);
hipError_t launch_fold_output(const mla_dims& d, int d_out, const void* w_o, const void* w_uv, void* w_fused,
                              bool packed, hipStream_t stream);
int linear_max_ksplit();
int linear_ksplit(int M, int N, int K, int block, int slots, int cus, int max_ks, int* per_out);
hipError_t launch_fused_query(const mla_dims& d, int d_in, int cus, const void* x, const void* q_rope,
                              const void* w_fused, void* q_cat, bool mfma, bool packed, hipStream_t stream);
hipError_t launch_fused_output(const mla_dims& d, int d_out, int cus, const float* o, const void* w_fused, void* y,
                               float* ws, bool mfma, bool packed, hipStream_t stream);

}  // namespace mla
