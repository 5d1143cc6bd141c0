// C-ABI front end of libmla: host-side validation, kernel selection, launches.
//
// Every entry point validates its arguments completely before the first HIP
// call, so an invalid call enqueues nothing and touches no buffer.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.h"
#include "internal.h"
#include "plan_body.h"
#include "mla.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxSplits = 4096;
constexpr int kMaxBatch = 1 << 20;
constexpr int kMaxDModel = 1 << 16;
// rows (B * q_len) of the fused products: the portable kernel's row blocks
// of 64 must fit a grid dimension
constexpr int64_t kMaxFusedRows = (int64_t)65535 * 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }

int check_dims(const mla_dims* d) {
  if (d == nullptr) return MLA_ERR_INVALID_ARG;
  if (d->batch <= 0 || d->q_len <= 0 || d->num_heads <= 0 || d->d_c <= 0 || d->d_rope < 0 || d->d_nope <= 0 ||
      d->d_v <= 0 || d->block_size <= 0 || d->max_blocks_per_seq <= 0 || d->num_blocks <= 0)
    return MLA_ERR_INVALID_ARG;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (d->batch > kMaxBatch) return MLA_ERR_UNSUPPORTED;
  if (d->q_len > 8) return MLA_ERR_UNSUPPORTED;
  if (d->d_c % 16 != 0 || d->d_c > 1024) return MLA_ERR_UNSUPPORTED;
  if (d->d_rope % 8 != 0 || d->d_c + d->d_rope > 1088) return MLA_ERR_UNSUPPORTED;
  if (d->d_nope > 1024 || d->d_v > 1024) return MLA_ERR_UNSUPPORTED;
  if (d->num_heads > 4096) return MLA_ERR_UNSUPPORTED;
  // every index the kernels form must fit comfortably in 31 bits per dimension product
  const int64_t max_len = (int64_t)d->max_blocks_per_seq * d->block_size;
  if (max_len > (int64_t)1 << 30) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Per-device compute-unit count, queried once per device.
int device_cus(int* cus) {
  static std::mutex mu;
  static int cache[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return MLA_ERR_HIP;
    cache[dev] = n;
  }
  *cus = cache[dev];
  return MLA_OK;
}

// Which kernels serve these dimensions.  MLA_KERNELS=portable forces the
// portable float32-VALU kernels for every step (both families are HIP; the
// switch exists to cross-check one against the other).
enum class DecodeKind { Generic, Mfma };

bool force_generic() {
  const char* e = std::getenv("MLA_KERNELS");
  return e != nullptr && std::strcmp(e, "portable") == 0;
}

DecodeKind pick_decode(const mla_dims& d) {
  if (!force_generic() && mla::decode_mfma_supported(d)) return DecodeKind::Mfma;
  return DecodeKind::Generic;
}

struct DecodeShape {
  int grid;       // workgroups launched along the split axis
  int min_chunk;  // smallest token range (in 64-token tiles) worth one workgroup
  int ov;         // overhead tiles the planner charges per sequence
  int hg_log2;    // the heads of a sequence run as 2^hg_log2 groups, each scheduled on its own
};

// Largest head grouping the dimensions allow (q_len = 1 and 64 or 128 heads:
// groups of 32 heads), whatever the device; the workspace is sized for it.
int max_hg_log2(const mla_dims& d) {
  if (d.q_len != 1) return 0;
  if (d.num_heads == 128) return 2;
  if (d.num_heads == 64) return 1;
  return 0;
}

// The schedule's view of the batch: head groups counted as sequences.
mla_dims grouped_dims(const mla_dims& d, int hg_log2) {
  mla_dims g = d;
  g.batch = d.batch << hg_log2;
  g.num_heads = d.num_heads >> hg_log2;
  return g;
}

int decode_shape(const mla_dims& d, bool fp8, DecodeShape* out) {
  int cus = 0;
  int st = device_cus(&cus);
  if (st != MLA_OK) return st;
  switch (pick_decode(d)) {
    case DecodeKind::Generic: {
      const int R = d.q_len * d.num_heads;
      const int row_groups = (R + mla::decode_generic_rows_per_group() - 1) / mla::decode_generic_rows_per_group();
      // about eight resident workgroups per CU over all row groups
      int g = (cus * 8 + row_groups - 1) / row_groups;
      out->grid = g < 1 ? 1 : g;
      out->min_chunk = 1;
      out->ov = 0;
      out->hg_log2 = 0;
      return MLA_OK;
    }
    case DecodeKind::Mfma: {
      // one 144 KiB-LDS workgroup per CU; a range must amortise the fixed
      // cost of a piece against the cache rows it streams.  Measured per
      // phase on MI355X, a piece costs about 1.5 tiles of pipeline fill plus
      // R * (1152 B of queries + 2048 B of partial result) at 0.9 times the
      // cost of streaming as many bytes of cache, in 64-row tiles of 73728 B:
      //   ov = round(1.5 + R * 3200 * 0.9 / 73728)   (7 at R = 128, 3 at R = 32)
      // An FP8 tile is half the bytes, so the same fixed cost is twice the
      // tiles (12 at R = 128) and the smallest worthwhile range doubles.
      // The smallest range is one tile (two for FP8): it binds only when the
      // whole batch has fewer tiles than the grid, where more workgroups
      // finish sooner (one 4096-token sequence: 28 us against 34 us with
      // four-tile ranges) and the merge reads the extra splits in parallel.
      //
      // Head groups: a batch too short to give every CU a tile keeps most
      // CUs idle, and each busy one pays for all 128 query rows and a
      // 128-row partial result per piece.  With q_len = 1 the heads are then
      // split into groups of 32 (or 64), each scheduled as a sequence of
      // its own on the same cache rows: 2 to 4 times the workgroups, each
      // with a quarter (half) of the fixed cost.  The grouping doubles while
      // the grouped count of the batch's largest possible tile total still
      // fits the grid; it depends only on the dimensions and the CU count, so
      // the planner and the attention call always agree on it (one
      // 4096-token sequence: 25 us against 34 us for plan and attention).
      const int64_t tile_bytes = fp8 ? 36864 : 73728;
      const int64_t max_tiles = (int64_t)d.batch * (((int64_t)d.max_blocks_per_seq * d.block_size +
                                                     mla::kPlanTile - 1) / mla::kPlanTile);
      int hg = 0;
      while (hg < max_hg_log2(d) && (max_tiles << (hg + 1)) <= (int64_t)cus) ++hg;
      const int R = (d.q_len * d.num_heads) >> hg;
      out->grid = cus;
      out->min_chunk = fp8 ? 2 : 1;
      const int ov = (int)(((int64_t)R * 2880 + 2 * tile_bytes) / tile_bytes);
      out->ov = ov < 1 ? 1 : ov;
      out->hg_log2 = hg;
      return MLA_OK;
    }
  }
  return MLA_ERR_UNSUPPORTED;
}

// ---- allocation-free decode: the schedule lives in a file-scope device array
//
// Each GPU holds its own copy of `scratch` until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a stand-in
// symbol): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// handed to the kernels.
constexpr int kScratchMaxBatch = 65536;
constexpr size_t kScratchWords = (size_t)mla::kWsCu + 2 * (size_t)kScratchMaxBatch + 1;
static __device__ __align__(256) int32_t scratch[kScratchWords];

// Device address of this device's scratch (nullptr and MLA_ERR_HIP on failure).
int scratch_address(int32_t** out) {
  static std::mutex mu;
  static int32_t* addr[kMaxDevices] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_HIP;
    addr[dev] = static_cast<int32_t*>(p);
  }
  *out = addr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_str(int s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dimensions or dtype";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int mla_version(void) { return 100; }

int mla_absorb_q(const mla_dims* d, const void* q_nope, const void* q_rope, const void* w_uk, void* q_cat,
                 void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!ptr_ok(q_nope) || !ptr_ok(w_uk) || !ptr_ok(q_cat) || (d->d_rope > 0 && !ptr_ok(q_rope)))
    return MLA_ERR_INVALID_ARG;
  if (!force_generic() && mla::absorb_mfma_supported(*d))
    return to_status(mla::launch_absorb_q_mfma(*d, q_nope, q_rope, w_uk, q_cat, (hipStream_t)stream));
  return to_status(mla::launch_absorb_q_generic(*d, q_nope, q_rope, w_uk, q_cat, (hipStream_t)stream));
}

int mla_decode_workspace_bytes(const mla_dims* d, int32_t num_splits, size_t* bytes) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (bytes == nullptr || num_splits < 1 || num_splits > kMaxSplits) return MLA_ERR_INVALID_ARG;
  const size_t b = mla::workspace_words(d->batch << max_hg_log2(*d)) * sizeof(int32_t);
  *bytes = (b + 255) / 256 * 256;
  return MLA_OK;
}

namespace {

int num_splits_impl(const mla_dims* d, int32_t max_seq_len, int64_t total_tokens, int32_t* num_splits, bool fp8) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (num_splits == nullptr || max_seq_len <= 0 || total_tokens < max_seq_len) return MLA_ERR_INVALID_ARG;
  DecodeShape sh;
  st = decode_shape(*d, fp8, &sh);
  if (st != MLA_OK) return st;
  const int64_t tile = 64;
  // lower bound of the planner's sum, so S is never too small; each head
  // group is scheduled as a sequence of the same length
  const int64_t total_tiles = ((total_tokens + tile - 1) / tile) << sh.hg_log2;
  int64_t chunk = (total_tiles + sh.grid - 1) / sh.grid;
  if (chunk < sh.min_chunk) chunk = sh.min_chunk;
  const int64_t maxn = (max_seq_len + tile - 1) / tile;
  int64_t s = (maxn <= 1) ? 1 : (maxn - 1 + chunk - 1) / chunk + 1;
  if (s < 2 && maxn > 1) s = 2;
  if (s > kMaxSplits) s = kMaxSplits;
  *num_splits = (int32_t)s;
  return MLA_OK;
}

int check_decode_common(const mla_dims* d, int32_t num_splits, const void* workspace, size_t workspace_bytes) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!ptr_ok(workspace)) return MLA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > kMaxSplits) return MLA_ERR_INVALID_ARG;
  size_t need = 0;
  mla_decode_workspace_bytes(d, num_splits, &need);
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
  return MLA_OK;
}

bool positive_finite(float x) { return x > 0.f && x == x && x != INFINITY; }

int check_attention_args(const mla_dims* d, const void* q_cat, const void* kv_cache, const int32_t* block_table,
                         float softmax_scale, void* o_partial, float* lse_partial, bool fp8, float kv_scale) {
  if (!ptr_ok(q_cat) || !ptr_ok(kv_cache) || !ptr_ok(block_table) || !ptr_ok(o_partial) || !ptr_ok(lse_partial))
    return MLA_ERR_INVALID_ARG;
  if (!positive_finite(softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (fp8 && !positive_finite(kv_scale)) return MLA_ERR_INVALID_ARG;
  (void)d;
  return MLA_OK;
}

hipError_t enqueue_plan(const mla_dims& d, const int32_t* seq_lens, int32_t num_splits, void* workspace,
                        const DecodeShape& sh, hipStream_t s) {
  return mla::launch_plan(grouped_dims(d, sh.hg_log2), seq_lens, num_splits, sh.grid, sh.min_chunk, sh.ov,
                          static_cast<int32_t*>(workspace), s, sh.hg_log2);
}

hipError_t enqueue_attention(const mla_dims& d, const void* q_cat, const void* kv_cache, const int32_t* block_table,
                             float softmax_scale, int32_t num_splits, const void* workspace, const DecodeShape& sh,
                             void* o_partial, float* lse_partial, hipStream_t s, bool fp8, float kv_scale) {
  const int32_t* ws = static_cast<const int32_t*>(workspace);
  const float kv = fp8 ? kv_scale : 1.f;
  switch (pick_decode(d)) {
    case DecodeKind::Generic:
      return mla::launch_decode_generic(d, q_cat, kv_cache, block_table, ws, softmax_scale, num_splits, sh.grid,
                                        o_partial, lse_partial, s, fp8, kv);
    case DecodeKind::Mfma:
      return mla::launch_decode_mfma(grouped_dims(d, sh.hg_log2), q_cat, kv_cache, block_table, ws, softmax_scale,
                                     num_splits, sh.grid, o_partial, lse_partial, s, fp8, kv, sh.hg_log2);
  }
  return hipErrorInvalidValue;
}

int plan_impl(const mla_dims* d, const int32_t* seq_lens, int32_t num_splits, void* workspace,
              size_t workspace_bytes, void* stream, bool fp8) {
  int st = check_decode_common(d, num_splits, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  if (!ptr_ok(seq_lens)) return MLA_ERR_INVALID_ARG;
  DecodeShape sh;
  st = decode_shape(*d, fp8, &sh);
  if (st != MLA_OK) return st;
  return to_status(enqueue_plan(*d, seq_lens, num_splits, workspace, sh, (hipStream_t)stream));
}

int planned_impl(const mla_dims* d, const void* q_cat, const void* kv_cache, const int32_t* block_table,
                 float softmax_scale, int32_t num_splits, const void* workspace, size_t workspace_bytes,
                 void* o_partial, float* lse_partial, void* stream, bool fp8, float kv_scale) {
  int st = check_decode_common(d, num_splits, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  st = check_attention_args(d, q_cat, kv_cache, block_table, softmax_scale, o_partial, lse_partial, fp8, kv_scale);
  if (st != MLA_OK) return st;
  DecodeShape sh;
  st = decode_shape(*d, fp8, &sh);
  if (st != MLA_OK) return st;
  return to_status(enqueue_attention(*d, q_cat, kv_cache, block_table, softmax_scale, num_splits, workspace, sh,
                                     o_partial, lse_partial, (hipStream_t)stream, fp8, kv_scale));
}

int decode_impl(const mla_dims* d, const void* q_cat, const void* kv_cache, const int32_t* block_table,
                const int32_t* seq_lens, float softmax_scale, int32_t num_splits, void* workspace,
                size_t workspace_bytes, void* o_partial, float* lse_partial, void* stream, bool fp8,
                float kv_scale) {
  int st = check_decode_common(d, num_splits, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  if (!ptr_ok(seq_lens)) return MLA_ERR_INVALID_ARG;
  st = check_attention_args(d, q_cat, kv_cache, block_table, softmax_scale, o_partial, lse_partial, fp8, kv_scale);
  if (st != MLA_OK) return st;
  DecodeShape sh;
  st = decode_shape(*d, fp8, &sh);
  if (st != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = enqueue_plan(*d, seq_lens, num_splits, workspace, sh, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  return to_status(enqueue_attention(*d, q_cat, kv_cache, block_table, softmax_scale, num_splits, workspace, sh,
                                     o_partial, lse_partial, s, fp8, kv_scale));
}

}  // namespace

int mla_decode_num_splits(const mla_dims* d, int32_t max_seq_len, int64_t total_tokens, int32_t* num_splits) {
  return num_splits_impl(d, max_seq_len, total_tokens, num_splits, false);
}

namespace {

// Longest sequence and total tokens from host lengths (each clamped into
// [0, MB * block_size]), or a batch of max_seq_len-long sequences.
int choose_splits_impl(const mla_dims* d, const int32_t* lens, int32_t max_seq_len, int32_t* num_splits, bool fp8) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (num_splits == nullptr) return MLA_ERR_INVALID_ARG;
  int64_t total = 0;
  int32_t mx = 0;
  if (lens != nullptr) {
    const int64_t cap = (int64_t)d->max_blocks_per_seq * d->block_size;
    for (int b = 0; b < d->batch; ++b) {
      const int64_t L = lens[b] < 0 ? 0 : (lens[b] > cap ? cap : lens[b]);
      total += L;
      if (L > mx) mx = (int32_t)L;
    }
  } else {
    mx = max_seq_len;
    total = (int64_t)d->batch * max_seq_len;
  }
  if (mx < 1) return MLA_ERR_INVALID_ARG;
  return num_splits_impl(d, mx, total, num_splits, fp8);
}

}  // namespace

int mla_choose_splits(const mla_dims* d, const int32_t* seq_lens_host, int32_t max_seq_len, int32_t* num_splits) {
  return choose_splits_impl(d, seq_lens_host, max_seq_len, num_splits, false);
}

int mla_choose_splits_fp8(const mla_dims* d, const int32_t* seq_lens_host, int32_t max_seq_len,
                          int32_t* num_splits) {
  return choose_splits_impl(d, seq_lens_host, max_seq_len, num_splits, true);
}

namespace {

static int absorb_q_plan_impl(const mla_dims* d, const void* q_nope, const void* q_rope, const void* w_uk, void* q_cat,
                       const int32_t* seq_lens, int32_t num_splits, void* workspace, size_t workspace_bytes,
                       void* stream, bool fp8) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!ptr_ok(q_nope) || !ptr_ok(w_uk) || !ptr_ok(q_cat) || (d->d_rope > 0 && !ptr_ok(q_rope)))
    return MLA_ERR_INVALID_ARG;
  st = check_decode_common(d, num_splits, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  if (!ptr_ok(seq_lens)) return MLA_ERR_INVALID_ARG;
  DecodeShape sh;
  st = decode_shape(*d, fp8, &sh);
  if (st != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (!force_generic() && mla::absorb_mfma_supported(*d)) {
    const mla::PlanArgs pa = mla::make_plan_args(grouped_dims(*d, sh.hg_log2), seq_lens, num_splits, sh.grid,
                                                  sh.min_chunk, sh.ov, static_cast<int32_t*>(workspace), sh.hg_log2);
    return to_status(mla::launch_absorb_q_mfma(*d, q_nope, q_rope, w_uk, q_cat, s, &pa));
  }
  hipError_t e = mla::launch_absorb_q_generic(*d, q_nope, q_rope, w_uk, q_cat, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  return to_status(enqueue_plan(*d, seq_lens, num_splits, workspace, sh, s));
}

}  // namespace

int mla_absorb_q_plan(const mla_dims* d, const void* q_nope, const void* q_rope, const void* w_uk, void* q_cat,
                      const int32_t* seq_lens, int32_t num_splits, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return absorb_q_plan_impl(d, q_nope, q_rope, w_uk, q_cat, seq_lens, num_splits, workspace, workspace_bytes, stream,
                            false);
}

int mla_absorb_q_plan_fp8(const mla_dims* d, const void* q_nope, const void* q_rope, const void* w_uk, void* q_cat,
                          const int32_t* seq_lens, int32_t num_splits, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return absorb_q_plan_impl(d, q_nope, q_rope, w_uk, q_cat, seq_lens, num_splits, workspace, workspace_bytes, stream,
                            true);
}

int mla_decode_plan(const mla_dims* d, const int32_t* seq_lens, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return plan_impl(d, seq_lens, num_splits, workspace, workspace_bytes, stream, false);
}

int mla_decode_planned(const mla_dims* d, const void* q_cat, const void* kv_cache, const int32_t* block_table,
                       float softmax_scale, int32_t num_splits, const void* workspace, size_t workspace_bytes,
                       void* o_partial, float* lse_partial, void* stream) {
  return planned_impl(d, q_cat, kv_cache, block_table, softmax_scale, num_splits, workspace, workspace_bytes,
                      o_partial, lse_partial, stream, false, 1.f);
}

int mla_decode(const mla_dims* d, const void* q_cat, const void* kv_cache, const int32_t* block_table,
               const int32_t* seq_lens, float softmax_scale, int32_t num_splits, void* workspace,
               size_t workspace_bytes, void* o_partial, float* lse_partial, void* stream) {
  return decode_impl(d, q_cat, kv_cache, block_table, seq_lens, softmax_scale, num_splits, workspace,
                     workspace_bytes, o_partial, lse_partial, stream, false, 1.f);
}

int mla_decode_noalloc(const mla_dims* d, const void* q_cat, const void* kv_cache, const int32_t* block_table,
                       const int32_t* seq_lens, float softmax_scale, int32_t num_splits, void* o_partial,
                       float* lse_partial, void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits) return MLA_ERR_INVALID_ARG;
  if (!ptr_ok(seq_lens)) return MLA_ERR_INVALID_ARG;
  st = check_attention_args(d, q_cat, kv_cache, block_table, softmax_scale, o_partial, lse_partial, false, 1.f);
  if (st != MLA_OK) return st;
  if (d->batch > kScratchMaxBatch) return MLA_ERR_WORKSPACE;
  int32_t* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MLA_OK) return st;
  DecodeShape sh;
  st = decode_shape(*d, false, &sh);
  if (st != MLA_OK) return st;
  if (((int64_t)d->batch << sh.hg_log2) > kScratchMaxBatch) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  // the planner writes every schedule word the attention kernel reads, so
  // nothing left from an earlier call needs clearing
  hipError_t e = enqueue_plan(*d, seq_lens, num_splits, ws, sh, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  return to_status(enqueue_attention(*d, q_cat, kv_cache, block_table, softmax_scale, num_splits, ws, sh, o_partial,
                                     lse_partial, s, false, 1.f));
}

int mla_decode_num_splits_fp8(const mla_dims* d, int32_t max_seq_len, int64_t total_tokens, int32_t* num_splits) {
  return num_splits_impl(d, max_seq_len, total_tokens, num_splits, true);
}

int mla_decode_plan_fp8(const mla_dims* d, const int32_t* seq_lens, int32_t num_splits, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return plan_impl(d, seq_lens, num_splits, workspace, workspace_bytes, stream, true);
}

int mla_decode_planned_fp8(const mla_dims* d, const void* q_cat, const uint8_t* kv_cache, float kv_scale,
                           const int32_t* block_table, float softmax_scale, int32_t num_splits, const void* workspace,
                           size_t workspace_bytes, void* o_partial, float* lse_partial, void* stream) {
  return planned_impl(d, q_cat, kv_cache, block_table, softmax_scale, num_splits, workspace, workspace_bytes,
                      o_partial, lse_partial, stream, true, kv_scale);
}

int mla_decode_fp8(const mla_dims* d, const void* q_cat, const uint8_t* kv_cache, float kv_scale,
                   const int32_t* block_table, const int32_t* seq_lens, float softmax_scale, int32_t num_splits,
                   void* workspace, size_t workspace_bytes, void* o_partial, float* lse_partial, void* stream) {
  return decode_impl(d, q_cat, kv_cache, block_table, seq_lens, softmax_scale, num_splits, workspace,
                     workspace_bytes, o_partial, lse_partial, stream, true, kv_scale);
}

int mla_combine(const mla_dims* d, int32_t num_splits, const void* o_partial, const float* lse_partial,
                float* o_latent, float* lse, void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!ptr_ok(o_partial) || !ptr_ok(lse_partial) || !ptr_ok(o_latent) || (lse != nullptr && !aligned16(lse)))
    return MLA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > kMaxSplits) return MLA_ERR_INVALID_ARG;
  return to_status(mla::launch_combine(*d, num_splits, o_partial, lse_partial, o_latent, lse, (hipStream_t)stream));
}

int mla_absorb_out(const mla_dims* d, const float* o_latent, const void* w_uv, void* out, void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!ptr_ok(o_latent) || !ptr_ok(w_uv) || !ptr_ok(out)) return MLA_ERR_INVALID_ARG;
  if (!force_generic() && mla::absorb_mfma_supported(*d))
    return to_status(mla::launch_absorb_out_mfma(*d, o_latent, w_uv, out, (hipStream_t)stream));
  return to_status(mla::launch_absorb_out_generic(*d, o_latent, w_uv, out, (hipStream_t)stream));
}

int mla_combine_absorb_out(const mla_dims* d, int32_t num_splits, const void* o_partial, const float* lse_partial,
                           const void* w_uv, void* out, float* o_latent, float* lse, void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (!ptr_ok(o_partial) || !ptr_ok(lse_partial) || !ptr_ok(w_uv) || !ptr_ok(out) ||
      (o_latent != nullptr && !aligned16(o_latent)) || (lse != nullptr && !aligned16(lse)))
    return MLA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > kMaxSplits) return MLA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (!force_generic() && mla::absorb_mfma_supported(*d)) {
    int cus = 0;
    st = device_cus(&cus);
    if (st != MLA_OK) return st;
    return to_status(
        mla::launch_combine_out_mfma(*d, num_splits, o_partial, lse_partial, w_uv, out, o_latent, lse, s, cus));
  }
  // two-kernel route: the merged latent output goes through o_latent
  if (o_latent == nullptr) return MLA_ERR_UNSUPPORTED;
  hipError_t e = mla::launch_combine(*d, num_splits, o_partial, lse_partial, o_latent, lse, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (!force_generic() && mla::absorb_mfma_supported(*d))
    return to_status(mla::launch_absorb_out_mfma(*d, o_latent, w_uv, out, s));
  return to_status(mla::launch_absorb_out_generic(*d, o_latent, w_uv, out, s));
}

int mla_cache_append_workspace_bytes(const mla_dims* d, int32_t d_model, size_t* bytes) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (bytes == nullptr || d_model < 1 || d_model > kMaxDModel) return MLA_ERR_INVALID_ARG;
  size_t b = 0;
  if (mla::append_mfma_supported(*d, d_model))  // float32 split-K partials [KS, B*Lq, d_c + d_rope]
    b = (size_t)mla::append_max_ksplit() * d->batch * d->q_len * (d->d_c + d->d_rope) * sizeof(float);
  *bytes = (b + 255) / 256 * 256;
  return MLA_OK;
}

namespace {

int cache_append_impl(const mla_dims* d, int32_t d_model, const void* h, const void* w_dkv, const void* w_kr,
                      float rope_base, const int32_t* block_table, const int32_t* seq_lens, void* kv_cache,
                      void* workspace, size_t workspace_bytes, void* stream, bool fp8, float kv_scale) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (fp8 && !positive_finite(kv_scale)) return MLA_ERR_INVALID_ARG;
  if (d_model < 1 || d_model > kMaxDModel) return MLA_ERR_INVALID_ARG;
  if (!ptr_ok(h) || !ptr_ok(w_dkv) || (d->d_rope > 0 && !ptr_ok(w_kr)) || !ptr_ok(block_table) ||
      !ptr_ok(seq_lens) || !ptr_ok(kv_cache))
    return MLA_ERR_INVALID_ARG;
  if (!(rope_base > 0.f) || rope_base == INFINITY) return MLA_ERR_INVALID_ARG;
  size_t need = 0;
  mla_cache_append_workspace_bytes(d, d_model, &need);
  if (need > 0 && !ptr_ok(workspace)) return MLA_ERR_INVALID_ARG;
  if (need > 0 && workspace_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (!force_generic() && mla::append_mfma_supported(*d, d_model)) {
    int cus = 0;
    st = device_cus(&cus);
    if (st != MLA_OK) return st;
    return to_status(mla::launch_append_mfma(*d, d_model, cus, h, w_dkv, w_kr, rope_base, block_table, seq_lens,
                                             kv_cache, static_cast<float*>(workspace), s, fp8, kv_scale));
  }
  return to_status(mla::launch_append_generic(*d, d_model, h, w_dkv, w_kr, rope_base, block_table, seq_lens,
                                              kv_cache, s, fp8, kv_scale));
}

}  // namespace

int mla_cache_append(const mla_dims* d, int32_t d_model, const void* h, const void* w_dkv, const void* w_kr,
                     float rope_base, const int32_t* block_table, const int32_t* seq_lens, void* kv_cache,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return cache_append_impl(d, d_model, h, w_dkv, w_kr, rope_base, block_table, seq_lens, kv_cache, workspace,
                           workspace_bytes, stream, false, 1.f);
}

int mla_cache_append_fp8(const mla_dims* d, int32_t d_model, const void* h, const void* w_dkv, const void* w_kr,
                         float rope_base, float kv_scale, const int32_t* block_table, const int32_t* seq_lens,
                         uint8_t* kv_cache, void* workspace, size_t workspace_bytes, void* stream) {
  return cache_append_impl(d, d_model, h, w_dkv, w_kr, rope_base, block_table, seq_lens, kv_cache, workspace,
                           workspace_bytes, stream, true, kv_scale);
}

int mla_prefill_workspace_bytes(const mla_dims* d, int32_t total_tokens, size_t* bytes) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (bytes == nullptr || total_tokens < 1) return MLA_ERR_INVALID_ARG;
  *bytes = (size_t)mla::prefill_layout(*d, total_tokens).total_bytes;
  return MLA_OK;
}

int mla_prefill(const mla_dims* d, int32_t total_tokens, int32_t max_seqlen, const int32_t* cu_seqlens,
                const void* q_nope, const void* q_rope, const void* c_kv, const void* k_rope, const void* w_uk,
                const void* w_uv, float softmax_scale, int32_t causal, void* out, float* lse, void* workspace,
                size_t workspace_bytes, void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (total_tokens < 1 || max_seqlen < 1 || max_seqlen > total_tokens || (causal != 0 && causal != 1))
    return MLA_ERR_INVALID_ARG;
  if (!ptr_ok(cu_seqlens) || !ptr_ok(q_nope) || !ptr_ok(c_kv) || !ptr_ok(w_uk) || !ptr_ok(w_uv) || !ptr_ok(out) ||
      !ptr_ok(workspace) || (d->d_rope > 0 && (!ptr_ok(q_rope) || !ptr_ok(k_rope))) ||
      (lse != nullptr && !aligned16(lse)))
    return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return MLA_ERR_INVALID_ARG;
  const mla::PrefillLayout lay = mla::prefill_layout(*d, total_tokens);
  if (workspace_bytes < (size_t)lay.total_bytes) return MLA_ERR_WORKSPACE;
  const bool mfma = !force_generic() && mla::prefill_mfma_supported(*d);
  // the matrix-core kernels address the workspace with 32-bit byte offsets,
  // and the attention grid's thread count must fit 32 bits
  if (mfma && lay.total_bytes >= ((int64_t)1 << 32)) return MLA_ERR_UNSUPPORTED;
  if (mfma && !mla::prefill_grid_fits(*d, max_seqlen)) return MLA_ERR_UNSUPPORTED;
  return to_status(mla::launch_prefill(*d, total_tokens, max_seqlen, cu_seqlens, q_nope, q_rope, c_kv, k_rope, w_uk,
                                       w_uv, softmax_scale, causal, out, lse, workspace, mfma, (hipStream_t)stream));
}

int mla_fold_query_weight(const mla_dims* d, int32_t d_in, const void* w_in, const void* w_uk, void* w_fused,
                          void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (d_in < 1 || d_in > kMaxDModel) return MLA_ERR_INVALID_ARG;
  if (!ptr_ok(w_in) || !ptr_ok(w_uk) || !ptr_ok(w_fused)) return MLA_ERR_INVALID_ARG;
  return to_status(mla::launch_fold_query(*d, d_in, w_in, w_uk, w_fused, mla::fused_query_mfma_supported(*d, d_in),
                                          (hipStream_t)stream));
}

int mla_fused_query(const mla_dims* d, int32_t d_in, const void* x, const void* q_rope, const void* w_fused,
                    void* q_cat, void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (d_in < 1 || d_in > kMaxDModel) return MLA_ERR_INVALID_ARG;
  if (!ptr_ok(x) || !ptr_ok(w_fused) || !ptr_ok(q_cat) || (d->d_rope > 0 && !ptr_ok(q_rope)))
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)d->batch * d->q_len > kMaxFusedRows) return MLA_ERR_UNSUPPORTED;
  const bool packed = mla::fused_query_mfma_supported(*d, d_in);
  const bool mfma = packed && !force_generic();
  int cus = 1;
  if (mfma && (st = device_cus(&cus)) != MLA_OK) return st;
  return to_status(
      mla::launch_fused_query(*d, d_in, cus, x, q_rope, w_fused, q_cat, mfma, packed, (hipStream_t)stream));
}

int mla_fold_output_weight(const mla_dims* d, int32_t d_out, const void* w_o, const void* w_uv, void* w_fused,
                           void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (d_out < 1 || d_out > kMaxDModel) return MLA_ERR_INVALID_ARG;
  if (!ptr_ok(w_o) || !ptr_ok(w_uv) || !ptr_ok(w_fused)) return MLA_ERR_INVALID_ARG;
  return to_status(mla::launch_fold_output(*d, d_out, w_o, w_uv, w_fused,
                                           mla::fused_output_mfma_supported(*d, d_out), (hipStream_t)stream));
}

int mla_fused_output_workspace_bytes(const mla_dims* d, int32_t d_out, size_t* bytes) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (bytes == nullptr || d_out < 1 || d_out > kMaxDModel) return MLA_ERR_INVALID_ARG;
  size_t b = 0;
  if (mla::fused_output_mfma_supported(*d, d_out))  // float32 split-K partials [KS, B*Lq, d_out]
    b = (size_t)mla::linear_max_ksplit() * d->batch * d->q_len * d_out * sizeof(float);
  *bytes = (b + 255) / 256 * 256;
  return MLA_OK;
}

int mla_fused_output(const mla_dims* d, int32_t d_out, const float* o_latent, const void* w_fused, void* y,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(d);
  if (st != MLA_OK) return st;
  if (d_out < 1 || d_out > kMaxDModel) return MLA_ERR_INVALID_ARG;
  if (!ptr_ok(o_latent) || !ptr_ok(w_fused) || !ptr_ok(y)) return MLA_ERR_INVALID_ARG;
  if ((int64_t)d->batch * d->q_len > kMaxFusedRows) return MLA_ERR_UNSUPPORTED;
  size_t need = 0;
  mla_fused_output_workspace_bytes(d, d_out, &need);
  if (need > 0 && !ptr_ok(workspace)) return MLA_ERR_INVALID_ARG;
  if (need > 0 && workspace_bytes < need) return MLA_ERR_WORKSPACE;
  const bool packed = mla::fused_output_mfma_supported(*d, d_out);
  const bool mfma = packed && !force_generic();
  int cus = 1;
  if (mfma && (st = device_cus(&cus)) != MLA_OK) return st;
  return to_status(mla::launch_fused_output(*d, d_out, cus, o_latent, w_fused, y, static_cast<float*>(workspace),
                                            mfma, packed, (hipStream_t)stream));
}

int mla_fused_query_weight_packed(const mla_dims* d, int32_t d_in) {
  if (check_dims(d) != MLA_OK || d_in < 1 || d_in > kMaxDModel) return 0;
  return mla::fused_query_mfma_supported(*d, d_in) ? 1 : 0;
}

int mla_fused_output_weight_packed(const mla_dims* d, int32_t d_out) {
  if (check_dims(d) != MLA_OK || d_out < 1 || d_out > kMaxDModel) return 0;
  return mla::fused_output_mfma_supported(*d, d_out) ? 1 : 0;
}

int mla_combine_absorb_out_fused(const mla_dims* d, int32_t num_splits) {
  if (check_dims(d) != MLA_OK || num_splits < 1 || num_splits > kMaxSplits) return 0;
  return (!force_generic() && mla::absorb_mfma_supported(*d)) ? 1 : 0;
}

}  // extern "C"
