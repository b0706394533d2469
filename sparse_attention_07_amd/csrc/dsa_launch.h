// Host-side launch interface between the C ABI (dsa_api.hip) and the kernels.
// Every launcher trusts that dsa_api.hip validated its arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct BatchArgs {
  int batch, num_q_rows, max_q_len, max_seq_len;
  const int32_t* cu_q;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int pt_stride, page_size, num_pages;
};

struct PoolArgs {
  const void* base;
  int format, dim;
  int64_t page_stride, row_stride;
};

// Lets `kernel` use up to the 160 KB of LDS of a gfx950 CU.  The attribute is
// set once per kernel and device; later calls only look it up.
hipError_t ensure_max_lds(const void* kernel);
// Compute units of the current device (cached per device).
int device_cu_count();

// Scores and top-k of the query rows [row_lo, row_hi) only; score row t is
// stored at scores + (t - row_lo) * ld (index rows keep their absolute t).
hipError_t launch_index_scores_bf16(const BatchArgs& ba, const void* q_idx, const float* w,
                                    const PoolArgs& pool, float* scores, int64_t ld,
                                    hipStream_t stream, int row_lo, int row_hi, bool q_fp8);
// Whether a batch's fp8-query launch fits the persistent form's LDS plan.
bool index_scores_fp8q_fits(const BatchArgs& ba);
hipError_t launch_index_scores_f32(const BatchArgs& ba, const void* q_idx, const float* w,
                                   const PoolArgs& pool, int n_heads, int head_dim, float* scores,
                                   int64_t ld, hipStream_t stream, int row_lo, int row_hi);

hipError_t launch_indexer_prepare(const BatchArgs& ba, const void* q_in, void* q_out, const void* k_in,
                                  int format, const float* gamma, const float* beta, float eps,
                                  const float* cos_tab, const float* sin_tab, int rope_rows,
                                  int rope_dim, int interleaved, const PoolArgs& pool, int n_heads,
                                  int head_dim, hipStream_t stream);

// With a workspace of topk_workspace_bytes(rows, max_seq_len, k) bytes, rows
// longer than the LDS cache are selected in two levels; without one (or when
// it is 0), one workgroup per row re-reads long rows in each pass.
size_t topk_workspace_bytes(int num_q_rows, int max_seq_len, int k);
hipError_t launch_topk(const BatchArgs& ba, const float* scores, int64_t ld, int k, int32_t* idx,
                       hipStream_t stream, int row_lo, int row_hi, void* ws = nullptr,
                       size_t ws_bytes = 0);

// Split plan of the MFMA sparse-MLA kernel (rows of each query cut into `splits`
// ranges of `rows_per_split`); workspace holds the partial results.
// The workspace starts with kMlaCounterBytes of arrival counters, one per
// (row, head group) of a split launch, always at the same place whatever the
// shape of the call; the split partials follow.  A launch splits only when it
// has fewer (row, head group) blocks than its workgroup target, so
// kMlaCounterSlots counters always suffice.
constexpr int kMlaCounterSlots = 512;
constexpr size_t kMlaCounterBytes = 4096;
struct MlaPlan {
  int splits;
  int rows_per_split;
  size_t ws_bytes;  // counters, then split partials (0 when splits == 1)
};
// q8: the latent rows are 8-bit (fp8 or int8), which changes the 16-head split.
MlaPlan plan_sparse_mla(int num_q_rows, int n_heads, int k, int dc, bool prefill, bool q8);
// Whether the MFMA kernel can stage a plan's rows per split in LDS (checked
// before launching; a plan that does not fit is refused as unsupported).
bool sparse_mla_plan_fits(const MlaPlan& plan, int n_heads);

hipError_t launch_sparse_mla_bf16(const BatchArgs& ba, const void* q, const PoolArgs& kv,
                                  const int32_t* idx, int k, int n_heads, float sm_scale,
                                  void* out, float* lse, void* ws, const MlaPlan& plan,
                                  hipStream_t stream);
hipError_t launch_sparse_mla_f32(const BatchArgs& ba, const void* q, const PoolArgs& kv,
                                 const int32_t* idx, int k, int n_heads, int dc, int dr,
                                 float sm_scale, void* out, float* lse, hipStream_t stream);

}  // namespace dsa
