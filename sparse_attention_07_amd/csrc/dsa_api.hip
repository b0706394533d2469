// C ABI of the DSA library: host-side validation, then kernel launches on the
// caller's stream.  Nothing here allocates, synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <set>
#include <utility>

#include "../../include/dsa.h"
#include "dsa_launch.h"

namespace dsa {

hipError_t ensure_max_lds(const void* kernel) {
  static std::mutex mu;
  static std::set<std::pair<int, const void*>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({dev, kernel})) return hipSuccess;
  hipFuncAttributes attr;
  e = hipFuncGetAttributes(&attr, kernel);
  if (e != hipSuccess) return e;
  const int dyn = 160 * 1024 - static_cast<int>(attr.sharedSizeBytes);  // static LDS counts too
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
  if (e == hipSuccess) done.insert({dev, kernel});
  return e;
}

int device_cu_count() {
  static std::mutex mu;
  static std::map<int, int> cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cus.find(dev);
  if (it != cus.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
  cus[dev] = n;
  return n;
}

}  // namespace dsa

namespace {

using dsa::BatchArgs;
using dsa::PoolArgs;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shared batch checks.  Returns DSA_OK and fills `ba`, or an error.  Calls
// that never touch a pool (top-k) pass paged = false: their page table may be
// NULL and the paging fields are not checked.
dsa_status check_batch(const dsa_batch* b, BatchArgs* ba, bool paged = true) {
  if (b == nullptr) return DSA_ERR_NULL;
  if (b->batch < 1 || b->num_q_rows < 0 || b->max_q_len < 0 || b->max_seq_len < 0)
    return DSA_ERR_SHAPE;
  if (paged && (b->page_size < 1 || b->pt_stride < 1 || b->num_pages < 0)) return DSA_ERR_SHAPE;
  if (b->num_q_rows > 0) {
    if (b->cu_q_lens == nullptr || b->seq_lens == nullptr || (paged && b->page_table == nullptr))
      return DSA_ERR_NULL;
    if (b->max_q_len < 1 || (int64_t)b->max_q_len * b->batch < b->num_q_rows) return DSA_ERR_SHAPE;
    if (!aligned(b->cu_q_lens, 4) || !aligned(b->seq_lens, 4) || (paged && !aligned(b->page_table, 4)))
      return DSA_ERR_ALIGN;
  }
  *ba = BatchArgs{b->batch, b->num_q_rows, b->max_q_len, b->max_seq_len, b->cu_q_lens,
                  b->seq_lens, b->page_table, b->pt_stride, b->page_size, b->num_pages};
  return DSA_OK;
}

dsa_status check_pool(const dsa_pool* p, int64_t row_bytes, size_t align, PoolArgs* pa) {
  if (p == nullptr || p->base == nullptr) return DSA_ERR_NULL;
  if (p->row_stride_bytes < row_bytes || p->page_stride_bytes < 0) return DSA_ERR_SHAPE;
  if (!aligned(p->base, align) || (p->row_stride_bytes % (int64_t)align) != 0 ||
      (p->page_stride_bytes % (int64_t)align) != 0)
    return DSA_ERR_ALIGN;
  *pa = PoolArgs{p->base, p->format, p->dim, p->page_stride_bytes, p->row_stride_bytes};
  return DSA_OK;
}

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// A validated indexer launch, shared by dsa_index_scores and dsa_index_topk.
struct IndexArgs {
  const void* q_idx;
  const float* w;
  PoolArgs pa;
  int q_format, n_heads, head_dim;  // q_format DSA_BF16 also stands for DSA_BF16_TO_FP8
  bool q_fp8;                       // DSA_BF16_TO_FP8: queries contracted as fp8 codes
};

dsa_status check_index(const BatchArgs& ba, const void* q_idx, int32_t q_format, const float* w,
                       const dsa_pool* k_idx, int32_t n_heads, int32_t head_dim, IndexArgs* ia) {
  if (q_idx == nullptr || w == nullptr || k_idx == nullptr) return DSA_ERR_NULL;
  if (n_heads < 1 || head_dim < 1) return DSA_ERR_SHAPE;
  // fp8 queries: bf16 in memory, quantised in the kernel; fp8 keys only
  const bool q_fp8 = q_format == DSA_BF16_TO_FP8;
  if (q_fp8 && k_idx->format != DSA_FP8_E4M3_B128) return DSA_ERR_UNSUPPORTED;
  if (q_fp8) q_format = DSA_BF16;
  const bool fp8_keys = q_format == DSA_BF16 && k_idx->format == DSA_FP8_E4M3_B128;
  if ((k_idx->format != q_format && !fp8_keys) || k_idx->dim != head_dim) return DSA_ERR_SHAPE;
  if (!aligned(w, 4)) return DSA_ERR_ALIGN;
  dsa_status st;
  *ia = IndexArgs{q_idx, w, PoolArgs{}, q_format, n_heads, head_dim, q_fp8};
  if (q_format == DSA_BF16) {
    if (n_heads != 64 || head_dim != 128) return DSA_ERR_UNSUPPORTED;
    if (fp8_keys) {
      // page-blocked: page_size rows of 128 codes, then page_size f32 scales
      if ((st = check_pool(k_idx, 128, 16, &ia->pa)) != DSA_OK) return st;
      if (k_idx->page_stride_bytes < (int64_t)ba.page_size * (k_idx->row_stride_bytes + 4))
        return DSA_ERR_SHAPE;
    } else if ((st = check_pool(k_idx, 256, 16, &ia->pa)) != DSA_OK) {
      return st;
    }
    if (!aligned(q_idx, 16) || !aligned(w, 16)) return DSA_ERR_ALIGN;
    if (q_fp8 && !dsa::index_scores_fp8q_fits(ba)) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
  }
  if (q_format == DSA_F32) {
    if (n_heads > 64 || head_dim > 256 || n_heads * head_dim > 8192) return DSA_ERR_UNSUPPORTED;
    if ((st = check_pool(k_idx, (int64_t)head_dim * 4, 4, &ia->pa)) != DSA_OK) return st;
    if (!aligned(q_idx, 4)) return DSA_ERR_ALIGN;
    return DSA_OK;
  }
  return DSA_ERR_UNSUPPORTED;
}

// Scores of the query rows [row_lo, row_hi), row t at scores + (t - row_lo) * ld.
hipError_t launch_index(const BatchArgs& ba, const IndexArgs& ia, float* scores, int64_t ld,
                        hipStream_t s, int row_lo, int row_hi) {
  if (ia.q_format == DSA_BF16) {
    if (ba.num_pages == 0) return hipSuccess;  // no token is mapped: nothing is written
    return dsa::launch_index_scores_bf16(ba, ia.q_idx, ia.w, ia.pa, scores, ld, s, row_lo, row_hi, ia.q_fp8);
  }
  return dsa::launch_index_scores_f32(ba, ia.q_idx, ia.w, ia.pa, ia.n_heads, ia.head_dim, scores, ld,
                                      s, row_lo, row_hi);
}

// Bytes of one workspace score row of dsa_index_topk: max_seq_len rounded up
// to 64 entries (256-byte rows).
int64_t score_row_bytes(int32_t max_seq_len) {
  const int64_t n = max_seq_len < 1 ? 1 : max_seq_len;
  return (n + 63) / 64 * 64 * 4;
}

// dsa_index_topk's workspace for a chunk of `rows` query rows: their score
// rows, then the two-level top-k candidates of those rows (none when the
// rows fit the top-k's LDS cache).
size_t index_topk_bytes(int64_t rows, int32_t max_seq_len, int32_t k) {
  return (size_t)(rows * score_row_bytes(max_seq_len)) + dsa::topk_workspace_bytes((int)rows, max_seq_len, k);
}

// The most query rows per chunk whose workspace fits in `bytes` (at most T).
int64_t index_topk_chunk_rows(int64_t T, int32_t max_seq_len, int32_t k, int64_t bytes) {
  // per-row cost: a score row plus, for two-level rows, k candidates (score
  // and position) per segment; the candidate layout pads once to 256 bytes
  const int64_t cand = dsa::topk_workspace_bytes(1, max_seq_len, k) > 0
                           ? (int64_t)(dsa::topk_workspace_bytes(2, max_seq_len, k) -
                                       dsa::topk_workspace_bytes(1, max_seq_len, k))
                           : 0;
  int64_t rows = std::min<int64_t>(T, bytes / (score_row_bytes(max_seq_len) + cand));
  while (rows > 0 && (int64_t)index_topk_bytes(rows, max_seq_len, k) > bytes) --rows;
  return rows;
}

// Workspace of dsa_sparse_mla_decode_static: a file-scope device array, one
// per GPU (each device holds its own copy at its own address until the
// process ends).  In host code `scratch` names a host-side stand-in, not the
// device array: only the address hipGetSymbolAddress returns for the current
// device is ever passed to a kernel or a copy.
constexpr size_t kScratchBytes = DSA_MLA_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void zero_counters(uint32_t* p, int words) {
  for (int i = (int)threadIdx.x; i < words; i += (int)blockDim.x) p[i] = 0u;
}

// The current device's address of `scratch`, looked up (and its arrival
// counters cleared by a small fill kernel on `stream`) on the first call on
// that device.  Returns nullptr when a HIP call fails.
void* scratch_for_current_device(hipStream_t stream) {
  static std::mutex mu;
  static std::map<int, void*> ptrs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = ptrs.find(dev);
  if (it != ptrs.end()) return it->second;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
  hipLaunchKernelGGL(zero_counters, dim3(1), dim3(256), 0, stream, static_cast<uint32_t*>(ptr),
                     (int)(dsa::kMlaCounterBytes / 4));
  if (hipGetLastError() != hipSuccess) return nullptr;
  ptrs[dev] = ptr;
  return ptr;
}

// ws == kUseScratch: the caller passes no workspace and the call uses the
// current device's `scratch` array (ws_bytes is then kScratchBytes).
void* const kUseScratch = reinterpret_cast<void*>(~uintptr_t(0));

dsa_status sparse_mla(const dsa_batch* batch, const void* q, int32_t q_format, const dsa_pool* kv,
                      const int32_t* idx, int32_t k, int32_t n_heads, int32_t dc, int32_t dr,
                      float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes,
                      hipStream_t stream, bool prefill) {
  BatchArgs ba;
  dsa_status st = check_batch(batch, &ba);
  if (st != DSA_OK) return st;
  if (ba.num_q_rows == 0) return DSA_OK;
  if (q == nullptr || kv == nullptr || idx == nullptr || out == nullptr) return DSA_ERR_NULL;
  if (k < 1 || n_heads < 1 || dc < 1 || dr < 0) return DSA_ERR_SHAPE;
  if (kv->dim != dc + dr) return DSA_ERR_SHAPE;
  // the kernels take the maximum of the unscaled scores and scale it, and
  // work in log2 units (sm_scale * log2 e must stay finite)
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale * 1.4426950408889634f)) return DSA_ERR_UNSUPPORTED;
  if (!aligned(idx, 4) || (lse != nullptr && !aligned(lse, 4))) return DSA_ERR_ALIGN;
  PoolArgs pa;
  if (q_format == DSA_BF16 && (kv->format == DSA_BF16 || kv->format == DSA_FP8_E4M3_B128 ||
                                kv->format == DSA_INT8_AFFINE_B128)) {
    if (dc != 512 || dr != 64 || n_heads % 16 != 0 || n_heads > 128) return DSA_ERR_UNSUPPORTED;
    const int64_t row_bytes = kv->format == DSA_BF16 ? 1152 : (kv->format == DSA_FP8_E4M3_B128 ? 656 : 672);
    if ((st = check_pool(kv, row_bytes, 16, &pa)) != DSA_OK) return st;
    if (!aligned(q, 16) || !aligned(out, 16)) return DSA_ERR_ALIGN;
    const dsa::MlaPlan plan = dsa::plan_sparse_mla(ba.num_q_rows, n_heads, k, dc, prefill,
                                                   kv->format != DSA_BF16);
    if (!dsa::sparse_mla_plan_fits(plan, n_heads)) return DSA_ERR_UNSUPPORTED;
    if (plan.ws_bytes > 0) {
      if (ws == nullptr) return DSA_ERR_WORKSPACE;
      if (ws_bytes < plan.ws_bytes) return DSA_ERR_WORKSPACE;
      if (ws != kUseScratch && !aligned(ws, 16)) return DSA_ERR_ALIGN;
    }
    if (ws == kUseScratch) {  // every check passed: only now touch the device
      ws = plan.ws_bytes > 0 ? scratch_for_current_device(stream) : nullptr;
      if (plan.ws_bytes > 0 && ws == nullptr) return DSA_ERR_HIP;
    }
    return hip_status(dsa::launch_sparse_mla_bf16(ba, q, pa, idx, k, n_heads, sm_scale, out, lse,
                                                  ws, plan, stream));
  }
  if (q_format == DSA_F32 && kv->format == DSA_F32) {
    if (dc + dr > 1024 || k > 4096) return DSA_ERR_UNSUPPORTED;
    if ((st = check_pool(kv, (int64_t)(dc + dr) * 4, 4, &pa)) != DSA_OK) return st;
    if (!aligned(q, 4) || !aligned(out, 4)) return DSA_ERR_ALIGN;
    return hip_status(dsa::launch_sparse_mla_f32(ba, q, pa, idx, k, n_heads, dc, dr, sm_scale, out,
                                                 lse, stream));
  }
  return DSA_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

int32_t dsa_version(void) { return 100; }

const char* dsa_status_string(dsa_status status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "inconsistent sizes";
    case DSA_ERR_UNSUPPORTED: return "format or dimension combination not supported";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP launch failed";
    case DSA_ERR_ALIGN: return "pointer or stride not aligned";
    default: return "unknown status";
  }
}

dsa_status dsa_index_scores(const dsa_batch* batch, const void* q_idx, int32_t q_format,
                            const float* w, const dsa_pool* k_idx, int32_t n_heads,
                            int32_t head_dim, float* scores, int64_t ld, void* stream) {
  BatchArgs ba;
  dsa_status st = check_batch(batch, &ba);
  if (st != DSA_OK) return st;
  if (ba.num_q_rows == 0) return DSA_OK;
  if (scores == nullptr) return DSA_ERR_NULL;
  IndexArgs ia;
  if ((st = check_index(ba, q_idx, q_format, w, k_idx, n_heads, head_dim, &ia)) != DSA_OK) return st;
  if (ld < 1 || ld < ba.max_seq_len) return DSA_ERR_SHAPE;
  if (!aligned(scores, 4)) return DSA_ERR_ALIGN;
  return hip_status(launch_index(ba, ia, scores, ld, static_cast<hipStream_t>(stream), 0, ba.num_q_rows));
}

size_t dsa_index_topk_workspace_bytes(int32_t num_q_rows, int32_t max_seq_len, int32_t k,
                                      int64_t budget_bytes) {
  if (num_q_rows <= 0 || max_seq_len < 0 || k < 1 || budget_bytes <= 0) return 0;
  const int64_t rows = index_topk_chunk_rows(num_q_rows, max_seq_len, k, budget_bytes);
  return rows < 1 ? 0 : index_topk_bytes(rows, max_seq_len, k);
}

dsa_status dsa_index_topk(const dsa_batch* batch, const void* q_idx, int32_t q_format, const float* w,
                          const dsa_pool* k_idx, int32_t n_heads, int32_t head_dim, int32_t k,
                          int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  BatchArgs ba;
  dsa_status st = check_batch(batch, &ba);
  if (st != DSA_OK) return st;
  if (ba.num_q_rows == 0) return DSA_OK;
  if (idx == nullptr) return DSA_ERR_NULL;
  IndexArgs ia;
  if ((st = check_index(ba, q_idx, q_format, w, k_idx, n_heads, head_dim, &ia)) != DSA_OK) return st;
  if (k < 1) return DSA_ERR_SHAPE;
  const int64_t row = score_row_bytes(ba.max_seq_len);
  const int64_t per =
      ws == nullptr ? 0 : index_topk_chunk_rows(ba.num_q_rows, ba.max_seq_len, k, (int64_t)ws_bytes);
  if (per < 1) return DSA_ERR_WORKSPACE;  // below the minimum: one row's scores (and candidates)
  if (!aligned(ws, 16) || !aligned(idx, 4)) return DSA_ERR_ALIGN;
  float* scores = static_cast<float*>(ws);
  // the chunk's two-level candidates follow its score rows (256-byte aligned)
  uint8_t* cand = static_cast<uint8_t*>(ws) + per * row;
  const size_t cand_bytes = dsa::topk_workspace_bytes((int)per, ba.max_seq_len, k);
  const int64_t ld = row / 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Chunks of `per` query rows: each chunk's scores, then at once its top-k.
  for (int r0 = 0; r0 < ba.num_q_rows; r0 += (int)per) {
    const int r1 = (int)std::min<int64_t>(ba.num_q_rows, r0 + per);
    if ((st = hip_status(launch_index(ba, ia, scores, ld, s, r0, r1))) != DSA_OK) return st;
    if ((st = hip_status(dsa::launch_topk(ba, scores, ld, k, idx, s, r0, r1, cand, cand_bytes))) != DSA_OK)
      return st;
  }
  return DSA_OK;
}

dsa_status dsa_indexer_prepare(const dsa_batch* batch, const void* q_in, void* q_out,
                               const void* k_in, int32_t format, const float* ln_weight,
                               const float* ln_bias, float ln_eps, const float* rope_cos,
                               const float* rope_sin, int32_t rope_rows, int32_t rope_dim,
                               int32_t rope_interleaved, const dsa_pool* k_idx, int32_t n_heads,
                               int32_t head_dim, void* stream) {
  BatchArgs ba;
  dsa_status st = check_batch(batch, &ba);
  if (st != DSA_OK) return st;
  if (ba.num_q_rows == 0) return DSA_OK;
  if (q_in == nullptr || q_out == nullptr || k_in == nullptr || ln_weight == nullptr ||
      ln_bias == nullptr || k_idx == nullptr)
    return DSA_ERR_NULL;
  if (rope_dim > 0 && (rope_cos == nullptr || rope_sin == nullptr)) return DSA_ERR_NULL;
  if (format != DSA_BF16 && format != DSA_F32) return DSA_ERR_UNSUPPORTED;
  const bool fp8_keys = k_idx->format == DSA_FP8_E4M3_B128;
  if (fp8_keys && (format != DSA_BF16 || head_dim != 128)) return DSA_ERR_UNSUPPORTED;
  if ((k_idx->format != format && !fp8_keys) || k_idx->dim != head_dim) return DSA_ERR_SHAPE;
  if (n_heads < 1 || head_dim < 1 || rope_dim < 0 || rope_dim > head_dim || !(ln_eps >= 0.f))
    return DSA_ERR_SHAPE;
  if (n_heads > 1024 || head_dim > 128 || head_dim % 16 != 0 || rope_dim % 16 != 0)
    return DSA_ERR_UNSUPPORTED;
  if (rope_dim > 0 && rope_rows < ba.max_seq_len) return DSA_ERR_SHAPE;
  if (rope_dim == 0) rope_rows = INT32_MAX;  // no table is read
  const int es = format == DSA_BF16 ? 2 : 4;
  PoolArgs pa;
  if (fp8_keys) {
    // page-blocked: page_size rows of 128 codes, then page_size f32 scales
    if ((st = check_pool(k_idx, 128, 16, &pa)) != DSA_OK) return st;
    if (k_idx->page_stride_bytes < (int64_t)ba.page_size * (k_idx->row_stride_bytes + 4))
      return DSA_ERR_SHAPE;
  } else if ((st = check_pool(k_idx, (int64_t)head_dim * es, 16, &pa)) != DSA_OK) {
    return st;
  }
  if (!aligned(q_in, 16) || !aligned(q_out, 16) || !aligned(k_in, 16) || !aligned(ln_weight, 4) ||
      !aligned(ln_bias, 4) || (rope_dim > 0 && (!aligned(rope_cos, 16) || !aligned(rope_sin, 16))))
    return DSA_ERR_ALIGN;
  return hip_status(dsa::launch_indexer_prepare(ba, q_in, q_out, k_in, format, ln_weight, ln_bias,
                                                ln_eps, rope_cos, rope_sin, rope_rows, rope_dim,
                                                rope_interleaved != 0, pa, n_heads, head_dim,
                                                static_cast<hipStream_t>(stream)));
}

size_t dsa_topk_workspace_bytes(int32_t num_q_rows, int32_t max_seq_len, int32_t k) {
  return dsa::topk_workspace_bytes(num_q_rows, max_seq_len, k);
}

dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  BatchArgs ba;
  dsa_status st = check_batch(batch, &ba, /*paged=*/false);
  if (st != DSA_OK) return st;
  if (ba.num_q_rows == 0) return DSA_OK;
  if (scores == nullptr || idx == nullptr) return DSA_ERR_NULL;
  if (k < 1 || ld < 1 || ld < ba.max_seq_len) return DSA_ERR_SHAPE;
  if (!aligned(scores, 4) || !aligned(idx, 4)) return DSA_ERR_ALIGN;
  const size_t need = dsa::topk_workspace_bytes(ba.num_q_rows, ba.max_seq_len, k);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need) return DSA_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return DSA_ERR_ALIGN;
  }
  return hip_status(dsa::launch_topk(ba, scores, ld, k, idx, static_cast<hipStream_t>(stream), 0,
                                     ba.num_q_rows, ws, ws_bytes));
}

size_t dsa_sparse_mla_workspace_bytes(int32_t num_q_rows, int32_t n_heads, int32_t k, int32_t dc,
                                      int32_t prefill) {
  // enough for every latent format (their split plans may differ)
  return std::max(dsa::plan_sparse_mla(num_q_rows, n_heads, k, dc, prefill != 0, false).ws_bytes,
                  dsa::plan_sparse_mla(num_q_rows, n_heads, k, dc, prefill != 0, true).ws_bytes);
}

dsa_status dsa_sparse_mla_decode(const dsa_batch* batch, const void* q, int32_t q_format,
                                 const dsa_pool* kv, const int32_t* idx, int32_t k,
                                 int32_t n_heads, int32_t dc, int32_t dr, float sm_scale,
                                 void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return sparse_mla(batch, q, q_format, kv, idx, k, n_heads, dc, dr, sm_scale, out, lse, ws,
                    ws_bytes, static_cast<hipStream_t>(stream), false);
}

dsa_status dsa_sparse_mla_decode_static(const dsa_batch* batch, const void* q, int32_t q_format,
                                        const dsa_pool* kv, const int32_t* idx, int32_t k,
                                        int32_t n_heads, int32_t dc, int32_t dr, float sm_scale,
                                        void* out, float* lse, void* stream) {
  return sparse_mla(batch, q, q_format, kv, idx, k, n_heads, dc, dr, sm_scale, out, lse, kUseScratch,
                    kScratchBytes, static_cast<hipStream_t>(stream), false);
}

dsa_status dsa_sparse_mla_prefill(const dsa_batch* batch, const void* q, int32_t q_format,
                                  const dsa_pool* kv, const int32_t* idx, int32_t k,
                                  int32_t n_heads, int32_t dc, int32_t dr, float sm_scale,
                                  void* out, float* lse, void* ws, size_t ws_bytes,
                                  void* stream) {
  return sparse_mla(batch, q, q_format, kv, idx, k, n_heads, dc, dr, sm_scale, out, lse, ws,
                    ws_bytes, static_cast<hipStream_t>(stream), true);
}

}  // extern "C"
