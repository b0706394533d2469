/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek-Sparse-Attention hot path.
 *
 * Three steps run per full layer, in this order, all on one HIP stream
 * (optionally preceded by dsa_indexer_prepare, which rotates the indexer
 * queries and stores this step's normalised, rotated index keys):
 *
 *   dsa_index_scores   lightning-indexer score of every earlier cached token
 *   dsa_topk           per query row, the index_topk best tokens
 *   dsa_sparse_mla_*   absorbed MLA over only the selected latent rows
 *
 * IndexShare "shared" layers skip the first two calls and pass the full
 * layer's index buffer to dsa_sparse_mla_* again (mlx-lm PR 1419 "GLM-5.2
 * (glm_moe_dsa) inference: IndexShare, indexer RoPE/eps, int8 MLA-KV",
 * description: only full layers run the indexer, shared layers reuse the
 * previous full layer's top-k).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named in dsa_batch / dsa_pool and every array argument are
 *   DEVICE pointers, except the two structs themselves, which live on the
 *   host and are read during the call only.  The caller owns all memory;
 *   the library allocates nothing and keeps no state between calls other
 *   than what a workspace holds.
 * - Every call only validates its host-side arguments and enqueues kernels
 *   on `stream` (a hipStream_t; NULL = the legacy default stream).  It never
 *   synchronises and never reads device memory on the host, so a sequence
 *   of calls can be captured into a HIP graph.  Grid sizes come from the
 *   host bounds max_q_len / max_seq_len, never from device data.
 * - A query row t of request b (cu_q_lens[b] <= t < cu_q_lens[b+1]) is the
 *   j-th new token of that request and sits at position
 *       pos(t) = seq_lens[b] - q_len[b] + j,   q_len[b] = cu_q_lens[b+1]-cu_q_lens[b].
 *   It sees cached tokens 0..pos(t): multi-token (MTP draft) rows are causal
 *   inside the draft (lmdeploy PR 4737 "feat: support GLM-5.2", section
 *   "Changes": multi-token query handling; mlx-lm PR 1419, the commit that
 *   re-masks gathered keys when a position has fewer valid keys than K).
 * - Token s of request b is stored in page page_table[b*pt_stride + s/page_size]
 *   at slot s % page_size.  Both pools (indexer keys and MLA latent) use the
 *   same page table.  Pages are read in place, never copied (lmdeploy PR 4737,
 *   section "Five-layer ablations": a zero-copy strided view replaced the
 *   materialised paged cache).
 * - Selected indices are LOGICAL token positions, ascending, padded with -1
 *   (lmdeploy PR 4968 "add glm5.3-flash support", commit notes: sparse
 *   FlashMLA indices are padded with invalid entries, negative means
 *   invalid).  The page-table remap happens inside the attention kernel.
 * - cu_q_lens must be consistent with batch and num_q_rows (cu_q_lens[B] = T).
 *   Other device data that contradicts the host bounds (seq_lens[b] >
 *   max_seq_len, a page id outside [0, num_pages), an index beyond pos) never
 *   causes an out-of-bounds access: such tokens are skipped.  Each pool must
 *   span num_pages * page_stride_bytes bytes.
 * - Device pointers must be 16-byte aligned (DSA_ERR_ALIGN otherwise).
 * - num_q_rows == 0 returns DSA_OK without launching anything.
 * - After each launch hipGetLastError() is checked (DSA_ERR_HIP).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dsa_status;
#define DSA_OK 0
#define DSA_ERR_NULL 1        /* a required pointer is NULL */
#define DSA_ERR_SHAPE 2       /* sizes inconsistent (e.g. ld < max_seq_len, k <= 0) */
#define DSA_ERR_UNSUPPORTED 3 /* format / dimension combination not built */
#define DSA_ERR_WORKSPACE 4   /* workspace NULL or smaller than the query says */
#define DSA_ERR_HIP 5         /* a HIP launch failed */
#define DSA_ERR_ALIGN 6       /* a device pointer or stride is not 16-byte aligned */

/* Element formats. */
#define DSA_F32 0
#define DSA_BF16 1
/* OCP e4m3fn values with an f32 scale per 128 elements; value = e4m3(byte) *
 * scale.  For the MLA latent pool (dc = 512, dr = 64): 656-byte rows of 512
 * e4m3 bytes (latent dims 0..511), four little-endian f32 scales (scale i
 * multiplies dims 128*i..128*i+127), then the 64 rope dims as bf16 (the
 * BF16/FP8 sparse cache paths of lmdeploy PR 4737, section "Changes"; the
 * block layout is this library's).  For an indexer key pool (dim 128): 128
 * codes per token and one scale per token, page-blocked (see
 * dsa_index_scores). */
#define DSA_FP8_E4M3_B128 2
/* Affine 8-bit latent rows (the int8 MLA latent cache of mlx-lm PR 1419's
 * description: only the latent is quantised, and it is dequantised on read;
 * the block layout is this library's): 672-byte rows of 512 unsigned codes,
 * four little-endian f32 scales, four f32 biases (pair i covers latent dims
 * 128*i..128*i+127), then the 64 rope dims as bf16;
 * latent dim d = scale[d/128] * code[d] + bias[d/128].  Latent pools only. */
#define DSA_INT8_AFFINE_B128 3
/* Indexer queries only (q_format of dsa_index_scores / dsa_index_topk, with
 * DSA_FP8_E4M3_B128 keys): bf16 queries in memory, contracted as fp8.  Each
 * (row, head) of 128 dims is scaled by 2^-e, e the smallest integer with the
 * head's largest magnitude <= 448 * 2^e (e = 0 for an all-zero head), and
 * rounded to e4m3fn codes (nearest, ties to even); the scores are the plain
 * formula over code * 2^e, on the fp8 matrix cores of gfx950 (the
 * "MFMA bf16/fp8 tiles" of the indexer's q.k; a reading of this library: the
 * pages quantise the keys, not how fp8 queries are scaled). */
#define DSA_BF16_TO_FP8 4

/* A ragged batch of B requests and T = cu_q_lens[B] query rows. */
typedef struct {
  int32_t batch;          /* B >= 1 */
  int32_t num_q_rows;     /* T >= 0; must equal cu_q_lens[B] */
  int32_t max_q_len;      /* >= every q_len[b] (host bound, sizes grids) */
  int32_t max_seq_len;    /* >= every seq_lens[b] (host bound, sizes grids) */
  const int32_t *cu_q_lens;  /* device [B+1], cu_q_lens[0] = 0, non-decreasing */
  const int32_t *seq_lens;   /* device [B], cache length including this step's rows */
  const int32_t *page_table; /* device [B, pt_stride]; -1 marks an unused entry */
  int32_t pt_stride;      /* entries per request in page_table */
  int32_t page_size;      /* tokens per page, >= 1 */
  int32_t num_pages;      /* pages in each pool */
} dsa_batch;

/* One paged pool viewed in place: token slot (page, i) starts at
 *   base + page*page_stride_bytes + i*row_stride_bytes. */
typedef struct {
  const void *base;          /* device */
  int32_t format;            /* DSA_F32 | DSA_BF16 | DSA_FP8_E4M3_B128 */
  int32_t dim;               /* elements per row: D_I for index keys, dc+dr for latent */
  int64_t page_stride_bytes;
  int64_t row_stride_bytes;
} dsa_pool;

/* Library version (major*10000 + minor*100 + patch). */
int32_t dsa_version(void);

/* Static description of a status code. */
const char *dsa_status_string(dsa_status status);

/*
 * Lightning-indexer scores (the DSA indexer of lmdeploy PR 4737, section
 * "Changes", and mlx-lm PR 1419's description; the pages give no formula,
 * this library computes the plain one):
 *
 *   scores[t*ld + s] = sum_h w[t,h] * max(0, dot(q_idx[t,h,:], k(s)))   for 0 <= s <= pos(t)
 *
 * q_idx    device [T, n_heads, head_dim], format q_format, contiguous
 * w        device [T, n_heads] f32 (any extra scale is folded in by the caller)
 * k_idx    indexer key pool, dim == head_dim, format == q_format -- or, with
 *          bf16 queries, DSA_FP8_E4M3_B128 keys: each page holds page_size
 *          rows of 128 e4m3fn codes (row_stride_bytes apart, a multiple of
 *          16, >= 128), followed at byte page_size*row_stride_bytes of the
 *          page by page_size little-endian f32 scales, one per token;
 *          k(s) = code * scale.  Scales must be non-negative (a quantiser's
 *          amax/448 is); page_stride_bytes >= page_size*(row_stride_bytes+4).
 *          (The FP8 index keys of the pages' "next" items: half the key bytes.)
 * scores   device [T, ld] f32, ld >= max_seq_len.  Entries s > pos(t), and
 *          entries of tokens whose page is not mapped, are NOT written.
 * Built combinations: (DSA_BF16, n_heads 64, head_dim 128) on MFMA, with bf16
 * or fp8 keys; (DSA_BF16_TO_FP8, n_heads 64, head_dim 128, fp8 keys) on fp8
 * MFMA -- DSA_ERR_UNSUPPORTED with other keys, and for batches whose tables
 * (about 24 bytes per request) leave no room for one unit of staged query
 * rows in LDS; (DSA_F32, n_heads <= 64, head_dim <= 256) on the vector ALUs.
 */
dsa_status dsa_index_scores(const dsa_batch *batch, const void *q_idx, int32_t q_format,
                            const float *w, const dsa_pool *k_idx, int32_t n_heads,
                            int32_t head_dim, float *scores, int64_t ld, void *stream);

/*
 * Indexer query/key preparation for this step's new rows, in one launch (the
 * fused indexer preparation of lmdeploy PR 4737, section "Changes", and its
 * section "DSA indexer fusion"; mlx-lm PR 1419's description: GLM-5.2's
 * indexer uses non-interleaved RoPE and LayerNorm eps 1e-6, DeepSeek-V3.2
 * interleaved RoPE and eps 1e-5).  For each query row t at position p = pos(t):
 *
 *   q_out[t,h,:] = rope(q_in[t,h,:], p)                      h < n_heads
 *   key(p)       = rope(layernorm(k_in[t,:]), p)   stored into k_idx at token p
 *
 *   layernorm(x) = (x - mean(x)) / sqrt(var(x) + ln_eps) * ln_weight + ln_bias
 *                  (var: mean squared deviation)
 *   rope(x, p)   turns the first rope_dim dims in rope_dim/2 pairs -- pair i is
 *                dims (i, i + rope_dim/2), or (2i, 2i+1) when rope_interleaved --
 *                by the angle with cosine rope_cos[p*rope_dim/2 + i] and sine
 *                rope_sin[p*rope_dim/2 + i]: (a, b) -> (a cos - b sin, a sin + b cos);
 *                the other dims pass through.
 *
 * q_in, q_out  device [T, n_heads, head_dim], `format` (DSA_BF16 or DSA_F32);
 *              q_out may equal q_in (in place) but may not overlap it otherwise
 * k_in         device [T, head_dim], `format`
 * ln_weight, ln_bias  device [head_dim] f32
 * rope_cos, rope_sin  device [rope_rows, rope_dim/2] f32 (caller-built tables,
 *              any frequency scaling included); rope_rows >= max_seq_len.  May
 *              be NULL when rope_dim == 0.
 * k_idx        the index-key pool (format == `format`, dim == head_dim), or,
 *              with bf16 inputs and head_dim 128, a DSA_FP8_E4M3_B128 key pool
 *              laid out as dsa_index_scores describes: the key is stored as
 *              e4m3fn codes of key / scale (rounded to nearest even) with
 *              scale = max|key| / 448 (1 for a zero key) in its scale slot.  Its
 *              base IS WRITTEN: the key of row t goes to token pos(t) of its
 *              request (nothing is written when that page is not mapped).
 * Work is done in f32; bf16 results are rounded to nearest even.  A row whose
 * position is outside [0, rope_rows) is left untouched.  Run it before
 * dsa_index_scores of the same step (which reads the keys it stores).
 * Built: head_dim a multiple of 16 up to 128, rope_dim a multiple of 16 up to
 * head_dim, n_heads <= 1024; fp8 key pools with bf16 inputs and head_dim 128.
 */
dsa_status dsa_indexer_prepare(const dsa_batch *batch, const void *q_in, void *q_out,
                               const void *k_in, int32_t format, const float *ln_weight,
                               const float *ln_bias, float ln_eps, const float *rope_cos,
                               const float *rope_sin, int32_t rope_rows, int32_t rope_dim,
                               int32_t rope_interleaved, const dsa_pool *k_idx, int32_t n_heads,
                               int32_t head_dim, void *stream);

/*
 * Scores and top-k in one call with a bounded score workspace (the bounded
 * "KPool" scoring of lmdeploy PR 4968, section "Capacity improvement":
 * a reserved score budget, deterministic top-k taken per query chunk at
 * once, the same selected indices as the unbounded path).  The query rows
 * are walked in chunks of as many rows as the workspace holds; each chunk's
 * scores (dsa_index_scores' formula) go to the workspace and its top-k
 * (dsa_topk's rule) is taken before the next chunk overwrites them.  idx is
 * bit-identical to dsa_index_scores followed by dsa_topk, whatever the
 * chunking, so a [T, max_seq_len] score buffer is never needed.
 *
 * q_idx, q_format, w, k_idx, n_heads, head_dim: as dsa_index_scores
 *          (every token below seq_len should be mapped: the score entry of an
 *          unmapped token is not written, so its place in the ranking is
 *          unspecified, though every access stays in bounds)
 * k, idx   as dsa_topk
 * ws       device workspace of ws_bytes; it must hold at least
 *          dsa_index_topk_workspace_bytes(1, max_seq_len, k, ...) bytes (one
 *          row), else DSA_ERR_WORKSPACE; the chunk length is the number of rows
 *          whose workspace fits in ws_bytes.  Its contents need no
 *          initialisation.
 */
dsa_status dsa_index_topk(const dsa_batch *batch, const void *q_idx, int32_t q_format, const float *w,
                          const dsa_pool *k_idx, int32_t n_heads, int32_t head_dim, int32_t k,
                          int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes dsa_index_topk uses within a budget, for chunks of as many
 * query rows (at most num_q_rows) as fit in budget_bytes.  Each row of a
 * chunk takes one score row of round_up(max_seq_len, 64) f32; when
 * max_seq_len exceeds both 32768 and k, it also takes the two-level top-k
 * candidates dsa_topk_workspace_bytes counts for one row (an f32 score and an
 * int32 position for each of k slots of each 32768-entry segment), so long
 * rows are selected in two levels here as in dsa_topk.  Returns 0 when the
 * budget is below the minimum of one row (or when num_q_rows <= 0 or
 * k < 1): such a budget cannot run the call. */
size_t dsa_index_topk_workspace_bytes(int32_t num_q_rows, int32_t max_seq_len, int32_t k,
                                      int64_t budget_bytes);

/* Workspace bytes dsa_topk needs for these sizes: 0 when max_seq_len <= 32768
 * or max_seq_len <= k; otherwise room for the candidates of a two-level
 * selection (an f32 score and an int32 position for each of k slots of each
 * 32768-entry segment of each row). */
size_t dsa_topk_workspace_bytes(int32_t num_q_rows, int32_t max_seq_len, int32_t k);

/*
 * Per-row top-k (radix top-k of lmdeploy PR 4737, section "Changes"):
 * among s = 0..pos(t), keep the k largest scores; equal scores go to the
 * lower s, and -0.0 equals +0.0.  When pos(t)+1 <= k every valid token is
 * kept (mstar PR 387 "GLM-5.2 with MLA, fp8 MoE and DSA", section "Body":
 * below index_topk the sparse pick is all tokens).  Output idx[t*k + j]:
 * selected positions in ascending order, then -1.  Only entries
 * s <= min(pos(t), ld-1) of each score row are used; when ld <= 32768 a
 * row's whole storage (ld entries) may be read, before pos(t) is known.
 * The used scores must be finite; the others may hold anything.
 * scores   device [T, ld] f32 (all T*ld entries allocated);  idx  device [T, k] int32
 * batch    only batch, num_q_rows, max_q_len, max_seq_len, cu_q_lens and
 *          seq_lens are used: page_table may be NULL and the paging fields
 *          are not checked.
 * ws       device workspace of dsa_topk_workspace_bytes() bytes (may be NULL when
 *          0; DSA_ERR_WORKSPACE when smaller).  Rows longer than 32768 entries
 *          are then selected in two levels: the exact top-k of each 32768-entry
 *          segment, then the top-k of those candidates.  Both levels use the
 *          order above, so the result is the same set in the same order.
 */
dsa_status dsa_topk(const dsa_batch *batch, const float *scores, int64_t ld, int32_t k,
                    int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes dsa_sparse_mla_decode (prefill != 0: _prefill) needs, for
 * any latent cache format (the split plan may differ between bf16 and 8-bit
 * rows; the size returned covers both). */
size_t dsa_sparse_mla_workspace_bytes(int32_t num_q_rows, int32_t n_heads, int32_t k,
                                      int32_t dc, int32_t prefill);

/*
 * Sparse weight-absorbed MLA over the selected latent rows (FlashMLA sparse
 * decode of lmdeploy PR 4737 section "Changes"; the single- and small-L
 * gather path of mlx-lm PR 1419; mstar PR 387 section "Shared code",
 * MLA with weight absorption).  For each row t and head h:
 *
 *   l_j = sm_scale * dot(q[t,h,0:dc+dr], row(idx[t,j])[0:dc+dr])   for usable j
 *   out[t,h,:] = sum_j softmax(l)_j * row(idx[t,j])[0:dc]
 *   lse[t,h]   = log(sum_j exp(l_j))          (natural log; NULL to skip)
 *
 * A j is usable when 0 <= idx[t,j] <= pos(t) and its page is mapped; others
 * are skipped.  A row with no usable j gives out = 0 and lse = -inf.
 * sm_scale must be positive, with sm_scale * log2(e) finite (the kernels take
 *          the maximum of the unscaled dot products and scale it, in log2
 *          units); DSA_ERR_UNSUPPORTED otherwise.
 * q        device [T, n_heads, dc+dr], format q_format, contiguous
 * kv       latent pool, dim == dc+dr
 * idx      device [T, k] int32 (the dsa_topk output, or a shared layer's copy)
 * out      device [T, n_heads, dc], format q_format
 * ws       device workspace of dsa_sparse_mla_workspace_bytes() bytes (it may
 *          be NULL when that is 0).  Its first 4096 bytes hold arrival
 *          counters, at that place for every shape, format and entry point;
 *          split partials follow them.  The caller zero-fills the workspace
 *          once before its first use; every call returns the counters to zero
 *          and never writes anything else into those 4096 bytes, so one
 *          workspace, sized for the largest call, serves calls of any shape in
 *          any order.  Calls that may run at the same time (other streams)
 *          need workspaces of their own.
 * Built combinations: q DSA_BF16 with kv DSA_BF16, DSA_FP8_E4M3_B128 or DSA_INT8_AFFINE_B128,
 * dc 512, dr 64, n_heads a multiple of 16 up to 128 (MFMA); q and kv DSA_F32
 * with dc+dr <= 1024, n_heads <= 128, k <= 4096 (vector ALUs).  The MFMA
 * kernels stage the byte offsets of all rows one workgroup attends in LDS:
 * with n_heads a multiple of 64, a workgroup that attends more than 5184 rows
 * (any prefill call with k > 5184; a decode call whose rows are not split,
 * which happens when num_q_rows * n_heads / 64 >= 384) does not fit, and the
 * call returns DSA_ERR_UNSUPPORTED before launching anything.
 * _decode and _prefill compute the same function; they differ only in how
 * the work is split across workgroups (decode splits the selected rows of
 * each query to fill the GPU, prefill does not).
 */
dsa_status dsa_sparse_mla_decode(const dsa_batch *batch, const void *q, int32_t q_format,
                                 const dsa_pool *kv, const int32_t *idx, int32_t k,
                                 int32_t n_heads, int32_t dc, int32_t dr, float sm_scale,
                                 void *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * dsa_sparse_mla_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same function, kernels and results, with the workspace
 * taken from a device array the library owns, DSA_MLA_SCRATCH_BYTES per GPU,
 * held by each GPU the library runs on until the process ends.  The call
 * allocates nothing.  The caller passes inputs and outputs as for
 * dsa_sparse_mla_decode, no workspace.
 * - A call whose split plan needs more workspace than DSA_MLA_SCRATCH_BYTES
 *   (what dsa_sparse_mla_workspace_bytes(num_q_rows, n_heads, k, dc, 0)
 *   returns) gets DSA_ERR_WORKSPACE before anything is launched.
 * - The first call on a device looks the array up on that device and clears
 *   its arrival counters with one small kernel on `stream`; every call leaves
 *   them at zero again.
 * - All calls on one GPU share its array, which keeps the last call's
 *   partials: calls that may overlap on one GPU (other streams, other host
 *   threads) race on it and must be serialised by the caller.
 */
#define DSA_MLA_SCRATCH_BYTES (64u << 20)
dsa_status dsa_sparse_mla_decode_static(const dsa_batch *batch, const void *q, int32_t q_format,
                                        const dsa_pool *kv, const int32_t *idx, int32_t k,
                                        int32_t n_heads, int32_t dc, int32_t dr, float sm_scale,
                                        void *out, float *lse, void *stream);

dsa_status dsa_sparse_mla_prefill(const dsa_batch *batch, const void *q, int32_t q_format,
                                  const dsa_pool *kv, const int32_t *idx, int32_t k,
                                  int32_t n_heads, int32_t dc, int32_t dr, float sm_scale,
                                  void *out, float *lse, void *ws, size_t ws_bytes,
                                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
