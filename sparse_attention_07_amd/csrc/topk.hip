// Per-row top-k of the indexer scores by radix select on gfx950 (the radix
// top-k of lmdeploy PR 4737 "feat: support GLM-5.2", section "Changes").
//
// Output: the selected positions in ascending order, then -1.  When
// pos(t)+1 <= k the row keeps every valid position (mstar PR 387, section
// "Body": below index_topk the pick is all tokens).  A workgroup of 1024
// threads selects one query row at a time: one row per workgroup when the
// rows fit the CUs (topk_radix), else a workgroup per CU walking its rows
// with the next row read ahead (topk_rows).  The selection itself (order,
// ties, passes, compaction) is in topk_select.h.  Rows of up to 32768 entries
// are cached in LDS after one read and then selected from registers; longer
// rows are re-read in each pass, or, when the caller gives a workspace,
// selected in two levels (topk_segments, then topk_merge).
#include "dsa_device.h"
#include "dsa_launch.h"
#include "topk_select.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kCache = 32768;

// Top-K of row[0, n): emit(o, s) for the o-th selected position s, o < K, in
// ascending s.  Cached: n <= kCache.  VEC: the row may be read as 16-byte
// quads (topk::quads_ok).  NPRE > 0 (cached, VEC rows only): pre holds the
// first NPRE quads per thread of the row's read.
template <bool Cached, int NPRE, bool VEC, typename Emit>
__device__ __attribute__((always_inline)) inline void select_emit(const float* __restrict__ row, int n, int K,
                                                                  uint32_t* cache, uint32_t* hist, uint32_t* wcount,
                                                                  uint32_t* pick, Emit emit,
                                                                  const f32x4* pre = nullptr) {
  const topk::RowReader<VEC> rd(row, n);
  if (Cached) {
    topk::select_cached<kThreads, NPRE, VEC>(rd, n, K, cache, hist, pick, wcount, emit, pre);
  } else {
    const topk::Threshold th = topk::select<kThreads, VEC>(rd, n, K, hist, pick);
    topk::compact<kThreads, false>(row, VEC, n, cache, th, wcount, [emit, K](uint32_t o, int s) {
      if (o < (uint32_t)K) emit(o, s);
    });
  }
}

// select_emit for a row of n <= kCache entries with `bound` entries of
// storage from row.
template <typename Emit>
__device__ __attribute__((always_inline)) inline void select_cached_row(const float* __restrict__ row, int n,
                                                                        int64_t bound, int K, uint32_t* cache,
                                                                        uint32_t* hist, uint32_t* wcount,
                                                                        uint32_t* pick, Emit emit) {
  if (topk::quads_ok(row, n, bound)) select_emit<true, 0, true>(row, n, K, cache, hist, wcount, pick, emit);
  else select_emit<true, 0, false>(row, n, K, cache, hist, wcount, pick, emit);
}

// The thread's index as a value the compiler cannot see through: in a loop
// over rows, everything derived from it is then computed inside the loop
// instead of being hoisted and held (or spilled) across it.
__device__ __attribute__((always_inline)) inline int opaque_tid() {
  int x = (int)threadIdx.x;
  asm volatile("" : "+v"(x));
  return x;
}

// The request lookup's first R rounds (requests 0 .. R * 64 - 1, as in
// locate_row): their loads are the same for every row, so a workgroup that
// handles several rows issues them once.  Later rounds are left to
// locate_row.
template <int R>
struct RequestTable {
  int lo[R], hi[R], sl[R];
  __device__ __attribute__((always_inline)) void load(const int32_t* __restrict__ cu_q,
                                                      const int32_t* __restrict__ seq_lens, int B, int lane) {
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int i = min(c * kWave + lane, B - 1);  // B >= 1
      lo[c] = cu_q[i];
      hi[c] = cu_q[i + 1];
      sl[c] = seq_lens[i];
    }
  }
  __device__ __attribute__((always_inline)) RowLoc find(const int32_t* __restrict__ cu_q,
                                                        const int32_t* __restrict__ seq_lens, int B, int t,
                                                        int lane) const {
    RowLoc loc{-1, 0};
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const uint64_t m = __ballot(c * kWave + lane < B && lo[c] <= t && t < hi[c]);
      if (m != 0 && loc.b < 0) {
        const int src = __ffsll((unsigned long long)m) - 1;
        const int q0 = __shfl(lo[c], src), q1 = __shfl(hi[c], src), s = __shfl(sl[c], src);
        loc = RowLoc{c * kWave + src, s - (q1 - q0) + (t - q0)};
      }
    }
    if (loc.b < 0) loc = locate_row(cu_q, seq_lens, B, t);
    return loc;
  }
};

__global__ __launch_bounds__(kThreads) void topk_radix(const int32_t* __restrict__ cu_q,
                                                       const int32_t* __restrict__ seq_lens, int B,
                                                       const float* __restrict__ scores, int64_t ld,
                                                       int K, int32_t* __restrict__ idx, int row_lo) {
  __shared__ __align__(16) uint32_t cache[kCache];
  __shared__ __align__(16) uint32_t hist[topk::kHistLdsWords];
  __shared__ uint32_t wcount[2 * kThreads / kWave];
  __shared__ uint32_t pick[3];

  const int t = row_lo + (int)blockIdx.x;  // score row t - row_lo, index row t
  const int tid = threadIdx.x;
  const float* row = scores + (int64_t)(t - row_lo) * ld;
  // Rows whose storage fits the cache as whole 16-byte quads, 16-byte
  // aligned, have the first part of their read issued before the lookup that
  // gives the row's length.
  const bool early = ld >= 4 && ld <= kCache && (ld & 3) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  // The lookup's loads go out first, then the row read, then the lookup's
  // search.
  const int lane = tid & (kWave - 1);
  RequestTable<4> req;
  req.load(cu_q, seq_lens, B, lane);
  f32x4 pre[topk::kReadBatch];
  if (early) topk::read_first_round<kThreads, topk::kEarlyBatch>(row, (int)ld, pre);
  const RowLoc loc = req.find(cu_q, seq_lens, B, t, lane);
  const int n = (int)max<int64_t>(0, min<int64_t>((int64_t)loc.pos + 1, ld));
  int32_t* out = idx + (int64_t)t * K;

  if (n <= K) {
    for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  auto emit = [out](uint32_t o, int s) { out[o] = s; };
  if (early) select_emit<true, topk::kEarlyBatch, true>(row, n, K, cache, hist, wcount, pick, emit, pre);
  else if (n <= kCache) select_cached_row(row, n, ld, K, cache, hist, wcount, pick, emit);
  else select_emit<false, 0, false>(row, n, K, cache, hist, wcount, pick, emit);  // rare: no workspace
}

// Persistent form for launches with more rows than CUs: workgroup w takes
// rows w, w + G, ... (G = gridDim.x).  Once a row is in registers (after its
// pass 0), the next row's whole storage is read blind into the registers pass
// 0 took the row from, so that read runs under the row's refining passes and
// compaction; the request lookup's loads go out once.  Needs a row storage
// that fits the cache as whole 16-byte quads (4 <= ld <= kCache, ld % 4 == 0,
// scores 16-byte aligned).
__global__ __launch_bounds__(kThreads) void topk_rows(const int32_t* __restrict__ cu_q,
                                                      const int32_t* __restrict__ seq_lens, int B,
                                                      const float* __restrict__ scores, int64_t ld, int K,
                                                      int32_t* __restrict__ idx, int row_lo, int rows) {
  __shared__ __align__(16) uint32_t cache[kCache];
  __shared__ __align__(16) uint32_t hist[topk::kHistLdsWords];
  __shared__ uint32_t wcount[2 * kThreads / kWave];
  __shared__ uint32_t pick[3];

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int G = (int)gridDim.x;
  RequestTable<1> req;  // registers are scarce here: one round, later ones from locate_row
  req.load(cu_q, seq_lens, B, lane);
  f32x4 nxt[topk::kReadBatch];
  topk::read_first_round<kThreads, topk::kReadBatch>(scores + (int64_t)blockIdx.x * ld, (int)ld, nxt);
  for (int rr = (int)blockIdx.x; rr < rows; rr += G) {
    const int tid_r = opaque_tid();
    const int t = row_lo + rr;
    const float* row = scores + (int64_t)rr * ld;
    const RowLoc loc = req.find(cu_q, seq_lens, B, t, lane);
    const int n = (int)max<int64_t>(0, min<int64_t>((int64_t)loc.pos + 1, ld));
    int32_t* out = idx + (int64_t)t * K;
    // the next row of this workgroup (the last row reads itself again: the
    // read stays in bounds and goes unused)
    const float* row_next = scores + (int64_t)(rr + G < rows ? rr + G : rr) * ld;
    auto read_next = [&]() { topk::read_first_round<kThreads, topk::kReadBatch>(row_next, (int)ld, nxt, tid_r); };
    if (n <= K) {
      for (int j = tid_r; j < K; j += kThreads) out[j] = j < n ? j : -1;
      read_next();
      continue;
    }
    topk::select_cached<kThreads, topk::kReadBatch, true>(topk::RowReader<true>(row, n), n, K, cache, hist, pick,
                                                          wcount, [out](uint32_t o, int s) { out[o] = s; }, nxt,
                                                          read_next, tid_r);
  }
}

// Two-level selection for rows longer than the LDS cache.  Level 1: each
// kSegLen-entry segment of a row gets its exact top-K (its entries cached in
// LDS), stored as candidates: scores and positions, segment after segment,
// ascending inside each segment, padded with (-inf, -1).  Level 2: the top-K
// of a row's candidates.  Both levels use the same order (higher score, then
// lower position), so the row's top-K lies in the union of its segments' and
// level 2 picks exactly it; candidate order is position order, so ties still
// go to the lower position.  Rows with n <= K use no candidates.  Segments
// are as long as the cache: each workgroup's selection is mostly a fixed
// chain of latencies, so fewer, fuller segments win (mtp_fp8 rows of 64-128K
// entries: 84 us at 32768, 93 at 16384, 127 at 8192, 112 single-level).
constexpr int kSegLen = kCache;

__global__ __launch_bounds__(kThreads) void topk_segments(const int32_t* __restrict__ cu_q,
                                                          const int32_t* __restrict__ seq_lens, int B,
                                                          const float* __restrict__ scores, int64_t ld,
                                                          int K, int row_lo, int segs, float* __restrict__ cand_sc,
                                                          int32_t* __restrict__ cand_ix) {
  __shared__ __align__(16) uint32_t cache[kSegLen];
  __shared__ __align__(16) uint32_t hist[topk::kHistLdsWords];
  __shared__ uint32_t wcount[2 * kThreads / kWave];
  __shared__ uint32_t pick[3];

  const int t = row_lo + (int)blockIdx.x, seg = (int)blockIdx.y;
  const int tid = threadIdx.x;
  const RowLoc loc = locate_row(cu_q, seq_lens, B, t);
  const int n = (int)max<int64_t>(0, min<int64_t>((int64_t)loc.pos + 1, ld));
  if (n <= K) return;  // topk_merge writes such rows directly
  const int64_t base = ((int64_t)(t - row_lo) * segs + seg) * K;
  const int s0 = seg * kSegLen, len = max(0, min(n - s0, kSegLen));
  const float* row = scores + (int64_t)(t - row_lo) * ld + s0;
  if (len <= K) {  // the whole segment, then padding
    for (int j = tid; j < K; j += kThreads) {
      cand_ix[base + j] = j < len ? s0 + j : -1;
      cand_sc[base + j] = j < len ? row[j] : -INFINITY;
    }
    return;
  }
  select_cached_row(row, len, ld - s0, K, cache, hist, wcount, pick, [=](uint32_t o, int s) {
    cand_ix[base + o] = s0 + s;
    cand_sc[base + o] = row[min(s, len - 1)];  // s < len always; the min only bounds the read
  });
}

__global__ __launch_bounds__(kThreads) void topk_merge(const int32_t* __restrict__ cu_q,
                                                       const int32_t* __restrict__ seq_lens, int B, int64_t ld,
                                                       int K, int32_t* __restrict__ idx, int row_lo, int segs,
                                                       const float* __restrict__ cand_sc,
                                                       const int32_t* __restrict__ cand_ix) {
  __shared__ __align__(16) uint32_t cache[kCache];
  __shared__ __align__(16) uint32_t hist[topk::kHistLdsWords];
  __shared__ uint32_t wcount[2 * kThreads / kWave];
  __shared__ uint32_t pick[3];

  const int t = row_lo + (int)blockIdx.x;
  const int tid = threadIdx.x;
  const RowLoc loc = locate_row(cu_q, seq_lens, B, t);
  const int n = (int)max<int64_t>(0, min<int64_t>((int64_t)loc.pos + 1, ld));
  int32_t* out = idx + (int64_t)t * K;
  if (n <= K) {
    for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const int n2 = segs * K;
  const float* row = cand_sc + (int64_t)(t - row_lo) * n2;
  const int32_t* ix = cand_ix + (int64_t)(t - row_lo) * n2;
  auto emit = [out, ix, n2](uint32_t o, int s) { out[o] = ix[min(s, n2 - 1)]; };  // s < n2 always
  if (n2 <= kCache) select_cached_row(row, n2, n2, K, cache, hist, wcount, pick, emit);
  else select_emit<false, 0, false>(row, n2, K, cache, hist, wcount, pick, emit);
}

}  // namespace

size_t topk_workspace_bytes(int num_q_rows, int max_seq_len, int k) {
  if (num_q_rows <= 0 || k <= 0 || max_seq_len <= kCache || max_seq_len <= k) return 0;
  const int64_t segs = (max_seq_len + kSegLen - 1) / kSegLen;
  const int64_t per = segs * k;  // candidates per row: a score and a position each
  return (size_t)((num_q_rows * per * 4 + 255) / 256 * 256 + num_q_rows * per * 4);
}

hipError_t launch_topk(const BatchArgs& ba, const float* scores, int64_t ld, int k, int32_t* idx,
                       hipStream_t stream, int row_lo, int row_hi, void* ws, size_t ws_bytes) {
  if (row_hi <= row_lo) return hipSuccess;
  const int rows = row_hi - row_lo;
  const size_t need = topk_workspace_bytes(rows, ba.max_seq_len, k);
  // topk_rows reads rows blind as whole 16-byte quads
  const bool rows_ok = ld >= 4 && ld % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  if (need > 0 && ws != nullptr && ws_bytes >= need) {
    const int segs = (ba.max_seq_len + kSegLen - 1) / kSegLen;
    float* cand_sc = static_cast<float*>(ws);
    int32_t* cand_ix = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) +
                                                  ((int64_t)rows * segs * k * 4 + 255) / 256 * 256);
    hipLaunchKernelGGL(topk_segments, dim3(rows, segs), dim3(kThreads), 0, stream, ba.cu_q, ba.seq_lens,
                       ba.batch, scores, ld, k, row_lo, segs, cand_sc, cand_ix);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge, dim3(rows), dim3(kThreads), 0, stream, ba.cu_q, ba.seq_lens, ba.batch, ld,
                       k, idx, row_lo, segs, cand_sc, cand_ix);
    return hipGetLastError();
  }
  if (rows_ok && ld <= kCache && rows > device_cu_count())
    hipLaunchKernelGGL(topk_rows, dim3(device_cu_count()), dim3(kThreads), 0, stream, ba.cu_q, ba.seq_lens,
                       ba.batch, scores, ld, k, idx, row_lo, rows);
  else
    hipLaunchKernelGGL(topk_radix, dim3(rows), dim3(kThreads), 0, stream, ba.cu_q,
                       ba.seq_lens, ba.batch, scores, ld, k, idx, row_lo);
  return hipGetLastError();
}

}  // namespace dsa
