// Per-row top-k of the indexer scores by radix select on gfx950 (the radix
// top-k of lmdeploy PR 4737 "feat: support GLM-5.2", section "Changes").
//
// Output: the selected positions in ascending order, then -1.  When
// pos(t)+1 <= k the row keeps every valid position (mstar PR 387, section
// "Body": below index_topk the pick is all tokens).  One workgroup of 1024
// threads per query row; the selection itself (order, ties, passes,
// compaction) is in topk_select.h.  Rows of up to 32768 entries are cached in
// LDS as keys after one read; longer rows are re-read in each pass (the two
// cases are separate instantiations).
#include "dsa_device.h"
#include "dsa_launch.h"
#include "topk_select.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kCache = 32768;

template <bool Cached>
__device__ inline void select_row(const float* __restrict__ row, int n, int K, int32_t* __restrict__ out,
                                  uint32_t* cache, uint32_t* hist, uint32_t* wcount, uint32_t* pick) {
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  const topk::Threshold th = topk::select<kThreads, Cached>(row, vec, n, K, cache, hist, pick);
  auto emit = [out, K](uint32_t o, int s) {
    if (o < (uint32_t)K) out[o] = s;
  };
  if (Cached) topk::compact_cached<kThreads>(n, cache, th, wcount, emit);
  else topk::compact<kThreads, Cached>(row, vec, n, cache, th, wcount, emit);
}

__global__ __launch_bounds__(kThreads) void topk_radix(const int32_t* __restrict__ cu_q,
                                                       const int32_t* __restrict__ seq_lens, int B,
                                                       const float* __restrict__ scores, int64_t ld,
                                                       int K, int32_t* __restrict__ idx, int row_lo) {
  __shared__ __align__(16) uint32_t cache[kCache];
  __shared__ __align__(16) uint32_t hist[2 * topk::kHistWords];
  __shared__ uint32_t wcount[2 * kThreads / kWave];
  __shared__ uint32_t pick[3];

  const int t = row_lo + (int)blockIdx.x;  // score row t - row_lo, index row t
  const int tid = threadIdx.x;
  const RowLoc loc = locate_row(cu_q, seq_lens, B, t);
  const int n = (int)max<int64_t>(0, min<int64_t>((int64_t)loc.pos + 1, ld));
  int32_t* out = idx + (int64_t)t * K;

  if (n <= K) {
    for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const float* row = scores + (int64_t)(t - row_lo) * ld;
  if (n <= kCache) select_row<true>(row, n, K, out, cache, hist, wcount, pick);
  else select_row<false>(row, n, K, out, cache, hist, wcount, pick);
}

}  // namespace

hipError_t launch_topk(const BatchArgs& ba, const float* scores, int64_t ld, int k, int32_t* idx,
                       hipStream_t stream, int row_lo, int row_hi) {
  if (row_hi <= row_lo) return hipSuccess;
  hipLaunchKernelGGL(topk_radix, dim3(row_hi - row_lo), dim3(kThreads), 0, stream, ba.cu_q,
                     ba.seq_lens, ba.batch, scores, ld, k, idx, row_lo);
  return hipGetLastError();
}

}  // namespace dsa
