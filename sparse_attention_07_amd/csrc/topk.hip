// Per-row top-k of the indexer scores by radix select on gfx950 (the radix
// top-k of lmdeploy PR 4737 "feat: support GLM-5.2", section "Changes").
//
// Order: higher score first, equal scores to the lower position, -0.0 equal
// to +0.0.  Output: the selected positions in ascending order, then -1.
// When pos(t)+1 <= k the row keeps every valid position (mstar PR 387,
// section "Body": below index_topk the pick is all tokens).
//
// One workgroup of 1024 threads per query row.  Scores map to 32-bit keys
// whose unsigned order is the score order.  Three histogram passes over
// 11, 11 and 10 key bits (LDS histograms, LDS atomics) narrow down the exact
// key tau of the k-th best element and how many elements equal to tau must
// be taken (the lowest-positioned ones).  A last pass walks the row in
// ascending position and compacts the selected positions with wave ballots
// and a workgroup prefix, which yields the ascending output directly and
// resolves the ties by position.  Rows of up to 32768 entries are cached in
// LDS as keys after one read; longer rows are re-read from global memory in
// each pass.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kCache = 32768;
constexpr int kBins = 2048;

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                          // -0.0 ranks with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);     // unsigned order == float order
}

// Exclusive prefix over the workgroup of a per-thread count; also returns the total.
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = wsum[w];
    before += (w < wave) ? s : 0u;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

__global__ __launch_bounds__(kThreads) void topk_radix(const int32_t* __restrict__ cu_q,
                                                       const int32_t* __restrict__ seq_lens, int B,
                                                       const float* __restrict__ scores, int64_t ld,
                                                       int K, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t cache[kCache];
  __shared__ uint32_t wsum[2][kWaves];
  __shared__ uint32_t pick[2];

  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = find_request(cu_q, B, t);
  const int64_t pos = row_position(cu_q, seq_lens, b, t);
  const int n = (int)max<int64_t>(0, min<int64_t>(pos + 1, ld));
  int32_t* out = idx + (int64_t)t * K;

  if (n <= K) {
    for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }

  const float* row = scores + (int64_t)t * ld;
  const bool cached = n <= kCache;
  if (cached)
    for (int s = tid; s < n; s += kThreads) cache[s] = order_key(row[s]);

  uint32_t prefix = 0, mask = 0, need = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int s = tid; s < n; s += kThreads) {
      const uint32_t u = cached ? cache[s] : order_key(row[s]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // Thread i owns bins nb-1-2i and nb-2-2i: a prefix in this order counts the
    // elements in higher bins.
    const int hb0 = nb - 1 - 2 * tid, hb1 = nb - 2 - 2 * tid;
    const uint32_t c0 = hb0 >= 0 ? hist[hb0] : 0u;
    const uint32_t c1 = hb1 >= 0 ? hist[hb1] : 0u;
    uint32_t total;
    const uint32_t above = block_excl_scan(c0 + c1, wsum[0], total);
    if (hb0 >= 0 && above < need && need <= above + c0) {
      pick[0] = (uint32_t)hb0;
      pick[1] = need - above;
    }
    if (hb1 >= 0 && above + c0 < need && need <= above + c0 + c1) {
      pick[0] = (uint32_t)hb1;
      pick[1] = need - above - c0;
    }
    __syncthreads();
    prefix |= pick[0] << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    need = pick[1];
    __syncthreads();
  }
  const uint32_t tau = prefix;  // key of the k-th best element; `need` of its equals are taken

  uint32_t run_gt = 0, run_tie = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll 1
  for (int base = 0; base < n; base += kThreads) {
    const int s = base + tid;
    const bool valid = s < n;
    const uint32_t u = valid ? (cached ? cache[s] : order_key(row[s])) : 0u;
    const bool gt = valid && u > tau;
    const bool tie = valid && u == tau;
    const uint64_t mg = __ballot(gt), mt = __ballot(tie);
    if (lane == 0) {
      wsum[0][wave] = (uint32_t)__popcll(mg);
      wsum[1][wave] = (uint32_t)__popcll(mt);
    }
    __syncthreads();
    uint32_t gt_before = (uint32_t)__popcll(mg & lt_mask), tie_before = (uint32_t)__popcll(mt & lt_mask);
    uint32_t gt_all = 0, tie_all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t g = wsum[0][w], e = wsum[1][w];
      gt_before += (w < wave) ? g : 0u;
      tie_before += (w < wave) ? e : 0u;
      gt_all += g;
      tie_all += e;
    }
    __syncthreads();
    const uint32_t tie_rank = run_tie + tie_before;
    if (gt || (tie && tie_rank < need)) {
      const uint32_t o = run_gt + gt_before + min(tie_rank, need);
      if (o < (uint32_t)K) out[o] = s;
    }
    run_gt += gt_all;
    run_tie += tie_all;
  }
}

}  // namespace

hipError_t launch_topk(const BatchArgs& ba, const float* scores, int64_t ld, int k, int32_t* idx,
                       hipStream_t stream) {
  if (ba.num_q_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_radix, dim3(ba.num_q_rows), dim3(kThreads), 0, stream, ba.cu_q,
                     ba.seq_lens, ba.batch, scores, ld, k, idx);
  return hipGetLastError();
}

}  // namespace dsa
