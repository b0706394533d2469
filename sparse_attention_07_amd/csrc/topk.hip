// Per-row top-k of the indexer scores by radix select on gfx950 (the radix
// top-k of lmdeploy PR 4737 "feat: support GLM-5.2", section "Changes").
//
// Order: higher score first, equal scores to the lower position, -0.0 equal
// to +0.0.  Output: the selected positions in ascending order, then -1.
// When pos(t)+1 <= k the row keeps every valid position (mstar PR 387,
// section "Body": below index_topk the pick is all tokens).
//
// One workgroup of 1024 threads per query row.  Scores map to 32-bit keys
// whose unsigned order is the score order.  Up to three histogram passes over
// 11, 11 and 10 key bits (LDS histograms, LDS atomics) narrow down the key
// prefix of the k-th best element; the first pass runs while the row is read
// (and cached in LDS as keys when it has at most 32768 entries), and the
// passes stop as soon as the chosen bin is taken whole.  After each pass a
// single wave scans the histogram (bins padded so that its lanes' ranges fall
// in distinct banks) to find the bin holding the k-th element.  The selection
// is then "key prefix above the chosen one, or equal to it and among the
// first `need` such positions".  Each wave owns a contiguous range of the row:
// it counts its selected elements with ballots, one workgroup-wide prefix over
// the sixteen wave counts places the ranges, and a second walk writes the
// positions, which yields the ascending order and breaks ties by position
// without sorting.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kCache = 32768;
constexpr int kBins = 2048;
constexpr int kHistWords = kBins + kBins / 32;  // one pad word per 32 bins

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                          // -0.0 ranks with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);     // unsigned order == float order
}

// Padded histogram slot of a bin: the 32 bins a lane of the picking wave owns
// then start on distinct banks.
__device__ inline int hslot(uint32_t bin) { return (int)(bin + (bin >> 5)); }

// Wave 0: in a histogram of nb bins (a larger bin holds larger keys) find the
// bin containing the need-th largest element; writes (bin, need left inside
// the bin, bin count) to pick[0..2].  Lane l owns bins nb-1-per*l down to
// nb-per*(l+1).  The histogram's total must be >= need.
__device__ inline void pick_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* pick) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per = nb / kWave;  // 32 or 16
  const int top = nb - 1 - per * lane;
  uint32_t sum = 0;
#pragma unroll 8
  for (int j = 0; j < per; ++j) sum += hist[hslot((uint32_t)(top - j))];
  uint32_t inc = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  // The one lane whose range holds the need-th element hands it to the wave,
  // which scans those bins one per lane.
  const uint64_t owner = __ballot(inc - sum < need && need <= inc);
  const int src = __ffsll((unsigned long long)owner) - 1;
  const int top_s = __shfl(top, src);
  const uint32_t acc = __shfl(inc - sum, src);
  const uint32_t c = lane < per ? hist[hslot((uint32_t)(top_s - lane))] : 0u;
  uint32_t ci = c;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t y = __shfl_up(ci, d);
    if (lane >= d) ci += y;
  }
  const uint32_t before = acc + ci - c;
  if (lane < per && before < need && need <= before + c) {
    pick[0] = (uint32_t)(top_s - lane);
    pick[1] = need - before;
    pick[2] = c;
  }
}

__global__ __launch_bounds__(kThreads) void topk_radix(const int32_t* __restrict__ cu_q,
                                                       const int32_t* __restrict__ seq_lens, int B,
                                                       const float* __restrict__ scores, int64_t ld,
                                                       int K, int32_t* __restrict__ idx) {
  __shared__ uint32_t cache[kCache];
  __shared__ uint32_t hist[2][kHistWords];
  __shared__ uint32_t wcount[2][kWaves];
  __shared__ uint32_t pick[3];

  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const RowLoc loc = locate_row(cu_q, seq_lens, B, t);
  const int n = (int)max<int64_t>(0, min<int64_t>((int64_t)loc.pos + 1, ld));
  int32_t* out = idx + (int64_t)t * K;

  if (n <= K) {
    for (int j = tid; j < K; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }

  const float* row = scores + (int64_t)t * ld;
  const bool cached = n <= kCache;
  for (int i = tid; i < 2 * kHistWords; i += kThreads) (&hist[0][0])[i] = 0u;
  __syncthreads();

  // Pass 0 (key bits 21..31) while the row is read; eight loads in flight per thread.
  for (int s0 = 0; s0 < n; s0 += 8 * kThreads) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = s0 + i * kThreads + tid;
      v[i] = s < n ? row[s] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = s0 + i * kThreads + tid;
      if (s < n) {
        const uint32_t u = order_key(v[i]);
        if (cached) cache[s] = u;
        atomicAdd(&hist[0][hslot(u >> 21)], 1u);
      }
    }
  }
  __syncthreads();
  if (wave == 0) pick_bin(hist[0], kBins, (uint32_t)K, pick);
  __syncthreads();
  uint32_t prefix = pick[0] << 21, mask = 0xFFE00000u, need = pick[1];
  bool done = pick[2] == need;  // the whole bin is taken

  // Passes 1 (bits 10..20) and 2 (bits 0..9) over the elements of the chosen prefix.
#pragma unroll 1
  for (int pass = 1; pass < 3 && !done; ++pass) {
    const int shift = pass == 1 ? 10 : 0;
    const int nb = pass == 1 ? 2048 : 1024;
    uint32_t* h = hist[pass & 1];
    if (pass == 1)  // pass 0's histogram was read before the last barrier; pass 2 reuses it
      for (int i = tid; i < kHistWords; i += kThreads) hist[0][i] = 0u;
    for (int s = tid; s < n; s += kThreads) {
      const uint32_t u = cached ? cache[s] : order_key(row[s]);
      if ((u & mask) == prefix) atomicAdd(&h[hslot((u >> shift) & (uint32_t)(nb - 1))], 1u);
    }
    __syncthreads();
    if (wave == 0) pick_bin(h, nb, need, pick);
    __syncthreads();
    prefix |= pick[0] << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    need = pick[1];
    done = pick[2] == need;
  }

  // Selected: (u & mask) > prefix, or (u & mask) == prefix among the first
  // `need` such positions.  Wave w owns positions [w*R, (w+1)*R).
  const int R = ((n + kWaves - 1) / kWaves + kWave - 1) / kWave * kWave;
  const int r0 = wave * R, r1 = min(n, r0 + R);
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t cg = 0, ce = 0;
  for (int c = r0; c < r1; c += kWave) {
    const int s = c + lane;
    const uint32_t u = s < r1 ? ((cached ? cache[s] : order_key(row[s])) & mask) : 0u;
    cg += (uint32_t)__popcll(__ballot(s < r1 && u > prefix));
    ce += (uint32_t)__popcll(__ballot(s < r1 && u == prefix));
  }
  if (lane == 0) {
    wcount[0][wave] = cg;
    wcount[1][wave] = ce;
  }
  __syncthreads();
  uint32_t run_gt = 0, run_eq = 0;
  for (int w = 0; w < wave; ++w) {
    run_gt += wcount[0][w];
    run_eq += wcount[1][w];
  }
  for (int c = r0; c < r1; c += kWave) {
    const int s = c + lane;
    const uint32_t u = s < r1 ? ((cached ? cache[s] : order_key(row[s])) & mask) : 0u;
    const bool gt = s < r1 && u > prefix, eq = s < r1 && u == prefix;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    const uint32_t eq_rank = run_eq + (uint32_t)__popcll(me & below);
    if (gt || (eq && eq_rank < need)) {
      const uint32_t o = run_gt + (uint32_t)__popcll(mg & below) + min(eq_rank, need);
      if (o < (uint32_t)K) out[o] = s;
    }
    run_gt += (uint32_t)__popcll(mg);
    run_eq += (uint32_t)__popcll(me);
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
