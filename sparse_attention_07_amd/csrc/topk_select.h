// Radix selection of a row's k best scores on gfx950: shared by the top-k
// kernel and by the 16-head sparse-MLA kernel that selects its own rows.
//
// Order: higher score first, equal scores to the lower position, -0.0 equal
// to +0.0.  Scores map to 32-bit keys whose unsigned order is the score
// order.  Up to three histogram passes over 11, 11 and 10 key bits (LDS
// histograms, LDS atomics) narrow down the key prefix of the k-th best
// element; the first pass runs while the row is read (and cached in LDS as
// keys when the caller has room), and the passes stop as soon as the chosen
// bin is taken whole.  After each pass a single wave scans the histogram
// (bins padded so that its lanes' ranges fall in distinct banks) to find the
// bin holding the k-th element.  The selection is then "key prefix above the
// chosen one, or equal to it and among the first `need` such positions".
// Compaction: each wave owns a contiguous range of the row, counts its
// selected elements with ballots, one workgroup-wide prefix over the wave
// counts places the ranges, and a second walk hands every selected position
// with its rank in ascending position order to the caller -- the ascending
// output and the position tie-break come without sorting.
#pragma once

#include "dsa_device.h"

namespace dsa {
namespace topk {

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

struct Threshold {
  uint32_t prefix, mask, need;
};

// Threshold of the k best of the n > k scores load(0) .. load(n-1), for a
// workgroup of NT threads.  hist: 2 * kHistWords LDS words; pick: 3 LDS
// words; cache: n LDS words, used when `cached`.  Begins and ends with a
// barrier.
template <int NT, typename Load>
__device__ inline Threshold select(Load load, int n, int k, bool cached, uint32_t* cache, uint32_t* hist,
                                   uint32_t* pick) {
  const int tid = threadIdx.x, wave = tid / kWave;
  for (int i = tid; i < 2 * kHistWords; i += NT) hist[i] = 0u;
  __syncthreads();
  // Pass 0 (key bits 21..31) while the row is read; eight loads in flight per thread.
  for (int s0 = 0; s0 < n; s0 += 8 * NT) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = s0 + i * NT + tid;
      v[i] = s < n ? load(s) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = s0 + i * NT + tid;
      if (s < n) {
        const uint32_t u = order_key(v[i]);
        if (cached) cache[s] = u;
        atomicAdd(&hist[hslot(u >> 21)], 1u);
      }
    }
  }
  __syncthreads();
  if (wave == 0) pick_bin(hist, kBins, (uint32_t)k, pick);
  __syncthreads();
  Threshold th{pick[0] << 21, 0xFFE00000u, pick[1]};
  bool done = pick[2] == th.need;  // the whole bin is taken
  // Passes 1 (bits 10..20) and 2 (bits 0..9) over the elements of the chosen prefix.
#pragma unroll 1
  for (int pass = 1; pass < 3 && !done; ++pass) {
    const int shift = pass == 1 ? 10 : 0;
    const int nb = pass == 1 ? 2048 : 1024;
    uint32_t* h = hist + (pass & 1) * kHistWords;
    if (pass == 1)  // pass 0's histogram was read before the last barrier; pass 2 reuses it
      for (int i = tid; i < kHistWords; i += NT) hist[i] = 0u;
    for (int s = tid; s < n; s += NT) {
      const uint32_t u = cached ? cache[s] : order_key(load(s));
      if ((u & th.mask) == th.prefix) atomicAdd(&h[hslot((u >> shift) & (uint32_t)(nb - 1))], 1u);
    }
    __syncthreads();
    if (wave == 0) pick_bin(h, nb, th.need, pick);
    __syncthreads();
    th.prefix |= pick[0] << shift;
    th.mask |= (uint32_t)(nb - 1) << shift;
    th.need = pick[1];
    done = pick[2] == th.need;
  }
  __syncthreads();  // pick may be rewritten by the next selection
  return th;
}

// Calls emit(o, s) for every selected position s, o = its rank (0 .. k-1) in
// ascending position order.  Selected: (key & mask) > prefix, or == prefix
// among the first `need` such positions.  wcount: 2 * NT / 64 LDS words.
template <int NT, typename Load, typename Emit>
__device__ inline void compact(Load load, int n, bool cached, const uint32_t* cache, Threshold th,
                               uint32_t* wcount, Emit emit) {
  constexpr int kW = NT / kWave;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int R = ((n + kW - 1) / kW + kWave - 1) / kWave * kWave;  // wave w owns [w R, (w+1) R)
  const int r0 = wave * R, r1 = min(n, r0 + R);
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t cg = 0, ce = 0;
  for (int c = r0; c < r1; c += kWave) {
    const int s = c + lane;
    const uint32_t u = s < r1 ? ((cached ? cache[s] : order_key(load(s))) & th.mask) : 0u;
    cg += (uint32_t)__popcll(__ballot(s < r1 && u > th.prefix));
    ce += (uint32_t)__popcll(__ballot(s < r1 && u == th.prefix));
  }
  if (lane == 0) {
    wcount[wave] = cg;
    wcount[kW + wave] = ce;
  }
  __syncthreads();
  uint32_t run_gt = 0, run_eq = 0;
  for (int w = 0; w < wave; ++w) {
    run_gt += wcount[w];
    run_eq += wcount[kW + w];
  }
  for (int c = r0; c < r1; c += kWave) {
    const int s = c + lane;
    const uint32_t u = s < r1 ? ((cached ? cache[s] : order_key(load(s))) & th.mask) : 0u;
    const bool gt = s < r1 && u > th.prefix, eq = s < r1 && u == th.prefix;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    const uint32_t eq_rank = run_eq + (uint32_t)__popcll(me & below);
    if (gt || (eq && eq_rank < th.need))
      emit(run_gt + (uint32_t)__popcll(mg & below) + min(eq_rank, th.need), s);
    run_gt += (uint32_t)__popcll(mg);
    run_eq += (uint32_t)__popcll(me);
  }
  __syncthreads();  // wcount may be rewritten by the next compaction
}

}  // namespace topk
}  // namespace dsa
