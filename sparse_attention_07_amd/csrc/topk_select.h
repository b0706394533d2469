// Radix selection of a row's k best scores on gfx950, for the top-k kernel.
//
// Order: higher score first, equal scores to the lower position, -0.0 equal
// to +0.0.  Scores map to 32-bit keys whose unsigned order is the score
// order.  Up to three histogram passes over 11, 11 and 10 key bits (LDS
// histograms, LDS atomics) narrow down the key prefix of the k-th best
// element; the first pass runs while the row is read (and cached in LDS as
// keys when it fits), and the passes stop as soon as the chosen bin is taken
// whole.  After each pass a single wave scans the histogram to find the bin
// holding the k-th element.  The selection is then "key prefix above the
// chosen one, or equal to it and among the first `need` such positions".
// Compaction: each wave owns a contiguous range of the row, counts its
// selected elements, one workgroup-wide prefix over the wave counts places
// the ranges, and a second walk hands every selected position with its rank
// in ascending position order to the caller -- the ascending output and the
// position tie-break come without sorting.
//
// The row is read in quads (four consecutive positions): 16-byte loads when
// the row is 16-byte aligned, and 16-byte LDS accesses for the key cache, so
// that one round of loads per thread covers a whole cached row.
#pragma once

#include "dsa_device.h"

namespace dsa {
namespace topk {

constexpr int kBins = 2048;
constexpr int kHistWords = kBins + kBins / 32 * 4;  // four pad words per 32 bins
// LDS histogram area: pass 0 counts into two copies (even and odd lanes; the
// second starts 16 banks further on), pass 1 into a third histogram, pass 2
// into the first copy again.  Scores crowd into a few of pass 0's bins, and
// LDS atomics of one instruction that hit one address or bank serialise:
// two copies halve the worst collisions.
constexpr int kHistCopy1 = kHistWords + 16;
constexpr int kHistPass1 = 2 * kHistWords + 16;
constexpr int kHistLdsWords = 3 * kHistWords + 16;

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                          // -0.0 ranks with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);     // unsigned order == float order
}

// Padded histogram slot of a bin.  A run of 16 or 32 bins starting at a
// multiple of its length is contiguous and 16-byte aligned, and the 32-bin
// runs of consecutive lanes start 36 words apart (distinct banks for 16-byte
// reads).
__device__ inline int hslot(uint32_t bin) { return (int)(bin + (bin >> 5) * 4); }

__device__ inline uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), kWave - 1);
}

// Wave 0: in a histogram of NB bins (a larger bin holds larger keys) find the
// bin containing the need-th largest element; writes (bin, need left inside
// the bin, bin count) to pick[0..2].  Lane l owns the PER bins
// NB-PER*(l+1) .. NB-1-PER*l.  The histogram's total must be >= need.
template <int NB, bool TWO = false>
__device__ inline void pick_bin(const uint32_t* hist, uint32_t need, uint32_t* pick,
                                const uint32_t* hist2 = nullptr) {
  constexpr int kPer = NB / kWave;  // 32 or 16
  const int lane = threadIdx.x & (kWave - 1);
  const int lo = NB - kPer * (lane + 1);
  const u32x4* p = reinterpret_cast<const u32x4*>(hist + hslot((uint32_t)lo));
  const u32x4* p2 = reinterpret_cast<const u32x4*>(hist2 + hslot((uint32_t)lo));
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < kPer / 4; ++j) {
    const u32x4 v = p[j];
    sum += v[0] + v[1] + v[2] + v[3];
    if (TWO) {
      const u32x4 v2 = p2[j];
      sum += v2[0] + v2[1] + v2[2] + v2[3];
    }
  }
  const uint32_t inc = wave_incl_scan(sum);
  // The one lane whose range holds the need-th element hands it to the wave,
  // which scans those bins (from the top) one per lane.
  const uint64_t owner = __ballot(inc - sum < need && need <= inc);
  const int src = __builtin_ctzll(owner);
  const int top_s = __builtin_amdgcn_readlane(lo + kPer - 1, src);
  const uint32_t acc = (uint32_t)__builtin_amdgcn_readlane((int)(inc - sum), src);
  uint32_t c = lane < kPer ? hist[hslot((uint32_t)(top_s - lane))] : 0u;
  if (TWO && lane < kPer) c += hist2[hslot((uint32_t)(top_s - lane))];
  const uint32_t before = acc + wave_incl_scan(c) - c;
  if (lane < kPer && before < need && need <= before + c) {
    pick[0] = (uint32_t)(top_s - lane);
    pick[1] = need - before;
    pick[2] = c;
  }
}

// Scores of positions 4q .. 4q+3 of a row of n (positions >= n read as 0).
// vec: the row is 16-byte aligned.
__device__ inline f32x4 load_quad(const float* __restrict__ row, int q, int n, bool vec) {
  const int s = 4 * q;
  if (vec && s + 3 < n) return *reinterpret_cast<const f32x4*>(row + s);
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (s + j < n) v[j] = row[s + j];
  return v;
}

__device__ inline u32x4 quad_keys(f32x4 v) {
  return u32x4{order_key(v[0]), order_key(v[1]), order_key(v[2]), order_key(v[3])};
}

// Lanes below this one whose bit is set in m.
__device__ inline uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

struct Threshold {
  uint32_t prefix, mask, need;
};

// Threshold of the k best of the n > k scores row[0] .. row[n-1], for a
// workgroup of NT threads.  hist: kHistLdsWords LDS words, 16-byte aligned;
// pick: 3 LDS words; cache (Cached only): round_up(n, 4) LDS words,
// 16-byte aligned.  Begins and ends with a barrier.
// Quads in flight per thread while a row is read: one round of them covers
// NT * kReadBatch * 4 positions.
constexpr int kReadBatch = 8;

// The early part of a row's first round: its first kEarlyBatch quads per
// thread (NT * kEarlyBatch * 4 positions), read up to `bound` positions (the
// row's storage) before the row's length is known, so that the read overlaps
// the request lookup.  Only this part is read blind: the rest of the row is
// read once the length is known, so a row much shorter than its storage
// costs little more than its own length.  Positions at or past the length
// are never used.
constexpr int kEarlyBatch = 2;
template <int NT>
__device__ inline void read_first_round(const float* __restrict__ row, bool vec, int bound,
                                        f32x4 (&v)[kReadBatch]) {
  const int nq = (bound + 3) >> 2;
#pragma unroll
  for (int i = 0; i < kEarlyBatch; ++i) {
    const int q = i * NT + threadIdx.x;
    if (q < nq) v[i] = load_quad(row, q, bound, vec);
  }
}

// pre (PRE only): the early part of the first round, from read_first_round
// with a bound >= n.
template <int NT, bool Cached, bool PRE = false>
__device__ inline Threshold select(const float* __restrict__ row, bool vec, int n, int k,
                                   uint32_t* cache, uint32_t* hist, uint32_t* pick,
                                   const f32x4* pre = nullptr) {
  constexpr int kBatch = kReadBatch;
  const int tid = threadIdx.x, wave = tid / kWave;
  const int nq = (n + 3) >> 2;
  u32x4* cache4 = reinterpret_cast<u32x4*>(cache);
  for (int i = tid; i < kHistLdsWords; i += NT) hist[i] = 0u;
  __syncthreads();
  uint32_t* h0 = hist + ((tid & 1) ? kHistCopy1 : 0);
  // Pass 0 (key bits 21..31) while the row is read.
  for (int q0 = 0; q0 < nq; q0 += kBatch * NT) {
    f32x4 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int q = q0 + i * NT + tid;
      if (PRE && q0 == 0 && i < kEarlyBatch) v[i] = pre[i];
      else if (q < nq) v[i] = load_quad(row, q, n, vec);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int q = q0 + i * NT + tid;
      if (q < nq) {
        const u32x4 u = quad_keys(v[i]);
        if (Cached) cache4[q] = u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * q + j < n) atomicAdd(&h0[hslot(u[j] >> 21)], 1u);
      }
    }
  }
  __syncthreads();
  if (wave == 0) pick_bin<kBins, true>(hist, (uint32_t)k, pick, hist + kHistCopy1);
  __syncthreads();
  Threshold th{pick[0] << 21, 0xFFE00000u, pick[1]};
  bool done = pick[2] == th.need;  // the whole bin is taken
  // Passes 1 (bits 10..20) and 2 (bits 0..9) over the elements of the chosen prefix.
#pragma unroll 1
  for (int pass = 1; pass < 3 && !done; ++pass) {
    const int shift = pass == 1 ? 10 : 0;
    const uint32_t bmask = pass == 1 ? 2047u : 1023u;
    uint32_t* h = pass == 1 ? hist + kHistPass1 : hist;
    if (pass == 1)  // pass 0's histograms were read before the last barrier; pass 2 reuses the first
      for (int i = tid; i < kHistWords; i += NT) hist[i] = 0u;
    for (int q0 = 0; q0 < nq; q0 += kBatch * NT) {
      u32x4 u[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int q = q0 + i * NT + tid;
        if (q < nq) u[i] = Cached ? cache4[q] : quad_keys(load_quad(row, q, n, vec));
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int q = q0 + i * NT + tid;
        if (q < nq) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (4 * q + j < n && (u[i][j] & th.mask) == th.prefix)
              atomicAdd(&h[hslot((u[i][j] >> shift) & bmask)], 1u);
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      if (pass == 1) pick_bin<2048>(h, th.need, pick);
      else pick_bin<1024>(h, th.need, pick);
    }
    __syncthreads();
    th.prefix |= pick[0] << shift;
    th.mask |= bmask << shift;
    th.need = pick[1];
    done = pick[2] == th.need;
  }
  __syncthreads();  // pick may be rewritten by the next selection
  return th;
}

// Calls emit(o, s) for every selected position s, o = its rank (0 .. k-1) in
// ascending position order.  Selected: (key & mask) > prefix, or == prefix
// among the first `need` such positions.  wcount: 2 * NT / 64 LDS words.
template <int NT, bool Cached, typename Emit>
__device__ inline void compact(const float* __restrict__ row, bool vec, int n, const uint32_t* cache,
                               Threshold th, uint32_t* wcount, Emit emit) {
  constexpr int kW = NT / kWave;
  constexpr int kChunk = 4 * kWave;          // positions per wave step: a quad per lane
  constexpr int kBatch = Cached ? 4 : 8;     // steps in flight
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // wave w owns [w R, (w+1) R), R a multiple of kChunk
  const int R = ((n + kW - 1) / kW + kChunk - 1) / kChunk * kChunk;
  const int r0 = wave * R, r1 = min(n, r0 + R);
  const u32x4* cache4 = reinterpret_cast<const u32x4*>(cache);
  // Masked keys of the quads at c + b*kChunk + 4*lane, b < kBatch (steps past r1 left unread).
  auto keys = [&](int c, u32x4 (&u)[kBatch]) {
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int q = (c + b * kChunk) / 4 + lane;
      u[b] = u32x4{0u, 0u, 0u, 0u};
      if (c + b * kChunk < r1) u[b] = Cached ? cache4[q] : quad_keys(load_quad(row, q, r1, vec));
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) u[b] &= th.mask;
  };
  uint32_t cg = 0, ce = 0;
  for (int c = r0; c < r1; c += kBatch * kChunk) {
    u32x4 u[kBatch];
    keys(c, u);
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = c + b * kChunk + 4 * lane + j < r1;
        cg += (in && u[b][j] > th.prefix) ? 1u : 0u;
        ce += (in && u[b][j] == th.prefix) ? 1u : 0u;
      }
  }
  cg = wave_sum(cg);
  ce = wave_sum(ce);
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
  for (int c = r0; c < r1; c += kBatch * kChunk) {
    u32x4 u[kBatch];
    keys(c, u);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (c + b * kChunk >= r1) break;  // wave-uniform
      const int s0 = c + b * kChunk + 4 * lane;
      uint32_t ng = 0, ne = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = s0 + j < r1;
        ng += (in && u[b][j] > th.prefix) ? 1u : 0u;
        ne += (in && u[b][j] == th.prefix) ? 1u : 0u;
      }
      // counts of the lanes below (per chunk at most 256 each: packed in 16 bits)
      const uint32_t packed = ng | (ne << 16);
      const uint32_t inc = wave_incl_scan(packed);
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
      uint32_t gtb = run_gt + ((inc - packed) & 0xFFFFu), eqb = run_eq + ((inc - packed) >> 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (s0 + j >= r1) continue;
        if (u[b][j] > th.prefix) {
          emit(gtb + min(eqb, th.need), s0 + j);
          ++gtb;
        } else if (u[b][j] == th.prefix) {
          if (eqb < th.need) emit(gtb + eqb, s0 + j);
          ++eqb;
        }
      }
      run_gt += tot & 0xFFFFu;
      run_eq += tot >> 16;
    }
  }
  __syncthreads();  // wcount may be rewritten by the next compaction
}

// compact() for a row cached in LDS as keys, in one walk of the row: each
// wave stages the positions of its range's elements above or at the
// threshold prefix in its own part of the cache (tagged by bit 31 when at
// it; the staged count never passes the positions already read, so it
// overwrites only keys already consumed), then, once the waves' counts are
// known, walks its staged list to apply the global cut among the elements at
// the prefix and emit.  Same result as compact().
template <int NT, typename Emit>
__device__ inline void compact_cached(int n, uint32_t* cache, Threshold th, uint32_t* wcount, Emit emit) {
  constexpr int kW = NT / kWave;
  constexpr int kBatch = 8;  // 64-position steps in flight
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int R = ((n + kW - 1) / kW + kWave - 1) / kWave * kWave;
  const int r0 = wave * R, r1 = min(n, r0 + R);
  uint32_t n_gt = 0, n_eq = 0, n_st = 0;  // wave-uniform
  for (int c = r0; c < r1; c += kBatch * kWave) {
    uint32_t u[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int s = c + b * kWave + lane;
      u[b] = s < r1 ? cache[s] & th.mask : 0u;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int s = c + b * kWave + lane;
      const bool in = s < r1;
      const bool gt = in && u[b] > th.prefix, eq = in && u[b] == th.prefix;
      const uint64_t mg = __ballot(gt), me = __ballot(eq), m = mg | me;
      if (gt || eq) cache[r0 + n_st + lanes_below(m)] = (uint32_t)s | (eq ? 0x80000000u : 0u);
      n_st += (uint32_t)__popcll(m);
      n_gt += (uint32_t)__popcll(mg);
      n_eq += (uint32_t)__popcll(me);
    }
  }
  if (lane == 0) {
    wcount[wave] = n_gt;
    wcount[kW + wave] = n_eq;
  }
  __syncthreads();
  uint32_t gt_before = 0, run_eq = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += wcount[w];
    run_eq += wcount[kW + w];
  }
  uint32_t run_sel = gt_before + min(run_eq, th.need);
  for (uint32_t i0 = 0; i0 < n_st; i0 += kWave) {
    const bool in = i0 + lane < n_st;
    const uint32_t e = in ? cache[r0 + i0 + lane] : 0u;
    const bool at = in && (e >> 31) != 0u;
    const uint64_t meq = __ballot(at);
    const bool sel = in && (!at || run_eq + lanes_below(meq) < th.need);
    const uint64_t msel = __ballot(sel);
    if (sel) emit(run_sel + lanes_below(msel), (int)(e & 0x7FFFFFFFu));
    run_sel += (uint32_t)__popcll(msel);
    run_eq += (uint32_t)__popcll(meq);
  }
  __syncthreads();  // wcount and the cache may be rewritten by the next row
}

}  // namespace topk
}  // namespace dsa
