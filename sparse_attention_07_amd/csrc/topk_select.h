// Radix selection of a row's k best scores on gfx950, for the top-k kernel.
//
// Order: higher score first, equal scores to the lower position, -0.0 equal
// to +0.0.  Scores map to 32-bit keys whose unsigned order is the score
// order.  Up to three histogram passes over 11, 11 and 10 key bits (LDS
// histograms, LDS atomics) narrow down the key prefix of the k-th best
// element; the first pass runs while the row is read, and the passes stop as
// soon as the chosen bin is taken whole.  After each pass a single wave scans
// the histogram to find the bin holding the k-th element.  The selection is
// then "key prefix above the chosen one, or equal to it and among the first
// `need` such positions", emitted in ascending position order, so the
// ascending output and the position tie-break come without sorting.
//
// Rows that fit the LDS cache are read once (coalesced 16-byte quads through
// a raw buffer resource, whose bounds check returns zeros past the row, so
// every load is issued without a branch), their keys cached in LDS, and then
// held in registers as one contiguous run per thread: the later passes and
// the compaction work from registers.  Longer rows are re-read in each pass
// and compacted by waves (compact()).
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
// 64 words after the histograms, one per lane: pass 0 adds an element past
// the row to its lane's word instead of branching around the add.
constexpr int kHistDummy = 3 * kHistWords + 16;
constexpr int kHistLdsWords = kHistDummy + kWave;

// Every function below is inlined into its kernel, so that LDS pointers stay
// in the LDS address space and the compiler can keep several LDS reads in
// flight (an out-of-line call sees generic pointers and waits after each).
#define DSA_TOPK_INLINE __device__ __attribute__((always_inline)) inline

DSA_TOPK_INLINE uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                          // -0.0 ranks with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);     // unsigned order == float order
}

// Padded histogram slot of a bin.  A run of 16 or 32 bins starting at a
// multiple of its length is contiguous and 16-byte aligned, and the 32-bin
// runs of consecutive lanes start 36 words apart (distinct banks for 16-byte
// reads).
DSA_TOPK_INLINE int hslot(uint32_t bin) { return (int)(bin + (bin >> 5) * 4); }

DSA_TOPK_INLINE uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), kWave - 1);
}

// Wave 0: in a histogram of NB bins (a larger bin holds larger keys) find the
// bin containing the need-th largest element; writes (bin, need left inside
// the bin, bin count) to pick[0..2].  Lane l owns the PER bins
// NB-PER*(l+1) .. NB-1-PER*l.  The histogram's total must be >= need.
template <int NB, bool TWO = false>
DSA_TOPK_INLINE void pick_bin(const uint32_t* hist, uint32_t need, uint32_t* pick,
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
// vec: the row is 16-byte aligned.  (Long rows' compaction.)
DSA_TOPK_INLINE f32x4 load_quad(const float* __restrict__ row, int q, int n, bool vec) {
  const int s = 4 * q;
  if (vec && s + 3 < n) return *reinterpret_cast<const f32x4*>(row + s);
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (s + j < n) v[j] = row[s + j];
  return v;
}

DSA_TOPK_INLINE u32x4 quad_keys(f32x4 v) {
  return u32x4{order_key(v[0]), order_key(v[1]), order_key(v[2]), order_key(v[3])};
}

// Lanes below this one whose bit is set in m.
DSA_TOPK_INLINE uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// A row's quads through a raw buffer resource.  VEC: one 16-byte load per
// quad over round_up(n, 4) entries (the row start 16-byte aligned and the
// storage holding that many); otherwise four 4-byte loads over exactly n.
// Loads past the resource return zeros without touching memory, so no load
// needs a branch; positions at or past n are never used.
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw buffer descriptor flags
template <bool VEC>
struct RowReader {
  __amdgpu_buffer_rsrc_t rs;
  // n is the same in every lane (readfirstlane tells the compiler so, which
  // keeps the descriptor in scalar registers).
  DSA_TOPK_INLINE RowReader(const float* row, int n)
      : rs(__builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), (short)0,
                                             __builtin_amdgcn_readfirstlane((VEC ? (n + 3) & ~3 : n) * 4),
                                             kRawBufferWord3)) {}
  DSA_TOPK_INLINE f32x4 quad(int q) const {
    if (VEC) return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, q * 16, 0, 0));
    f32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (4 * q + j) * 4, 0, 0));
    return v;
  }
};

// Whether a row of n entries at `row`, with `bound` >= n entries of storage
// from there, may be read as 16-byte quads.
DSA_TOPK_INLINE bool quads_ok(const float* row, int n, int64_t bound) {
  return (reinterpret_cast<uintptr_t>(row) & 15) == 0 && (int64_t)((n + 3) & ~3) <= bound;
}

struct Threshold {
  uint32_t prefix, mask, need;
};

// Quads in flight per thread while a row is read: one round of them covers
// NT * kReadBatch * 4 positions, a whole cached row.
constexpr int kReadBatch = 8;

// The early part of a row's first round: its first kEarlyBatch quads per
// thread (NT * kEarlyBatch * 4 positions), read before the row's length is
// known so that the read overlaps the request lookup, within the row's
// storage of `bound` entries (a multiple of 4, the row 16-byte aligned).
// Only this part is read blind: the rest of the row is read once the length
// is known, so a row much shorter than its storage costs little more than its
// own length.  Positions at or past the length are never used.  Plain global
// loads (lanes past the storage re-read its last quad): the lookup's loads
// are global too, and the compiler then waits for exactly those.
constexpr int kEarlyBatch = 2;
// The first NPRE quads per thread of a row's round, from a row storage of
// `bound` entries (bound >= 4 and a multiple of 4, the row 16-byte aligned).
template <int NT, int NPRE>
DSA_TOPK_INLINE void read_first_round(const float* __restrict__ row, int bound, f32x4 (&v)[kReadBatch],
                                      int tid = (int)threadIdx.x) {
  const int last = (bound >> 2) - 1;
#pragma unroll
  for (int i = 0; i < NPRE; ++i) v[i] = *reinterpret_cast<const f32x4*>(row + 4 * min(i * NT + tid, last));
}

// Pass 0 (key bits 21..31) while the row is read, the bin pick after it.
// Cached (n <= NT * kReadBatch * 4, one round of reads): the keys are also
// written to cache.  pre: the round's first NPRE quads per thread, already
// read (read_first_round).  Begins by clearing the histograms and ends with a
// barrier after the pick.
template <int NT, bool Cached, int NPRE, bool VEC>
DSA_TOPK_INLINE Threshold pass0(const RowReader<VEC>& rd, int n, int k, uint32_t* cache, uint32_t* hist,
                                uint32_t* pick, const f32x4* pre, bool& done, int tid) {
  constexpr int kBatch = kReadBatch;
  const int wave = tid / kWave;
  const int nq = (n + 3) >> 2;
  u32x4* cache4 = reinterpret_cast<u32x4*>(cache);
  for (int i = tid; i < kHistLdsWords; i += NT) hist[i] = 0u;
  __syncthreads();
  uint32_t* h0 = hist + ((tid & 1) ? kHistCopy1 : 0);
  uint32_t* dummy = hist + kHistDummy + (tid & (kWave - 1));
  const int rounds = Cached ? 1 : (nq + kBatch * NT - 1) / (kBatch * NT);
  for (int r = 0; r < rounds; ++r) {
    const int q0 = r * kBatch * NT;
    f32x4 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (i < NPRE) v[i] = pre[i];
      else v[i] = rd.quad(q0 + i * NT + tid);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int q = q0 + i * NT + tid;
      if (q < nq) {
        const u32x4 u = quad_keys(v[i]);
        if (Cached) cache4[q] = u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          atomicAdd(4 * q + j < n ? &h0[hslot(u[j] >> 21)] : dummy, 1u);
      }
    }
  }
  __syncthreads();
  if (wave == 0) pick_bin<kBins, true>(hist, (uint32_t)k, pick, hist + kHistCopy1);
  __syncthreads();
  const Threshold th{pick[0] << 21, 0xFFE00000u, pick[1]};
  done = pick[2] == th.need;  // the whole bin is taken
  return th;
}

// After a refining pass's counting: the bin of its histogram holding the
// need-th element narrows the threshold.  Begins and ends with a barrier.
template <int NT>
DSA_TOPK_INLINE void refine(Threshold& th, bool& done, int pass, const uint32_t* h, uint32_t* pick, int tid) {
  const int wave = tid / kWave;
  const int shift = pass == 1 ? 10 : 0;
  const uint32_t bmask = pass == 1 ? 2047u : 1023u;
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

// Threshold of the k best of the n > k scores of a row longer than the LDS
// cache, re-reading the row in every pass.  hist: kHistLdsWords LDS words,
// 16-byte aligned; pick: 3 LDS words.  Begins and ends with a barrier.
template <int NT, bool VEC>
DSA_TOPK_INLINE Threshold select(const RowReader<VEC>& rd, int n, int k, uint32_t* hist, uint32_t* pick) {
  constexpr int kBatch = kReadBatch;
  const int tid = (int)threadIdx.x;
  const int nq = (n + 3) >> 2;
  bool done;
  Threshold th = pass0<NT, false, 0, VEC>(rd, n, k, nullptr, hist, pick, nullptr, done, tid);
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
      for (int i = 0; i < kBatch; ++i) u[i] = quad_keys(rd.quad(q0 + i * NT + tid));
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int q = q0 + i * NT + tid;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (q < nq && 4 * q + j < n && (u[i][j] & th.mask) == th.prefix)
            atomicAdd(&h[hslot((u[i][j] >> shift) & bmask)], 1u);
      }
    }
    refine<NT>(th, done, pass, h, pick, tid);
  }
  __syncthreads();  // pick may be rewritten by the next selection
  return th;
}

// Most quads a thread holds when a cached row is walked from registers: rows
// of up to 4 * NT * kRegQuads positions (36864 at NT = 1024).
constexpr int kRegQuads = 9;

// Selection of the k best of the n > k scores of a row of at most
// 4 * NT * kReadBatch positions, calling emit(o, s) for every selected
// position s with o its rank (0 .. k-1) in ascending position order; the
// calls go out in order of o, consecutive o to consecutive threads.
//
// Pass 0 reads the row (coalesced, quads interleaved over the threads) and
// caches its keys in LDS.  Then every thread takes a contiguous run of Q
// quads from the cache into registers, Q odd so that the 16-byte reads of 16
// lanes, 16 Q bytes apart, meet 16 distinct bank quartets.  The later passes
// count the runs' keys from registers.  The compaction counts each run's
// selected elements, places the runs by one packed wave scan and one
// workgroup prefix over the wave totals, and stages every selected position
// at its rank in LDS (over the cache, which every thread has read by then),
// from where the workgroup emits them.  pre: the first NPRE quads per thread
// of pass 0's round, already read.  after_pass0() runs once the row is in
// registers: pre (and the cache until the compaction) is free from then on,
// so a caller can start reading its next row there.
// cache: 4 * NT * kReadBatch LDS words, 16-byte aligned (k <= that many);
// hist: kHistLdsWords LDS words, 16-byte aligned; pick: 3 LDS words; wcount:
// NT / 64 LDS words.  Begins and ends with a barrier.
struct NoHook {
  DSA_TOPK_INLINE void operator()() const {}
};
template <int NT, int NPRE, bool VEC, typename Emit, typename Hook = NoHook>
DSA_TOPK_INLINE void select_cached(const RowReader<VEC>& rd, int n, int k, uint32_t* cache, uint32_t* hist,
                                   uint32_t* pick, uint32_t* wcount, Emit emit, const f32x4* pre = nullptr,
                                   Hook after_pass0 = Hook(), int tid = (int)threadIdx.x) {
  static_assert(kRegQuads * NT >= kReadBatch * NT + NT, "a run of Q <= kRegQuads quads covers a cached row");
  constexpr int kW = NT / kWave;
  const int lane = tid % kWave, wave = tid / kWave;
  const int nq = (n + 3) >> 2;
  bool done;
  Threshold th = pass0<NT, true, NPRE, VEC>(rd, n, k, cache, hist, pick, pre, done, tid);
  // This thread's run: quads tid*Q .. tid*Q+Q-1 (the cache was complete at
  // pass 0's last barrier).  Positions at or past n hold key 0, the lowest:
  // they all lie after the row's last position, so even when 0 is the
  // threshold prefix they are never staged (at least `need` elements of the
  // row at the prefix come first); and were they counted in a refining pass's
  // lowest bin, the pick would not change, since the need-th element lies in
  // that bin only when no other bin can hold it.
  const int Q = __builtin_amdgcn_readfirstlane(((nq + NT - 1) / NT) | 1);
  const int q_first = tid * Q;
  const int p_first = 4 * q_first;
  const u32x4* cache4 = reinterpret_cast<const u32x4*>(cache);
  u32x4 r[kRegQuads];
#pragma unroll
  for (int j = 0; j < kRegQuads; ++j) {
    r[j] = u32x4{0u, 0u, 0u, 0u};
    if (j < Q) {
      if (q_first + j < nq) r[j] = cache4[q_first + j];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[j][e] = p_first + 4 * j + e < n ? r[j][e] : 0u;
    }
  }
  after_pass0();
#pragma unroll 1
  for (int pass = 1; pass < 3 && !done; ++pass) {
    const int shift = pass == 1 ? 10 : 0;
    const uint32_t bmask = pass == 1 ? 2047u : 1023u;
    uint32_t* h = pass == 1 ? hist + kHistPass1 : hist;
    if (pass == 1)  // pass 0's histograms were read before the last barrier; pass 2 reuses the first
      for (int i = tid; i < kHistWords; i += NT) hist[i] = 0u;
#pragma unroll
    for (int j = 0; j < kRegQuads; ++j) {
      if (j < Q) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((r[j][e] & th.mask) == th.prefix) atomicAdd(&h[hslot((r[j][e] >> shift) & bmask)], 1u);
      }
    }
    refine<NT>(th, done, pass, h, pick, tid);
  }
  // Compaction.  Bit 4j+e of gm / em: element e of quad j of the run is
  // above / at the threshold prefix.  Counts packed: above in the low half,
  // at in the high half (a row's totals stay below 2^16).
  uint64_t gm = 0, em = 0;
#pragma unroll
  for (int j = 0; j < kRegQuads; ++j) {
    if (j < Q) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = r[j][e] & th.mask;
        gm |= (uint64_t)(u > th.prefix ? 1u : 0u) << (4 * j + e);
        em |= (uint64_t)(u == th.prefix ? 1u : 0u) << (4 * j + e);
      }
    }
  }
  const uint32_t cnt = (uint32_t)__popcll(gm) | ((uint32_t)__popcll(em) << 16);
  const uint32_t inc = wave_incl_scan(cnt);
  if (lane == kWave - 1) wcount[wave] = inc;
  __syncthreads();  // also: every thread has read its run from the cache
  uint32_t before = inc - cnt;
#pragma unroll
  for (int w = 0; w < kW; ++w) before += w < wave ? wcount[w] : 0u;
  uint32_t gt = before & 0xFFFFu, eq = before >> 16;
  // The run's selected elements in position order, each staged at its rank.
  for (uint64_t m = gm | em; m != 0; m &= m - 1) {
    const int b = __builtin_ctzll(m);
    const uint32_t pos = (uint32_t)(p_first + b);
    if ((gm >> b) & 1u) {
      cache[gt + min(eq, th.need)] = pos;
      ++gt;
    } else {
      if (eq < th.need) cache[gt + eq] = pos;
      ++eq;
    }
  }
  __syncthreads();
  for (int o = tid; o < k; o += NT) emit((uint32_t)o, (int)cache[o]);
  __syncthreads();  // pick, wcount and the cache may be rewritten by the next selection
}

// Calls emit(o, s) for every selected position s, o = its rank (0 .. k-1) in
// ascending position order.  Selected: (key & mask) > prefix, or == prefix
// among the first `need` such positions.  wcount: 2 * NT / 64 LDS words.
template <int NT, bool Cached, typename Emit>
DSA_TOPK_INLINE void compact(const float* __restrict__ row, bool vec, int n, const uint32_t* cache,
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

}  // namespace topk
}  // namespace dsa
