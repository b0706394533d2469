// Sparse weight-absorbed MLA over selected latent rows on gfx950.
//
// For query row t and head h (mlx-lm PR 1419, the commit extending the gather
// path to small L: keys and values are both the latent row and the value
// up-projection follows attention; mstar PR 387 "GLM-5.2 with MLA, fp8 MoE and
// DSA", section "Shared code": MLA with weight absorption):
//
//   l_j = scale * q[t,h,:576] . row(idx[t,j])[:576]      (usable j only)
//   out[t,h,:512] = sum_j softmax(l)_j row(idx[t,j])[:512],   lse = log sum_j exp(l_j)
//
// Rows are gathered straight from their pages through the page table (the
// zero-copy paged view of lmdeploy PR 4737 "feat: support GLM-5.2", section
// "Five-layer ablations"); an index is usable when 0 <= s <= pos(t) and its
// page is mapped, otherwise it is masked (lmdeploy PR 4968, invalid -1
// entries; mlx-lm PR 1419, re-masking of gathered keys).
//
// Both MFMA kernels run four waves per workgroup on one query row and one
// range of its selected rows:
//
// * Gather.  A prologue turns the range's indices into byte offsets (page
//   table applied, unusable entries marked) in LDS.  Tiles of 32 rows are then
//   copied from HBM straight into an LDS ring of 2-4 buffers with 16-byte
//   global_load_lds (no register staging), each wave issuing the same number
//   of copies per tile, so "all copies of tile i are done" is one
//   s_waitcnt vmcnt(copies issued after tile i).  Up to three tiles are in
//   flight while one is computed.  Rows are padded to 1168 B so that 16 lanes
//   reading 16 rows at one column hit 16 distinct bank groups.  Unusable rows
//   are copied from a usable row of the same range (finite data) and masked
//   in the softmax.  fp8 rows arrive raw (656 B) and a pass decodes them
//   (e4m3 * block scale -> bf16) into one compute tile.
// * QK^T.  S^T = rows x q^T on MFMA with the rows as the A operand read from
//   LDS and q held in registers as the B operand for the whole range.
// * Softmax.  Online, in registers, in log2 units; the running max is only
//   raised (and O rescaled) when a new tile beats it by more than 2^8, which
//   keeps the O rescale off the common path without changing the result.
// * PV.  P comes straight from the S^T accumulators as the A operand (the
//   accumulator layout defines which row feeds which k slot); V is the B
//   operand, read transposed from the row-major tile with ds_read_b64_tr_b16
//   (in each 16-lane group, lane i receives element i%4 of the 8-byte blocks
//   addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4), so every lane gets eight
//   rows of one output column without register shuffles.
//
// Both use v_mfma_f32_16x16x32_bf16 with 16 heads per wave.  For 16-head
// workloads every wave computes the (cheap) 32x16 score tile and then its own
// quarter of the 512 output columns, so one query's work spreads over four
// SIMDs.  For 64+ heads a workgroup owns 64 heads, 16 per wave, each wave all
// 512 columns (one wave per SIMD: 72 VGPRs of q, a 128-register accumulator).
// (32 heads per wave would halve the LDS operand traffic, but 144 VGPRs of q
// next to a 256-register accumulator do not fit and q ends up spilled.)
//
// When the selected rows of a query are split across workgroups, each writes
// (m, l, unnormalised O) partials and a second kernel merges them by
// log-sum-exp.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kD = kDc + kDr;
constexpr int kThreads = 256;                          // four waves
constexpr int kTileRows = 32;
constexpr int kSlotsPerRow = 73;                       // 72 chunks of 16 B + 1 pad chunk
constexpr int kRowLds = kSlotsPerRow * 16;             // 1168 B
constexpr int kTileSlots = kTileRows * kSlotsPerRow;   // 2336
constexpr int kTileLds = kTileSlots * 16;              // 37376 B
constexpr int kBf16Copies = (kTileSlots + kThreads - 1) / kThreads;   // 10 per thread
constexpr int kBf16CopiesMin = kTileSlots / kThreads;                 // 9 for the waves past the end
constexpr int kFp8Chunks = 41;                         // 656-byte row
constexpr int kFp8TileSlots = kTileRows * kFp8Chunks;  // 1312
constexpr int kFp8TileLds = kFp8TileSlots * 16;        // 20992 B
constexpr int kFp8Copies = (kFp8TileSlots + kThreads - 1) / kThreads; // 6
constexpr int kFp8CopiesMin = kFp8TileSlots / kThreads;               // 5
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.f;                   // log2 units

static_assert(kBf16CopiesMin == 9 && kFp8CopiesMin == 5, "wait immediates below assume these");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Wait until at most `after` tiles' copies are still outstanding for this wave,
// then barrier.  The inline asm is also a compiler memory barrier, and no
// other wait is implied (a C++ fence would add vmcnt(0) and drain the ring).
template <int L>
__device__ inline void wait_tiles_barrier(int after) {
  static_assert(L == 9 || L == 5, "immediates");
  if (L == 9) {
    switch (after) {
      case 0: asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(18)\n\ts_barrier" ::: "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(27)\n\ts_barrier" ::: "memory"); break;
    }
  } else {
    switch (after) {
      case 0: asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(5)\n\ts_barrier" ::: "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(15)\n\ts_barrier" ::: "memory"); break;
    }
  }
}

// All of this wave's LDS accesses are done, then barrier.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline void copy16_to_lds(const uint8_t* src, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                   (lds_void_t*)(lds_wave_base), 16, 0, 0);
}

__device__ inline s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

__device__ inline bf16x8 join(s16x4 a, s16x4 b) {
  const s16x8 w = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

// e4m3fn (OCP OFP8) byte -> float, exact.  Exponent bias 7, subnormals
// m/8 * 2^-6; the NaN code (S.1111.111) is not expected in a cache.
__device__ inline float e4m3_to_f32(uint32_t byte) {
  const uint32_t sign = (byte & 0x80u) << 24;
  const uint32_t e = (byte >> 3) & 0xFu, m = byte & 0x7u;
  float mag;
  if (e == 0)
    mag = (float)m * 0.001953125f;  // m * 2^-9
  else
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));  // rebias 7 -> 127
  return __uint_as_float(__float_as_uint(mag) | sign);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Copies of one bf16 tile: slot q -> (row q/73, chunk q%73); chunk 72 pads.
// Every wave issues the same copies per tile except the last round (only wave 0).
__device__ inline void issue_bf16_tile(uint8_t* buf, const int64_t* offs, int64_t fallback,
                                       const uint8_t* kv, int tid) {
#pragma unroll
  for (int it = 0; it < kBf16Copies; ++it) {
    const int q = it * kThreads + tid;
    if (it < kBf16CopiesMin || q < kTileSlots) {
      const int row = q / kSlotsPerRow;
      const int ch = q - row * kSlotsPerRow;
      int64_t off = offs[row];
      if (off < 0) off = fallback;
      copy16_to_lds(kv + off + (ch < 72 ? ch * 16 : 0), buf + (it * kThreads + (tid & ~63)) * 16);
    }
  }
}

// Copies of one raw fp8 tile: 41 chunks of 16 B per 656-byte row, unpadded.
__device__ inline void issue_fp8_tile(uint8_t* buf, const int64_t* offs, int64_t fallback,
                                      const uint8_t* kv, int tid) {
#pragma unroll
  for (int it = 0; it < kFp8Copies; ++it) {
    const int q = it * kThreads + tid;
    if (it < kFp8CopiesMin || q < kFp8TileSlots) {
      const int row = q / kFp8Chunks;
      const int ch = q - row * kFp8Chunks;
      int64_t off = offs[row];
      if (off < 0) off = fallback;
      copy16_to_lds(kv + off + ch * 16, buf + (it * kThreads + (tid & ~63)) * 16);
    }
  }
}

// Raw fp8 tile -> bf16 compute tile (value = e4m3 * block scale, rounded to bf16).
__device__ inline void decode_fp8_tile(const uint8_t* raw, uint8_t* tile, int tid) {
  for (int c = tid; c < kTileRows * 40; c += kThreads) {
    const int r = c / 40, ch = c - r * 40;
    const uint8_t* rr = raw + r * 656;
    uint8_t* dst = tile + r * kRowLds;
    if (ch < 32) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(rr + ch * 16);
      const float sc = *reinterpret_cast<const float*>(rr + 512 + (ch >> 3) * 4);
      u32x4 lo, hi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = v[w];
        const uint32_t p0 = pack_bf16x2(e4m3_to_f32(x & 0xFFu) * sc, e4m3_to_f32((x >> 8) & 0xFFu) * sc);
        const uint32_t p1 = pack_bf16x2(e4m3_to_f32((x >> 16) & 0xFFu) * sc, e4m3_to_f32(x >> 24) * sc);
        if (w < 2) { lo[2 * w] = p0; lo[2 * w + 1] = p1; }
        else { hi[2 * w - 4] = p0; hi[2 * w - 3] = p1; }
      }
      *reinterpret_cast<u32x4*>(dst + ch * 32) = lo;
      *reinterpret_cast<u32x4*>(dst + ch * 32 + 16) = hi;
    } else {
      *reinterpret_cast<u32x4*>(dst + 1024 + (ch - 32) * 16) =
          *reinterpret_cast<const u32x4*>(rr + 528 + (ch - 32) * 16);
    }
  }
}

// Prologue: byte offsets of the range's rows (page table applied; -1 when not
// usable), padded with -1 to whole tiles.  Returns the first usable slot, or
// INT32_MAX when the range has none.  Ends with a barrier.
__device__ inline int build_offsets(int64_t* offs, int* first_valid, const int32_t* idx_row,
                                    int j_begin, int j_end, int n_pad, int pos, int b,
                                    const int32_t* page_table, int pt_stride, int page_size,
                                    int num_pages, int64_t page_stride, int64_t row_stride, int tid) {
  if (tid == 0) *first_valid = INT32_MAX;
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  for (int i = tid; i < n_pad; i += kThreads) {
    const int j = j_begin + i;
    int64_t off = -1;
    if (j < j_end) {
      const int s = idx_row[j];
      if (s >= 0 && s <= pos)
        off = token_offset(page_table, pt_stride, page_size, num_pages, b, s, page_stride, row_stride);
    }
    offs[i] = off;
    if (off >= 0) atomicMin(first_valid, i);
  }
  __syncthreads();
  return *first_valid;
}

struct MlaArgs {
  const int32_t* cu_q;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int B, pt_stride, page_size, num_pages;
  const uint16_t* q;
  const uint8_t* kv;
  int64_t page_stride, row_stride;
  const int32_t* idx;
  int K, H;
  float scale_log2;
  uint16_t* out;
  float* lse;
  float* ws;
  int splits, rows_per_split, nbuf;
};

// Online-softmax bookkeeping shared by both kernels.  `mt` is this lane's
// tile max for its head (already reduced over the lanes holding that head).
// Returns true when the wave must rescale O by `alpha`.
__device__ inline bool softmax_step(float mt, float& m_run, float& alpha) {
  const bool raise = mt > m_run + kRescaleSlack;
  alpha = 1.f;
  if (__any(raise)) {
    const float m_new = raise ? mt : m_run;
    alpha = (m_run == kNegInf) ? 0.f : exp2f(m_run - m_new);
    m_run = m_new;
    return true;
  }
  return false;
}

// ---------------------------------------------------------------- kernel

// DSPLIT = 4: a workgroup owns 16 heads; each wave computes the 32x16 score
// tile and a quarter (128) of the output columns.  DSPLIT = 1: a workgroup
// owns 64 heads, 16 per wave, each wave all 512 columns (1 wave per SIMD:
// 72 VGPRs of q plus a 128-register accumulator).  With several head groups
// per query, linear workgroup ids are laid out so that the groups of one query
// are 8 ids apart: they land on the same XCD at about the same time and the
// second gather of each tile is served by that XCD's L2.
template <int DSPLIT, bool FP8>
__global__ __launch_bounds__(kThreads) void sparse_mla_tiles(MlaArgs a, int n_groups, int T) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int kHeadsPerGroup = 64 / DSPLIT;
  constexpr int kCols = kDc / DSPLIT;          // output columns per wave
  constexpr int kColTiles = kCols / 16;
  const int x = blockIdx.x, sp = blockIdx.z;
  const int t = (x / (8 * n_groups)) * 8 + (x & 7);
  const int grp = (x >> 3) % n_groups;
  if (t >= T) return;                          // padding ids of the XCD-aware layout
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int head0 = grp * kHeadsPerGroup + (DSPLIT == 1 ? 16 * wave : 0);
  const int col0 = DSPLIT == 1 ? 0 : kCols * wave;
  const bool writes_stats = DSPLIT == 1 || wave == 0;
  const int j_begin = sp * a.rows_per_split;
  const int j_end = min(a.K, j_begin + a.rows_per_split);
  const int ntiles = (j_end - j_begin + kTileRows - 1) / kTileRows;
  const int b = find_request(a.cu_q, a.B, t);
  const int pos = row_position(a.cu_q, a.seq_lens, b, t);
  const int buf_bytes = FP8 ? kFp8TileLds : kTileLds;
  const int nbuf = a.nbuf;
  uint8_t* ctile = smem + nbuf * buf_bytes;  // fp8 decode target
  int64_t* offs = reinterpret_cast<int64_t*>(ctile + (FP8 ? kTileLds : 0));
  int* first_valid = reinterpret_cast<int*>(offs + ntiles * kTileRows);

  const int fv = build_offsets(offs, first_valid, a.idx + (int64_t)t * a.K, j_begin, j_end,
                               ntiles * kTileRows, pos, b, a.page_table, a.pt_stride, a.page_size,
                               a.num_pages, a.page_stride, a.row_stride, tid);

  f32x4 o[kColTiles];
#pragma unroll
  for (int i = 0; i < kColTiles; ++i) o[i] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;

  if (fv != INT32_MAX) {
    const int64_t fallback = offs[fv];
    // q as the B operand of S^T: lane (head c16, group g) holds dims 32 ks + 8 g .. +7.
    bf16x8 qreg[18];
    {
      const uint16_t* qp = a.q + ((int64_t)t * a.H + head0 + c16) * kD + g * 8;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
    }
    const int D = nbuf - 1;
    for (int i = 0; i < D && i < ntiles; ++i) {
      if (FP8) issue_fp8_tile(smem + i * buf_bytes, offs + i * kTileRows, fallback, a.kv, tid);
      else issue_bf16_tile(smem + i * buf_bytes, offs + i * kTileRows, fallback, a.kv, tid);
    }
#pragma unroll 1
    for (int i = 0; i < ntiles; ++i) {
      if (i + D < ntiles) {
        uint8_t* nb = smem + ((i + D) % nbuf) * buf_bytes;
        if (FP8) issue_fp8_tile(nb, offs + (i + D) * kTileRows, fallback, a.kv, tid);
        else issue_bf16_tile(nb, offs + (i + D) * kTileRows, fallback, a.kv, tid);
      }
      const int after = min(D, ntiles - 1 - i);
      if (FP8) wait_tiles_barrier<kFp8CopiesMin>(after);
      else wait_tiles_barrier<kBf16CopiesMin>(after);
      const uint8_t* tile = smem + (i % nbuf) * buf_bytes;
      if (FP8) {
        decode_fp8_tile(tile, ctile, tid);
        lds_barrier();
        tile = ctile;
      }
      const int64_t* toffs = offs + i * kTileRows;

      // S^T: accumulator r of lane = tile row nt*16 + 4g + r, head c16.
      f32x4 s0 = f32x4{}, s1 = f32x4{};
      const uint8_t* ap = tile + c16 * kRowLds + g * 16;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        s0 = mfma16(*reinterpret_cast<const bf16x8*>(ap + ks * 64), qreg[ks], s0);
        s1 = mfma16(*reinterpret_cast<const bf16x8*>(ap + 16 * kRowLds + ks * 64), qreg[ks], s1);
      }
      float xv[8];
      float mt = kNegInf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        xv[r] = toffs[4 * g + r] >= 0 ? s0[r] * a.scale_log2 : kNegInf;
        xv[4 + r] = toffs[16 + 4 * g + r] >= 0 ? s1[r] * a.scale_log2 : kNegInf;
        mt = fmaxf(mt, fmaxf(xv[r], xv[4 + r]));
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      float alpha;
      if (softmax_step(mt, m_run, alpha)) {
        l_run *= alpha;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(alpha, 4 * g + r);  // O row r holds head 4g + r
#pragma unroll
          for (int i2 = 0; i2 < kColTiles; ++i2) o[i2][r] *= ar;
        }
      }
      bf16x8 pa;
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) {
        const float p = xv[i2] == kNegInf ? 0.f : exp2f(xv[i2] - m_run);
        l_run += p;
        pa[i2] = (__bf16)p;
      }
      // O[:, col0 + 16 i .. +16] += P V.  k slot (g, e) <-> tile row 4g + e,
      // (g, 4 + e) <-> 16 + 4g + e, matching the S^T accumulator rows.
      const uint8_t* vp = tile + (4 * g + (c16 >> 2)) * kRowLds + (col0 + 4 * (c16 & 3)) * 2;
#pragma unroll
      for (int i2 = 0; i2 < kColTiles; ++i2) {
        const s16x4 v1 = lds_read_tr16(vp + i2 * 32);
        const s16x4 v2 = lds_read_tr16(vp + 16 * kRowLds + i2 * 32);
        o[i2] = mfma16(pa, join(v1, v2), o[i2]);
        if ((i2 & 7) == 7) __builtin_amdgcn_sched_barrier(0);  // bound operand prefetch
      }
      lds_barrier();
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  // O accumulator r of lane: head 4g + r, column col0 + 16 i + c16.
  if (a.splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g + r;
      const float lh = __shfl(l_run, h);
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      uint16_t* op = a.out + ((int64_t)t * a.H + head0 + h) * kDc + col0 + c16;
#pragma unroll
      for (int i2 = 0; i2 < kColTiles; ++i2)
        op[16 * i2] = __builtin_bit_cast(uint16_t, (__bf16)(o[i2][r] * inv));
    }
    if (a.lse != nullptr && writes_stats && lane < 16)
      a.lse[(int64_t)t * a.H + head0 + lane] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : kNegInf;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g + r;
      float* wp = a.ws + (((int64_t)t * a.H + head0 + h) * a.splits + sp) * 516 + col0 + c16;
#pragma unroll
      for (int i2 = 0; i2 < kColTiles; ++i2) wp[16 * i2] = o[i2][r];
    }
    if (writes_stats && lane < 16) {
      float* wp = a.ws + (((int64_t)t * a.H + head0 + lane) * a.splits + sp) * 516 + 512;
      wp[0] = m_run;
      wp[1] = l_run;
    }
  }
}

// Merge per-split partials: one wave per (row, head); lane covers 8 columns.
__global__ __launch_bounds__(kWave) void sparse_mla_combine(const float* __restrict__ ws, int H,
                                                            int splits, uint16_t* __restrict__ out,
                                                            float* __restrict__ lse) {
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const float* base = ws + ((int64_t)t * H + h) * splits * 516;
  float M = kNegInf;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, base[s * 516 + 512]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < splits; ++s) {
      const float* p = base + s * 516;
      const float wgt = exp2f(p[512] - M);  // an empty split has m = -inf, weight 0
      L += wgt * p[513];
      const f32x4 a = *reinterpret_cast<const f32x4*>(p + lane * 8);
      const f32x4 c = *reinterpret_cast<const f32x4*>(p + lane * 8 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += wgt * a[i];
        acc[4 + i] += wgt * c[i];
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  u32x4 pk;
#pragma unroll
  for (int c = 0; c < 4; ++c) pk[c] = pack_bf16x2(acc[2 * c] * inv, acc[2 * c + 1] * inv);
  *reinterpret_cast<u32x4*>(out + ((int64_t)t * H + h) * kDc + lane * 8) = pk;
  if (lse != nullptr && lane == 0)
    lse[(int64_t)t * H + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
}

// f32 path on the vector ALUs: one wave per (row, head), up to 4096 selected
// rows and 1024 dims; two passes (logits, then the weighted sum).
constexpr int kF32MaxK = 4096;
constexpr int kF32MaxD = 1024;

__global__ __launch_bounds__(kWave) void sparse_mla_f32_valu(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, int B, int pt_stride, int page_size, int num_pages,
    const float* __restrict__ q, const uint8_t* __restrict__ kv_base, int64_t kv_page_stride,
    int64_t kv_row_stride, const int32_t* __restrict__ idx, int K, int H, int Dc, int Dr,
    float scale, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float qs[kF32MaxD];
  __shared__ float logit[kF32MaxK];
  __shared__ int64_t offs[kF32MaxK];
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int D = Dc + Dr;
  const int b = find_request(cu_q, B, t);
  const int pos = row_position(cu_q, seq_lens, b, t);
  for (int d = lane; d < D; d += kWave) qs[d] = q[((int64_t)t * H + h) * D + d];
  __syncthreads();
  float m = kNegInf;
  for (int j = lane; j < K; j += kWave) {
    const int s = idx[(int64_t)t * K + j];
    int64_t off = -1;
    if (s >= 0 && s <= pos)
      off = token_offset(page_table, pt_stride, page_size, num_pages, b, s, kv_page_stride, kv_row_stride);
    offs[j] = off;
    float l = kNegInf;
    if (off >= 0) {
      const float* row = reinterpret_cast<const float*>(kv_base + off);
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], row[d], dot);
      l = dot * scale;
    }
    logit[j] = l;
    m = fmaxf(m, l);
  }
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  __syncthreads();
  float sum = 0.f;
  if (m != kNegInf)
    for (int j = lane; j < K; j += kWave) sum += offs[j] >= 0 ? expf(logit[j] - m) : 0.f;
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  for (int d = lane; d < Dc; d += kWave) {
    float acc = 0.f;
    if (m != kNegInf)
      for (int j = 0; j < K; ++j) {
        const int64_t off = offs[j];
        if (off >= 0) acc = fmaf(expf(logit[j] - m), reinterpret_cast<const float*>(kv_base + off)[d], acc);
      }
    out[((int64_t)t * H + h) * Dc + d] = acc * inv;
  }
  if (lse != nullptr && lane == 0) lse[(int64_t)t * H + h] = sum > 0.f ? m + logf(sum) : kNegInf;
}

}  // namespace

MlaPlan plan_sparse_mla(int num_q_rows, int n_heads, int k, int dc, bool prefill) {
  MlaPlan p{1, k, 0};
  if (dc != kDc || n_heads % 16 != 0 || k <= 0 || num_q_rows <= 0) return p;
  const bool wide = n_heads % 64 == 0;
  const int64_t blocks = (int64_t)num_q_rows * (wide ? n_heads / 64 : n_heads / 16);
  int splits = 1;
  if (!prefill) {
    const int64_t target = wide ? 384 : 512;
    const int max_splits = k / 256 > 1 ? k / 256 : 1;
    const int64_t want = (target + blocks - 1) / blocks;
    splits = (int)(want < 1 ? 1 : (want > max_splits ? max_splits : want));
  }
  int rps = (k + splits - 1) / splits;
  rps = (rps + kTileRows - 1) / kTileRows * kTileRows;
  splits = (k + rps - 1) / rps;
  p.splits = splits;
  p.rows_per_split = rps;
  p.ws_bytes = splits > 1 ? (size_t)num_q_rows * n_heads * splits * 516 * sizeof(float) : 0;
  return p;
}

namespace {

constexpr size_t kMaxLds = 160 * 1024;

// LDS bytes of a launch with `nbuf` ring buffers.
size_t mla_lds(bool wide, bool fp8, int nbuf, int rps) {
  const size_t buf = fp8 ? kFp8TileLds : kTileLds;
  (void)wide;
  return nbuf * buf + (fp8 ? kTileLds : 0) +
         (size_t)(rps + kTileRows - 1) / kTileRows * kTileRows * 8 + 16;
}

template <typename Kernel>
hipError_t launch_with_lds(Kernel kernel, dim3 grid, size_t lds, hipStream_t stream, const MlaArgs& args,
                           int n_groups, int T) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), lds, stream, args, n_groups, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla_bf16(const BatchArgs& ba, const void* q, const PoolArgs& kv,
                                  const int32_t* idx, int k, int n_heads, float sm_scale,
                                  void* out, float* lse, void* ws, const MlaPlan& plan,
                                  hipStream_t stream) {
  const bool wide = n_heads % 64 == 0;
  const bool fp8 = kv.format == 2;
  int nbuf = 4;
  while (nbuf > 2 && mla_lds(wide, fp8, nbuf, plan.rows_per_split) > kMaxLds) --nbuf;
  const size_t lds = mla_lds(wide, fp8, nbuf, plan.rows_per_split);
  if (lds > kMaxLds) return hipErrorInvalidValue;
  MlaArgs args{ba.cu_q, ba.seq_lens, ba.page_table, ba.batch, ba.pt_stride, ba.page_size,
               ba.num_pages, static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(kv.base),
               kv.page_stride, kv.row_stride, idx, k, n_heads, sm_scale * kLog2e,
               static_cast<uint16_t*>(out), lse, static_cast<float*>(ws), plan.splits,
               plan.rows_per_split, nbuf};
  const int T = ba.num_q_rows;
  const int n_groups = wide ? n_heads / 64 : n_heads / 16;
  const dim3 grid((unsigned)((T + 7) / 8 * 8 * n_groups), 1, plan.splits);
  hipError_t e;
  if (wide)
    e = fp8 ? launch_with_lds(sparse_mla_tiles<1, true>, grid, lds, stream, args, n_groups, T)
            : launch_with_lds(sparse_mla_tiles<1, false>, grid, lds, stream, args, n_groups, T);
  else
    e = fp8 ? launch_with_lds(sparse_mla_tiles<4, true>, grid, lds, stream, args, n_groups, T)
            : launch_with_lds(sparse_mla_tiles<4, false>, grid, lds, stream, args, n_groups, T);
  if (e != hipSuccess || plan.splits == 1) return e;
  hipLaunchKernelGGL(sparse_mla_combine, dim3(ba.num_q_rows, n_heads), dim3(kWave), 0, stream,
                     static_cast<const float*>(ws), n_heads, plan.splits,
                     static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

hipError_t launch_sparse_mla_f32(const BatchArgs& ba, const void* q, const PoolArgs& kv,
                                 const int32_t* idx, int k, int n_heads, int dc, int dr,
                                 float sm_scale, void* out, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(sparse_mla_f32_valu, dim3(ba.num_q_rows, n_heads), dim3(kWave), 0, stream,
                     ba.cu_q, ba.seq_lens, ba.page_table, ba.batch, ba.pt_stride, ba.page_size,
                     ba.num_pages, static_cast<const float*>(q), static_cast<const uint8_t*>(kv.base),
                     kv.page_stride, kv.row_stride, idx, k, n_heads, dc, dr, sm_scale,
                     static_cast<float*>(out), lse);
  return hipGetLastError();
}

}  // namespace dsa
