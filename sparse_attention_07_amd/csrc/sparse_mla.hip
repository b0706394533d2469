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
// The kernel runs four waves per workgroup on one query row and one range of
// its selected rows:
//
// * Gather.  A prologue turns the range's indices into byte offsets (page
//   table applied, unusable entries marked -1) and a usable-row bitmask per
//   32-row tile, in LDS.  Each tile is loaded with plain 16-byte global loads
//   into registers (9 per thread for bf16 rows; 5 for fp8 rows, which are
//   decoded to bf16 as e4m3 * block scale on the way), one to three tiles ahead
//   of the tile being computed, and written to a single LDS tile whose rows
//   are padded to 1168 B (16 lanes reading 16 rows at one column then hit 16
//   distinct bank groups).  Measured on MI355X, random 1152-byte row gathers
//   this way run at the rate of a sequential read (about 6 TB/s), while
//   global_load_lds copies of the same rows reached only 2-3.4 TB/s.
// * QK^T.  S^T = rows x q^T on MFMA with the rows as the A operand read from
//   LDS (kept four k steps ahead of their MFMAs) and q held in registers as
//   the B operand for the whole range.
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
// Both variants use v_mfma_f32_16x16x32_bf16 with 16 heads per wave.  For
// 16-head workloads every wave computes the (cheap) 32x16 score tile and then
// its own quarter of the 512 output columns, so one query's work spreads over
// four SIMDs.  For 64+ heads a workgroup owns 64 heads, 16 per wave, each wave
// all 512 columns (one wave per SIMD: 72 VGPRs of q, a 128-register
// accumulator).  (32 heads per wave would halve the LDS operand traffic, but
// 144 VGPRs of q next to a 256-register accumulator do not fit and q ends up
// spilled.)
//
// When the selected rows of a query are split across workgroups, each writes
// (m, l, unnormalised O) partials; the last split of a (query, head group) to
// finish, found with an arrival counter, merges them by log-sum-exp in the
// same launch.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kD = kDc + kDr;
constexpr int kThreads = 256;                          // four waves
constexpr int kTileRows = 32;
constexpr int kRowLds = 73 * 16;                       // 1152 B of row + one 16-byte pad
constexpr int kTileLds = kTileRows * kRowLds;          // 37376 B
constexpr int kSbufLds = kThreads * 16;                // one f32x4 of partial scores per thread
constexpr int kQ8TabLds = 2 * 4 * 4 * 16 * 4;           // 8-bit rows: block scales and biases, [wave][block][16 rows]
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.f;                   // log2 units

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// All of this wave's LDS accesses are done, then barrier.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ inline bf16x8 lds16(const uint8_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ inline s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

__device__ inline bf16x8 join(s16x4 a, s16x4 b) {
  const s16x8 w = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Four e4m3 bytes (one dword, byte 0 first) -> four bf16 of e4m3 * sc.  The
// hardware conversion to f32 at scale 1 is exact (its scale operand only
// takes a power of two), then the block scale is applied in f32 and the
// product rounded to bf16 once: two conversions, four multiplies and two
// packs per four codes.
__device__ inline uint2 fp8x4_to_bf16x4(uint32_t x, float sc) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.0f, false);  // bytes 0, 1
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.0f, true);   // bytes 2, 3
  return uint2{pack_bf16x2(a[0] * sc, a[1] * sc), pack_bf16x2(b[0] * sc, b[1] * sc)};
}

// Four unsigned 8-bit codes (one dword, byte 0 first) -> four bf16 of
// sc * code + bi, each computed with one f32 fma and rounded to bf16 once.
__device__ inline uint2 u8x4_to_bf16x4(uint32_t x, float sc, float bi) {
  const float v0 = fmaf((float)(x & 0xFFu), sc, bi), v1 = fmaf((float)((x >> 8) & 0xFFu), sc, bi);
  const float v2 = fmaf((float)((x >> 16) & 0xFFu), sc, bi), v3 = fmaf((float)(x >> 24), sc, bi);
  return uint2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
}

// Latent cache formats of the MFMA kernels: bf16 rows (1152 B), fp8 rows
// (656 B: 512 e4m3 codes, 4 block scales, bf16 rope) and affine int8 rows
// (672 B: 512 unsigned codes, 4 block scales, 4 block biases, bf16 rope).
// Both 8-bit forms keep one scale (and bias) per 128 latent dims.
constexpr int kFmtBf16 = 0, kFmtFp8 = 1, kFmtInt8 = 2;
template <int F>
constexpr bool kQ8 = F != kFmtBf16;  // 8-bit latent codes
template <int F>
constexpr int kRopeOff = F == kFmtBf16 ? 1024 : (F == kFmtFp8 ? 528 : 544);

// Four latent codes of 8-bit format F -> four bf16.
template <int F>
__device__ inline uint2 decode4(uint32_t x, float sc, float bi) {
  if (F == kFmtFp8) return fp8x4_to_bf16x4(x, sc);
  return u8x4_to_bf16x4(x, sc, bi);
}

// One tile's latent rows in flight in the registers of the 64-head kernel's
// two gather waves (128 threads, gt = thread - 256): bf16 rows -- latent
// chunk gt % 64 (16 B) of rows gt / 64 + 2k, k < 16; 8-bit rows -- latent
// chunk gt % 32 (16 codes, with its block scale and bias) of rows gt / 32 +
// 4k, k < 8.  Each load of a wave reads 1 KB of one row (bf16) or 512 B of
// each of two rows (8-bit).  The rope of a tile is gathered by the value
// waves (one 16-byte chunk per thread).
constexpr int kGatherThreads = 128;

template <int F>
struct Stage {
  static constexpr int kLat = kQ8<F> ? 8 : 16;   // latent items
  static constexpr int kStep = kQ8<F> ? 4 : 2;   // row step between items
  u32x4 lat[kLat];
  float sc[kQ8<F> ? kLat : 1];
  float bi[F == kFmtInt8 ? kLat : 1];
};

__device__ inline u32x4 ld_global16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Registers of a stage into one LDS tile buffer (row-major rows of
// kRowLds bytes: latent as bf16 at bytes 0..1023, rope at 1024..1151);
// 8-bit codes are decoded here.
template <int F>
__device__ inline void stage_store(const Stage<F>& st, uint8_t* tile, int gt) {
  constexpr bool Q8 = kQ8<F>;
  constexpr int kLat = Stage<F>::kLat, kStep = Stage<F>::kStep;
  const int ch = Q8 ? (gt & 31) : (gt & 63);
  const int r0 = Q8 ? (gt >> 5) : (gt >> 6);
#pragma unroll
  for (int k = 0; k < kLat; ++k) {
    uint8_t* dst = tile + (r0 + kStep * k) * kRowLds;
    if (!Q8) {
      *reinterpret_cast<u32x4*>(dst + ch * 16) = st.lat[k];
    } else {
      u32x4 lo, hi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint2 pr = decode4<F>(st.lat[k][w], st.sc[k], F == kFmtInt8 ? st.bi[k] : 0.f);
        if (w < 2) { lo[2 * w] = pr.x; lo[2 * w + 1] = pr.y; }
        else { hi[2 * w - 4] = pr.x; hi[2 * w - 3] = pr.y; }
      }
      *reinterpret_cast<u32x4*>(dst + ch * 32) = lo;
      *reinterpret_cast<u32x4*>(dst + ch * 32 + 16) = hi;
    }
  }
}

// Prologue: byte offsets of the range's rows (page table applied; -1 when not
// usable), padded with -1 to whole tiles, and a usable-row bitmask per tile.
// Each thread handles rows tid, tid+NT, ...; the index loads of a batch of
// eight rows are all issued before the dependent page-table loads, so the
// prologue costs two memory latencies per 2048 rows rather than two per row.
// Returns the first usable slot, or INT32_MAX when the range has none.  Ends
// with a barrier.
constexpr int kIdxBatch = 8;

// The first batch of a range's indices (thread tid: entries tid + NT k).
// They depend only on the row, so they are loaded before the row's request
// and position are known.
template <int NT = kThreads>
__device__ inline void preload_indices(int (&sv)[kIdxBatch], const int32_t* idx_row, int j_begin,
                                       int j_end, int n_pad, int tid) {
#pragma unroll
  for (int k = 0; k < kIdxBatch; ++k) {
    const int i = k * NT + tid;
    const int j = j_begin + i;
    sv[k] = (i < n_pad && j < j_end) ? idx_row[j] : -1;
  }
}

// Per-wave slots after the tile masks in LDS: the waves' first usable slots,
// then one flag the split merge uses.
constexpr int kWaveSlots = 8;

template <int NT = kThreads>
__device__ inline int build_offsets(int64_t* offs, uint32_t* vmask, int* wmin,
                                    const int (&sv0)[kIdxBatch], const int32_t* idx_row,
                                    int j_begin, int j_end, int n_pad, int pos, int b,
                                    const int32_t* page_table, int pt_stride, int page_size,
                                    int num_pages, int64_t page_stride, int64_t row_stride, int tid) {
  constexpr int kBatch = kIdxBatch, kW = NT / kWave;
  static_assert(kW <= kWaveSlots, "one LDS slot per wave");
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  // The first usable slot of this wave's rows (rows grow with k and base, so
  // the first non-empty ballot holds it).  Masks and minima come from ballots:
  // LDS atomics from every row to one word serialised for microseconds.
  int my_first = INT32_MAX;
  for (int base = 0; base < n_pad; base += kBatch * NT) {
    int sv[kBatch], pg[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = base + k * NT + tid;
      const int j = j_begin + i;
      sv[k] = base == 0 ? sv0[k] : ((i < n_pad && j < j_end) ? idx_row[j] : -1);
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int sk = sv[k];
      const bool ok = sk >= 0 && sk <= pos && sk / page_size < pt_stride;
      pg[k] = ok ? page_table[(int64_t)b * pt_stride + sk / page_size] : -1;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = base + k * NT + tid;
      int64_t off = -1;
      if (i < n_pad && pg[k] >= 0 && pg[k] < num_pages)
        off = (int64_t)pg[k] * page_stride + (int64_t)(sv[k] % page_size) * row_stride;
      if (i < n_pad) offs[i] = off;
      // this wave's 64 rows start at a multiple of 64: tiles r0/32 and r0/32 + 1
      const uint64_t m = __ballot(off >= 0);
      const int r0 = base + k * NT + kWave * wave;
      if (lane == 0 && r0 < n_pad) {  // n_pad is a multiple of 32: whole tiles
        vmask[r0 / kTileRows] = (uint32_t)m;
        if (r0 + kTileRows < n_pad) vmask[r0 / kTileRows + 1] = (uint32_t)(m >> 32);
      }
      if (m != 0 && my_first == INT32_MAX) my_first = r0 + __ffsll((unsigned long long)m) - 1;
    }
  }
  if (lane == 0) wmin[wave] = my_first;
  __syncthreads();
  int fv = INT32_MAX;
#pragma unroll
  for (int w = 0; w < kW; ++w) fv = min(fv, wmin[w]);
  return fv;
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
  float* ws;       // split partials: [T, head groups, splits] blocks of kPartBytes(heads per group)
  int* counters;   // [T * head groups] arrivals per row and head group (< kMlaCounterSlots)
  int splits, rows_per_split;
};

// Reductions over the four lane groups (lanes l, l^16, l^32, l^48) that hold
// one head's scores: a permlane swap exchanges row pairs of a wave in one
// VALU instruction, and each lane ends up with its own and its partner's
// value in a fixed order (same result in both lanes of a pair).
__device__ inline float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline float sum_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x on the hardware exponential (v_exp_f32); results below the normal
// range flush to zero, which no softmax weight here can notice.
__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Online softmax of one 32-row tile for 16 heads, in log2 units.  s0 / s1:
// S^T accumulators (lane (g, c16): rows 4g+r and 16+4g+r, head c16);
// valid: usable-row bits of the tile.  The running max is raised (and O and
// l rescaled) only when the tile beats it by more than kRescaleSlack.
// Returns P as the PV A operand (k slot (g, e) <-> row 4g + e, (g, 4 + e) <->
// row 16 + 4g + e).  O accumulator r of lane (g, c16) holds head 4g + r.
// SCALED (8-bit rows, block scale deferred to P): P is multiplied by the k
// slot's row scale psc before it is rounded to bf16, and with BIAS (affine
// int8) bacc += p * the slot's row bias, rescaled with O; l takes p itself.
template <int TILES, bool SCALED = false, bool BIAS = false>
__device__ inline bf16x8 tile_softmax(const f32x4& s0, const f32x4& s1, uint32_t valid, float scale_log2,
                                      float& m_run, float& l_run, f32x4 (&o)[TILES],
                                      const float* psc = nullptr, const float* pbi = nullptr,
                                      float* bacc = nullptr) {
  const int lane = threadIdx.x & (kWave - 1), g = lane >> 4;
  float xv[8];
  if (valid == 0xFFFFFFFFu) {  // wave-uniform: every row usable
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      xv[r] = s0[r] * scale_log2;
      xv[4 + r] = s1[r] * scale_log2;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      xv[r] = (valid >> (4 * g + r)) & 1u ? s0[r] * scale_log2 : kNegInf;
      xv[4 + r] = (valid >> (16 + 4 * g + r)) & 1u ? s1[r] * scale_log2 : kNegInf;
    }
  }
  float mt = fmaxf(fmaxf(fmaxf(xv[0], xv[1]), fmaxf(xv[2], xv[3])),
                   fmaxf(fmaxf(xv[4], xv[5]), fmaxf(xv[6], xv[7])));
  mt = max_over_groups(mt);
  const bool raise = mt > m_run + kRescaleSlack;
  if (__any(raise)) {
    const float m_new = raise ? mt : m_run;
    const float alpha = (m_run == kNegInf) ? 0.f : exp2_fast(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    if (BIAS) *bacc *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * g + r);  // O row r holds head 4g + r
#pragma unroll
      for (int i2 = 0; i2 < TILES; ++i2) o[i2][r] *= ar;
    }
  }
  bf16x8 pa;
  if (valid == 0xFFFFFFFFu) {  // finite scores, finite running max
#pragma unroll
    for (int i2 = 0; i2 < 8; ++i2) {
      const float p = exp2_fast(xv[i2] - m_run);
      l_run += p;
      if (BIAS) *bacc = fmaf(p, pbi[i2], *bacc);
      pa[i2] = (__bf16)(SCALED ? p * psc[i2] : p);
    }
  } else {
#pragma unroll
    for (int i2 = 0; i2 < 8; ++i2) {
      const float p = xv[i2] == kNegInf ? 0.f : exp2_fast(xv[i2] - m_run);
      l_run += p;
      if (BIAS) *bacc = fmaf(p, pbi[i2], *bacc);
      pa[i2] = (__bf16)(SCALED ? p * psc[i2] : p);
    }
  }
  return pa;
}

// Split partials are exchanged between workgroups with device-scope (sc1)
// buffer stores and loads, the cache policy the compiler gives relaxed
// agent-scope atomics on gfx950: they are performed at the device coherence
// point, past the per-XCD L2, so the only ordering needed is that a
// workgroup's partial stores are complete before its arrival is counted.  (A
// device-scope fence would also do, but its release writes back the XCD's
// whole L2, and hundreds of workgroups doing that serialise.)  Buffer
// intrinsics keep the accesses visible to the compiler's wait counting, and
// the descriptor's size bounds them.
constexpr int kSc1 = 16;                     // cache policy: device scope
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw buffer descriptor flags

__device__ inline __amdgpu_buffer_rsrc_t raw_buffer(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, kRawBufferWord3);
}

// Partials of one (row, head group, split), kPartBytes(nh) bytes: O / l as
// bf16, exactly as the waves hold it -- [wave][16-column tile][lane] x 4 heads
// (the heads 4g..4g+3 of lane group g at one column), so each store
// instruction writes 512 B contiguous -- then (m, l) per head as f32.
// Normalised partials are bounded by the values attended, so bf16 keeps them
// within the output's own rounding.
__host__ __device__ constexpr int kPartBytes(int nh) { return nh * (kDc * 2 + 8); }

// Descriptor over the partials of every split of (row t, head group grp).
__device__ inline __amdgpu_buffer_rsrc_t split_blocks(const MlaArgs& a, int t, int grp, int n_groups, int nh) {
  uint8_t* p = reinterpret_cast<uint8_t*>(a.ws) + ((int64_t)t * n_groups + grp) * a.splits * (int64_t)kPartBytes(nh);
  return raw_buffer(p, a.splits * kPartBytes(nh));
}

// A split's partials: O / l of this lane's four heads (4g..4g+3) at its
// columns as bf16 (layout tiles slot0 .. slot0+TILES-1), and when
// stat_h0 >= 0 (one wave per 16 heads) the (m, l) of heads stat_h0 + lane for
// lanes < 16.  l_run is already the full sum.
template <int NH, int TILES>
__device__ inline void store_partials(const MlaArgs& a, int t, int grp, int n_groups, int sp, int slot0,
                                      int lane, const f32x4 (&o)[TILES], float m_run, float l_run,
                                      int stat_h0) {
  const __amdgpu_buffer_rsrc_t rs = split_blocks(a, t, grp, n_groups, NH);
  const int base = sp * kPartBytes(NH);
  const int g = lane >> 4;
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lh = __shfl(l_run, 4 * g + r);  // lane h holds head h's l
    inv[r] = lh > 0.f ? __builtin_amdgcn_rcpf(lh) : 0.f;
  }
#pragma unroll
  for (int i2 = 0; i2 < TILES; ++i2) {
    uint2 pk;
    pk.x = pack_bf16x2(o[i2][0] * inv[0], o[i2][1] * inv[1]);
    pk.y = pack_bf16x2(o[i2][2] * inv[2], o[i2][3] * inv[3]);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(2 * sizeof(int)))) int, pk), rs,
                                          base + ((slot0 + i2) * 64 + lane) * 8, 0, kSc1);
  }
  if (stat_h0 >= 0 && lane < 16) {
    uint2 ml;
    ml.x = __float_as_uint(m_run);
    ml.y = __float_as_uint(l_run);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(2 * sizeof(int)))) int, ml), rs,
                                          base + NH * kDc * 2 + 8 * (stat_h0 + lane), 0, kSc1);
  }
}

// Called by every thread of a workgroup after it stored its split's block.
// The last of the (row, head group)'s splits to arrive, found with an arrival
// counter, merges all splits by log-sum-exp into out/lse and resets the
// counter to zero, so no separate merge launch is needed and the counters are
// left as they were found.  WIDE: 64 heads, each wave 16 heads x 512 columns;
// else 16 heads, each wave 16 heads x 128 columns.  `wgt` is LDS space for
// 2 * nh * splits floats (the tile buffer, free by now); `is_last` one LDS int.
template <bool WIDE, int NT = kThreads>
__device__ inline void merge_splits_if_last(const MlaArgs& a, int t, int grp, int n_groups,
                                            int* counter, float* wgt, int* is_last, int tid) {
  constexpr int kThreads = NT;
  constexpr int kNh = WIDE ? 64 : 16;
  constexpr int kTiles = WIDE ? 32 : 8;  // 16-column tiles per wave
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores are done
  __syncthreads();                                    // ... and every other thread's
  if (tid == 0)
    *is_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               a.splits - 1;
  __syncthreads();
  if (!*is_last) return;
  const int S = a.splits, h0 = grp * kNh;
  const __amdgpu_buffer_rsrc_t rs = split_blocks(a, t, grp, n_groups, kNh);
  constexpr int kStride = kPartBytes(kNh);
  // The statistics are loaded first and the first round of O loads right
  // after them, so the weights are computed while O is in flight.
  // 16-byte chunks of O per split; 1024 of them per load round
  constexpr int kIt = 1024 / NT, kSp = 8, kChunks = kNh * kDc * 2 / 16;
  u32x4 v[kIt][kSp];
  auto issue = [&](int c0, int s0) {
#pragma unroll
    for (int u = 0; u < kIt; ++u)
#pragma unroll
      for (int s = 0; s < kSp; ++s)
        if (s0 + s < S)
          v[u][s] = __builtin_amdgcn_raw_buffer_load_b128(rs, (s0 + s) * kStride + (c0 + u * kThreads) * 16, 0, kSc1);
  };
  float* ls = wgt + kNh * S;
  constexpr int kStatIt = (kNh * 64 + kThreads - 1) / kThreads;  // S <= 64
  uint2 ml[kStatIt];
#pragma unroll
  for (int k = 0; k < kStatIt; ++k) {  // i = h * S + s
    const int i = tid + k * kThreads;
    ml[k] = i < kNh * S ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                        rs, (i % S) * kStride + kNh * kDc * 2 + 8 * (i / S), 0, kSc1))
                        : uint2{0u, 0u};
  }
  issue(tid, 0);
#pragma unroll
  for (int k = 0; k < kStatIt; ++k) {
    const int i = tid + k * kThreads;
    if (i < kNh * S) {
      wgt[i] = __uint_as_float(ml[k].x);
      ls[i] = __uint_as_float(ml[k].y);
    }
  }
  __syncthreads();
  // Merge weight of (head h, split s): l_s exp2(m_s - M) / L, one thread per pair.
  float wnew[(kNh * 64 + kThreads - 1) / kThreads];
#pragma unroll
  for (int k = 0; k < (kNh * 64 + kThreads - 1) / kThreads; ++k) {
    const int i = tid + k * kThreads, h = i / S;
    wnew[k] = 0.f;
    if (i < kNh * S) {
      const float* mh = wgt + h * S;
      const float* lh = ls + h * S;
      float M = kNegInf;
      for (int s = 0; s < S; ++s) M = fmaxf(M, mh[s]);
      float L = 0.f;
      if (M != kNegInf)
        for (int s = 0; s < S; ++s) L += exp2_fast(mh[s] - M) * lh[s];  // empty split: 0
      const float ms = mh[i % S];
      wnew[k] = L > 0.f ? exp2_fast(ms - M) * lh[i % S] / L : 0.f;
      if (i % S == 0 && a.lse != nullptr)
        a.lse[(int64_t)t * a.H + h0 + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < (kNh * 64 + kThreads - 1) / kThreads; ++k)
    if (tid + k * kThreads < kNh * S) wgt[tid + k * kThreads] = wnew[k];
  __syncthreads();
  // Chunk c holds lanes 2m, 2m+1 (m = c % 32) of tile (c / 32) % kTiles of
  // wave c / (32 kTiles): heads hb..hb+3 at columns col, col+1.  A thread's
  // chunks c0 + NT u (u < kIt) share m and, as NT kIt is 1024 = 32 kTiles
  // (wide) or the heads do not depend on the wave, also hb: the weights of
  // the thread's heads are read once per round.
  static_assert(!WIDE || kThreads * kIt == 32 * kTiles, "one wave slot per round");
  for (int c0 = tid; c0 < kChunks; c0 += kThreads * kIt) {
    float acc[kIt][8];
#pragma unroll
    for (int u = 0; u < kIt; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;
    const int hb = (WIDE ? 16 * (c0 / (32 * kTiles)) : 0) + 4 * ((2 * (c0 & 31)) >> 4);
    for (int s0 = 0; s0 < S; s0 += kSp) {
      if (c0 != tid || s0 != 0) issue(c0, s0);
      float wt[4][kSp];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < kSp; ++s) wt[r][s] = s0 + s < S ? wgt[(hb + r) * S + s0 + s] : 0.f;
#pragma unroll
      for (int u = 0; u < kIt; ++u) {
#pragma unroll
        for (int s = 0; s < kSp; ++s) {
          if (s0 + s < S) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t x = v[u][s][e];
              acc[u][2 * e] += wt[(2 * e) % 4][s] * __uint_as_float(x << 16);
              acc[u][2 * e + 1] += wt[(2 * e + 1) % 4][s] * __uint_as_float(x & 0xFFFF0000u);
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kIt; ++u) {
      const int c = c0 + u * kThreads, lane = 2 * (c & 31), w = c / (32 * kTiles), i2 = (c / 32) % kTiles;
      const int hb = (WIDE ? 16 * w : 0) + 4 * (lane >> 4);
      const int col = (WIDE ? 0 : 128 * w) + 16 * i2 + (lane & 15);
      // acc[u][e]: e < 4 -> head hb + e at col, e >= 4 -> head hb + e - 4 at col + 1
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<uint32_t*>(a.out + ((int64_t)t * a.H + h0 + hb + r) * kDc + col) =
            pack_bf16x2(acc[u][r], acc[u][4 + r]);
    }
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- 64 heads, 8 waves

// A workgroup owns 64 heads of one query row and one range of its selected
// rows, with eight waves in three roles.  Waves w and w + 4 share a SIMD
// (waves 0..3 sit on four distinct SIMDs), so the roles are placed to give
// every SIMD about the same MFMA time per 32-row tile:
// * score waves 0, 1 (head block g = w, 32 heads): S^T = K Q^T for all 32
//   tile rows on v_mfma_f32_32x32x16_bf16 over the 576 dims (36 MFMAs), q
//   held as the B operand (144 VGPRs).  Each lane then holds 16 of the 32
//   rows of one head, so the tile maximum needs one permlane swap and no
//   LDS exchange; the wave takes the online-softmax step for its heads and
//   writes P (bf16) and the rescale factors into LDS.
// * value waves 2, 3, 6, 7 (column quarter cq): O += P V for all 64 heads
//   and 128 columns (16 MFMAs, 128 accumulator registers), V read once per
//   tile with ds_read_b64_tr_b16.
// * gather waves 4, 5: the tiles' latent gathers, three tiles in flight in
//   registers (one stage per tile), stored into the LDS tile buffers; the
//   value waves gather the rope (16 B per thread per tile) the same way.
// Per phase i (each ends with a barrier): score waves QK + softmax of tile
// i+1; value waves PV of tile i; gather and value waves store tile i+2
// (waiting for exactly its loads) and issue the gathers of tile i+5.  Tile j lives in LDS
// buffer j % 3 and register stage j % 3; P and rescale factors of tile j in
// slot j % 2.  The gathers are branch-free (an unusable row loads the pool's
// first row, and the tile's unusable rows are zeroed in LDS when it is stored).
//
// The output (O / l, bf16) is staged in LDS as [head][column] and written
// with 16-byte stores: to `out` when the rows are not split, else to the
// split's partial block, which the last split to finish merges.
constexpr int kH64Threads = 512;
constexpr int kH64Bufs = 3;                          // LDS tile buffers
constexpr int kH64Stages = 3;                        // register stages of the gather waves
constexpr int kH64Pslot = 64 * 32 * 2;               // P of one tile: [row half][k step][64 heads][8] bf16
constexpr int kH64Aslot = 64 * 4 + 16;               // rescale factors [64 heads], then 2 flags
constexpr int kH64Stats = 64 * 12;                   // per head: m, l, 0
constexpr int kH64Fixed = kH64Bufs * kTileLds + 2 * kH64Pslot + 2 * kH64Aslot + kH64Stats;
static_assert(kH64Fixed % 16 == 0 && kH64Aslot % 16 == 0 && kH64Pslot % 16 == 0, "16-byte aligned regions");
static_assert(kH64Bufs * kTileLds >= 64 * kDc * 2, "the output staging fits the tile buffers");

// Loads per gather thread per stage (they are all issued together).
template <int F>
constexpr int kStageLoads = F == kFmtBf16 ? 16 : (F == kFmtFp8 ? 16 : 24);

// One tile's gathers, branch-free: an unusable row (offset < 0) loads the
// pool's first row instead (zeroed when the tile is stored).
template <int F>
__device__ inline void stage_load_all(Stage<F>& st, const int64_t* toffs, const uint8_t* kv, int gt) {
  constexpr bool Q8 = kQ8<F>;
  constexpr int kLat = Stage<F>::kLat, kStep = Stage<F>::kStep;
  const int ch = Q8 ? (gt & 31) : (gt & 63);
  const int r0 = Q8 ? (gt >> 5) : (gt >> 6);
  if (!Q8) {
    // bf16: a wave's rows r0 + 2k are wave-uniform.  Lane k < 16 reads row
    // r0 + 2k's offset; each row base then moves to scalar registers, and the
    // loads take it as their scalar base with a 32-bit lane offset.
    const int64_t mine = toffs[r0 + 2 * (gt & 15)];
    const int lo = (int)(uint32_t)mine, hi = (int)(mine >> 32);
#pragma unroll
    for (int k = 0; k < kLat; ++k) {
      const int64_t o = ((int64_t)__builtin_amdgcn_readlane(hi, k) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane(lo, k);
      st.lat[k] = ld_global16(kv + (o < 0 ? 0 : o) + (uint32_t)(ch * 16));
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < kLat; ++k) {
    // at most six rows' addresses live at once (the gather waves hold three
    // stages in their registers)
    if (k % 6 == 0 && k > 0) asm volatile("" ::: "memory");
    const int64_t o = toffs[r0 + kStep * k];
    const uint8_t* row = kv + (o < 0 ? 0 : o);
    st.lat[k] = ld_global16(row + ch * 16);
    if (Q8) st.sc[k] = *reinterpret_cast<const float*>(row + 512 + (ch >> 3) * 4);
    if (F == kFmtInt8) st.bi[k] = *reinterpret_cast<const float*>(row + 528 + (ch >> 3) * 4);
  }
}

// The rope chunk vt % 8 (bf16 dims 8 (vt % 8) .. +7) of tile row vt / 8, for
// value-wave thread vt < 256; an unusable row loads the pool's first row.
template <int F>
__device__ inline u32x4 rope_load(const int64_t* toffs, const uint8_t* kv, int vt) {
  const int64_t o = toffs[vt >> 3];
  return ld_global16(kv + (o < 0 ? 0 : o) + kRopeOff<F> + (vt & 7) * 16);
}

// ... into the tile buffer, zeros for an unusable row (clear bit of `vm`).
__device__ inline void rope_store(u32x4 x, uint32_t vm, uint8_t* tile, int vt) {
  const int r = vt >> 3;
  *reinterpret_cast<u32x4*>(tile + r * kRowLds + 1024 + (vt & 7) * 16) = ((vm >> r) & 1u) ? x : u32x4{};
}

// stage_store, then zeros over this thread's latent items of the unusable
// rows (clear bits of the tile's usable-row mask `vm`).
template <int F>
__device__ inline void stage_store_masked(const Stage<F>& st, uint32_t vm, uint8_t* tile, int gt) {
  constexpr bool Q8 = kQ8<F>;
  stage_store<F>(st, tile, gt);
  if (vm != 0xFFFFFFFFu) {
    constexpr int kLat = Stage<F>::kLat, kStep = Stage<F>::kStep;
    const int ch = Q8 ? (gt & 31) : (gt & 63);
    const int r0 = Q8 ? (gt >> 5) : (gt >> 6);
#pragma unroll
    for (int k = 0; k < kLat; ++k) {
      const int r = r0 + kStep * k;
      if (!((vm >> r) & 1u)) {
        uint8_t* dst = tile + r * kRowLds + ch * (Q8 ? 32 : 16);
        *reinterpret_cast<u32x4*>(dst) = u32x4{};
        if (Q8) *reinterpret_cast<u32x4*>(dst + 16) = u32x4{};
      }
    }
  }
}

// stage_store_masked of one tile, then stage_load_all of the next one into the
// same stage.  For bf16 rows the two are interleaved item by item, so the
// texture path takes the next tile's loads while LDS takes this tile's stores.
template <int F>
__device__ inline void stage_cycle(Stage<F>& st, uint32_t vm, uint8_t* tile, const int64_t* next_offs,
                                   const uint8_t* kv, int gt) {
  if (kQ8<F>) {
    stage_store_masked<F>(st, vm, tile, gt);
    stage_load_all<F>(st, next_offs, kv, gt);
    return;
  }
  constexpr int kLat = Stage<F>::kLat;
  const int ch = gt & 63, r0 = gt >> 6;
  const int64_t mine = next_offs[r0 + 2 * (gt & 15)];
  const int lo = (int)(uint32_t)mine, hi = (int)(mine >> 32);
#pragma unroll
  for (int k = 0; k < kLat; ++k) {
    *reinterpret_cast<u32x4*>(tile + (r0 + 2 * k) * kRowLds + ch * 16) = st.lat[k];
    const int64_t o = ((int64_t)__builtin_amdgcn_readlane(hi, k) << 32) | (uint32_t)__builtin_amdgcn_readlane(lo, k);
    st.lat[k] = ld_global16(kv + (o < 0 ? 0 : o) + (uint32_t)(ch * 16));
  }
  if (vm != 0xFFFFFFFFu) {
#pragma unroll
    for (int k = 0; k < kLat; ++k)
      if (!((vm >> (r0 + 2 * k)) & 1u)) *reinterpret_cast<u32x4*>(tile + (r0 + 2 * k) * kRowLds + ch * 16) = u32x4{};
  }
}

// Merge of the split partials of one (row, 64-head group) by the last split
// to arrive (called by every thread after its split's block is stored).  A
// block is O / l as bf16 [64 heads][512 columns], then (m, l) per head.
template <int NT>
__device__ inline void merge_splits_h64(const MlaArgs& a, int t, int grp, int n_groups, int* counter,
                                        float* wgt, int* is_last, int tid) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores are done
  __syncthreads();                                    // ... and every other thread's
  if (tid == 0)
    *is_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               a.splits - 1;
  __syncthreads();
  if (!*is_last) return;
  constexpr int kNh = 64;
  const int S = a.splits, h0 = grp * kNh;
  const __amdgpu_buffer_rsrc_t rs = split_blocks(a, t, grp, n_groups, kNh);
  constexpr int kStride = kPartBytes(kNh);
  float* ls = wgt + kNh * S;
  // statistics of (head h, split s) at index i = h * S + s
  for (int i = tid; i < kNh * S; i += NT) {
    const uint2 ml = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                   rs, (i % S) * kStride + kNh * kDc * 2 + 8 * (i / S), 0, kSc1));
    wgt[i] = __uint_as_float(ml.x);
    ls[i] = __uint_as_float(ml.y);
  }
  __syncthreads();
  // merge weight of (h, s): l_s exp2(m_s - M) / L
  float wnew[(kNh * 64 + NT - 1) / NT];
#pragma unroll
  for (int k = 0; k < (kNh * 64 + NT - 1) / NT; ++k) {
    const int i = tid + k * NT, h = i / S;
    wnew[k] = 0.f;
    if (i < kNh * S) {
      const float* mh = wgt + h * S;
      const float* lh = ls + h * S;
      float M = kNegInf;
      for (int s = 0; s < S; ++s) M = fmaxf(M, mh[s]);
      float L = 0.f;
      if (M != kNegInf)
        for (int s = 0; s < S; ++s) L += exp2_fast(mh[s] - M) * lh[s];  // empty split: 0
      wnew[k] = L > 0.f ? exp2_fast(mh[i % S] - M) * lh[i % S] / L : 0.f;
      if (i % S == 0 && a.lse != nullptr)
        a.lse[(int64_t)t * a.H + h0 + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < (kNh * 64 + NT - 1) / NT; ++k)
    if (tid + k * NT < kNh * S) wgt[tid + k * NT] = wnew[k];
  __syncthreads();
  // 16-byte chunks c = h * 64 + col / 8 of the [64][512] block, eight rounds
  // of NT chunks; each round loads up to kSp splits at once.
  constexpr int kSp = 8, kRounds = kNh * kDc * 2 / 16 / NT;
  uint16_t* outp = a.out + ((int64_t)t * a.H + h0) * kDc;
#pragma unroll 1
  for (int u = 0; u < kRounds; ++u) {
    const int c = tid + u * NT, h = c >> 6;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int s0 = 0; s0 < S; s0 += kSp) {
      u32x4 v[kSp];
#pragma unroll
      for (int s = 0; s < kSp; ++s)
        if (s0 + s < S) v[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, (s0 + s) * kStride + c * 16, 0, kSc1);
#pragma unroll
      for (int s = 0; s < kSp; ++s) {
        if (s0 + s < S) {
          const float wt = wgt[h * S + s0 + s];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += wt * __uint_as_float(v[s][e] << 16);
            acc[2 * e + 1] += wt * __uint_as_float(v[s][e] & 0xFFFF0000u);
          }
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
    *reinterpret_cast<u32x4*>(outp + c * 8) = o;
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS regions of the 64-head kernel.
struct H64Lds {
  uint8_t* tiles;   // three tile buffers; at the end, the output staging area
  uint8_t* pbuf;    // P, two slots of kH64Pslot bytes
  float* alpha;     // rescale factors, two slots: [64 heads], then 2 int flags (per head block)
  float* stats;     // per head: m, l, 0
};

__device__ inline float* alpha_slot(const H64Lds& L, int slot) { return L.alpha + slot * (kH64Aslot / 4); }
__device__ inline int* flag_slot(const H64Lds& L, int slot) {
  return reinterpret_cast<int*>(alpha_slot(L, slot) + 64);
}

// Byte offset in a P slot of the 8 bf16 that score lane (head, row half hb)
// holds for k step ks of the PV operand: [hb][ks][64 heads][8], so the score
// waves' writes and the value waves' operand reads are lane-linear 16-byte
// accesses.
__device__ inline int p_off(int hb, int ks, int head) { return ((hb * 2 + ks) * 64 + head) * 16; }

// Max / sum of a lane's value and that of the lane 32 away (one permlane swap;
// both lanes get the same result).
__device__ inline float max_over_halves(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_over_halves(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

constexpr int kRoleScore = 0, kRoleValue = 1, kRoleGather = 2;

// The tile pipeline of one role (every role runs the same barriers in the
// same order), then its part of the epilogue: the score waves publish (m, l)
// per head, the value waves write O / l as bf16 [64 heads][512 columns] into
// the staging area.  Every register array lives in one role only.
template <int F, int ROLE>
__device__ inline void h64_role(const MlaArgs& a, const H64Lds& L, const int64_t* offs,
                                const uint32_t* vmask, int t, int grp, int ntiles, bool any_usable,
                                int tid) {
  constexpr bool S = ROLE == kRoleScore, V = ROLE == kRoleValue, G = ROLE == kRoleGather;
  static_assert(kH64Bufs == 3 && kH64Stages == 3, "the tile loop is unrolled for three buffers and stages");
  constexpr int kQSteps = 36;                  // k steps of 16 over the 576 dims
  constexpr int kColTiles = 4;                 // value waves: 128 columns in tiles of 32
  constexpr int kL = kStageLoads<F>;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hb = lane >> 5;   // 32x32 layouts: column, lane half
  uint8_t* tiles = L.tiles;

  // ---- score waves: head block g (32 heads)
  const int g = wave & 1;
  bf16x8 q[S ? kQSteps : 1];                   // lane: head 32 g + l32, dims 16 ks + 8 hb .. +7
  float m_run = kNegInf;                       // running max (log2 units) of head 32 g + l32
  float l_run = 0.f;                           // this lane's share of that head's sum
  // ---- value waves: column quarter cq
  const int cq = (wave & 1) | ((wave >> 1) & 2);
  f32x16 o[V ? 2 : 1][V ? kColTiles : 1];
#pragma unroll
  for (int mb = 0; mb < (V ? 2 : 1); ++mb)
#pragma unroll
    for (int ct = 0; ct < (V ? kColTiles : 1); ++ct) o[mb][ct] = f32x16{};
  u32x4 rs[V ? kH64Stages : 1];                // rope of the tiles in flight (value waves)
  const int vt = cq * 64 + lane;
  // ---- gather waves
  const int gt = tid - 4 * 64;
  Stage<F> st[G ? kH64Stages : 1];

  // Score waves: S^T of the tile (A operand: lane row l32, dims 16 ks + 8 hb
  // .. +7, read from LDS four k steps ahead; B: q); then the online-softmax
  // step.  D lane (l32, hb) register i holds
  // tile row 8 (i / 4) + 4 hb + i % 4 of head 32 g + l32.  The running max is
  // raised (O and l rescaled) only when the tile beats it by more than
  // kRescaleSlack; the decision is taken per wave, and the factors (1 for
  // heads not raised) go to LDS with a flag.  P goes to `slot` as bf16,
  // registers 8 ks .. 8 ks + 7 as k step ks of the PV operand.
  // * The MFMAs form one accumulator chain, so each waits for its A operand:
  //   the scheduling barrier after every step keeps each read four steps
  //   ahead of its MFMA (left to itself the compiler issues the reads in
  //   pairs right before their MFMAs, and every pair waits out a whole LDS
  //   round trip: 640 against 570 us for three decode128 layers).
  // * The scale (positive, checked by the caller) is applied in the exponent's
  //   fma: the maximum of the scaled scores is the scaled maximum.
  auto qk_softmax = [&](const uint8_t* tl, uint32_t valid, int slot) {
    constexpr int kAhead = 4;
    const uint8_t* ap = tl + l32 * kRowLds + 16 * hb;
    bf16x8 ra[kAhead];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) ra[k] = lds16(ap + 32 * k);
    f32x16 c = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      c = mfma32(ra[ks % kAhead], q[S ? ks : 0], c);
      if (ks + kAhead < kQSteps) ra[ks % kAhead] = lds16(ap + 32 * (ks + kAhead));
      __builtin_amdgcn_sched_barrier(0);
    }
    float sv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = c[i];
    if (valid != 0xFFFFFFFFu) {                // a partial tile (uniform branch)
      // this lane half's rows: bit 8 (i / 4) + i % 4 of vs (literal masks,
      // nothing kept in registers across the loop)
      const uint32_t vs = valid >> (4 * hb);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!(vs & (1u << (8 * (i >> 2) + (i & 3))))) sv[i] = kNegInf;
    }
    float m = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, sv[i]);
    m = max_over_halves(m) * a.scale_log2;
    const bool raise = m > m_run + kRescaleSlack;
    const bool any_raise = __any(raise);
    if (any_raise) {
      const float m_new = raise ? m : m_run;
      const float al = (m_run == kNegInf) ? 0.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= al;
      if (hb == 0) alpha_slot(L, slot)[32 * g + l32] = al;
    }
    if (lane == 0) flag_slot(L, slot)[g] = any_raise ? 1 : 0;
    // exp2(-inf - m) is 0 for a finite m; m_run is -inf only while every
    // score seen so far is -inf
    const float mu = m_run == kNegInf ? 0.f : m_run;
    u32x4 pk[2];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = exp2_fast(fmaf(sv[i], a.scale_log2, -mu));
      const float p1 = exp2_fast(fmaf(sv[i + 1], a.scale_log2, -mu));
      l_run += p0 + p1;
      pk[i >> 3][(i & 7) >> 1] = pack_bf16x2(p0, p1);
    }
    uint8_t* pslot = L.pbuf + slot * kH64Pslot;
    *reinterpret_cast<u32x4*>(pslot + p_off(hb, 0, 32 * g + l32)) = pk[0];
    *reinterpret_cast<u32x4*>(pslot + p_off(hb, 1, 32 * g + l32)) = pk[1];
  };

  // Value waves: O[64 heads][128 columns] += P V over the tile, after the
  // rescale of the head blocks the score waves flagged.  P is the A operand
  // (lane: head 32 mb + l32, k step ks: tile rows 16 ks + 8 (e / 4) + 4 hb +
  // e % 4); V the B operand (lane: column l32 of the column tile, the same
  // rows), two ds_read_b64_tr_b16 per operand: in each 16-lane group lane j
  // addresses tile row base + j / 4 at column block 4 (j % 4) of the group's
  // 16 columns and receives column j of the four rows.
  auto pv = [&](const uint8_t* tl, int slot) {
    // the P operands, the first V operands and the flags are read together,
    // so the wave waits for LDS once before its MFMAs
    const uint8_t* pslot = L.pbuf + slot * kH64Pslot;
    bf16x8 pa[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pa[mb][ks] = lds16(pslot + p_off(hb, ks, 32 * mb + l32));
    const int jj = lane & 15, g16 = (lane >> 4) & 1;
    const uint8_t* vp = tl + (4 * hb + (jj >> 2)) * kRowLds + (cq * 128 + 16 * g16 + 4 * (jj & 3)) * 2;
    constexpr int kAhead = 3;
    // operand n: k step n / 4, column tile n % 4
    auto vread = [&](int n) {
      const uint8_t* pp = vp + (n >> 2) * 16 * kRowLds + (n & 3) * 64;
      return join(lds_read_tr16(pp), lds_read_tr16(pp + 8 * kRowLds));
    };
    bf16x8 vb[kAhead];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) vb[n] = vread(n);
    const int2 fl = *reinterpret_cast<const int2*>(flag_slot(L, slot));
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (mb == 0 ? fl.x : fl.y) {
        const float* al_s = alpha_slot(L, slot);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 al = *reinterpret_cast<const f32x4*>(al_s + 32 * mb + 8 * j + 4 * hb);
#pragma unroll
          for (int ct = 0; ct < (V ? kColTiles : 1); ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[V ? mb : 0][ct][4 * j + r] *= al[r];
        }
      }
    }
#pragma unroll
    for (int n = 0; n < 2 * kColTiles; ++n) {
      const bf16x8 v = vb[n % kAhead];
      if (n + kAhead < 2 * kColTiles) vb[n % kAhead] = vread(n + kAhead);
      const int ct = V ? (n & 3) : 0;
#pragma unroll
      for (int mb = 0; mb < (V ? 2 : 1); ++mb) o[mb][ct] = mfma32(pa[mb][n >> 2], v, o[mb][ct]);
    }
  };

  // Gather waves: tile j from stage j % 3 into buffer j % 3 (its loads are
  // the oldest in flight: the two later tiles' loads may still be pending),
  // then the gathers of tile j + 3 into the same stage.  Tile numbers are
  // clamped to the last tile, so every call issues the same loads (a tile
  // past the end lands in a buffer no phase reads).
  // The value waves do the same for the tile's rope (one load per tile).
  // 8-bit rows: the gather wave decodes them on the score wave's SIMD and
  // takes issue priority over it meanwhile (decode128 fp8 690 -> 652 us, int8
  // 673 -> 641, three layers; bf16 rows, with no decode, lose 2% with it).
  auto store_issue = [&](int j, int sx) {
    if (G) {
      if constexpr (kQ8<F>) __builtin_amdgcn_s_setprio(2);
      wait_vmcnt<2 * kL>();
      stage_cycle<F>(st[sx], vmask[min(j, ntiles - 1)], tiles + sx * kTileLds,
                     offs + min(j + 3, ntiles - 1) * kTileRows, a.kv, gt);
      if constexpr (kQ8<F>) __builtin_amdgcn_s_setprio(0);
    } else if (V) {
      wait_vmcnt<2>();
      rope_store(rs[sx], vmask[min(j, ntiles - 1)], tiles + sx * kTileLds, vt);
      rs[sx] = rope_load<F>(offs + min(j + 3, ntiles - 1) * kTileRows, a.kv, vt);
    }
  };

  if (any_usable) {
    if (G) {
#pragma unroll
      for (int j = 0; j < kH64Stages; ++j)
        stage_load_all<F>(st[j], offs + min(j, ntiles - 1) * kTileRows, a.kv, gt);
    }
    if (V) {
#pragma unroll
      for (int j = 0; j < kH64Stages; ++j) rs[j] = rope_load<F>(offs + min(j, ntiles - 1) * kTileRows, a.kv, vt);
    }
    store_issue(0, 0);
    if (S) {
      const uint16_t* qp = a.q + ((int64_t)t * a.H + grp * 64 + 32 * g + l32) * kD + 8 * hb;
#pragma unroll
      for (int ks = 0; ks < (S ? kQSteps : 1); ++ks) q[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
    }
    lds_barrier();
    if (S) qk_softmax(tiles, vmask[0], 0);
    store_issue(1, 1);  // unconditional (tile 1 clamped), so the loop sees one wait state
    lds_barrier();
    // phase i (i3 = i % 3, i2 = i % 2); `checked` phases test the tile count
    auto phase = [&](int i, int i3, int i2, bool checked) {
      if (S && (!checked || i + 1 < ntiles)) qk_softmax(tiles + (i3 == 2 ? 0 : i3 + 1) * kTileLds, vmask[i + 1], i2 ^ 1);
      if (V) pv(tiles + i3 * kTileLds, i2);
      if (!checked || i + 2 < ntiles) store_issue(i + 2, i3 == 0 ? 2 : i3 - 1);
      lds_barrier();
    };
    // whole trips of six phases in which every role has its work, then the rest
    int i = 0;
#pragma unroll 1
    for (; i + 8 <= ntiles; i += 6) {
      phase(i, 0, 0, false);
      phase(i + 1, 1, 1, false);
      phase(i + 2, 2, 0, false);
      phase(i + 3, 0, 1, false);
      phase(i + 4, 1, 0, false);
      phase(i + 5, 2, 1, false);
    }
    if (i < ntiles) phase(i, 0, 0, true);
    if (i + 1 < ntiles) phase(i + 1, 1, 1, true);
    if (i + 2 < ntiles) phase(i + 2, 2, 0, true);
    if (i + 3 < ntiles) phase(i + 3, 0, 1, true);
    if (i + 4 < ntiles) phase(i + 4, 1, 0, true);
    if (i + 5 < ntiles) phase(i + 5, 2, 1, true);
    if (i + 6 < ntiles) phase(i + 6, 0, 0, true);
    wait_vmcnt<0>();  // the last gathers (of no tile) are done
  }

  // m and l per head, from the score waves
  if (S) {
    const float l = sum_over_halves(l_run);
    if (hb == 0) {
      const int h = 32 * g + l32;
      L.stats[3 * h] = m_run;
      L.stats[3 * h + 1] = l;
      L.stats[3 * h + 2] = 0.f;
    }
  }
  lds_barrier();
  // O / l as bf16 into the staging area, [64 heads][512 columns]
  if (V) {
    uint16_t* stage_out = reinterpret_cast<uint16_t*>(tiles);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = 32 * mb + 8 * j + 4 * hb + r;
          const float l = L.stats[3 * h + 1] + L.stats[3 * h + 2];
          const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;
#pragma unroll
          for (int ct = 0; ct < kColTiles; ++ct)
            stage_out[h * kDc + cq * 128 + ct * 32 + l32] =
                __builtin_bit_cast(uint16_t, (__bf16)(o[V ? mb : 0][V ? ct : 0][4 * j + r] * inv));
        }
      }
    }
  }
  lds_barrier();
}

template <int F>
__global__ __launch_bounds__(kH64Threads, 1) void sparse_mla_h64(MlaArgs a, int n_groups, int T) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int NT = kH64Threads;
  static_assert(NT == 8 * 64 && kGatherThreads == 2 * 64, "two score, four value and two gather waves");
  const int x = blockIdx.x, sp = blockIdx.z;
  const int t = (x / (8 * n_groups)) * 8 + (x & 7);
  const int grp = (x >> 3) % n_groups;
  if (t >= T) return;                          // padding ids of the XCD-aware layout
  const int tid = threadIdx.x, wave = tid >> 6;
  const int j_begin = sp * a.rows_per_split;
  const int j_end = min(a.K, j_begin + a.rows_per_split);
  const int ntiles = (j_end - j_begin + kTileRows - 1) / kTileRows;
  int sv0[kIdxBatch];
  preload_indices<NT>(sv0, a.idx + (int64_t)t * a.K, j_begin, j_end, ntiles * kTileRows, tid);
  const RowLoc loc = locate_row(a.cu_q, a.seq_lens, a.B, t);
  H64Lds L;
  uint8_t* p = smem;
  L.tiles = p;
  p += kH64Bufs * kTileLds;
  L.pbuf = p;
  p += 2 * kH64Pslot;
  L.alpha = reinterpret_cast<float*>(p);
  p += 2 * kH64Aslot;
  L.stats = reinterpret_cast<float*>(p);
  int64_t* offs = reinterpret_cast<int64_t*>(smem + kH64Fixed);
  uint32_t* vmask = reinterpret_cast<uint32_t*>(offs + ntiles * kTileRows);
  int* wmin = reinterpret_cast<int*>(vmask + ntiles);  // kWaveSlots, then the merge's flag

  const int fv = build_offsets<NT>(offs, vmask, wmin, sv0, a.idx + (int64_t)t * a.K, j_begin, j_end,
                                   ntiles * kTileRows, loc.pos, loc.b, a.page_table, a.pt_stride,
                                   a.page_size, a.num_pages, a.page_stride, a.row_stride, tid);
  const bool any = fv != INT32_MAX;
  if (wave < 2) h64_role<F, kRoleScore>(a, L, offs, vmask, t, grp, ntiles, any, tid);
  else if (wave == 4 || wave == 5) h64_role<F, kRoleGather>(a, L, offs, vmask, t, grp, ntiles, any, tid);
  else h64_role<F, kRoleValue>(a, L, offs, vmask, t, grp, ntiles, any, tid);

  const uint16_t* stage_out = reinterpret_cast<const uint16_t*>(L.tiles);
  constexpr int kChunks = 64 * kDc * 2 / 16 / NT;  // 16-byte chunks per thread
  if (a.splits == 1) {
    uint16_t* outp = a.out + ((int64_t)t * a.H + grp * 64) * kDc;
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int c = tid + u * NT;
      *reinterpret_cast<u32x4*>(outp + c * 8) = *reinterpret_cast<const u32x4*>(stage_out + c * 8);
    }
    if (a.lse != nullptr && tid < 64) {
      const float m = L.stats[3 * tid], l = L.stats[3 * tid + 1] + L.stats[3 * tid + 2];
      a.lse[(int64_t)t * a.H + grp * 64 + tid] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
    }
  } else {
    const __amdgpu_buffer_rsrc_t rs = split_blocks(a, t, grp, n_groups, 64);
    const int base = sp * kPartBytes(64);
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int c = tid + u * NT;
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(stage_out + c * 8), rs,
                                             base + c * 16, 0, kSc1);
    }
    if (tid < 64) {
      const uint2 ml{__float_as_uint(L.stats[3 * tid]),
                     __float_as_uint(L.stats[3 * tid + 1] + L.stats[3 * tid + 2])};
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(2 * sizeof(int)))) int, ml),
                                            rs, base + 64 * kDc * 2 + 8 * tid, 0, kSc1);
    }
    // the merge's weights overwrite the staging area only after every
    // thread's copy out of it is complete (it waits and synchronises first)
    merge_splits_h64<NT>(a, t, grp, n_groups, a.counters + (int64_t)t * n_groups + grp,
                         reinterpret_cast<float*>(L.tiles), wmin + kWaveSlots, tid);
  }
}

// ---------------------------------------------------------------- 16 heads

// One workgroup owns 16 heads of one query row and one range of its selected
// rows.  Wave w splits QK with its siblings: it owns tile rows 16(w&1) .. +15
// and k steps 9(w>>1) .. +8 (half of the 576 dims).  It loads exactly that
// part of each tile from HBM into registers, already in the A-operand layout
// of v_mfma_f32_16x16x32_bf16 (lane: row c16, dims 32 ks + 8 g .. +7), so QK
// reads no LDS at all; the latent dims are also written to the LDS tile, from
// which every wave then reads V for its quarter (128) of the output columns.
// Partial scores of the two k halves are summed through LDS in a fixed order.
// Registers: 36 of q, 32 of accumulator, 36 per tile in flight (two tiles).
// 8-bit rows: the first of the 8 latent dims lane group g supplies in k step
// ks < 16 (the sum over dims runs in any order; q follows the same map).
__host__ __device__ constexpr int q8_dim(int ks, int g) { return 64 * (ks >> 1) + 16 * g + 8 * (ks & 1); }

template <int F>
struct RegTile {
  u32x4 v[9];   // bf16: 16 B per k step; 8-bit: 8 latent codes (v.x, v.y) or 16 B of rope
  f32x4 sc;     // 8-bit: block scales of the row
  f32x4 bi;     // int8: block biases of the row
};

template <int F>
__device__ inline void regtile_load(RegTile<F>& st, int64_t off, const uint8_t* kv, int ks0, int g) {
  constexpr bool Q8 = kQ8<F>;
#pragma unroll
  for (int k = 0; k < 9; ++k) st.v[k] = u32x4{};
  st.sc = f32x4{};
  st.bi = f32x4{};
  if (off < 0) return;
  const uint8_t* row = kv + off;
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int ks = ks0 + k;
    if (!Q8) {
      st.v[k] = ld_global16(row + ks * 64 + g * 16);
    } else if (ks < 16) {
      // 8-bit: k steps 2j and 2j+1 take dims 64 j + 16 g .. +15 (q8_dim), so
      // one 16-byte load serves both when the wave has both steps
      if ((ks & 1) == 0 && k + 1 < 9) {
        const u32x4 x = ld_global16(row + q8_dim(ks, g));
        st.v[k] = u32x4{x[0], x[1], 0u, 0u};
        st.v[k + 1] = u32x4{x[2], x[3], 0u, 0u};
      } else if ((ks & 1) == 1 && k == 0) {
        const uint2 x = *reinterpret_cast<const uint2*>(row + q8_dim(ks, g));
        st.v[k] = u32x4{x.x, x.y, 0u, 0u};
      } else if ((ks & 1) == 0) {
        const uint2 x = *reinterpret_cast<const uint2*>(row + q8_dim(ks, g));
        st.v[k] = u32x4{x.x, x.y, 0u, 0u};
      }
    } else {
      st.v[k] = ld_global16(row + kRopeOff<F> + ((ks - 16) * 32 + g * 8) * 2);
    }
  }
  if (Q8) st.sc = *reinterpret_cast<const f32x4*>(row + 512);
  if (F == kFmtInt8) st.bi = *reinterpret_cast<const f32x4*>(row + 528);
}

// The bf16 A operand of k step ks.  8-bit latent dims give their codes
// exactly (every e4m3 value is a bf16; int8 codes centred, code - 128, an
// integer in -128..127); the block scale, and the int8 bias (then bi + 128
// sc), is applied to the scores and to P instead.  Centring keeps sc times
// the code near the decoded value when a block's range is centred near zero,
// so rounding P times the scale to bf16 costs no more than rounding the
// decoded value would.
template <int F>
__device__ inline bf16x8 regtile_operand(const RegTile<F>& st, int k, int ks) {
  if (!kQ8<F> || ks >= 16) return __builtin_bit_cast(bf16x8, st.v[k]);
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t x = st.v[k][h];
    if (F == kFmtFp8) {
      r[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
      r[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
    } else {
      r[2 * h] = pack_bf16x2((float)(x & 0xFFu) - 128.f, (float)((x >> 8) & 0xFFu) - 128.f);
      r[2 * h + 1] = pack_bf16x2((float)((x >> 16) & 0xFFu) - 128.f, (float)(x >> 24) - 128.f);
    }
  }
  return __builtin_bit_cast(bf16x8, r);
}

// QK of one tile for the k steps KS0 .. KS0+8 of 8-bit rows: one accumulator
// per 128-dim block the steps touch (the rope steps 16, 17 in the last), each
// scaled by its row's block scale (and, int8, plus the row's block bias for
// the centred codes times q's sum over the wave's dims of the block), as
// exact codes go in.  sct /
// bit: this wave's [block][16 rows] scale and bias tables in LDS; rows of the
// D layout: 4 g + i.  trow: the lane's LDS tile row (latent codes as bf16).
template <int F, int KS0>
__device__ inline f32x4 qk_q8(const RegTile<F>& st, const bf16x8 (&qreg)[9], uint8_t* trow,
                              const float* sct, const float* bit, const float (&qsum)[3], int g) {
  f32x4 acc[3] = {f32x4{}, f32x4{}, f32x4{}};
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int ks = KS0 + k;
    const bf16x8 av = regtile_operand<F>(st, k, ks);
    if (ks < 16) *reinterpret_cast<bf16x8*>(trow + 2 * q8_dim(ks, g)) = av;  // latent codes feed PV
    const int slot = (ks < 16 ? ks >> 2 : 4) - (KS0 >> 2);
    acc[slot] = mfma16(av, qreg[k], acc[slot]);
  }
  f32x4 s = f32x4{};
#pragma unroll
  for (int slot = 0; slot < 3; ++slot) {
    const int b = slot + (KS0 >> 2);  // 4: the rope
    if (b < 4) {
      const f32x4 sc = *reinterpret_cast<const f32x4*>(sct + b * 16 + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = fmaf(acc[slot][i], sc[i], s[i]);
      if (F == kFmtInt8) {
        const f32x4 bi = *reinterpret_cast<const f32x4*>(bit + b * 16 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = fmaf(bi[i], qsum[slot], s[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += acc[slot][i];
    }
  }
  return s;
}

// q's sum over the dims of each block slot of the k steps KS0 .. KS0+8
// (lane: head c16, the lane's 8 dims per step; summed over the four lane
// groups), for the int8 bias term of the scores.
template <int KS0>
__device__ inline void qsum_q8(const bf16x8 (&qreg)[9], float (&qsum)[3]) {
  float part[3] = {0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int ks = KS0 + k;
    const int slot = (ks < 16 ? ks >> 2 : 4) - (KS0 >> 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) part[slot] += (float)qreg[k][e];
  }
#pragma unroll
  for (int slot = 0; slot < 3; ++slot) qsum[slot] = sum_over_groups(part[slot]);
}

// MINW: workgroups per CU the register budget is sized for (1 when the grid
// fits the CUs in one round, so each wave may use a SIMD's whole register file).
template <int F, int STAGES, int MINW>
__global__ __launch_bounds__(kThreads, MINW) void sparse_mla_q16(MlaArgs a, int n_groups, int T) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // Workgroup ids: head group outermost over a block of P = (T * splits
  // rounded up to 8) ids, so the head groups of one (row, split) are a
  // multiple of 8 apart -- same XCD, sharing the gathered rows in its L2 --
  // while consecutive splits and rows go to different XCDs and every XCD gets
  // a like share of long and short rows.
  const int P = (T * a.splits + 7) / 8 * 8;
  const int grp = (int)blockIdx.x / P, u = (int)blockIdx.x % P;
  if (u >= T * a.splits) return;               // padding ids
  const int t = u / a.splits, sp = u % a.splits;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int rb = wave & 1, ks0 = 9 * (wave >> 1);
  const int head0 = grp * 16;
  const int col0 = 128 * wave;
  const int j_begin = sp * a.rows_per_split;
  const int j_end = min(a.K, j_begin + a.rows_per_split);
  const int ntiles = (j_end - j_begin + kTileRows - 1) / kTileRows;
  int sv0[kIdxBatch];
  preload_indices(sv0, a.idx + (int64_t)t * a.K, j_begin, j_end, ntiles * kTileRows, tid);
  const RowLoc loc = locate_row(a.cu_q, a.seq_lens, a.B, t);
  const int b = loc.b, pos = loc.pos;
  uint8_t* tile = smem;
  f32x4* sbuf = reinterpret_cast<f32x4*>(smem + kTileLds);
  float* q8tab = reinterpret_cast<float*>(smem + kTileLds + kSbufLds);  // [scale, bias][wave][block][16 rows]
  int64_t* offs = reinterpret_cast<int64_t*>(smem + kTileLds + kSbufLds + kQ8TabLds);
  uint32_t* vmask = reinterpret_cast<uint32_t*>(offs + ntiles * kTileRows);
  int* wmin = reinterpret_cast<int*>(vmask + ntiles);  // kWaveSlots, then the merge's flag

  // q for this wave's k half: lane (head c16, group g) holds dims 32 ks + 8 g .. +7.
  bf16x8 qreg[9];
  {
    const uint16_t* qh = a.q + ((int64_t)t * a.H + head0 + c16) * kD;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const int ks = ks0 + k;
      const int d = (kQ8<F> && ks < 16) ? q8_dim(ks, g) : 32 * ks + 8 * g;  // 8-bit rows: their dim map
      qreg[k] = *reinterpret_cast<const bf16x8*>(qh + d);
    }
  }
  const int fv = build_offsets(offs, vmask, wmin, sv0, a.idx + (int64_t)t * a.K, j_begin, j_end,
                               ntiles * kTileRows, pos, b, a.page_table, a.pt_stride, a.page_size,
                               a.num_pages, a.page_stride, a.row_stride, tid);

  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;
  constexpr bool Q8 = kQ8<F>, BIAS = F == kFmtInt8;
  float qsum[3] = {0.f, 0.f, 0.f};  // int8: q summed over each block slot of the wave's dims
  if (BIAS) {
    if (ks0 == 0) qsum_q8<0>(qreg, qsum);
    else qsum_q8<9>(qreg, qsum);
  }
  float bacc = 0.f;                 // int8: this lane's share of sum_r p * bias (head c16), rescaled with O
  float* sct = q8tab + wave * 64;   // this wave's [block][16 rows] scales; biases 256 floats on
  float* bit = sct + 256;

  if (fv != INT32_MAX) {
    const int my_row = 16 * rb + c16;
    auto step = [&](RegTile<F>& st, int i) {
      lds_barrier();                                       // every wave is done with tile i-1
      f32x4 spart = f32x4{};
      uint8_t* trow = tile + my_row * kRowLds + g * 16;
      if (Q8) {
        // the rows' block scales (and biases) into this wave's tables: lane
        // (g, c16) writes block g of row c16
        sct[g * 16 + c16] = st.sc[g];
        if (BIAS) bit[g * 16 + c16] = fmaf(128.f, st.sc[g], st.bi[g]);  // the centred codes' bias
        uint8_t* trow8 = tile + my_row * kRowLds;
        spart = ks0 == 0 ? qk_q8<F, 0>(st, qreg, trow8, sct, bit, qsum, g)
                         : qk_q8<F, 9>(st, qreg, trow8, sct, bit, qsum, g);
      } else {
#pragma unroll
        for (int k = 0; k < 9; ++k) {
          const int ks = ks0 + k;
          const bf16x8 av = regtile_operand<F>(st, k, ks);
          if (ks < 16) *reinterpret_cast<bf16x8*>(trow + ks * 64) = av;  // latent dims feed PV
          spart = mfma16(av, qreg[k], spart);
        }
      }
      sbuf[wave * 64 + lane] = spart;
      if (i + STAGES < ntiles) regtile_load<F>(st, offs[(i + STAGES) * kTileRows + my_row], a.kv, ks0, g);
      lds_barrier();                                       // tile i and partial scores visible
      const uint32_t valid = vmask[i];
      // rows 0..15 from waves 0 and 2, rows 16..31 from waves 1 and 3; k half 0 first
      const f32x4 s0 = sbuf[0 * 64 + lane] + sbuf[2 * 64 + lane];
      const f32x4 s1 = sbuf[1 * 64 + lane] + sbuf[3 * 64 + lane];
      bf16x8 pa;
      if (Q8) {
        // P for this wave's columns (block `wave`) carries the rows' scale of
        // that block: k slot (g, e) is row 4g + e (waves 0, 2 hold rows 0..15),
        // (g, 4 + e) row 16 + 4g + e (waves 1, 3)
        float psc[8], pbi[8];
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(q8tab + 0 * 64 + wave * 16 + 4 * g);
        const f32x4 c1 = *reinterpret_cast<const f32x4*>(q8tab + 1 * 64 + wave * 16 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          psc[e] = c0[e];
          psc[4 + e] = c1[e];
        }
        if (BIAS) {
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(q8tab + 256 + 0 * 64 + wave * 16 + 4 * g);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(q8tab + 256 + 1 * 64 + wave * 16 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pbi[e] = d0[e];
            pbi[4 + e] = d1[e];
          }
        }
        pa = tile_softmax<8, true, BIAS>(s0, s1, valid, a.scale_log2, m_run, l_run, o, psc, pbi, &bacc);
      } else {
        pa = tile_softmax(s0, s1, valid, a.scale_log2, m_run, l_run, o);
      }
      // O[:, col0 + 16 i .. +16] += P V.  k slot (g, e) <-> tile row 4g + e,
      // (g, 4 + e) <-> 16 + 4g + e, matching the S^T accumulator rows.
      const uint8_t* vp = tile + (4 * g + (c16 >> 2)) * kRowLds + (col0 + 4 * (c16 & 3)) * 2;
      s16x4 tv1[8], tv2[8];
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) {
        tv1[i2] = lds_read_tr16(vp + i2 * 32);
        tv2[i2] = lds_read_tr16(vp + 16 * kRowLds + i2 * 32);
      }
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) o[i2] = mfma16(pa, join(tv1[i2], tv2[i2]), o[i2]);
    };
    RegTile<F> st[STAGES];
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < ntiles) regtile_load<F>(st[s], offs[s * kTileRows + my_row], a.kv, ks0, g);
#pragma unroll 1
    for (int i = 0; i < ntiles; i += STAGES) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s)
        if (i + s < ntiles) step(st[s], i + s);
    }
  }

  if (BIAS) {  // the bias term, the same for every column of the wave's block
    const float bt = sum_over_groups(bacc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float br = __shfl(bt, 4 * g + r);
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) o[i2][r] += br;
    }
  }
  l_run = sum_over_groups(l_run);
  // O accumulator r of lane: head 4g + r, column col0 + 16 i + c16.
  if (a.splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g + r;
      const float lh = __shfl(l_run, h);
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      uint16_t* op = a.out + ((int64_t)t * a.H + head0 + h) * kDc + col0 + c16;
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) op[16 * i2] = __builtin_bit_cast(uint16_t, (__bf16)(o[i2][r] * inv));
    }
    if (a.lse != nullptr && wave == 0 && lane < 16)
      a.lse[(int64_t)t * a.H + head0 + lane] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : kNegInf;
  } else {
    store_partials<16, 8>(a, t, grp, n_groups, sp, wave * 8, lane, o, m_run, l_run, wave == 0 ? 0 : -1);
    merge_splits_if_last<false>(a, t, grp, n_groups, a.counters + (int64_t)t * n_groups + grp,
                                reinterpret_cast<float*>(tile), wmin + kWaveSlots, tid);
  }
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
  const RowLoc loc = locate_row(cu_q, seq_lens, B, t);
  const int b = loc.b, pos = loc.pos;
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

MlaPlan plan_sparse_mla(int num_q_rows, int n_heads, int k, int dc, bool prefill, bool q8) {
  MlaPlan p{1, k, 0};
  if (dc != kDc || n_heads % 16 != 0 || k <= 0 || num_q_rows <= 0) return p;
  const bool wide = n_heads % 64 == 0;
  const int64_t blocks = (int64_t)num_q_rows * (wide ? n_heads / 64 : n_heads / 16);
  int splits = 1;
  if (!prefill) {
    // Workgroups wanted.  16-head groups over bf16 rows: one per CU (a lone
    // resident workgroup streams a longer range and leaves half the split
    // partials to merge; two per CU measured 6% slower at 64 decode rows).
    // Over 8-bit rows, whose decode is VALU work, two per CU (a second wave
    // per SIMD hides it: 57 against 73+ us at 64 decode rows).  64-head
    // groups: 1.5 waves of the 512-thread workgroups.
    const int64_t target = wide ? 384 : (q8 ? 512 : 256);
    // at most 64 splits: the merge keeps 2 x 64 heads x splits floats in the tile buffer
    const int max_splits = k / 256 > 64 ? 64 : (k / 256 > 1 ? k / 256 : 1);
    const int64_t want = (target + blocks - 1) / blocks;
    splits = (int)(want < 1 ? 1 : (want > max_splits ? max_splits : want));
  }
  int rps = (k + splits - 1) / splits;
  rps = (rps + kTileRows - 1) / kTileRows * kTileRows;
  splits = (k + rps - 1) / rps;
  p.splits = splits;
  p.rows_per_split = rps;
  if (splits > 1) {
    // want > 1 means blocks < target <= kMlaCounterSlots: one counter per block fits
    static_assert(kMlaCounterSlots >= 512, "a counter for every block of a split launch");
    p.ws_bytes = kMlaCounterBytes + (size_t)num_q_rows * n_heads * splits * kPartBytes(16) / 16;
  }
  return p;
}

namespace {

constexpr size_t kMaxLds = 160 * 1024;

// LDS bytes: the first tile, `more` bytes of further tiles and partial
// scores, then the range's row offsets, tile masks and a flag.
size_t mla_lds(int rps, size_t more) {
  const size_t ntiles = (size_t)(rps + kTileRows - 1) / kTileRows;
  return kTileLds + more + ntiles * (kTileRows * 8 + 4) + (kWaveSlots + 4) * sizeof(int);
}

template <typename Kernel>
hipError_t launch_with_lds(Kernel kernel, dim3 grid, int threads, size_t lds, hipStream_t stream,
                           const MlaArgs& args, int n_groups, int T) {
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(kernel));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, grid, dim3(threads), lds, stream, args, n_groups, T);
  return hipGetLastError();
}

size_t plan_lds(const MlaPlan& plan, int n_heads) {
  return n_heads % 64 == 0 ? mla_lds(plan.rows_per_split, kH64Fixed - kTileLds)
                           : mla_lds(plan.rows_per_split, kSbufLds + kQ8TabLds);
}

}  // namespace

bool sparse_mla_plan_fits(const MlaPlan& plan, int n_heads) { return plan_lds(plan, n_heads) <= kMaxLds; }

hipError_t launch_sparse_mla_bf16(const BatchArgs& ba, const void* q, const PoolArgs& kv,
                                  const int32_t* idx, int k, int n_heads, float sm_scale,
                                  void* out, float* lse, void* ws, const MlaPlan& plan,
                                  hipStream_t stream) {
  const bool wide = n_heads % 64 == 0;
  const int fmt = kv.format == 2 ? kFmtFp8 : (kv.format == 3 ? kFmtInt8 : kFmtBf16);
  const size_t lds = plan_lds(plan, n_heads);
  if (lds > kMaxLds) return hipErrorInvalidValue;  // the API refuses such plans before launching
  MlaArgs args{ba.cu_q, ba.seq_lens, ba.page_table, ba.batch, ba.pt_stride, ba.page_size,
               ba.num_pages, static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(kv.base),
               kv.page_stride, kv.row_stride, idx, k, n_heads, sm_scale * kLog2e,
               static_cast<uint16_t*>(out), lse,
               plan.splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kMlaCounterBytes) : nullptr,
               plan.splits > 1 ? static_cast<int*>(ws) : nullptr,
               plan.splits, plan.rows_per_split};
  const int T = ba.num_q_rows;
  const int n_groups = wide ? n_heads / 64 : n_heads / 16;
  // 64-head groups: ids t, split on z (row-major XCD layout); 16-head groups: see sparse_mla_q16.
  const dim3 grid = wide ? dim3((unsigned)((T + 7) / 8 * 8 * n_groups), 1, plan.splits)
                         : dim3((unsigned)(n_groups * ((T * plan.splits + 7) / 8 * 8)), 1, 1);
  hipError_t e;
  // Tiles of loads in flight per workgroup: two or three.
  if (wide)
    e = fmt == kFmtFp8    ? launch_with_lds(sparse_mla_h64<kFmtFp8>, grid, kH64Threads, lds, stream, args, n_groups, T)
        : fmt == kFmtInt8 ? launch_with_lds(sparse_mla_h64<kFmtInt8>, grid, kH64Threads, lds, stream, args, n_groups, T)
                          : launch_with_lds(sparse_mla_h64<kFmtBf16>, grid, kH64Threads, lds, stream, args, n_groups, T);
  else if (fmt == kFmtFp8)
    e = launch_with_lds(sparse_mla_q16<kFmtFp8, 2, 2>, grid, kThreads, lds, stream, args, n_groups, T);
  else if (fmt == kFmtInt8)
    e = launch_with_lds(sparse_mla_q16<kFmtInt8, 2, 2>, grid, kThreads, lds, stream, args, n_groups, T);
  else if ((int)grid.x <= device_cu_count())  // one round of workgroups: one per CU
    e = launch_with_lds(sparse_mla_q16<kFmtBf16, 3, 1>, grid, kThreads, lds, stream, args, n_groups, T);
  else
    e = launch_with_lds(sparse_mla_q16<kFmtBf16, 3, 2>, grid, kThreads, lds, stream, args, n_groups, T);
  return e;
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
