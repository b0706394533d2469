// Lightning-indexer scores on gfx950.
//
//   score[t, s] = sum_h w[t, h] * max(0, q_I[t, h, :] . k_I[s, :]),  0 <= s <= pos(t)
//
// (the DSA indexer of lmdeploy PR 4737 "feat: support GLM-5.2", section
// "Changes", and of mlx-lm PR 1419's description; the pages name the
// indexer without a formula and this is its plain reading.)
//
// MFMA kernels (bf16, 64 heads x 128 dims).  The grid form (kept for
// launches the persistent form below cannot stage): a workgroup of four waves
// owns one request, a chunk of 512 consecutive cached tokens (chunk index
// outermost in the grid, so that requests' empty tails dispatch last) and a
// group of up to eight consecutive query rows of that request.  Each wave
// walks two blocks of 64 tokens; a block's keys are loaded straight from their pages into
// registers, already in the B-operand layout of v_mfma_f32_32x32x16_bf16, and
// used for every row of the group (two waves per SIMD hide each other's load
// latency).  The group's query rows sit in LDS (copied in with
// global_load_lds while the page lookups and first keys load) and feed the A operand
// (heads on M, tokens on N).  The ReLU, the per-head weight and the sum over
// heads are applied to the accumulators in registers: a lane owns one token
// column and half of the heads, so one cross-lane add finishes each score.
// Keys are read in place (no copy of the cache), once per row group.
//
// Reduction-index layout: the dot product over the 128 dims is summed in any
// order, so the k slots of each MFMA are mapped to dims to suit the key
// loads.  bf16 keys (256 B, two 128-byte lines per token): lane l (group g =
// l/32) supplies dims 16 ks + 8 g .. +7 in step ks, so lanes l and l + 32 read
// neighbouring 16 bytes of one line and a load instruction touches 32 lines,
// not 64.  fp8 keys (128 B, one line per token): dims g*64 + ks*8 .. +7, each
// lane reading 64 contiguous bytes.  The query operand uses the keys' mapping.
#include <algorithm>
#include <type_traits>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

namespace {

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kKeysPerStep = 64;                                  // per wave and step
constexpr int kSteps = 2;                                         // steps per wave
constexpr int kKeysPerBlock = kWaves * kSteps * kKeysPerStep;     // 512 per workgroup
constexpr int kHeadSlots = 17;                                    // 16 chunks of 16 B + 1 pad
constexpr int kHeadStrideLds = kHeadSlots * 16;                   // 272 B: heads start on distinct banks
constexpr int kRowSlots = kHeads * kHeadSlots;                    // 1088
constexpr int kRowBytesLds = kRowSlots * 16;                      // 17408 B per staged query row
// fp8 queries (codes in the keys' dim order, 128 B per head): heads 144 B
// apart, so the 16-byte operand reads of 16 lanes (16 heads) meet distinct
// bank quartets.
constexpr int kHeadStrideLds8 = 144;
constexpr int kRowBytesLds8 = kHeads * kHeadStrideLds8;             // 9216 B per staged query row
template <bool QFP8>
constexpr int kQRowBytes = QFP8 ? kRowBytesLds8 : kRowBytesLds;

typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;            // fp8 MFMA operand
typedef __attribute__((__vector_size__(8 * sizeof(uint32_t)))) uint32_t u32x8;
typedef short s16x2 __attribute__((ext_vector_type(2)));                        // packed fp8 pair

// 16-byte copy HBM -> LDS for every active lane of the wave: lane i's bytes land
// at lds_wave_base + 16 i (global_load_lds_dwordx4, LDS base in M0).
__device__ inline void copy16_to_lds(const void* src, uint8_t* lds_wave_base) {
  const uint32_t l = (uint32_t)(uintptr_t)(lds_u8_t*)lds_wave_base;
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(l))
               : "memory");
}

__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Keys of one wave step: two 32-token column tiles x eight k steps.  The loads
// are unconditional (a token without a mapped page reads the pool's first row
// and its score is not written), so every step issues exactly 16 loads per lane.
struct Keys {
  bf16x8 v[2][8];
};

__device__ inline void load_keys(Keys& kk, const int64_t (&off)[2], const uint8_t* k_base, int lane, int,
                                 int, int64_t) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint8_t* p = k_base + (off[nt] < 0 ? 0 : off[nt]) + (lane >> 5) * 16;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kk.v[nt][ks] = *reinterpret_cast<const bf16x8*>(p + ks * 32);
  }
}

// fp8 keys (e4m3, one f32 scale per token, page-blocked: a page holds
// page_size rows of 128 codes, row_stride bytes apart, then the page_size
// scales).  Raw codes of one wave step: this lane's 64 dims of its two tokens,
// plus the tokens' scales; every step issues exactly 10 loads per lane (a
// token without a mapped page reads page 0 and its score is not written).
struct Keys8 {
  u32x4 v[2][4];
  float sc[2];
};

__device__ inline void load_keys(Keys8& kk, const int64_t (&off)[2], const uint8_t* k_base, int lane,
                                 int s_first, int page_size, int64_t row_stride) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t o = off[nt] < 0 ? 0 : off[nt];
    const uint8_t* p = k_base + o + (lane >> 5) * 64;
#pragma unroll
    for (int c = 0; c < 4; ++c) kk.v[nt][c] = *reinterpret_cast<const u32x4*>(p + c * 16);
    // row offset o = page * page_stride + slot * row_stride; the scale sits at
    // page * page_stride + page_size * row_stride + slot * 4
    const int slot = off[nt] < 0 ? 0 : (s_first + nt * 32 + (lane & 31)) % page_size;
    kk.sc[nt] = *reinterpret_cast<const float*>(k_base + o + (int64_t)(page_size - slot) * row_stride + slot * 4);
  }
}

// e4m3 codes -> bf16 (exact: every e4m3 value is a bf16), step ks: dims
// 8 ks .. +7 of the lane's 64 (the fp8 keys' mapping).
__device__ inline void keys_from_fp8(Keys& kk, const Keys8& k8) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 b;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const uint32_t x = k8.v[nt][c][2 * half + d];
          b[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
          b[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
        }
        kk.v[nt][2 * c + half] = __builtin_bit_cast(bf16x8, b);
      }
}

template <bool KFP8>
using KeyRegs = typename std::conditional<KFP8, Keys8, Keys>::type;
template <bool KFP8>
constexpr int kLoadsPerStep = KFP8 ? 10 : 16;

// One wave: scores of a 64-token block (keys kk, tokens s_base + 32 nt + lane%32,
// page offsets off, -1 when unmapped) against the nr staged query rows; row r
// sits at position pos_first + r (clamped to ld_last) and its output row is
// row0 + r.
constexpr int kMaxUnitRows = 8;  // query rows scored against one key block

// max(x, 0) as a signed-integer max of the bit pattern: a negative float is a
// negative integer (and -0 gives +0).  One v_max_i32, where fmaxf on an MFMA
// result also costs a NaN-quieting v_max_f32 first.
__device__ inline float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Where a wave's scores of one block go.  put(r, s, lane, score, valid):
// lane's token s of unit row r, valid when s is at or before the row's
// position and its page is mapped; skip(r): row r has no token in the block.
// GlobalSink stores the valid scores straight into the score rows.
struct GlobalSink {
  float* __restrict__ scores;
  int64_t row0, ld;
  __device__ void put(int r, int s, int, float score, bool valid) const {
    if (valid) scores[(row0 + r) * ld + s] = score;
  }
  __device__ void skip(int) const {}
};

// The kernel's dynamic LDS (the same array in every function that names it).
__device__ inline uint8_t* dyn_lds() {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  return smem;
}

// The persistent kernel's sink: with `defer` (uniform), the block's scores
// go to slot slot0 + r of an LDS stage (64 floats each, from byte data_off)
// and the ballot of valid tokens to the slot's mask (from byte mask_off), to
// be written out once every key of the segment has been read
// (flush_scores); otherwise as GlobalSink.  The stage is named by 32-bit LDS
// offsets: a generic pointer would cost the kernel a register pair it does
// not have.
struct ScoreSink {
  bool defer;
  uint32_t data_off, mask_off;
  int slot0;
  float* __restrict__ scores;
  int64_t row0, ld;
  __device__ void put(int r, int s, int lane, float score, bool valid) const {
    if (defer) {
      reinterpret_cast<float*>(dyn_lds() + data_off)[(slot0 + r) * kWave + lane] = score;
      const uint64_t m = __ballot(valid);
      if (lane == 0) reinterpret_cast<uint64_t*>(dyn_lds() + mask_off)[slot0 + r] = m;
    } else if (valid) {
      scores[(row0 + r) * ld + s] = score;
    }
  }
  __device__ void skip(int r) const {
    if (defer) {
      // every lane writes the same zero mask; the zero is made here (a
      // hoisted constant would hold a register pair through the loop)
      uint32_t z = 0;
      asm volatile("" : "+v"(z));
      uint32_t* m = reinterpret_cast<uint32_t*>(dyn_lds() + mask_off) + 2 * (slot0 + r);
      m[0] = z;
      m[1] = z;
    }
  }
};

template <bool SCALED, typename Sink>
__device__ inline void score_block(const Keys& kk, const int64_t (&off)[2], const uint8_t* q_lds,
                                   const float* w_lds, int nr, int s_base, int pos_first,
                                   int64_t ld_last, const Sink& sink, int lane, const float* ksc = nullptr) {
  // Unrolled over the at most kMaxUnitRows rows: as a loop with score stores
  // and no loads, the compiler would wait for every load in flight (the next
  // block's keys included) before entering it.
#pragma unroll
  for (int r = 0; r < kMaxUnitRows; ++r) {
    if (r >= nr) break;
    const int pos_r = (int)min<int64_t>((int64_t)pos_first + r, ld_last);
    if (s_base > pos_r) {
      sink.skip(r);
      continue;
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) acc[i][jj] = f32x16{};
    // the query operand in the keys' dim mapping (bf16 keys: 16 ks + 8 g; fp8: 64 g + 8 ks)
    const uint8_t* qa = q_lds + r * kRowBytesLds + (lane & 31) * kHeadStrideLds + (lane >> 5) * (SCALED ? 128 : 16);
    constexpr int kStepBytes = SCALED ? 16 : 32;
    // The sibling wave on this SIMD is usually in its epilogue (VALU); issuing
    // this row's MFMAs first keeps the matrix core fed (prefill indexer -1.6%).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(qa + ks * kStepBytes);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(qa + 32 * kHeadStrideLds + ks * kStepBytes);
      acc[0][0] = mfma32(a0, kk.v[0][ks], acc[0][0]);
      acc[0][1] = mfma32(a1, kk.v[0][ks], acc[0][1]);
      acc[1][0] = mfma32(a0, kk.v[1][ks], acc[1][0]);
      acc[1][1] = mfma32(a1, kk.v[1][ks], acc[1][1]);
    }
    __builtin_amdgcn_s_setprio(0);
    // Accumulator (i, lane) of a 32x32 tile holds head 8*(i/4) + 4*(lane/32) + i%4
    // and token column lane%32.
    const float* wr = w_lds + r * kHeads + 4 * (lane >> 5);
    float part[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      part[nt] = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 wq = *reinterpret_cast<const f32x4*>(wr + mt * 32 + 8 * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) part[nt] += wq[e] * relu_bits(acc[nt][mt][4 * q4 + e]);
        }
    }
    // Each token's head sum is split over lanes l and l + 32.  One swap of the
    // upper half of part[0] with the lower half of part[1] puts both halves of
    // token l (first 32 tokens) in lane l < 32 and of token l (last 32) in
    // lane l >= 32, so after one add lane l holds the score of token s_base + l.
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                     false, false);
    float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int nt = lane >> 5;
    // a token's non-negative scale factors out of the ReLU and the head sum
    if (SCALED) score *= nt ? ksc[1] : ksc[0];
    const int s = s_base + lane;
    sink.put(r, s, lane, score, s <= pos_r && (nt ? off[1] : off[0]) >= 0);
  }
}

// Scores of one key step from its key registers (fp8 codes are converted to
// bf16 first and each token's scale applied to its scores).
template <typename Sink>
__device__ inline void score_keys(const Keys& kk, const int64_t (&off)[2], const uint8_t* q_lds,
                                  const float* w_lds, int nr, int s_base, int pos_first, int64_t ld_last,
                                  const Sink& sink, int lane) {
  score_block<false>(kk, off, q_lds, w_lds, nr, s_base, pos_first, ld_last, sink, lane);
}

template <typename Sink>
__device__ inline void score_keys(const Keys8& k8, const int64_t (&off)[2], const uint8_t* q_lds,
                                  const float* w_lds, int nr, int s_base, int pos_first, int64_t ld_last,
                                  const Sink& sink, int lane) {
  Keys kk;
  keys_from_fp8(kk, k8);
  score_block<true>(kk, off, q_lds, w_lds, nr, s_base, pos_first, ld_last, sink, lane, k8.sc);
}

// fp8 queries against fp8 keys on v_mfma_scale_f32_32x32x64_f8f6f4 (scales
// 1): per row two 64-dim k steps for each of the four 32x32 (heads, tokens)
// tiles.  A lane's 32 codes of step i are dims 64 g + 32 i .. +31 (g = lane
// half) in both operands, the keys' load layout: the keys' codes enter the
// contraction as loaded.  The query heads' power-of-two scales are in the
// staged weights and each token's key scale multiplies its score, as in
// score_block<true>.
__device__ inline i32x8 join8(u32x4 lo, u32x4 hi) {
  return __builtin_bit_cast(i32x8, u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

__device__ inline f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <typename Sink>
__device__ inline void score_keys_fp8q(const Keys8& k8, const int64_t (&off)[2], const uint8_t* q_lds,
                                       const float* w_lds, int nr, int s_base, int pos_first, int64_t ld_last,
                                       const Sink& sink, int lane) {
  i32x8 kb[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int i = 0; i < 2; ++i) kb[nt][i] = join8(k8.v[nt][2 * i], k8.v[nt][2 * i + 1]);
#pragma unroll
  for (int r = 0; r < kMaxUnitRows; ++r) {
    if (r >= nr) break;
    const int pos_r = (int)min<int64_t>((int64_t)pos_first + r, ld_last);
    if (s_base > pos_r) {
      sink.skip(r);
      continue;
    }
    const uint8_t* qa = q_lds + r * kRowBytesLds8 + (lane & 31) * kHeadStrideLds8 + (lane >> 5) * 64;
    i32x8 qa8[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint8_t* p = qa + mt * 32 * kHeadStrideLds8 + i * 32;
        qa8[mt][i] = join8(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 16));
      }
    f32x16 acc[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[nt][mt] = f32x16{};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[nt][mt] = mfma32_fp8(qa8[mt][i], kb[nt][i], acc[nt][mt]);
    __builtin_amdgcn_s_setprio(0);
    const float* wr = w_lds + r * kHeads + 4 * (lane >> 5);
    float part[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      part[nt] = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 wq = *reinterpret_cast<const f32x4*>(wr + mt * 32 + 8 * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) part[nt] += wq[e] * relu_bits(acc[nt][mt][4 * q4 + e]);
        }
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                     false, false);
    const int nt = lane >> 5;
    const float score = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * (nt ? k8.sc[1] : k8.sc[0]);
    const int s = s_base + lane;
    sink.put(r, s, lane, score, s <= pos_r && (nt ? off[1] : off[0]) >= 0);
  }
}

// Quantised staging of one unit's query rows for fp8 contraction: each head's
// 128 dims are scaled by 2^-e, e the smallest exponent with the head's
// largest magnitude <= 448 * 2^e (0 for an all-zero head), and rounded to
// e4m3 codes (nearest, ties to even); 2^e goes into the head's staged
// weight.  A thread takes 8 dims (16 bytes) of one head, the 16 threads of a
// head are 16 consecutive lanes.
__device__ inline void stage_fp8_queries(const uint16_t* __restrict__ qsrc, const float* __restrict__ wsrc,
                                         int nr, uint8_t* qd, float* wd, int tid, int nthreads) {
  const int n_chunks = nr * kHeads * 16;
  for (int c0 = 0; c0 < n_chunks; c0 += nthreads) {
    const int c = c0 + tid;
    const bool in = c < n_chunks;
    const int r = c / (kHeads * 16), h = (c / 16) % kHeads, ch = c % 16;
    u32x4 raw = in ? *reinterpret_cast<const u32x4*>(qsrc + ((r * kHeads + h) * kDim + ch * 8)) : u32x4{};
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(raw[j] << 16);
      x[2 * j + 1] = __uint_as_float(raw[j] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    int k = 0;
    const float mant = frexpf(amax, &k);  // amax = mant * 2^k, mant in [0.5, 1)
    const int e = amax == 0.f ? 0 : (mant <= 0.875f ? k - 9 : k - 8);
    s16x2 pk[2] = {{0, 0}, {0, 0}};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      pk[j] = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk[j], ldexpf(x[4 * j], -e), ldexpf(x[4 * j + 1], -e),
                                                       1.0f, false);
      pk[j] = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk[j], ldexpf(x[4 * j + 2], -e),
                                                       ldexpf(x[4 * j + 3], -e), 1.0f, true);
    }
    if (in) {
      *reinterpret_cast<uint2*>(qd + r * kRowBytesLds8 + h * kHeadStrideLds8 + ch * 8) =
          uint2{__builtin_bit_cast(uint32_t, pk[0]), __builtin_bit_cast(uint32_t, pk[1])};
      if (ch == 0) wd[r * kHeads + h] = ldexpf(wsrc[r * kHeads + h], e);
    }
  }
}

template <bool KFP8>
__global__ __launch_bounds__(kThreads, 2) void index_scores_bf16_mfma(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, int pt_stride, int page_size, int num_pages,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_base, int64_t k_page_stride, int64_t k_row_stride,
    float* __restrict__ scores, int64_t ld, int row_group, int row_lo, int row_hi) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* q_lds = smem;
  float* w_lds = reinterpret_cast<float*>(smem + (size_t)row_group * kRowBytesLds);

  const int b = blockIdx.x;
  const int q0 = cu_q[b];
  const int q_len = cu_q[b + 1] - q0;
  // this group's rows, clipped to the window [row_lo, row_hi)
  const int g0 = blockIdx.y * row_group;
  const int r0 = max(g0, row_lo - q0), r1 = min(min(q_len, g0 + row_group), row_hi - q0);
  if (r0 >= r1) return;
  const int nr = r1 - r0;
  const int pos_first = seq_lens[b] - q_len + r0;
  const int64_t ld_last = ld - 1;
  const int pos_last = (int)min<int64_t>((int64_t)pos_first + nr - 1, ld_last);
  const int k0 = blockIdx.z * kKeysPerBlock;
  if (k0 > pos_last) return;  // uniform across the block: causal skip

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t row0 = (int64_t)q0 + r0;

  // 1. Query rows -> LDS (padded per head; the pad slot repeats chunk 15).
  {
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(q_idx + row0 * kHeads * kDim);
    const int n_slots = nr * kRowSlots;
    for (int base = 0; base < n_slots; base += kThreads) {
      const int slot = base + tid;
      const int r = slot / kRowSlots, rem = slot - r * kRowSlots;
      const int h = rem / kHeadSlots, ch = min(rem - h * kHeadSlots, 15);
      if (slot < n_slots)
        copy16_to_lds(qsrc + ((r * kHeads + h) * kDim + ch * 8) * 2, smem + (base + wave * kWave) * 16);
    }
  }
  float wv[2] = {0.f, 0.f};  // nr * 64 <= 512 weights, two per thread
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (tid + k * kThreads < nr * kHeads) wv[k] = w[row0 * kHeads + tid + k * kThreads];

  // 2. Page lookups for this wave's tokens, then the first step's 16 key loads.
  int64_t off[kSteps][2];
#pragma unroll
  for (int j = 0; j < kSteps; ++j)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int s = k0 + (j * kWaves + wave) * kKeysPerStep + nt * 32 + (lane & 31);
      off[j][nt] = s <= pos_last ? token_offset(page_table, pt_stride, page_size, num_pages, b, s,
                                                k_page_stride, k_row_stride)
                                 : -1;
    }
  // Both steps' keys go out at once (32 loads per lane).
  KeyRegs<KFP8> kk[kSteps];
#pragma unroll
  for (int j = 0; j < kSteps; ++j)
    load_keys(kk[j], off[j], k_base, lane, k0 + (j * kWaves + wave) * kKeysPerStep, page_size, k_row_stride);
  // Everything issued before those key loads (the copies above) is complete.
  static_assert(kSteps * kLoadsPerStep<KFP8> == (KFP8 ? 20 : 32), "vmcnt below");
  if (KFP8) asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (tid + k * kThreads < nr * kHeads) w_lds[tid + k * kThreads] = wv[k];
  lds_barrier();  // q and w visible to every wave; the keys stay in flight

  // 3. Steps of 64 tokens: every row of the group against the step's keys.
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    const int s_base = k0 + (j * kWaves + wave) * kKeysPerStep;
    if (s_base > pos_last) break;                        // later steps are further right
    score_keys(kk[j], off[j], q_lds, w_lds, nr, s_base, pos_first, ld_last, GlobalSink{scores, row0 - row_lo, ld},
               lane);
  }
}

// Persistent form, used for every batch: one workgroup of eight waves per CU.
// A request's query rows are cut into units of up to rg consecutive rows (the
// whole draft at decode, eight rows of a prefill chunk); a unit's work is the
// 64-token key blocks up to its last row's position.  Each workgroup takes an
// equal share of all units' blocks (concatenated unit after unit), so no
// workgroup is empty and none waits for a second round.  The share is walked
// in segments of one unit: the unit's query rows and weights are staged in LDS
// (all units of the share at once when they fit), then wave w scores blocks
// w, w+8, ... of the segment with the page lookups two blocks ahead and the
// key loads one block ahead.  A segment's scores go straight to the score
// rows, or (DEFER) are held in the staged-row slots the segment leaves
// unused and written in one burst once its keys are read.
constexpr int kFlatWaves = 8;
constexpr int kFlatThreads = kFlatWaves * kWave;

// A lane's two tokens in a block: s = blk_tok0 + 32 nt + lane % 32.  Their
// page ids are loaded unconditionally (the table index is clamped to the
// request's row, so every load is in bounds) and only checked when the
// offsets are formed: no branch depends on a load, so the loads can stay in
// flight while the wave does other work.  Vector loads complete in issue
// order, so a wave sends a block's page ids before the keys of the block
// ahead of it; forming that block's offsets then never waits on keys.
__device__ inline void block_pages(int (&pid)[2], int blk_tok0, const int32_t* __restrict__ page_table,
                                   int pt_stride, int page_size, int b, int lane) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int s = blk_tok0 + nt * 32 + (lane & 31);
    pid[nt] = page_table[(int64_t)b * pt_stride + min(s / page_size, pt_stride - 1)];
  }
}

// Offsets of those tokens from their page ids, as token_offset gives them
// (-1 past pos_last, past the table row, or for a page id outside the pool).
__device__ inline void block_offsets(int64_t (&off)[2], const int (&pid)[2], int blk_tok0, int pos_last,
                                     int pt_stride, int page_size, int num_pages, int64_t page_stride,
                                     int64_t row_stride, int lane) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int s = blk_tok0 + nt * 32 + (lane & 31);
    const int lp = s / page_size;
    const bool ok = s <= pos_last && lp < pt_stride && pid[nt] >= 0 && pid[nt] < num_pages;
    off[nt] = ok ? (int64_t)pid[nt] * page_stride + (int64_t)(s - lp * page_size) * row_stride : -1;
  }
}


// Last request b in [0, B) whose first block is at or below blk (the owner of
// block blk; requests without blocks are passed over).  pre is in LDS.
__device__ inline int last_at_or_below(const int* pre, int B, int blk) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= blk) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

struct FlatBlock {
  int u, tok;       // unit and its first token of the block
  int pid[2];       // page ids of this lane's two tokens (loads possibly in flight)
  int64_t off[2];   // their offsets, once formed
};

// Unit and page-id loads of block blk, walking forward from unit u_from.
__device__ inline void prep_pages(FlatBlock& x, int blk, int u_from, const int* pre, const int* ub,
                                  const int32_t* __restrict__ page_table, int pt_stride, int page_size,
                                  int lane) {
  int u = u_from;
  while (pre[u + 1] <= blk) ++u;
  x.u = u;
  x.tok = (blk - pre[u]) * kKeysPerStep;
  block_pages(x.pid, x.tok, page_table, pt_stride, page_size, ub[u], lane);
}

// prep_pages, or for a block past the wave's range the same two loads of
// table entries that exist (request 0): every path issues the same loads, so
// the compiler's wait counts stay exact.
__device__ inline void prep_pages_or_none(FlatBlock& x, bool valid, int blk, int u_from, const int* pre,
                                          const int* ub, const int32_t* __restrict__ page_table,
                                          int pt_stride, int page_size, int lane) {
  if (valid) {
    prep_pages(x, blk, u_from, pre, ub, page_table, pt_stride, page_size, lane);
  } else {
    x.u = u_from;
    x.tok = 0;
    block_pages(x.pid, 0, page_table, pt_stride, page_size, 0, lane);
  }
}

// Offsets of block x from its page ids (waits for those loads only).
__device__ inline void finish_block(FlatBlock& x, const int* unr, const int* upf, int64_t ld_last,
                                     int pt_stride, int page_size, int num_pages, int64_t page_stride,
                                     int64_t row_stride, int lane) {
  const int pos_last = (int)min<int64_t>((int64_t)upf[x.u] + unr[x.u] - 1, ld_last);
  block_offsets(x.off, x.pid, x.tok, pos_last, pt_stride, page_size, num_pages, page_stride, row_stride, lane);
}

// Block exclusive scan over the workgroup of one int per thread (carry added);
// returns this thread's exclusive prefix and adds the total to carry.
__device__ inline int flat_excl_scan(int v, int* wsum, int& carry, int lane, int wave) {
  const int x = (int)wave_incl_scan((uint32_t)v);
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  int before = carry, all = 0;
#pragma unroll
  for (int w = 0; w < kFlatWaves; ++w) {
    const int c = wsum[w];
    before += w < wave ? c : 0;
    all += c;
  }
  carry += all;
  __syncthreads();
  return before + x - v;
}

// Segments of at least this many blocks hold their scores back when they fit
// (for fewer the write burst buys nothing and its latency shows).
constexpr int kDeferMinBlocks = 64;

// Writes a segment's held-back scores: row r of block lo + b from stage slot
// b * rg + r, 16 bytes per thread and step, the blocks in order so each
// row's stores run contiguously; tokens whose mask bit is clear are not
// written.
__device__ inline void flush_scores(const float* sdata, const uint64_t* smask, int lo, int hi, int rg, int u0,
                                    const int* pre, const int* unr, const int* uq0, float* __restrict__ scores,
                                    int64_t ld, int row_lo, int tid, int nthreads) {
  const int items = (hi - lo) * rg * 16;
  int u = u0;
  for (int q = tid; q < items; q += nthreads) {
    const int bi = q / (rg * 16), rem = q - bi * rg * 16, r = rem >> 4, c = rem & 15;
    const int blk = lo + bi;
    while (pre[u + 1] <= blk) ++u;  // blocks grow with q: walk forward
    if (r >= unr[u]) continue;
    const uint32_t bits = (uint32_t)(smask[bi * rg + r] >> (4 * c)) & 0xFu;
    if (bits == 0) continue;
    const float* src = sdata + (bi * rg + r) * kWave + 4 * c;
    float* dst = scores + ((int64_t)uq0[u] - row_lo + r) * ld + (int64_t)(blk - pre[u]) * kKeysPerStep + 4 * c;
    if (bits == 0xFu && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(src);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((bits >> e) & 1u) dst[e] = src[e];
    }
  }
}

// Scores of one key step: fp8 queries (QFP8, fp8 keys only) on the fp8
// matrix cores, else score_keys.
template <bool QFP8, typename K, typename Sink>
__device__ inline void score_step(const K& kk, const int64_t (&off)[2], const uint8_t* q_lds, const float* w_lds,
                                  int nr, int s_base, int pos_first, int64_t ld_last, const Sink& sink, int lane) {
  if constexpr (QFP8) score_keys_fp8q(kk, off, q_lds, w_lds, nr, s_base, pos_first, ld_last, sink, lane);
  else score_keys(kk, off, q_lds, w_lds, nr, s_base, pos_first, ld_last, sink, lane);
}

// QFP8: the query rows are staged as fp8 codes (stage_fp8_queries) and
// contracted on the fp8 matrix cores; fp8 keys only.
// DEFER: segments may hold their scores back (the launcher instantiates it
// for units of up to four rows; longer units keep the direct stores).
template <bool KFP8, bool QFP8, bool DEFER>
__global__ __launch_bounds__(kFlatThreads, 1) void index_scores_flat(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int B,
    const int32_t* __restrict__ page_table, int pt_stride, int page_size, int num_pages,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_base, int64_t k_page_stride, int64_t k_row_stride,
    float* __restrict__ scores, int64_t ld, int rg, int nslots, int u_max, int row_lo, int row_hi) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // LDS: nslots staged units (query rows, then their weights), then the tables.
  uint8_t* q_area = smem;
  static_assert(!QFP8 || KFP8, "fp8 queries contract with fp8 keys");
  float* w_area = reinterpret_cast<float*>(smem + (size_t)nslots * rg * kQRowBytes<QFP8>);
  int* rq0 = reinterpret_cast<int*>(w_area + nslots * rg * kHeads);  // [B] first row in the window
  int* rql = rq0 + B;                                             // [B] its rows in the window
  int* rpf = rql + B;                                             // [B] position of the first
  int* ubase = rpf + B;                                           // [B+1] first unit of each request
  int* pre = ubase + B + 1;                                       // [u_max+1] first block of each unit
  int* uq0 = pre + u_max + 1;                                     // [u_max] first row of the unit
  int* unr = uq0 + u_max;                                         // [u_max] rows in the unit
  int* upf = unr + u_max;                                         // [u_max] position of its first row
  int* ub = upf + u_max;                                          // [u_max] its request
  int* wsum = ub + u_max;                                         // [kFlatWaves]
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t ld_last = ld - 1;

  // 1. Units: runs of up to rg consecutive rows of one request, counting only
  //    rows inside [row_lo, row_hi).  When no request has more than rg rows
  //    (decode, drafts), unit u is request u (a request without rows in the
  //    window is an empty unit) and no scan is needed.
  const bool per_request = u_max == B;
  int n_units = 0;
  if (per_request) {
    for (int bb = tid; bb < B; bb += kFlatThreads) {
      const int q0 = cu_q[bb], q1 = cu_q[bb + 1];
      const int lo = max(q0, row_lo), hi = min(q1, row_hi);
      rq0[bb] = lo;
      rql[bb] = max(0, hi - lo);
      rpf[bb] = seq_lens[bb] - (q1 - q0) + (lo - q0);
      ubase[bb] = bb;
    }
    n_units = B;
  } else {
    for (int c0 = 0; c0 < B; c0 += kFlatThreads) {
      const int bb = c0 + tid;
      int nu = 0;
      if (bb < B) {
        const int q0 = cu_q[bb], q1 = cu_q[bb + 1];
        const int lo = max(q0, row_lo), hi = min(q1, row_hi), ql = max(0, hi - lo);
        rq0[bb] = lo;
        rql[bb] = ql;
        rpf[bb] = seq_lens[bb] - (q1 - q0) + (lo - q0);
        nu = ql > 0 ? (ql + rg - 1) / rg : 0;
      }
      const int e = flat_excl_scan(nu, wsum, n_units, lane, wave);
      if (bb < B) ubase[bb] = e;
    }
    n_units = min(n_units, u_max);  // rows beyond the host bound are not scored
  }
  if (tid == 0) ubase[B] = n_units;
  __syncthreads();
  // 2. Per unit: rows, position, and its 64-token blocks, ceil(min(pos_last + 1, ld) / 64).
  int carry = 0;
  for (int c0 = 0; c0 < n_units; c0 += kFlatThreads) {
    const int u = c0 + tid;
    int nb = 0;
    if (u < n_units) {
      const int b = per_request ? u : last_at_or_below(ubase, B, u), j = u - ubase[b];
      const int nr = min(rg, rql[b] - rg * j);
      const int pf = rpf[b] + rg * j;
      uq0[u] = rq0[b] + rg * j;
      unr[u] = nr;
      upf[u] = pf;
      ub[u] = b;
      const int64_t n = min<int64_t>((int64_t)pf + nr, ld);
      nb = (nr > 0 && n > 0) ? (int)((n + kKeysPerStep - 1) / kKeysPerStep) : 0;  // an empty unit has none
    }
    const int e = flat_excl_scan(nb, wsum, carry, lane, wave);
    if (u < n_units) pre[u] = e;
  }
  if (tid == 0) pre[n_units] = carry;
  __syncthreads();
  const int per = (carry + (int)gridDim.x - 1) / (int)gridDim.x;
  const int start = (int)blockIdx.x * per, end = min(carry, start + per);

  if (start >= end) return;

  // 3. The units the share touches are staged in LDS all at once when they
  //    fit (slot = unit - first staged unit); otherwise the share is walked
  //    one unit at a time through slot 0.
  const int u_first = last_at_or_below(pre, n_units, start), u_last = last_at_or_below(pre, n_units, end - 1);
  const bool all_staged = u_last - u_first + 1 <= nslots;
  int lo = start, u0 = u_first;
  while (lo < end) {
    const int hi = all_staged ? end : min(end, pre[u0 + 1]);
    const int u_hi = all_staged ? u_last : u0;
    // The staged-row slots this segment leaves unused hold its scores back
    // when they all fit: they leave in one burst once every key of the
    // segment has been read, instead of as 256-byte writes between the key
    // loads (written between them, decode128's 17.8 MB of scores cost 23-25
    // us of the stream).
    const int n_used = u_hi - u0 + 1;
    const size_t free_bytes = (size_t)(nslots - n_used) * rg * kQRowBytes<QFP8>;
    const bool defer = DEFER && hi - lo >= kDeferMinBlocks &&
                       (size_t)(hi - lo) * rg * (kWave * sizeof(float) + sizeof(uint64_t)) <= free_bytes;
    // (scalar: the values come from LDS tables the compiler cannot see are uniform)
    const uint32_t sdata_off = __builtin_amdgcn_readfirstlane((uint32_t)(q_area - smem) +
                                                             (uint32_t)n_used * rg * kQRowBytes<QFP8>);
    const uint32_t smask_off =
        __builtin_amdgcn_readfirstlane(sdata_off + (uint32_t)(hi - lo) * rg * kWave * sizeof(float));
    // This wave's blocks lo + wave + 8 i < hi.  A, B, C: the block being scored
    // and the next two (keys of B in flight, page ids of C in flight).  The
    // first three blocks' page ids go out together; then A's keys, the
    // staging copies and B's keys.
    int j = lo + wave;
    FlatBlock A{u0, 0, {0, 0}, {-1, -1}}, Bk = A, C = A;
    prep_pages_or_none(A, j < hi, j, u0, pre, ub, page_table, pt_stride, page_size, lane);
    prep_pages_or_none(Bk, j + kFlatWaves < hi, j + kFlatWaves, A.u, pre, ub, page_table, pt_stride,
                       page_size, lane);
    prep_pages_or_none(C, j + 2 * kFlatWaves < hi, j + 2 * kFlatWaves, Bk.u, pre, ub, page_table, pt_stride,
                       page_size, lane);
#define DSA_FINISH(X) \
  finish_block(X, unr, upf, ld_last, pt_stride, page_size, num_pages, k_page_stride, k_row_stride, lane)
    if (j < hi) DSA_FINISH(A);
    KeyRegs<KFP8> k0, k1;
    load_keys(k0, A.off, k_base, lane, A.tok, page_size, k_row_stride);
    for (int uu = u0; uu <= u_hi; ++uu) {  // query rows and weights -> LDS slot uu - u0
      const int q0 = uq0[uu], nr = unr[uu];
      uint8_t* qd = q_area + (size_t)(uu - u0) * rg * kQRowBytes<QFP8>;
      if constexpr (QFP8) {
        stage_fp8_queries(q_idx + (int64_t)q0 * kHeads * kDim, w + (int64_t)q0 * kHeads, nr, qd,
                          w_area + (size_t)(uu - u0) * rg * kHeads, tid, kFlatThreads);
        continue;
      }
      const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(q_idx + (int64_t)q0 * kHeads * kDim);
      const int n_slots = nr * kRowSlots;  // padded per head; the pad slot repeats chunk 15
      for (int base = 0; base < n_slots; base += kFlatThreads) {
        const int slot = base + tid;
        const int r = slot / kRowSlots, rem = slot - r * kRowSlots;
        const int h = rem / kHeadSlots, ch = min(rem - h * kHeadSlots, 15);
        if (slot < n_slots)
          copy16_to_lds(qsrc + ((r * kHeads + h) * kDim + ch * 8) * 2, qd + (base + wave * kWave) * 16);
      }
      uint8_t* wd = reinterpret_cast<uint8_t*>(w_area + (size_t)(uu - u0) * rg * kHeads);
      const uint8_t* wsrc = reinterpret_cast<const uint8_t*>(w + (int64_t)q0 * kHeads);
      for (int base = 0; base < nr * (kHeads / 4); base += kFlatThreads)
        if (base + tid < nr * (kHeads / 4)) copy16_to_lds(wsrc + (base + tid) * 16, wd + (base + wave * kWave) * 16);
    }

    // B's keys (or, past the range, a harmless read at pool offset 0) go out
    // after the copies on every path, then everything but them is waited
    // for: A's keys, the page ids and the copies.
    if (j + kFlatWaves < hi) DSA_FINISH(Bk);
    load_keys(k1, Bk.off, k_base, lane, Bk.tok, page_size, k_row_stride);
    wait_vmcnt<kLoadsPerStep<KFP8>>();
    lds_barrier();

    // JB: the block's number; past the range (a placeholder block, no valid
    // token) nothing is written anywhere
#define DSA_SCORE(KK, X, JB)                                                                         \
  do {                                                                                               \
    const uint8_t* qx = q_area + (size_t)(X.u - u0) * rg * kQRowBytes<QFP8>;                        \
    const float* wx = w_area + (size_t)(X.u - u0) * rg * kHeads;                                     \
    if constexpr (DEFER)                                                                             \
      score_step<QFP8>(KK, X.off, qx, wx, unr[X.u], X.tok, upf[X.u], ld_last,                        \
                       ScoreSink{defer && (JB) < hi, sdata_off, smask_off,                           \
                                 __builtin_amdgcn_readfirstlane(((JB) - lo) * rg), scores,           \
                                 (int64_t)uq0[X.u] - row_lo, ld},                                    \
                       lane);                                                                        \
    else                                                                                             \
      score_step<QFP8>(KK, X.off, qx, wx, unr[X.u], X.tok, upf[X.u], ld_last,                        \
                       GlobalSink{scores, (int64_t)uq0[X.u] - row_lo, ld}, lane);                    \
  } while (0)
    // Each step issues the page ids two blocks ahead, then the keys one block
    // ahead (into the registers just scored), whether or not those blocks
    // exist, so the compiler's waits before scoring cover exactly the block
    // being scored.  The empty asm statements pin the issue order: page ids,
    // then keys, then the next block's scoring.
    // block j: keys in k0; block j + 8: keys in k1 (in flight); block j + 16:
    // page ids in flight.  The first block is scored before the loop, whose
    // steps each issue loads and then score: every scoring then follows its
    // own wait on the same path.
    wait_vmcnt<kLoadsPerStep<KFP8>>();  // all but the newest block's keys
    DSA_SCORE(k0, A, j);
    while (j + kFlatWaves < hi) {
      j += kFlatWaves;
      A = Bk;
      Bk = C;
      prep_pages_or_none(C, j + 2 * kFlatWaves < hi, j + 2 * kFlatWaves, Bk.u, pre, ub, page_table,
                         pt_stride, page_size, lane);
      asm volatile("" ::: "memory");
      if (j + kFlatWaves < hi) DSA_FINISH(Bk);
      else Bk.off[0] = Bk.off[1] = -1;
      load_keys(k0, Bk.off, k_base, lane, Bk.tok, page_size, k_row_stride);
      asm volatile("" ::: "memory");
      wait_vmcnt<kLoadsPerStep<KFP8>>();
      DSA_SCORE(k1, A, j);
      if (j + kFlatWaves >= hi) break;
      j += kFlatWaves;
      A = Bk;
      Bk = C;
      prep_pages_or_none(C, j + 2 * kFlatWaves < hi, j + 2 * kFlatWaves, Bk.u, pre, ub, page_table,
                         pt_stride, page_size, lane);
      asm volatile("" ::: "memory");
      if (j + kFlatWaves < hi) DSA_FINISH(Bk);
      else Bk.off[0] = Bk.off[1] = -1;
      load_keys(k1, Bk.off, k_base, lane, Bk.tok, page_size, k_row_stride);
      asm volatile("" ::: "memory");
      wait_vmcnt<kLoadsPerStep<KFP8>>();
      DSA_SCORE(k0, A, j);
    }
#undef DSA_SCORE
#undef DSA_FINISH
    lds_barrier();  // every wave is done with the staged rows and the stage
    if (DEFER && defer) {
      flush_scores(reinterpret_cast<const float*>(smem + sdata_off), reinterpret_cast<const uint64_t*>(smem + smask_off),
                   lo, hi, rg, u0, pre, unr, uq0, scores, ld, row_lo, tid, kFlatThreads);
      lds_barrier();  // the stage is read before the next segment's copies land there
    }
    lo = hi;
    if (lo < end) u0 = last_at_or_below(pre, n_units, lo);
  }
}

// f32 path on the vector ALUs: one thread per (row, token).
__global__ __launch_bounds__(256) void index_scores_f32_valu(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, int B, int pt_stride, int page_size, int num_pages,
    const float* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_base, int64_t k_page_stride, int64_t k_row_stride,
    int n_heads, int head_dim, float* __restrict__ scores, int64_t ld, int row_lo) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* qs = reinterpret_cast<float*>(smem);
  float* ws = qs + n_heads * head_dim;
  const int t = row_lo + (int)blockIdx.y;
  const RowLoc loc = locate_row(cu_q, seq_lens, B, t);
  const int b = loc.b;
  const int pos = (int)min<int64_t>(loc.pos, ld - 1);
  const int s0 = blockIdx.x * 256;
  if (s0 > pos) return;
  for (int i = threadIdx.x; i < n_heads * head_dim; i += 256) qs[i] = q_idx[(int64_t)t * n_heads * head_dim + i];
  for (int i = threadIdx.x; i < n_heads; i += 256) ws[i] = w[(int64_t)t * n_heads + i];
  __syncthreads();
  const int s = s0 + threadIdx.x;
  if (s > pos) return;
  const int64_t off = token_offset(page_table, pt_stride, page_size, num_pages, b, s, k_page_stride, k_row_stride);
  if (off < 0) return;
  const float* k = reinterpret_cast<const float*>(k_base + off);
  float acc = 0.f;
  for (int h = 0; h < n_heads; ++h) {
    float dot = 0.f;
    for (int d = 0; d < head_dim; ++d) dot = fmaf(qs[h * head_dim + d], k[d], dot);
    acc = fmaf(ws[h], fmaxf(dot, 0.f), acc);
  }
  scores[(int64_t)(t - row_lo) * ld + s] = acc;
}


}  // namespace

namespace {

template <bool KFP8, bool QFP8, bool DEFER>
hipError_t launch_flat(const BatchArgs& ba, const void* q_idx, const float* w, const PoolArgs& pool,
                       float* scores, int64_t ld, hipStream_t stream, int row_lo, int row_hi, int rg,
                       int nslots, int64_t u_max, size_t lds) {
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(index_scores_flat<KFP8, QFP8, DEFER>));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((index_scores_flat<KFP8, QFP8, DEFER>), dim3(device_cu_count()), dim3(kFlatThreads), lds,
                     stream, ba.cu_q, ba.seq_lens, ba.batch, ba.page_table, ba.pt_stride, ba.page_size,
                     ba.num_pages, static_cast<const uint16_t*>(q_idx), w,
                     static_cast<const uint8_t*>(pool.base), pool.page_stride, pool.row_stride,
                     scores, ld, rg, nslots, (int)u_max, row_lo, row_hi);
  return hipGetLastError();
}

template <bool KFP8, bool QFP8>
hipError_t launch_index_scores_mfma(const BatchArgs& ba, const void* q_idx, const float* w,
                                    const PoolArgs& pool, float* scores, int64_t ld,
                                    hipStream_t stream, int row_lo, int row_hi) {
  if (ba.max_q_len >= 1) {
    // Units of up to rg rows (the whole draft for decode-sized q_len, eight
    // rows -- the most whose query rows fit in LDS -- for long prefill chunks,
    // so each key block loaded serves eight rows); up to 8 units staged at
    // once, as many as fit next to the tables.
    const int rg = ba.max_q_len <= 8 ? ba.max_q_len : 8;
    const int64_t u_max = (int64_t)ba.batch * ((ba.max_q_len + rg - 1) / rg);
    const size_t tables = ((size_t)(4 * (int64_t)ba.batch + 1 + 5 * u_max + 1 + kFlatWaves) * sizeof(int) + 15) / 16 * 16;
    const size_t per_unit = (size_t)rg * (kQRowBytes<QFP8> + kHeads * sizeof(float));
    const size_t avail = tables < 160 * 1024 ? 160 * 1024 - tables : 0;
    const int nslots = (int)std::min<size_t>(8, avail / per_unit);
    const size_t lds = tables + (size_t)nslots * per_unit;
    // Units of up to four rows (decode, short drafts) may hold their scores
    // back when a workgroup's share can reach kDeferMinBlocks blocks (bounded
    // from the host's batch bounds); longer units, and launches too small for
    // that, store them as they are made.
    const int64_t max_blocks = u_max * (((int64_t)ba.max_seq_len + kKeysPerStep - 1) / kKeysPerStep);
    const bool defer = rg <= 4 && max_blocks >= (int64_t)kDeferMinBlocks * device_cu_count();
    if (nslots >= 1)
      return defer ? launch_flat<KFP8, QFP8, true>(ba, q_idx, w, pool, scores, ld, stream, row_lo, row_hi, rg,
                                                    nslots, u_max, lds)
                   : launch_flat<KFP8, QFP8, false>(ba, q_idx, w, pool, scores, ld, stream, row_lo, row_hi, rg,
                                                     nslots, u_max, lds);
  }
  // fp8 queries have no grid form: the API refuses such launches up front
  // (index_scores_fp8q_fits)
  if (QFP8) return hipErrorNotSupported;
  // Row groups: the whole draft for decode-sized q_len, four rows for long
  // prefill chunks (LDS: 17 KB per staged row).
  int rg = ba.max_q_len <= 8 ? ba.max_q_len : 4;
  if (rg < 1) rg = 1;
  const size_t lds = (size_t)rg * kRowBytesLds + (size_t)rg * kHeads * sizeof(float);
  // Token chunks outermost: the early chunks, which every request has, are
  // dispatched first and the empty tails of short requests last, so that they
  // do not hold dispatch slots while real work waits.
  dim3 grid(ba.batch, (ba.max_q_len + rg - 1) / rg,
            (ba.max_seq_len + kKeysPerBlock - 1) / kKeysPerBlock);
  if (grid.y == 0 || grid.z == 0) return hipSuccess;
  hipError_t e = ensure_max_lds(reinterpret_cast<const void*>(index_scores_bf16_mfma<KFP8>));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(index_scores_bf16_mfma<KFP8>, grid, dim3(kThreads), lds, stream,
                     ba.cu_q, ba.seq_lens, ba.page_table, ba.pt_stride, ba.page_size, ba.num_pages,
                     static_cast<const uint16_t*>(q_idx), w, static_cast<const uint8_t*>(pool.base),
                     pool.page_stride, pool.row_stride, scores, ld, rg, row_lo, row_hi);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scores_bf16(const BatchArgs& ba, const void* q_idx, const float* w,
                                    const PoolArgs& pool, float* scores, int64_t ld,
                                    hipStream_t stream, int row_lo, int row_hi, bool q_fp8) {
  if (q_fp8) return launch_index_scores_mfma<true, true>(ba, q_idx, w, pool, scores, ld, stream, row_lo, row_hi);
  return pool.format == 2
             ? launch_index_scores_mfma<true, false>(ba, q_idx, w, pool, scores, ld, stream, row_lo, row_hi)
             : launch_index_scores_mfma<false, false>(ba, q_idx, w, pool, scores, ld, stream, row_lo, row_hi);
}

bool index_scores_fp8q_fits(const BatchArgs& ba) {
  const int rg = ba.max_q_len <= 8 ? std::max(ba.max_q_len, 1) : 8;
  const int64_t u_max = (int64_t)ba.batch * ((ba.max_q_len + rg - 1) / rg);
  const size_t tables = ((size_t)(4 * (int64_t)ba.batch + 1 + 5 * u_max + 1 + kFlatWaves) * sizeof(int) + 15) / 16 * 16;
  const size_t per_unit = (size_t)rg * (kRowBytesLds8 + kHeads * sizeof(float));
  return tables + per_unit <= 160 * 1024;
}

hipError_t launch_index_scores_f32(const BatchArgs& ba, const void* q_idx, const float* w,
                                   const PoolArgs& pool, int n_heads, int head_dim, float* scores,
                                   int64_t ld, hipStream_t stream, int row_lo, int row_hi) {
  const size_t lds = (size_t)(n_heads * head_dim + n_heads) * sizeof(float);
  dim3 grid((ba.max_seq_len + 255) / 256, row_hi - row_lo);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL(index_scores_f32_valu, grid, dim3(256), lds, stream, ba.cu_q, ba.seq_lens,
                     ba.page_table, ba.batch, ba.pt_stride, ba.page_size, ba.num_pages,
                     static_cast<const float*>(q_idx), w, static_cast<const uint8_t*>(pool.base),
                     pool.page_stride, pool.row_stride, n_heads, head_dim, scores, ld, row_lo);
  return hipGetLastError();
}

}  // namespace dsa
