// Internal device helpers shared by the gfx950 kernels of the DSA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Request b owning query row t (cu_q[b] <= t < cu_q[b+1]) and the row's
// position seq_len[b] - q_len[b] + (t - cu_q[b]), found by one wave in one
// round of loads per 256 requests: lane i tests request i of each 64-request
// chunk and the owner's values are broadcast from its lane.  Every lane of
// the wave must call it (wave-uniform result).  With inconsistent device data
// (no owner) it returns request B-1, so callers stay in bounds.
struct RowLoc {
  int b, pos;
};

__device__ inline RowLoc locate_row(const int32_t* __restrict__ cu_q,
                                    const int32_t* __restrict__ seq_lens, int B, int t) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int i0 = 0; i0 < B; i0 += 4 * kWave) {
    int lo[4], hi[4], sl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = i0 + c * kWave + lane;
      lo[c] = hi[c] = sl[c] = 0;
      if (i < B) {
        lo[c] = cu_q[i];
        hi[c] = cu_q[i + 1];
        sl[c] = seq_lens[i];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t m = __ballot(lo[c] <= t && t < hi[c]);
      if (m != 0) {
        const int src = __ffsll((unsigned long long)m) - 1;
        const int q0 = __shfl(lo[c], src), q1 = __shfl(hi[c], src), s = __shfl(sl[c], src);
        return RowLoc{i0 + c * kWave + src, s - (q1 - q0) + (t - q0)};
      }
    }
  }
  const int q0 = cu_q[B - 1], q1 = cu_q[B];
  return RowLoc{B - 1, seq_lens[B - 1] - (q1 - q0) + (t - q0)};
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts inside
// each row of 16 lanes, then row broadcasts of lanes 15 and 31).
__device__ inline uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Byte offset of logical token s of request b inside a pool, or -1 when the
// token is not mapped (negative s, logical page beyond the table, or a page
// id outside [0, num_pages)).
__device__ inline int64_t token_offset(const int32_t* __restrict__ page_table, int pt_stride,
                                       int page_size, int num_pages, int b, int s,
                                       int64_t page_stride, int64_t row_stride) {
  if (s < 0) return -1;
  int lp = s / page_size;
  if (lp >= pt_stride) return -1;
  int page = page_table[(int64_t)b * pt_stride + lp];
  if (page < 0 || page >= num_pages) return -1;
  return (int64_t)page * page_stride + (int64_t)(s - lp * page_size) * row_stride;
}

// s_waitcnt vmcnt(N) through the builtin, so that the compiler's own wait
// tracking sees it (an inline-asm wait is opaque to it).  gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt (6:4) and lgkmcnt (11:8) at their maxima.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ inline float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace dsa
