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

// Query row t belongs to the request b with cu_q[b] <= t < cu_q[b+1].  The
// search is clamped to [0, B-1] so inconsistent device data cannot index out
// of bounds.
__device__ inline int find_request(const int32_t* __restrict__ cu_q, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Position of row t (request b) in its sequence: seq_len - q_len + j.
__device__ inline int row_position(const int32_t* __restrict__ cu_q,
                                   const int32_t* __restrict__ seq_lens, int b, int t) {
  int q0 = cu_q[b], q1 = cu_q[b + 1];
  return seq_lens[b] - (q1 - q0) + (t - q0);
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

__device__ inline float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace dsa
