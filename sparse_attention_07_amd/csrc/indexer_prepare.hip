// Indexer query/key preparation in one launch: RoPE of every query head, key
// LayerNorm and RoPE, and the key's store into the paged index-key pool at the
// row's position (the fused indexer preparation of lmdeploy PR 4737, section
// "Changes", measured there as a cut of thirteen graph kernels per layer in
// section "DSA indexer fusion"; mlx-lm PR 1419's description fixes the GLM
// indexer's non-interleaved RoPE and LayerNorm eps 1e-6 against DeepSeek-V3.2's
// interleaved RoPE and eps 1e-5).
//
// One workgroup of 256 threads per query row.  Wave 0 normalises the key (one
// or two dims per lane, two-pass mean and variance by wave reductions) into
// LDS while every wave rotates the query heads in 16-element units; after one
// barrier the key's units are rotated from LDS and stored into the pool.  An
// fp8 key pool (page-blocked: P rows of 128 e4m3 codes, then P f32 scales)
// gets the rotated key's codes at scale amax/448 and that scale.
//
// A unit is two 8-element chunks of one head: a rotated unit holds whole
// rotation pairs -- chunks u and u + R/16 when not interleaved (dims i and
// i + R/2), chunks 2u and 2u + 1 when interleaved (dims 2i and 2i + 1) -- and
// uses the eight table entries 8u .. 8u + 7 of the row's position.  Units past
// the rotated dims copy two chunks (skipped when q_out == q_in).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace {

constexpr int kPrepThreads = 256;
constexpr int kPrepMaxDim = 128;

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

struct PrepArgs {
  const int32_t* cu_q;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int batch, pt_stride, page_size, num_pages;
  const uint8_t* q_in;
  uint8_t* q_out;
  const uint8_t* k_in;
  const float* gamma;
  const float* beta;
  float eps;
  const float* cos_tab;
  const float* sin_tab;
  int rope_rows, rope_dim, interleaved;
  int n_heads, head_dim;
  uint8_t* pool;
  int64_t page_stride, row_stride;
  int key_fp8;
};

typedef short __attribute__((ext_vector_type(2))) s16x2;

// Eight elements of one chunk as f32 (bf16: one 16-byte load; f32: two).
template <bool BF16>
__device__ inline void load8(const uint8_t* p, float (&x)[8]) {
  if (BF16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(v[i] << 16);
      x[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
}

// Stores eight f32 values (bf16: rounded to nearest even).
template <bool BF16>
__device__ inline void store8(uint8_t* p, const float (&x)[8]) {
  if (BF16) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * i], x[2 * i + 1]}, bf16x2));
    *reinterpret_cast<u32x4*>(p) = v;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 16) = f32x4{x[4], x[5], x[6], x[7]};
  }
}

// Rotates one unit's pairs in place: (a, b) -> (a c - b s, a s + b c).
__device__ inline void rotate_unit(float (&x0)[8], float (&x1)[8], const float (&c)[8], const float (&s)[8],
                                   bool interleaved) {
  if (!interleaved) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = x0[e], b = x1[e];
      x0[e] = a * c[e] - b * s[e];
      x1[e] = a * s[e] + b * c[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = x0[2 * e], b = x0[2 * e + 1];
      x0[2 * e] = a * c[e] - b * s[e];
      x0[2 * e + 1] = a * s[e] + b * c[e];
      a = x1[2 * e];
      b = x1[2 * e + 1];
      x1[2 * e] = a * c[4 + e] - b * s[4 + e];
      x1[2 * e + 1] = a * s[4 + e] + b * c[4 + e];
    }
  }
}

// Chunks (c0, c1) of unit u and whether it is rotated.
__device__ inline bool unit_chunks(int u, int R, bool interleaved, int& c0, int& c1) {
  const int ru = R / 16;
  if (u < ru) {
    c0 = interleaved ? 2 * u : u;
    c1 = interleaved ? 2 * u + 1 : u + ru;
    return true;
  }
  c0 = R / 8 + 2 * (u - ru);
  c1 = c0 + 1;
  return false;
}

__device__ inline float wave_sum_f32(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

template <bool BF16>
__global__ __launch_bounds__(kPrepThreads) void indexer_prepare_kernel(PrepArgs a) {
  __shared__ float kn[kPrepMaxDim];
  constexpr int es = BF16 ? 2 : 4;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const RowLoc loc = locate_row(a.cu_q, a.seq_lens, a.batch, t);
  const int pos = loc.pos;
  if (pos < 0 || pos >= a.rope_rows) return;  // whole workgroup: no rotation angle for this row
  const int D = a.head_dim, R = a.rope_dim, H = a.n_heads;
  const bool inter = a.interleaved != 0;
  const int upr = D / 16;  // units per head (and per key)

  // Key LayerNorm (wave 0): dims lane and lane + 64.
  if (wave == 0) {
    const uint8_t* kr = a.k_in + (int64_t)t * D * es;
    float x0 = 0.f, x1 = 0.f;
    if (lane < D) x0 = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(kr)[lane])
                            : reinterpret_cast<const float*>(kr)[lane];
    if (lane + 64 < D) x1 = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(kr)[lane + 64])
                                 : reinterpret_cast<const float*>(kr)[lane + 64];
    const float mean = wave_sum_f32(x0 + x1) / (float)D;
    const float d0 = lane < D ? x0 - mean : 0.f, d1 = lane + 64 < D ? x1 - mean : 0.f;
    const float var = wave_sum_f32(d0 * d0 + d1 * d1) / (float)D;
    const float inv = 1.0f / __builtin_sqrtf(var + a.eps);
    if (lane < D) kn[lane] = d0 * inv * a.gamma[lane] + a.beta[lane];
    if (lane + 64 < D) kn[lane + 64] = d1 * inv * a.gamma[lane + 64] + a.beta[lane + 64];
  }

  // Query heads.
  const float* ct = a.cos_tab + (int64_t)pos * (R / 2);
  const float* st = a.sin_tab + (int64_t)pos * (R / 2);
  const bool in_place = a.q_out == a.q_in;
  const int64_t qrow = (int64_t)t * H * D * es;
  for (int it = tid; it < H * upr; it += kPrepThreads) {
    const int h = it / upr, u = it - h * upr;
    int c0, c1;
    const bool rot = unit_chunks(u, R, inter, c0, c1);
    if (!rot && in_place) continue;
    const int64_t base = qrow + (int64_t)h * D * es;
    float x0[8], x1[8];
    load8<BF16>(a.q_in + base + c0 * 8 * es, x0);
    load8<BF16>(a.q_in + base + c1 * 8 * es, x1);
    if (rot) {
      float c[8], s[8];
      const f32x4 ca = *reinterpret_cast<const f32x4*>(ct + 8 * u), cb = *reinterpret_cast<const f32x4*>(ct + 8 * u + 4);
      const f32x4 sa = *reinterpret_cast<const f32x4*>(st + 8 * u), sb = *reinterpret_cast<const f32x4*>(st + 8 * u + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = ca[i];
        c[4 + i] = cb[i];
        s[i] = sa[i];
        s[4 + i] = sb[i];
      }
      rotate_unit(x0, x1, c, s, inter);
    }
    store8<BF16>(a.q_out + base + c0 * 8 * es, x0);
    store8<BF16>(a.q_out + base + c1 * 8 * es, x1);
  }
  __syncthreads();

  // Key: rotate from LDS and store at the row's token slot.
  const int64_t off = token_offset(a.page_table, a.pt_stride, a.page_size, a.num_pages, loc.b, pos,
                                   a.page_stride, a.row_stride);
  if (tid < upr) {
    int c0, c1;
    const bool rot = unit_chunks(tid, R, inter, c0, c1);
    float x0[8], x1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x0[e] = kn[c0 * 8 + e];
      x1[e] = kn[c1 * 8 + e];
    }
    if (rot) {
      float c[8], s[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        c[e] = ct[8 * tid + e];
        s[e] = st[8 * tid + e];
      }
      rotate_unit(x0, x1, c, s, inter);
    }
    if (!a.key_fp8) {
      if (off >= 0) {
        store8<BF16>(a.pool + off + c0 * 8 * es, x0);
        store8<BF16>(a.pool + off + c1 * 8 * es, x1);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // the rotated key back in place (same unit, same thread)
        kn[c0 * 8 + e] = x0[e];
        kn[c1 * 8 + e] = x1[e];
      }
    }
  }
  if (!a.key_fp8) return;
  __syncthreads();
  if (wave != 0) return;
  // fp8 key (D = 128): lane l quantises dims 2l and 2l+1 at scale amax / 448.
  const float v0 = kn[2 * lane], v1 = kn[2 * lane + 1];
  float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  if (off >= 0) {
    s16x2 pk = {0, 0};
    pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, v0 / scale, v1 / scale, 1.0f, false);
    *reinterpret_cast<uint16_t*>(a.pool + off + 2 * lane) = (uint16_t)pk[0];
    if (lane == 0) {
      const int slot = pos % a.page_size;  // off = page * page_stride + slot * row_stride
      *reinterpret_cast<float*>(a.pool + off + (int64_t)(a.page_size - slot) * a.row_stride + slot * 4) = scale;
    }
  }
}

}  // namespace

hipError_t launch_indexer_prepare(const BatchArgs& ba, const void* q_in, void* q_out, const void* k_in,
                                  int format, const float* gamma, const float* beta, float eps,
                                  const float* cos_tab, const float* sin_tab, int rope_rows,
                                  int rope_dim, int interleaved, const PoolArgs& pool, int n_heads,
                                  int head_dim, hipStream_t stream) {
  PrepArgs a;
  a.key_fp8 = pool.format == 2;
  a.cu_q = ba.cu_q;
  a.seq_lens = ba.seq_lens;
  a.page_table = ba.page_table;
  a.batch = ba.batch;
  a.pt_stride = ba.pt_stride;
  a.page_size = ba.page_size;
  a.num_pages = ba.num_pages;
  a.q_in = static_cast<const uint8_t*>(q_in);
  a.q_out = static_cast<uint8_t*>(q_out);
  a.k_in = static_cast<const uint8_t*>(k_in);
  a.gamma = gamma;
  a.beta = beta;
  a.eps = eps;
  a.cos_tab = cos_tab;
  a.sin_tab = sin_tab;
  a.rope_rows = rope_rows;
  a.rope_dim = rope_dim;
  a.interleaved = interleaved;
  a.n_heads = n_heads;
  a.head_dim = head_dim;
  // the pool is written here: the library's pool view is read-only elsewhere
  a.pool = static_cast<uint8_t*>(const_cast<void*>(pool.base));
  a.page_stride = pool.page_stride;
  a.row_stride = pool.row_stride;
  const dim3 grid(ba.num_q_rows), block(kPrepThreads);
  if (format == 1)
    hipLaunchKernelGGL(indexer_prepare_kernel<true>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(indexer_prepare_kernel<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
