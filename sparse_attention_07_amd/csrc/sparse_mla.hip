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
// MFMA kernel.  A workgroup owns one query row, NW blocks of 16 heads (one
// per wave) and a range of the selected rows.  Tiles of 32 rows are gathered
// into LDS (fp8 rows are decoded to bf16 on the way, value = e4m3 * block
// scale) and shared by all waves.  Per tile each wave computes
// S^T = rows x q^T with v_mfma_f32_16x16x32_bf16 (rows on M, heads on N, the
// 576 dims as K), runs the online softmax in registers, and accumulates
// O += P V with P as the A operand straight from the S^T accumulators.  The V
// operand needs eight rows per lane for one output column; each lane reads
// eight 16-byte row pieces and regroups them, so that MFMA instance c of a
// group covers output columns 8*(lane%16) + c.  When the rows of a query are
// split across workgroups, each writes (m, l, unnormalised O) partials and a
// second kernel merges them by log-sum-exp.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kD = kDc + kDr;
constexpr int kTileRows = 32;
constexpr int kRowLds = kD * 2 + 16;                 // 1168 B: consecutive rows start 36 banks apart
constexpr int kTileLds = kTileRows * kRowLds;        // 37376 B
constexpr float kNegInf = -__builtin_inff();

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

template <int NW, bool FP8>
__global__ __launch_bounds__(NW * kWave) void sparse_mla_mfma(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, int B, int pt_stride, int page_size, int num_pages,
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_base, int64_t kv_page_stride,
    int64_t kv_row_stride, const int32_t* __restrict__ idx, int K, int H, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws, int splits,
    int rows_per_split) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileLds];
  __shared__ int64_t row_off[kTileRows];

  const int t = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int head0 = (blockIdx.y * NW + wave) * 16;
  const int sp = blockIdx.z;
  const int j_begin = sp * rows_per_split;
  const int j_end = min(K, j_begin + rows_per_split);
  const int b = find_request(cu_q, B, t);
  const int pos = row_position(cu_q, seq_lens, b, t);

  // q as the B operand of S^T: lane (head c16, group g) holds dims ks*32 + g*8 .. +7.
  bf16x8 qreg[18];
  {
    const uint16_t* qp = q + ((int64_t)t * H + head0 + c16) * kD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
  }

  f32x4 o[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[i][c] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;

#pragma unroll 1
  for (int j0 = j_begin; j0 < j_end; j0 += kTileRows) {
    if (tid < kTileRows) {
      const int j = j0 + tid;
      int64_t off = -1;
      if (j < j_end) {
        const int s = idx[(int64_t)t * K + j];
        if (s >= 0 && s <= pos)
          off = token_offset(page_table, pt_stride, page_size, num_pages, b, s, kv_page_stride,
                             kv_row_stride);
      }
      row_off[tid] = off;
    }
    __syncthreads();
    if constexpr (!FP8) {
      for (int c = tid; c < kTileRows * 72; c += NW * kWave) {
        const int r = c / 72, ch = c - r * 72;
        const int64_t off = row_off[r];
        u32x4 v = u32x4{};
        if (off >= 0) v = *reinterpret_cast<const u32x4*>(kv_base + off + ch * 16);
        *reinterpret_cast<u32x4*>(tile + r * kRowLds + ch * 16) = v;
      }
    } else {
      // 32 chunks of 16 e4m3 latent bytes and 8 chunks of bf16 rope per row.
      for (int c = tid; c < kTileRows * 40; c += NW * kWave) {
        const int r = c / 40, ch = c - r * 40;
        const int64_t off = row_off[r];
        if (ch < 32) {
          u32x4 v = u32x4{};
          float sc = 0.f;
          if (off >= 0) {
            v = *reinterpret_cast<const u32x4*>(kv_base + off + ch * 16);
            sc = *reinterpret_cast<const float*>(kv_base + off + 512 + (ch >> 3) * 4);
          }
          u32x4 lo, hi;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t x = v[w];
            const uint32_t p0 = pack_bf16x2(e4m3_to_f32(x & 0xFFu) * sc, e4m3_to_f32((x >> 8) & 0xFFu) * sc);
            const uint32_t p1 = pack_bf16x2(e4m3_to_f32((x >> 16) & 0xFFu) * sc, e4m3_to_f32(x >> 24) * sc);
            if (w < 2) { lo[2 * w] = p0; lo[2 * w + 1] = p1; }
            else { hi[2 * w - 4] = p0; hi[2 * w - 3] = p1; }
          }
          *reinterpret_cast<u32x4*>(tile + r * kRowLds + ch * 32) = lo;
          *reinterpret_cast<u32x4*>(tile + r * kRowLds + ch * 32 + 16) = hi;
        } else {
          u32x4 v = u32x4{};
          if (off >= 0) v = *reinterpret_cast<const u32x4*>(kv_base + off + 528 + (ch - 32) * 16);
          *reinterpret_cast<u32x4*>(tile + r * kRowLds + 1024 + (ch - 32) * 16) = v;
        }
      }
    }
    __syncthreads();

    // S^T (rows x heads): accumulator r of lane = row nt*16 + 4g + r, head c16.
    f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint8_t* ap = tile + (nt * 16 + c16) * kRowLds + g * 16;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        s[nt] = mfma16(*reinterpret_cast<const bf16x8*>(ap + ks * 64), qreg[ks], s[nt]);
    }
    float x[8];
    float mt = kNegInf;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = row_off[nt * 16 + 4 * g + r] >= 0 ? s[nt][r] * scale_log2 : kNegInf;
        x[nt * 4 + r] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const bool none = m_new == kNegInf;
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8 pa;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = none ? 0.f : exp2f(x[i] - m_new);
      psum += p;
      pa[i] = (__bf16)p;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // Rescale O: its accumulator r holds head 4g + r.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int G = 0; G < 4; ++G)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[G][c][r] *= a;
    }

    // O += P V.  K slot (g, i) of the A operand is tile row 4g + i (i < 4) or
    // 16 + 4g + i - 4 (i >= 4), matching the S^T accumulator layout.
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      bf16x8 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = (i < 4) ? (4 * g + i) : (16 + 4 * g + i - 4);
        v[i] = *reinterpret_cast<const bf16x8*>(tile + j * kRowLds + G * 256 + c16 * 16);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bf16x8 bc;
#pragma unroll
        for (int i = 0; i < 8; ++i) bc[i] = v[i][c];
        o[G][c] = mfma16(pa, bc, o[G][c]);
      }
    }
    __syncthreads();
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g + r;
      const float lh = __shfl(l_run, h);
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      uint16_t* op = out + ((int64_t)t * H + head0 + h) * kDc + c16 * 8;
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        u32x4 pk;
#pragma unroll
        for (int c = 0; c < 4; ++c) pk[c] = pack_bf16x2(o[G][2 * c][r] * inv, o[G][2 * c + 1][r] * inv);
        *reinterpret_cast<u32x4*>(op + G * 128) = pk;
      }
    }
    if (lse != nullptr && lane < 16)
      lse[(int64_t)t * H + head0 + lane] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : kNegInf;
  } else {
    // Partials: ws[((t*H + head)*splits + sp)] = {512 floats O, m, l, pad to 516}
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * g + r;
      float* wp = ws + (((int64_t)t * H + head0 + h) * splits + sp) * 516 + c16 * 8;
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        f32x4 lo = {o[G][0][r], o[G][1][r], o[G][2][r], o[G][3][r]};
        f32x4 hi = {o[G][4][r], o[G][5][r], o[G][6][r], o[G][7][r]};
        *reinterpret_cast<f32x4*>(wp + G * 128) = lo;
        *reinterpret_cast<f32x4*>(wp + G * 128 + 4) = hi;
      }
    }
    if (lane < 16) {
      float* wp = ws + (((int64_t)t * H + head0 + lane) * splits + sp) * 516 + 512;
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

// Waves (16-head blocks) per workgroup: the largest of 4, 2, 1 that divides
// the number of head blocks, so every head is covered exactly once.  (A wave
// needs ~400 registers with its 16x576 q slice and 16x512 f32 accumulator,
// so one wave per SIMD; eight waves per workgroup would spill.)
static int mla_waves(int head_blocks) {
  for (int nw = 4; nw > 1; nw >>= 1)
    if (head_blocks % nw == 0) return nw;
  return 1;
}

MlaPlan plan_sparse_mla(int num_q_rows, int n_heads, int k, int dc, bool prefill) {
  MlaPlan p{1, k, 0};
  if (dc != kDc || n_heads % 16 != 0 || k <= 0 || num_q_rows <= 0) return p;
  const int nw = mla_waves(n_heads / 16);
  const int64_t blocks = (int64_t)num_q_rows * (n_heads / (16 * nw));
  int splits = 1;
  if (!prefill) {
    const int64_t target = nw >= 4 ? 256 : 1024;
    const int max_splits = k / 128 > 1 ? k / 128 : 1;
    int64_t want = (target + blocks - 1) / blocks;
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

template <int NW, bool FP8>
static void launch_mla(dim3 grid, hipStream_t stream, const BatchArgs& ba, const void* q,
                       const PoolArgs& kv, const int32_t* idx, int k, int n_heads, float scale_log2,
                       void* out, float* lse, void* ws, const MlaPlan& plan) {
  hipLaunchKernelGGL((sparse_mla_mfma<NW, FP8>), grid, dim3(NW * kWave), 0, stream, ba.cu_q,
                     ba.seq_lens, ba.page_table, ba.batch, ba.pt_stride, ba.page_size, ba.num_pages,
                     static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(kv.base),
                     kv.page_stride, kv.row_stride, idx, k, n_heads, scale_log2,
                     static_cast<uint16_t*>(out), lse, static_cast<float*>(ws), plan.splits,
                     plan.rows_per_split);
}

hipError_t launch_sparse_mla_bf16(const BatchArgs& ba, const void* q, const PoolArgs& kv,
                                  const int32_t* idx, int k, int n_heads, float sm_scale,
                                  void* out, float* lse, void* ws, const MlaPlan& plan,
                                  hipStream_t stream) {
  const int hb = n_heads / 16;
  const int nw = mla_waves(hb);
  dim3 grid(ba.num_q_rows, hb / nw, plan.splits);
  const float sl2 = sm_scale * kLog2e;
  const bool fp8 = kv.format == 2;
#define DSA_MLA_CASE(N)                                                                        \
  case N:                                                                                      \
    if (fp8) launch_mla<N, true>(grid, stream, ba, q, kv, idx, k, n_heads, sl2, out, lse, ws, plan); \
    else launch_mla<N, false>(grid, stream, ba, q, kv, idx, k, n_heads, sl2, out, lse, ws, plan);   \
    break;
  switch (nw) {
    DSA_MLA_CASE(1)
    DSA_MLA_CASE(2)
    DSA_MLA_CASE(4)
  }
#undef DSA_MLA_CASE
  hipError_t e = hipGetLastError();
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
