// Lightning-indexer scores on gfx950.
//
//   score[t, s] = sum_h w[t, h] * max(0, q_I[t, h, :] . k_I[s, :]),  0 <= s <= pos(t)
//
// (the DSA indexer of lmdeploy PR 4737 "feat: support GLM-5.2", section
// "Changes", and of mlx-lm PR 1419's description; the pages name the
// indexer without a formula and this is its plain reading.)
//
// MFMA kernel (bf16, 64 heads x 128 dims).  One workgroup of four waves owns
// one request, a chunk of 256 consecutive cached tokens and a group of up to
// eight consecutive query rows of that request.  Each wave holds the keys of
// 64 tokens in registers, already in the B-operand layout of
// v_mfma_f32_32x32x16_bf16, and reuses them for every row of the group; the
// query rows sit in LDS and feed the A operand (heads on M, tokens on N).
// The ReLU, the per-head weight and the sum over heads are applied to the
// accumulators in registers: a lane owns one token column and half of the
// heads, so one cross-lane add finishes each score.  Keys are read straight
// from their pages (no copy of the cache), once per row group.
//
// Reduction-index layout: the dot product over the 128 dims is summed in any
// order, so the k slots of each MFMA are mapped to dims such that every lane
// reads 128 contiguous bytes of one key: lane l (group g = l/32) supplies dims
// g*64 + ks*8 .. +7 in step ks.  The query operand uses the same mapping.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

namespace {

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kWaves = 4;
constexpr int kKeysPerWave = 64;
constexpr int kKeysPerBlock = kWaves * kKeysPerWave;  // 256
constexpr int kHeadStrideLds = kDim * 2 + 16;         // 272 B: rows start on different banks
constexpr int kRowBytesLds = kHeads * kHeadStrideLds; // 17408 B per staged query row

__global__ __launch_bounds__(kWaves * kWave) void index_scores_bf16_mfma(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, int pt_stride, int page_size, int num_pages,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_base, int64_t k_page_stride, int64_t k_row_stride,
    float* __restrict__ scores, int64_t ld, int row_group) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* q_lds = smem;
  float* w_lds = reinterpret_cast<float*>(smem + (size_t)row_group * kRowBytesLds);

  const int b = blockIdx.z;
  const int q0 = cu_q[b];
  const int q_len = cu_q[b + 1] - q0;
  const int r0 = blockIdx.y * row_group;
  if (r0 >= q_len) return;
  const int nr = min(row_group, q_len - r0);
  const int pos_first = seq_lens[b] - q_len + r0;
  const int64_t ld_last = ld - 1;
  const int pos_last = (int)min<int64_t>((int64_t)pos_first + nr - 1, ld_last);
  const int k0 = blockIdx.x * kKeysPerBlock;
  if (k0 > pos_last) return;  // uniform across the block: causal skip

  // Stage the group's query rows (16 B chunks) and weights into LDS.
  const int64_t row0 = (int64_t)q0 + r0;
  for (int c = threadIdx.x; c < nr * kHeads * 16; c += kWaves * kWave) {
    const int r = c >> 10, h = (c >> 4) & 63, ch = c & 15;
    const u32x4 v = *reinterpret_cast<const u32x4*>(q_idx + ((row0 + r) * kHeads + h) * kDim + ch * 8);
    *reinterpret_cast<u32x4*>(q_lds + r * kRowBytesLds + h * kHeadStrideLds + ch * 16) = v;
  }
  for (int c = threadIdx.x; c < nr * kHeads; c += kWaves * kWave) w_lds[c] = w[row0 * kHeads + c];
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s_base = k0 + wave * kKeysPerWave;
  if (s_base > pos_last) return;  // no barrier follows

  // Keys of this wave's 64 tokens: two 32-token column tiles, eight K steps.
  bf16x8 bk[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int s = s_base + nt * 32 + (lane & 31);
    int64_t off = -1;
    if (s <= pos_last)
      off = token_offset(page_table, pt_stride, page_size, num_pages, b, s, k_page_stride, k_row_stride);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bk[nt][ks] = bf16x8{};
    if (off >= 0) {
      const uint8_t* p = k_base + off + (lane >> 5) * 128;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) bk[nt][ks] = *reinterpret_cast<const bf16x8*>(p + ks * 16);
    }
  }

  for (int r = 0; r < nr; ++r) {
    const int pos_r = (int)min<int64_t>((int64_t)pos_first + r, ld_last);
    if (s_base > pos_r) continue;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    const uint8_t* qa = q_lds + r * kRowBytesLds + (lane & 31) * kHeadStrideLds + (lane >> 5) * 128;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(qa + ks * 16);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(qa + 32 * kHeadStrideLds + ks * 16);
      acc[0][0] = mfma32(a0, bk[0][ks], acc[0][0]);
      acc[0][1] = mfma32(a1, bk[0][ks], acc[0][1]);
      acc[1][0] = mfma32(a0, bk[1][ks], acc[1][0]);
      acc[1][1] = mfma32(a1, bk[1][ks], acc[1][1]);
    }
    // Accumulator (i, lane) of a 32x32 tile holds head 8*(i/4) + 4*(lane/32) + i%4
    // and token column lane%32.
    const float* wr = w_lds + r * kHeads + 4 * (lane >> 5);
    float wv[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) wv[mt][i] = wr[mt * 32 + 8 * (i >> 2) + (i & 3)];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float part = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) part += wv[mt][i] * fmaxf(acc[nt][mt][i], 0.f);
      part += __shfl_xor(part, 32);
      const int s = s_base + nt * 32 + (lane & 31);
      if (lane < 32 && s <= pos_r) scores[(row0 + r) * ld + s] = part;
    }
  }
}

// f32 path on the vector ALUs: one thread per (row, token).
__global__ __launch_bounds__(256) void index_scores_f32_valu(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ page_table, int B, int pt_stride, int page_size, int num_pages,
    const float* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_base, int64_t k_page_stride, int64_t k_row_stride,
    int n_heads, int head_dim, float* __restrict__ scores, int64_t ld) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* qs = reinterpret_cast<float*>(smem);
  float* ws = qs + n_heads * head_dim;
  const int t = blockIdx.y;
  const int b = find_request(cu_q, B, t);
  const int pos = (int)min<int64_t>(row_position(cu_q, seq_lens, b, t), ld - 1);
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
  scores[(int64_t)t * ld + s] = acc;
}

}  // namespace

hipError_t launch_index_scores_bf16(const BatchArgs& ba, const void* q_idx, const float* w,
                                    const PoolArgs& pool, float* scores, int64_t ld,
                                    hipStream_t stream) {
  // Row groups: one row per group for single-token decode, the whole draft
  // for short multi-token rows, four rows for long prefill chunks.
  int rg = ba.max_q_len <= 8 ? ba.max_q_len : 4;
  if (rg < 1) rg = 1;
  const size_t lds = (size_t)rg * kRowBytesLds + (size_t)rg * kHeads * sizeof(float);
  dim3 grid((ba.max_seq_len + kKeysPerBlock - 1) / kKeysPerBlock,
            (ba.max_q_len + rg - 1) / rg, ba.batch);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(index_scores_bf16_mfma),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(index_scores_bf16_mfma, grid, dim3(kWaves * kWave), lds, stream,
                     ba.cu_q, ba.seq_lens, ba.page_table, ba.pt_stride, ba.page_size, ba.num_pages,
                     static_cast<const uint16_t*>(q_idx), w, static_cast<const uint8_t*>(pool.base),
                     pool.page_stride, pool.row_stride, scores, ld, rg);
  return hipGetLastError();
}

hipError_t launch_index_scores_f32(const BatchArgs& ba, const void* q_idx, const float* w,
                                   const PoolArgs& pool, int n_heads, int head_dim, float* scores,
                                   int64_t ld, hipStream_t stream) {
  const size_t lds = (size_t)(n_heads * head_dim + n_heads) * sizeof(float);
  dim3 grid((ba.max_seq_len + 255) / 256, ba.num_q_rows);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL(index_scores_f32_valu, grid, dim3(256), lds, stream, ba.cu_q, ba.seq_lens,
                     ba.page_table, ba.batch, ba.pt_stride, ba.page_size, ba.num_pages,
                     static_cast<const float*>(q_idx), w, static_cast<const uint8_t*>(pool.base),
                     pool.page_stride, pool.row_stride, n_heads, head_dim, scores, ld);
  return hipGetLastError();
}

}  // namespace dsa
