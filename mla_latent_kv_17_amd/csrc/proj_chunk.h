// One workgroup's share of a skinny product X = H W^T with bf16 rows of
// length d_model on both sides (the tokens' hidden states H, a weight W of
// n_cols rows), used by the cache append and the MoE gate: the fp32 partial
// sums over one 512-wide chunk of d_model for 32 tokens and 32 output
// columns (small tiles, so that even one token tile spreads the weight
// stream over many compute units), on the matrix cores (v_mfma_f32_32x32x16_bf16, exact products,
// fp32 sums).  The row slices are staged in LDS with fully coalesced loads (a
// wave's load is 1 KB of one row; the operands' own lane layout would touch
// 32 rows per load); each of the four waves multiplies a quarter of the
// chunk, and the partial tiles sum through LDS.
#pragma once

#include "mla_device.h"

namespace mla {

constexpr int kProjChunk = 512;

// Workgroup (256 threads) for columns n0 .. n0+31, chunk `chunk`,
// tokens m0 .. m0+31.  wrow(n) is W's row n for n < n_cols; columns at or past
// n_cols, tokens at or past `tokens` and bytes past d_model stage zeros.
// Writes part[(chunk * tokens + r) * part_stride + n] for the valid r, n.
template <typename WRow>
__device__ __forceinline__ void proj_chunk_bf16(const uint16_t* h, int tokens, int d_model, int n_cols, WRow wrow,
                                                int n0, int chunk, int m0, float* part, int part_stride) {
  constexpr int kPad = 33;          // LDS row stride (floats) of the partial tiles
  constexpr int kRow = 1024 + 16;   // LDS row stride (bytes) of the staged operands
  constexpr int kCols = 32;         // output columns per workgroup
  constexpr int kNT = kCols / 32;   // 32-column blocks
  __shared__ __attribute__((aligned(16))) uint8_t ws[kCols * kRow];  // W rows n0 .., this chunk
  __shared__ __attribute__((aligned(16))) uint8_t hs[32 * kRow];  // H rows m0 .. m0+31, this chunk
  __shared__ float red[4][kNT][32 * kPad];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, n32 = lane & 31;
  const int k_lo = chunk * kProjChunk;
  const int klen = min(kProjChunk, d_model - k_lo);  // a multiple of 64
  // ---- staging: every load is issued before the first store
  const int cb = lane * 16;  // byte of the row slice this lane moves
  const bool in_k = cb < 2 * klen;
  u32x4 wv[kCols / 4], hv[8];
#pragma unroll
  for (int i = 0; i < kCols / 4; ++i) {
    const int n = n0 + 4 * i + wave;
    const uint16_t* row = wrow(n < n_cols ? n : 0);
    wv[i] = *(const u32x4*)((const uint8_t*)(row + k_lo) + (in_k ? cb : 0));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = m0 + 4 * i + wave;
    hv[i] = *(const u32x4*)((const uint8_t*)(h + (int64_t)(r < tokens ? r : 0) * d_model + k_lo) + (in_k ? cb : 0));
  }
#pragma unroll
  for (int i = 0; i < kCols / 4; ++i) {
    const bool live = in_k && n0 + 4 * i + wave < n_cols;
    *(MLA_LDS u32x4*)((MLA_LDS uint8_t*)ws + (4 * i + wave) * kRow + cb) = live ? wv[i] : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool live = in_k && m0 + 4 * i + wave < tokens;
    *(MLA_LDS u32x4*)((MLA_LDS uint8_t*)hs + (4 * i + wave) * kRow + cb) = live ? hv[i] : u32x4{0, 0, 0, 0};
  }
  __syncthreads();
  // ---- products: wave w takes k-steps 8w .. 8w+7 of the chunk (16 k each):
  // A = H rows (token n32, k + 8g .. +7), B = W rows (column 32 nt + n32, same k)
  f32x16 acc[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) acc[nt] = f32x16{};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int kb = (16 * (8 * wave + j) + 8 * g) * 2;
    const bf16x8 av = *(const MLA_LDS bf16x8*)((const MLA_LDS uint8_t*)hs + n32 * kRow + kb);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const bf16x8 bv = *(const MLA_LDS bf16x8*)((const MLA_LDS uint8_t*)ws + (32 * nt + n32) * kRow + kb);
      acc[nt] = mfma32x32x16(av, bv, acc[nt]);
    }
  }
  // D lane l, register i: token (i/4)*8 + 4g + i%4 of the tile, column n32 of the 32-column block
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave][nt][((i >> 2) * 8 + 4 * g + (i & 3)) * kPad + n32] = acc[nt][i];
  __syncthreads();
  float* pc = part + (int64_t)chunk * tokens * part_stride;
#pragma unroll
  for (int i = 0; i < kCols / 8; ++i) {
    const int idx = i * 256 + tid;
    const int row = idx / kCols, d = idx % kCols, nt = d >> 5, n = d & 31;
    const float v = red[0][nt][row * kPad + n] + red[1][nt][row * kPad + n] + red[2][nt][row * kPad + n] +
                    red[3][nt][row * kPad + n];
    if (m0 + row < tokens && n0 + d < n_cols) pc[(int64_t)(m0 + row) * part_stride + n0 + d] = v;
  }
}

}  // namespace mla
