// Kernel argument blocks and kernel declarations shared by the host entry
// points and the kernel sources.  Strides inside these blocks are in BYTES.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeArgs {
  const uint16_t* q_lat;   // [B*S_q][H][512]  bf16 bits (fp32 for the f32 path)
  const uint16_t* q_rope;  // [B*S_q][H][64]
  const uint8_t* latent;   // cache latent rows
  const uint8_t* rope;     // cache RoPE-key rows
  const uint8_t* kv_scale_bytes;  // fp8 per-token scales (fp32)
  int64_t lat_bs, lat_rs, rope_bs, rope_rs, scale_bs;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* o;    // o_lat [slot][rows][512], slot = b * num_splits + split
  float* lse;  // [slot][rows]
  int batch, sq, heads, rows, row_blocks, num_splits, units, max_blocks;
  float softmax_scale, scale_log2;
};

__global__ void decode_mfma_bf16(const DecodeArgs a);
__global__ void decode_mfma_fp8(const DecodeArgs a);
constexpr int kDecodeRowsPerWg = 64;
__global__ void decode_f32(const DecodeArgs a);

struct AbsorbArgs {
  const void* q_nope;  // [R][H][128]
  const void* w;       // [H][128][512]
  void* q_lat;         // [R][H][512]
  int rows, heads;     // rows = B * S_q
};
template <bool kOutBf16>
__global__ void absorb_q_mfma(const AbsorbArgs a);   // bf16 inputs
template <bool kOutBf16>
__global__ void absorb_q_f32(const AbsorbArgs a);    // fp32 inputs

struct CombineArgs {
  const float* o_part;    // [B][ns][S_q][H][512]
  const float* lse_part;  // [B][ns][S_q][H]
  float* o_lat;           // [B*S_q][H][512]
  float* lse;             // [B*S_q][H] or null
  int batch, num_splits, rows;  // rows = S_q * H
};
__global__ void split_combine(const CombineArgs a);

struct OutUvArgs {
  const float* o_lat;     // [R][H][512] (unmerged form)
  const void* w;          // [H][128][512]
  void* out;              // [R][H][128], fp32 or (out_bf16) bf16 bits
  int rows, heads;        // R = B * S_q
  // merged form: o_lat = log-sum-exp merge of the chunk partials
  const float* o_part;    // [B][ns][S_q][H][512]
  const float* lse_part;  // [B][ns][S_q][H]
  float* lse;             // [R][H] or null
  int num_splits, sq;
  int out_bf16;           // 1: round the fp32 sums to bf16 (nearest even)
};
__global__ void out_uv_mfma(const OutUvArgs a);        // bf16 weights, hi/lo split of o_lat
__global__ void merge_out_uv_mfma(const OutUvArgs a);  // the same with the chunk merge on the way
template <bool kMerge>
__global__ void out_uv_f32(const OutUvArgs a);   // fp32 weights

// Cache append (c_t = W_DKV h_t, k^R_t = RoPE_p(W_KR h_t), written to the
// paged cache).  Projections in two steps: fp32 partial sums over 512-wide
// chunks of d_model into the caller's workspace, then per token the chunk
// sums, the rotation, the encoding and the paged write.
constexpr int kAppendChunk = 512;
constexpr int kAppendCols = 576;  // W_DKV rows, then W_KR rows
struct AppendArgs {
  const void* h;      // [tokens][d_model]
  const void* w_dkv;  // [512][d_model]
  const void* w_kr;   // [64][d_model]
  float* part;        // [chunks][tokens][576]
  uint8_t* latent;    // cache latent rows (byte strides below)
  uint8_t* rope;      // cache RoPE-key rows
  float* scale;       // fp8: per-token scales
  int64_t lat_bs, lat_rs, rope_bs, rope_rs, scale_bs;  // bytes; scale_bs in floats
  const int32_t* block_table;
  const int32_t* seq_lens;
  int tokens, sq, d_model, chunks, max_blocks;
  double log2_theta;  // log2(rope_theta)
};
__global__ void append_proj_mfma(const AppendArgs a);  // bf16 inputs
__global__ void append_proj_f32(const AppendArgs a);   // fp32 inputs
template <int kFmt>  // 0 fp32, 1 bf16, 2 fp8 cache
__global__ void append_finish(const AppendArgs a);

}  // namespace mla
