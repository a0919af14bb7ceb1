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
  void* o;     // o_lat [slot][rows][512], slot = b * num_splits + split: fp32, or fp16 if o_f16
  float* lse;  // [slot][rows]
  int o_f16;   // 1: chunk partials written as binary16 (round to nearest even)
  int batch, sq, heads, rows, row_blocks, num_splits, units, max_blocks;
  float softmax_scale, scale_log2;
};

template <int kRows>  // query rows per workgroup: 64, or 32 for launches with few units
__global__ void decode_mfma_bf16(const DecodeArgs a);
__global__ void decode_mfma_fp8(const DecodeArgs a);
constexpr int kDecodeRowsPerWg = 64;  // the fp8 kernel's, and the bf16 kernel's by default
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
  const void* o_part;     // [B][ns][S_q][H][512], fp32 or fp16 (the kernel's template argument)
  const float* lse_part;  // [B][ns][S_q][H]
  float* o_lat;           // [B*S_q][H][512]
  float* lse;             // [B*S_q][H] or null
  int batch, num_splits, rows;  // rows = S_q * H
};
constexpr int kCombineSoloMaxSplits = 16;  // up to this many chunks: one wave per query row
template <typename PT, bool kSolo>  // partial type: float or _Float16
__global__ void split_combine(const CombineArgs a);

struct OutUvArgs {
  const float* o_lat;     // [R][H][512] (unmerged form)
  const void* w;          // [H][128][512]
  void* out;              // [R][H][128], fp32 or (out_bf16) bf16 bits
  int rows, heads;        // R = B * S_q
  // merged form: o_lat = log-sum-exp merge of the chunk partials
  const void* o_part;     // [B][ns][S_q][H][512], fp32 or fp16 (part_f16)
  const float* lse_part;  // [B][ns][S_q][H]
  float* lse;             // [R][H] or null
  int num_splits, sq;
  int out_bf16;           // 1: round the fp32 sums to bf16 (nearest even)
  int part_f16;           // merged form: 1 if the partials are fp16
  int groups;             // merge_out_uv16: workgroups per head (each takes every groups-th 16-row tile)
};
__global__ void out_uv_mfma(const OutUvArgs a);        // bf16 weights, hi/lo split of o_lat
template <typename PT, int kF>  // partial type: float or _Float16; chunks of the first round: 4, or 1 for one chunk
__global__ void merge_out_uv16(const OutUvArgs a);  // the same with the chunk merge on the way (16-row tiles)
template <typename PT>
__global__ void merge_out_uv_few(const OutUvArgs a);  // the same for few query rows and many chunks
constexpr int kMergeFewRows = 8;  // query rows up to which merge_out_uv_few is used beyond 8 chunks
template <bool kMerge>
__global__ void out_uv_f32(const OutUvArgs a);   // fp32 weights

// Explicit form (k = [W_UK c ; k^R], v = W_UV c rebuilt per head, then
// attention on them).  Workspace, per sequence b and head h, with
// tokens = the token capacity (a multiple of 256):
//   K   [B][H][tokens][128] bf16: token-major rebuilt keys (no RoPE part)
//   V^T [B][H][tokens / 32][128][32] bf16: rebuilt values per group of 32
//       tokens, a dimension's 32 values adjacent; position 8 q + 4 k + i of a
//       group holds token 16 k + 4 q + i (q < 4, k < 2, i < 4), the order in
//       which the attention's value product consumes them.
struct ExplicitArgs {
  const uint16_t* q_nope;  // [B*S_q][H][128] bf16
  const uint16_t* q_rope;  // [B*S_q][H][64] bf16
  const uint8_t* latent;   // cache latent rows (bf16)
  const uint8_t* rope;     // cache RoPE-key rows (bf16)
  int64_t lat_bs, lat_rs, rope_bs, rope_rs;  // bytes
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint16_t* w_uk;    // [H][128][512] bf16
  const uint16_t* w_uv;    // [H][128][512] bf16
  uint16_t* k;             // workspace K
  uint16_t* vt;            // workspace V^T
  void* out;               // [B*S_q][H][128], fp32 or (out_bf16) bf16
  float* lse;              // [B*S_q][H] or null
  int batch, sq, heads, max_blocks, tokens;  // tokens: workspace token capacity
  int tiles;               // rebuild: 256-token tiles per sequence
  int qblocks;             // attention: 128-query blocks per sequence
  int out_bf16;
  float scale_log2;        // softmax_scale * log2(e)
};
constexpr int kRebuildTok = 256;  // tokens per rebuild workgroup
constexpr int kRbBlockT = 4, kRbBlockH = 8;  // rebuild placement block: token tiles x heads
constexpr int kAtWaves = 8;       // waves per attention workgroup (32 query tokens each)
constexpr int kExplicitQ = 32 * kAtWaves;  // query tokens per attention workgroup
__global__ void rebuild_kv(const ExplicitArgs a);
__global__ void attend_explicit(const ExplicitArgs a);

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
