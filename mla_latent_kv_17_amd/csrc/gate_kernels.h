// Kernels of the MoE gate and their argument block (the launches are in
// api.hip).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace mla {

// MoE gate (s_i = softmax over the routed experts of u^T e_i; the top_k
// largest kept, g_i = s_i).  Affinities in two steps as in the append: fp32
// partial sums over 512-wide chunks of d_model into the caller's workspace,
// then per token the chunk sums, the softmax and the selection.
constexpr int kGateChunk = 512;  // width of the d_model chunks of the partial sums
constexpr int kGateMaxExperts = 256;
constexpr int kGateMaxTopK = 16;
struct GateArgs {
  const void* u;   // [tokens][d_model]
  const void* e;   // [n_experts][d_model] expert centroids
  float* part;     // [chunks][tokens][part_stride]
  int32_t* idx;    // [tokens][top_k]
  float* weight;   // [tokens][top_k]
  float* scores;   // [tokens][n_experts] or null
  int tokens, d_model, n_experts, top_k;
  int chunks;  // partial sums per token: d_model slices of kslice (the last shorter)
  int kslice;       // a multiple of 64
  int part_stride;  // n_experts rounded up to a multiple of 4 (16-byte rows)
};
constexpr int kGateTallM = 128;        // tokens per workgroup of gate_proj_tall
constexpr int kGateTallMinTokens = 768;  // from this many tokens on, gate_proj_tall
__global__ void gate_proj_mfma(const GateArgs a);  // bf16 inputs, few tokens
template <int kNT>  // ceil(n_experts / 32)
__global__ void gate_proj_tall(const GateArgs a);  // bf16 inputs, many tokens
__global__ void gate_proj_f32(const GateArgs a);   // fp32 inputs
template <int kS4, int kL>  // experts per lane / 4, lanes per token
__global__ void gate_finish(const GateArgs a);
constexpr int kGateWideFinishMaxTokens = 2047;  // up to this many tokens: 64 lanes per token

}  // namespace mla
