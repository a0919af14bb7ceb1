// MoE gate: which routed experts each token uses, and with what weight.
//
// deepforge.srivtx.xyz "DeepSeek-V2", section 1, "Make the feed-forward layer
// sparse" and its formula box "Top-K routed MoE layer": the affinity of token
// u and expert i is u^T e_i (e_i the expert's centroid), s_i is the softmax
// of the affinities over the routed experts, and the K_r largest s_i are
// kept with gate value g_i = s_i (no renormalisation; every other g_i is 0).
// DeepSeek-V2 routes over 160 experts and keeps 6; its 2 shared experts take
// every token and need no gate.
//
// Two launches:
//  * gate_proj_mfma (bf16 inputs) / gate_proj_f32: the affinities U E^T as
//    fp32 partial sums over 512-wide chunks of d_model in the caller's
//    workspace (proj_chunk_bf16: LDS-staged coalesced rows, matrix cores).
//    The centroids (n_experts x d_model) are the traffic, read once.
//  * gate_finish: one wave per token.  Lane l owns experts l, l+64, l+128,
//    l+192: the chunk sums, the softmax (max, exp, sum across the wave),
//    then top_k rounds of a wave argmax.  The selection compares the fp32
//    affinities, not the rounded scores: the softmax is strictly increasing
//    in each affinity, so the order is the scores' order, and two distinct
//    affinities never tie through the rounding of exp.  Equal affinities
//    rank the lower expert index first.
#include "mla_device.h"
#include "gate_kernels.h"
#include "proj_chunk.h"

namespace mla {

static_assert(kGateMaxExperts == 4 * 64, "four experts per lane");
static_assert(kGateChunk == kProjChunk, "the gate's chunk is the projection routine's");

__global__ void __launch_bounds__(256) gate_proj_mfma(const GateArgs a) {
  const uint16_t* e = (const uint16_t*)a.e;
  const int64_t dm = a.d_model;
  auto wrow = [&](int n) __attribute__((always_inline)) -> const uint16_t* { return e + n * dm; };
  proj_chunk_bf16((const uint16_t*)a.u, a.tokens, a.d_model, a.n_experts, wrow, blockIdx.x * 64, blockIdx.y,
                  blockIdx.z * 32, a.part, a.n_experts);
}

// fp32 inputs: wave w of workgroup x computes expert 4x + w of one token
// (grid y): its 64 lanes stride along d_model, then a shuffle sum.
__global__ void __launch_bounds__(256) gate_proj_f32(const GateArgs a) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6), r = blockIdx.y, lane = threadIdx.x & 63;
  if (n >= a.n_experts) return;  // uniform per wave; no barrier follows
  const float* u = (const float*)a.u + (int64_t)r * a.d_model;
  const float* e = (const float*)a.e + (int64_t)n * a.d_model;
  float acc = 0.f;
  for (int k = lane; k < a.d_model; k += 64) acc = fmaf(u[k], e[k], acc);
  acc = wave_sum(acc);
  if (lane == 0) a.part[(int64_t)r * a.n_experts + n] = acc;
}

namespace {

// (v, i) ranks before (w, j): larger value, or equal value and lower index.
__device__ __forceinline__ bool ranks_before(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

}  // namespace

__global__ void __launch_bounds__(256) gate_finish(const GateArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.tokens) return;  // uniform per wave; no barrier in this kernel
  const int N = a.n_experts;
  // the chunk sums, chunk order fixed, eight chunks' loads for all four of a
  // lane's experts in flight at a time with no branch between them
  const int64_t cstride = (int64_t)a.tokens * N;
  const float* pp = a.part + (int64_t)t * N;
  float x[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.chunks; c0 += 8) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = min(lane + 64 * u, N - 1);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[u][k] = pp[min(c0 + k, a.chunks - 1) * cstride + n];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) x[u] += c0 + k < a.chunks ? v[u][k] : 0.f;
  }
  bool live[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) live[u] = lane + 64 * u < N;
  // softmax over the routed experts
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (live[u]) m = fmaxf(m, x[u]);
  m = wave_max(m);
  float z[4], zs = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    z[u] = live[u] ? expf(x[u] - m) : 0.f;
    zs += z[u];
  }
  zs = wave_sum(zs);
  const float inv = 1.0f / zs;
  float s[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) s[u] = z[u] * inv;
  if (a.scores) {
    float* so = a.scores + (int64_t)t * N;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (live[u]) so[lane + 64 * u] = s[u];
  }
  // top_k rounds: the lane's best remaining expert, then the wave's
  bool taken[4] = {!live[0], !live[1], !live[2], !live[3]};
  for (int k = 0; k < a.top_k; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (!taken[u] && ranks_before(x[u], lane + 64 * u, bv, bi)) {
        bv = x[u];
        bi = lane + 64 * u;
      }
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // every lane now holds the winner bi; its owner marks it and writes it
    if ((bi & 63) == lane) {
      const int u = bi >> 6;
      float w = s[0];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q == u) {
          taken[q] = true;
          w = s[q];
        }
      a.idx[(int64_t)t * a.top_k + k] = bi;
      a.weight[(int64_t)t * a.top_k + k] = w;
    }
  }
}

}  // namespace mla
