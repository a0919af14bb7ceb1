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
//  * the affinities U E^T as fp32 partial sums over slices of d_model in the
//    caller's workspace, on the matrix cores (exact products, fp32 sums):
//    - gate_proj_mfma (few tokens): one workgroup per (64 experts, 512-wide
//      slice, 32 tokens) through proj_chunk_bf16, so that even one token
//      tile spreads the centroid read (the traffic) over many CUs;
//    - gate_proj_tall (many tokens): one workgroup per (64 tokens, slice of
//      d_model) covering every expert, looping over its slice in 64-wide
//      stages staged through LDS, so that each token row is read once and
//      the partial sums stay few; the centroids (n_experts x d_model, 1.6 MB
//      for DeepSeek-V2) are re-read from L2.
//  * gate_finish: one wave per token.  Lane l owns experts l, l+64, l+128,
//    l+192: the slice sums, the softmax (max, exp, sum across the wave),
//    then top_k rounds of a wave argmax.  The selection compares the fp32
//    affinities, not the rounded scores: the softmax is strictly increasing
//    in each affinity, so the order is the scores' order, and two distinct
//    affinities never tie through the rounding of exp.  Equal affinities
//    rank the lower expert index first.  Cross-lane steps use DPP moves
//    within rows of 16 lanes and four lane reads across the rows.
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

// Many tokens: workgroup (slice x, token tile y) computes the affinities of
// tokens 64y .. 64y+63 with every expert over d_model slice x.  Per 64-wide
// stage the 64 token rows and the centroid rows (2 * kTilesPerWave * 32, the
// ones past n_experts zero) are loaded as 128-byte rows, 8 rows per wave
// load, into one of two LDS buffers (rows padded to 144 bytes so that the
// operand reads, 8 rows per pass at one column, hit distinct banks); the
// loads of the next two stages are in flight while one is multiplied.  Wave w
// owns token tile (w & 1) and expert tiles (w >> 1) * kTilesPerWave + j,
// accumulating over all four 16-wide k-steps of a stage.
template <int kTilesPerWave>
__global__ void __launch_bounds__(256) gate_proj_tall(const GateArgs a) {
  constexpr int kRow = 144;
  constexpr int kER = 2 * kTilesPerWave * 32;  // staged centroid rows
  constexpr int kLoads = (kGateTallM + kER) / 32;
  __shared__ __attribute__((aligned(16))) uint8_t us[2][kGateTallM * kRow];
  __shared__ __attribute__((aligned(16))) uint8_t es[2][kER * kRow];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, n32 = lane & 31, sub = lane >> 3, piece = lane & 7;
  const int T = a.tokens, N = a.n_experts, NT = (N + 31) / 32;
  const int m0 = blockIdx.y * kGateTallM;
  const int k_lo = blockIdx.x * a.kslice;
  const int stages = (min(a.d_model, k_lo + a.kslice) - k_lo) / 64;
  const uint16_t* u = (const uint16_t*)a.u;
  const uint16_t* e = (const uint16_t*)a.e;
  const int64_t dm = a.d_model;
  // two register sets hold the next two stages' rows while one is multiplied
  u32x4 va[kLoads], vb[kLoads];
  auto load = [&](u32x4 (&v)[kLoads], int st) __attribute__((always_inline)) {
    const int k0 = k_lo + 64 * st;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = 32 * i + 8 * wave + sub;
      const uint16_t* src = i < kGateTallM / 32 ? u + min(m0 + r, T - 1) * dm : e + min(r - kGateTallM, N - 1) * dm;
      v[i] = *(const u32x4*)(src + k0 + 8 * piece);
    }
  };
  auto store = [&](const u32x4 (&v)[kLoads], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int r = 32 * i + 8 * wave + sub;
      const bool live = i < kGateTallM / 32 ? m0 + r < T : r - kGateTallM < N;
      uint8_t* dst = i < kGateTallM / 32 ? &us[b][r * kRow] : &es[b][(r - kGateTallM) * kRow];
      *(MLA_LDS u32x4*)(dst + 16 * piece) = live ? v[i] : u32x4{0, 0, 0, 0};
    }
  };
  const int mt = wave & 1, nt0 = (wave >> 1) * kTilesPerWave;
  f32x16 acc[kTilesPerWave];
#pragma unroll
  for (int j = 0; j < kTilesPerWave; ++j) acc[j] = f32x16{};
  auto compute = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = 32 * ks + 16 * g;
      const bf16x8 av = *(const MLA_LDS bf16x8*)&us[b][(32 * mt + n32) * kRow + kb];
#pragma unroll
      for (int j = 0; j < kTilesPerWave; ++j)
        if (nt0 + j < NT) {
          const bf16x8 bv = *(const MLA_LDS bf16x8*)&es[b][(32 * (nt0 + j) + n32) * kRow + kb];
          acc[j] = mfma32x32x16(av, bv, acc[j]);
        }
    }
  };
  // stage s sits in LDS buffer s & 1 while it is multiplied; stage s + 1 is
  // stored into the other buffer after that (its readers, stage s - 1, are
  // past the barrier), and the freed register set starts loading stage s + 3
  load(va, 0);
  store(va, 0);
  if (stages > 1) load(va, 1);
  if (stages > 2) load(vb, 2);
  __syncthreads();
  for (int st = 0; st < stages; st += 2) {
    compute(0);
    if (st + 1 < stages) {
      store(va, 1);
      if (st + 3 < stages) load(va, st + 3);
    }
    __syncthreads();
    if (st + 1 >= stages) break;
    compute(1);
    if (st + 2 < stages) {
      store(vb, 0);
      if (st + 4 < stages) load(vb, st + 4);
    }
    __syncthreads();
  }
  // D lane l, register i: token (i/4)*8 + 4g + i%4 of the wave's tile, expert n32 of tile nt0 + j
  float* pc = a.part + (int64_t)blockIdx.x * T * N;
#pragma unroll
  for (int j = 0; j < kTilesPerWave; ++j) {
    const int n = 32 * (nt0 + j) + n32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = m0 + 32 * mt + (i >> 2) * 8 + 4 * g + (i & 3);
      if (t < T && n < N) pc[(int64_t)t * N + n] = acc[j][i];
    }
  }
}

template __global__ void gate_proj_tall<1>(const GateArgs);
template __global__ void gate_proj_tall<2>(const GateArgs);
template __global__ void gate_proj_tall<3>(const GateArgs);
template __global__ void gate_proj_tall<4>(const GateArgs);

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

// Lane moves within rows of 16 lanes (every lane has a source in these
// patterns): swap neighbours, swap pairs, mirror within 8, mirror within 16.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(dpp<kCtrl>(__float_as_int(v)));
}

__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Every lane receives the maximum / the sum over the wave (fixed order).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

template <int kCtrl>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = dpp<kCtrl>(v);
  const int oi = dpp<kCtrl>(i);
  if (ranks_before(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// The wave's first-ranked (value, index) pair, returned to every lane.
__device__ __forceinline__ int wave_argmax(float v, int i) {
  argmax_step<kDppXor1>(v, i);
  argmax_step<kDppXor2>(v, i);
  argmax_step<kDppHalfMirror>(v, i);
  argmax_step<kDppMirror>(v, i);
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float rv = lane_f(v, r);
    const int ri = __builtin_amdgcn_readlane(i, r);
    if (ranks_before(rv, ri, bv, bi)) {
      bv = rv;
      bi = ri;
    }
  }
  return bi;
}

}  // namespace

__global__ void __launch_bounds__(256) gate_finish(const GateArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.tokens) return;  // uniform per wave; no barrier in this kernel
  const int N = a.n_experts;
  // the slice sums, slice order fixed, sixteen slices' loads for all four
  // of a lane's experts in flight at a time with no branch between them
  const int64_t cstride = (int64_t)a.tokens * N;
  const float* pp = a.part + (int64_t)t * N;
  float x[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.chunks; c0 += 16) {
    float v[4][16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n = min(lane + 64 * u, N - 1);
#pragma unroll
      for (int k = 0; k < 16; ++k) v[u][k] = pp[min(c0 + k, a.chunks - 1) * cstride + n];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 16; ++k) x[u] += c0 + k < a.chunks ? v[u][k] : 0.f;
  }
  bool live[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) live[u] = lane + 64 * u < N;
  // softmax over the routed experts
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (live[u]) m = fmaxf(m, x[u]);
  m = wave_max_dpp(m);
  float z[4], zs = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    z[u] = live[u] ? expf(x[u] - m) : 0.f;
    zs += z[u];
  }
  zs = wave_sum_dpp(zs);
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
    bi = wave_argmax(bv, bi);
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
