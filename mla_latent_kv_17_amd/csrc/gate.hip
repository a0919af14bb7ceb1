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
//    - gate_proj_mfma (few tokens): one workgroup per (32 experts, 512-wide
//      slice, 32 tokens) through proj_chunk_bf16, so that even one token
//      tile spreads the centroid read (the traffic) over many CUs;
//    - gate_proj_tall (many tokens): one workgroup per (128 tokens, slice of
//      d_model) covering every expert, looping over its slice in 64-wide
//      stages staged through LDS, so that each token row is read once, each
//      centroid row staged serves 128 tokens, and the partial sums stay
//      few; the centroids (n_experts x d_model, 1.6 MB for DeepSeek-V2) are
//      re-read from L2.
//  * gate_finish: 16 lanes per token (many tokens) or 64 (few), each lane
//    owning a run of 4 to 16 experts (16-byte loads per slice): the slice
//    sums, the softmax (max, exp, sum across the token's lanes), then top_k
//    rounds of an argmax over 64-bit keys (the affinity's ordered bits, then
//    the complemented index).  The selection compares the fp32
//    affinities, not the rounded scores: the softmax is strictly increasing
//    in each affinity, so the order is the scores' order, and two distinct
//    affinities never tie through the rounding of exp.  Equal affinities
//    rank the lower expert index first.  Cross-lane steps are DPP moves
//    within rows of 16 lanes, plus one lane read per row for 64 lanes.
#include "mla_device.h"
#include "mla_copy.h"
#include "gate_kernels.h"
#include "proj_chunk.h"

namespace mla {

static_assert(kGateMaxExperts == 4 * 64, "four experts per lane");
static_assert(kGateTallM == 4 * 32, "one 32-token tile per wave");
static_assert(kGateChunk == kProjChunk, "the gate's chunk is the projection routine's");

__global__ void __launch_bounds__(256) gate_proj_mfma(const GateArgs a) {
  const uint16_t* e = (const uint16_t*)a.e;
  const int64_t dm = a.d_model;
  auto wrow = [&](int n) __attribute__((always_inline)) -> const uint16_t* { return e + n * dm; };
  proj_chunk_bf16((const uint16_t*)a.u, a.tokens, a.d_model, a.n_experts, wrow, blockIdx.x * 32, blockIdx.y,
                  blockIdx.z * 32, a.part, a.part_stride);
}

// Many tokens: workgroup (slice x, token tile y) computes the affinities of
// tokens 128y .. 128y+127 with every expert over d_model slice x.  Per
// 64-wide stage the 128 token rows and the 32 * kNT centroid rows (rows past
// the last token or expert repeat it; their results are never stored) go
// HBM -> LDS by DMA as 128-byte rows, 1 KB (eight rows) per copy, into a
// ring of kS stage slots, kS - 1 stages in flight while one is multiplied
// (one barrier per stage).  The copies are contiguous in LDS, so the row's
// 16-byte pieces are permuted at the source instead of padding the rows:
// piece p of row r sits at slot p ^ ((r >> 1) & 7), and the operand reads (16
// rows per pass at one piece) hit 16 distinct bank groups.  Wave w owns
// token tile w (32 tokens) against all kNT expert tiles, so each staged
// centroid row serves 128 tokens.  The results leave through LDS: each wave
// writes its tile there and stores rows of 16-byte pieces.
template <int kNT>
__global__ void __launch_bounds__(256) gate_proj_tall(const GateArgs a) {
  constexpr int kRows = kGateTallM + 32 * kNT;             // staged rows per stage
  constexpr int kStage = kRows * 128;                      // bytes of a stage slot
  constexpr int kS = 147456 / kStage < 4 ? 147456 / kStage : 4;  // ring slots
  constexpr int kPer = kRows / 8 / 4;                      // 1 KB copies per wave per stage
  static_assert(kS >= 3 && kPer * 4 * 8 == kRows && kPer * (kS - 2) < 64, "ring shape");
  constexpr int kOutRow = 128 * 4 + 16;                    // output staging row: 128 fp32 + pad
  constexpr int kOutWave = 32 * kOutRow;                   // one wave's output staging
  constexpr int kLds = kS * kStage > 4 * kOutWave ? kS * kStage : 4 * kOutWave;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, n32 = lane & 31;
  const int T = a.tokens, N = a.n_experts;
  const int m0 = blockIdx.y * kGateTallM;
  const int k_lo = blockIdx.x * a.kslice;
  const int stages = (min(a.d_model, k_lo + a.kslice) - k_lo) / 64;
  const int64_t dm = a.d_model;
  const uint32_t lds0 = (uint32_t)(size_t)(MLA_LDS uint8_t*)lds;
  // copy c = kPer wave + k brings rows 8c .. 8c+7: lane i reads source piece
  // (i & 7) ^ swz(row) of row 8c + i / 8 (a fixed address per copy, plus the
  // stage's column offset)
  const uint8_t* src[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int r = 8 * (kPer * wave + k) + (lane >> 3);
    const uint16_t* row = r < kGateTallM ? (const uint16_t*)a.u + min(m0 + r, T - 1) * dm
                                         : (const uint16_t*)a.e + min(r - kGateTallM, N - 1) * dm;
    src[k] = (const uint8_t*)(row + k_lo) + 16 * ((lane & 7) ^ ((r >> 1) & 7));
  }
  auto issue = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      dma16(src[k] + 128 * st, lds0 + (uint32_t)((st % kS) * kStage + (kPer * wave + k) * 1024));
  };
  f32x16 acc[kNT];
#pragma unroll
  for (int j = 0; j < kNT; ++j) acc[j] = f32x16{};
  // operand rows: 32 wave + n32 (tokens), kGateTallM + 32 j + n32 (experts);
  // k-step ks reads piece 2 ks + g
  const int ra = 32 * wave + n32;
  auto compute = [&](int st) __attribute__((always_inline)) {
    const MLA_LDS uint8_t* buf = (const MLA_LDS uint8_t*)lds + (st % kS) * kStage;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int p = 2 * ks + g;
      const bf16x8 av = *(const MLA_LDS bf16x8*)(buf + ra * 128 + 16 * (p ^ ((ra >> 1) & 7)));
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        const int rb = kGateTallM + 32 * j + n32;
        const bf16x8 bv = *(const MLA_LDS bf16x8*)(buf + rb * 128 + 16 * (p ^ ((rb >> 1) & 7)));
        acc[j] = mfma32x32x16(av, bv, acc[j]);
      }
    }
  };
  // stages 0 .. kS-2 go out first; before barrier B_st each wave waits for
  // its copies of stage st (the ones issued after it may stay in flight);
  // after B_st every wave is done with stage st-1, whose slot takes stage
  // st+kS-1
  const int last = stages - 1;
  for (int st = 0; st <= min(kS - 2, last); ++st) issue(st);
  for (int st = 0; st < stages; ++st) {
    wait_groups<kPer, kS - 2>(min(kS - 2, last - st));
    __syncthreads();  // B_st
    if (st + kS - 1 <= last) issue(st + kS - 1);
    compute(st);
  }
  __syncthreads();  // every wave is done with the stage slots
  // out: up to four expert tiles (128 columns) at a time through the wave's
  // own LDS area.  D lane l, register i: token (i/4)*8 + 4g + i%4 of the
  // wave's tile, expert n32 of the tile
  uint8_t* ow = &lds[wave * kOutWave];
  const int ps = a.part_stride;
  float* pc = a.part + (int64_t)blockIdx.x * T * ps;
  const int t0 = m0 + 32 * wave;
#pragma unroll
  for (int p = 0; p < kNT; p += 4) {
#pragma unroll
    for (int j = p; j < p + 4 && j < kNT; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        *(MLA_LDS float*)&ow[((i >> 2) * 8 + 4 * g + (i & 3)) * kOutRow + 4 * (32 * (j - p) + n32)] = acc[j][i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 32 rows x 128 columns: lane l takes 16-byte piece l % 32 of rows 2q + l / 32
    const int cols = min(128, ps - 128 * (p / 4));
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = 2 * q + (lane >> 5), c = 4 * (lane & 31);
      const f32x4 v = *(const MLA_LDS f32x4*)&ow[r * kOutRow + 4 * c];
      if (t0 + r < T && c < cols) *(f32x4*)&pc[(int64_t)(t0 + r) * ps + 128 * (p / 4) + c] = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template __global__ void gate_proj_tall<1>(const GateArgs);
template __global__ void gate_proj_tall<2>(const GateArgs);
template __global__ void gate_proj_tall<3>(const GateArgs);
template __global__ void gate_proj_tall<4>(const GateArgs);
template __global__ void gate_proj_tall<5>(const GateArgs);
template __global__ void gate_proj_tall<6>(const GateArgs);
template __global__ void gate_proj_tall<7>(const GateArgs);
template __global__ void gate_proj_tall<8>(const GateArgs);

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
  if (lane == 0) a.part[(int64_t)r * a.part_stride + n] = acc;
}

namespace {

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)dpp<kCtrl>((int)(uint32_t)v), hi = (uint32_t)dpp<kCtrl>((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// The row's largest key, returned to every lane of the row.
__device__ __forceinline__ uint64_t row_max64(uint64_t v) {
  v = max64(v, dpp64<kDppXor1>(v));
  v = max64(v, dpp64<kDppXor2>(v));
  v = max64(v, dpp64<kDppHalfMirror>(v));
  return max64(v, dpp64<kDppMirror>(v));
}

__device__ __forceinline__ uint64_t lane64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max64_rows(uint64_t v) {
  v = row_max64(v);
  return max64(max64(lane64(v, 0), lane64(v, 16)), max64(lane64(v, 32), lane64(v, 48)));
}

// A key whose unsigned order is the ranking of (affinity, expert): the
// affinity's bits made monotone in its value (-0 taken as +0), then the
// complement of the index, so that of equal affinities the lower index is
// the larger key.  Every key of a finite affinity exceeds 0.
__device__ __forceinline__ uint64_t rank_key(float x, int i) {
  const uint32_t b = __float_as_uint(x + 0.0f);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (0xFFFFFFFFu - (uint32_t)i);
}

}  // namespace

// kL lanes per token (16: four tokens per wave, one per row; 64: one token
// per wave); lane j of a token owns the S = 4 * kS4 experts from S * j on
// (16-byte loads per slice from rows padded to a multiple of 4).
// Reductions by DPP moves within rows, and for 64 lanes the four rows'
// results read from one lane each.  Sixteen lanes per token spend fewer
// instructions per token (many tokens); 64 lanes give each lane fewer
// experts and so a shorter chain (few tokens).
template <int kS4, int kL>
__global__ void __launch_bounds__(256) gate_finish(const GateArgs a) {
  static_assert(kL == 16 || kL == 64, "a row or a wave per token");
  constexpr int S = 4 * kS4, kTpw = 64 / kL;
  const int lane = threadIdx.x & 63, j = lane % kL;
  const int w0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kTpw;  // the wave's first token
  if (w0 >= a.tokens) return;  // uniform per wave; no barrier in this kernel
  const int t = w0 + lane / kL;
  const int tc = min(t, a.tokens - 1);  // rows past the last token compute on it and write nothing
  const int N = a.n_experts, ps = a.part_stride;
  const int e0 = S * j;
  auto vmax = [](float v) __attribute__((always_inline)) { return kL == 16 ? row_max(v) : wave_max_rows(v); };
  auto vsum = [](float v) __attribute__((always_inline)) { return kL == 16 ? row_sum(v) : wave_sum_rows(v); };
  auto kmax = [](uint64_t v) __attribute__((always_inline)) { return kL == 16 ? row_max64(v) : wave_max64_rows(v); };
  // the slice sums in slice order, kRound slices' loads in flight at a time
  // with no branch between them (16 with one run of 4 experts per lane: a
  // 5120-wide d_model in one round of loads)
  constexpr int kRound = kS4 == 1 ? 16 : 8;
  const int64_t cstride = (int64_t)a.tokens * ps;
  const float* pp = a.part + (int64_t)tc * ps;
  f32x4 x[kS4];
#pragma unroll
  for (int q = 0; q < kS4; ++q) x[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.chunks; c0 += kRound) {
    f32x4 v[kRound][kS4];
#pragma unroll
    for (int k = 0; k < kRound; ++k)
#pragma unroll
      for (int q = 0; q < kS4; ++q)
        v[k][q] = *(const f32x4*)(pp + min(c0 + k, a.chunks - 1) * cstride + min(e0 + 4 * q, ps - 4));
#pragma unroll
    for (int k = 0; k < kRound; ++k)
#pragma unroll
      for (int q = 0; q < kS4; ++q)
        if (c0 + k < a.chunks) x[q] += v[k][q];
  }
  // softmax over the routed experts
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < S; ++i)
    if (e0 + i < N) m = fmaxf(m, x[i / 4][i % 4]);
  m = vmax(m);
  float sc[S], zs = 0.f;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    sc[i] = e0 + i < N ? expf(x[i / 4][i % 4] - m) : 0.f;
    zs += sc[i];
  }
  zs = vsum(zs);
  const float inv = 1.0f / zs;
#pragma unroll
  for (int i = 0; i < S; ++i) sc[i] *= inv;
  const bool tok = t < a.tokens;
  if (a.scores && tok) {
    float* so = a.scores + (int64_t)t * N;
#pragma unroll
    for (int i = 0; i < S; ++i)
      if (e0 + i < N) so[e0 + i] = sc[i];
  }
  // top_k rounds: the token's largest key; its owner clears it, writes the
  // expert and its score, and finds its next largest key
  uint64_t key[S], best = 0;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    key[i] = e0 + i < N ? rank_key(x[i / 4][i % 4], e0 + i) : 0;
    best = max64(best, key[i]);
  }
  for (int k = 0; k < a.top_k; ++k) {
    const uint64_t r = kmax(best);
    const int bi = (int)(0xFFFFFFFFu - (uint32_t)r);
    if (bi - e0 >= 0 && bi - e0 < S) {
      float w = 0.f;
      best = 0;
#pragma unroll
      for (int i = 0; i < S; ++i) {
        if (e0 + i == bi) {
          w = sc[i];
          key[i] = 0;
        }
        best = max64(best, key[i]);
      }
      if (tok) {
        a.idx[(int64_t)t * a.top_k + k] = bi;
        a.weight[(int64_t)t * a.top_k + k] = w;
      }
    }
  }
}

template __global__ void gate_finish<1, 16>(const GateArgs);
template __global__ void gate_finish<2, 16>(const GateArgs);
template __global__ void gate_finish<3, 16>(const GateArgs);
template __global__ void gate_finish<4, 16>(const GateArgs);
template __global__ void gate_finish<1, 64>(const GateArgs);

}  // namespace mla
