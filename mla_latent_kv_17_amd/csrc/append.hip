// Cache append: the S_q newest tokens of each sequence enter the paged cache.
//
// deepforge.srivtx.xyz "DeepSeek-V2", section 1, "Store a latent, rebuild the
// keys and values" and its formula box: the cache holds, per token per layer,
// the down-projected latent c_t = W_DKV h_t (512 wide) and one 64-wide key
// that carries the position (RoPE cannot pass through the absorbed
// projections, so it is kept apart from the latent).  Here that key is
// k^R_t = RoPE_p(W_KR h_t) at the token's position p: pairs (2j, 2j+1) turned
// by the angle p * theta^(-2j/64).
//
// Two launches:
//  * append_proj_mfma (bf16 inputs): X = h W^T with W = [W_DKV; W_KR]
//    (576 x d_model), a [tokens x 576] product over K = d_model, one
//    workgroup per (32 output columns, 512-wide chunk of d_model, 32 tokens:
//    180 workgroups at d_model 5120, so the weight stream spreads over most
//    compute units)
//    (proj_chunk_bf16: LDS-staged coalesced rows, matrix cores, fp32 chunk
//    partials into the caller's workspace).  The weights are the traffic
//    (576 x d_model x 2 bytes) and are read once; the small h is read once
//    per column tile.
//  * append_finish (one workgroup per token): the chunk sums, the rotation
//    (angles and sin/cos in fp64, so large positions keep their precision),
//    then the cache encoding and the write into the token's page row.
#include "mla_device.h"
#include "mla_kernels.h"
#include "proj_chunk.h"

namespace mla {

static_assert(kAppendChunk == kProjChunk, "the append's chunk is the projection routine's");

__global__ void __launch_bounds__(256) append_proj_mfma(const AppendArgs a) {
  const uint16_t* w_dkv = (const uint16_t*)a.w_dkv;
  const uint16_t* w_kr = (const uint16_t*)a.w_kr;
  const int64_t dm = a.d_model;
  auto wrow = [&](int n) __attribute__((always_inline)) -> const uint16_t* {
    return n < 512 ? w_dkv + n * dm : w_kr + (n - 512) * dm;  // W_DKV rows, then W_KR rows
  };
  proj_chunk_bf16((const uint16_t*)a.h, a.tokens, a.d_model, kAppendCols, wrow, blockIdx.x * 32, blockIdx.y,
                  blockIdx.z * 32, a.part, kAppendCols);
}

// fp32 inputs: wave w of workgroup x computes column 4x + w of one token
// (grid y): its 64 lanes stride along d_model, then a shuffle sum.
__global__ void __launch_bounds__(256) append_proj_f32(const AppendArgs a) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6), r = blockIdx.y, lane = threadIdx.x & 63;
  const float* h = (const float*)a.h + (int64_t)r * a.d_model;
  const float* w = n < 512 ? (const float*)a.w_dkv + (int64_t)n * a.d_model
                           : (const float*)a.w_kr + (int64_t)(n - 512) * a.d_model;
  float acc = 0.f;
  for (int k = lane; k < a.d_model; k += 64) acc = fmaf(h[k], w[k], acc);
  acc = wave_sum(acc);
  if (lane == 0) a.part[(int64_t)r * kAppendCols + n] = acc;
}

namespace {

// OCP E4M3FN code of a finite float with |x| <= 448, nearest with ties to
// even, from the format's definition: at or above 2^-6 the float's exponent
// and top three mantissa bits rounded as one field (a carry moves into the
// exponent) and re-biased from 127 to 7; below 2^-6 the nearest-even count
// of 2^-9.  The sign goes to bit 7.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = fabsf(x);
  uint32_t code;
  if (ax >= 0.015625f) {
    const uint32_t b = __float_as_uint(ax);
    code = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
  } else {
    code = (uint32_t)rintf(ax * 512.0f);
  }
  return sign | code;
}

}  // namespace

template <int kFmt>
__global__ void __launch_bounds__(256) append_finish(const AppendArgs a) {
  __shared__ float x[kAppendCols];
  __shared__ float wmax[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  // the token's position and page row (read first: their latency overlaps
  // the chunk sums; a token without a position reads entry 0 and leaves)
  const int b = r / a.sq, i = r - b * a.sq;
  const int p = a.seq_lens[b] - a.sq + i;
  const int64_t blk = a.block_table[(int64_t)b * a.max_blocks + (max(p, 0) >> 6)];
  const int row = p & 63;
  // the chunk sums (they do not depend on the token's position), chunk
  // order fixed, the loads of sixteen chunks (d_model up to 8192 in one
  // round) for all of a thread's columns in flight at a time with no branch
  // between them
  constexpr int kRound = 16;
  const int64_t cstride = (int64_t)a.tokens * kAppendCols;
  const float* pp = a.part + (int64_t)r * kAppendCols;
  float sum[3] = {0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.chunks; c0 += kRound) {
    float v[3][kRound];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int n = min(tid + 256 * u, kAppendCols - 1);
#pragma unroll
      for (int k = 0; k < kRound; ++k) v[u][k] = pp[min(c0 + k, a.chunks - 1) * cstride + n];
    }
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
      for (int k = 0; k < kRound; ++k) sum[u] += c0 + k < a.chunks ? v[u][k] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < 3; ++u)
    if (tid + 256 * u < kAppendCols) x[tid + 256 * u] = sum[u];
  if (p < 0) return;  // uniform: the whole workgroup leaves before any barrier
  __syncthreads();
  if (tid < 32) {
    // pair j = tid of the RoPE key: angle p * theta^(-2j/64)
    const double ang = (double)p * exp2(-(double)(2 * tid) / 64.0 * a.log2_theta);
    double sn, cs;
    sincos(ang, &sn, &cs);
    const double x0 = x[512 + 2 * tid], x1 = x[512 + 2 * tid + 1];
    x[512 + 2 * tid] = (float)(x0 * cs - x1 * sn);
    x[512 + 2 * tid + 1] = (float)(x0 * sn + x1 * cs);
  }
  __syncthreads();
  uint8_t* lrow = a.latent + blk * a.lat_bs + (int64_t)row * a.lat_rs;
  uint8_t* rrow = a.rope + blk * a.rope_bs + (int64_t)row * a.rope_rs;
  if (kFmt == 0) {
    for (int n = tid; n < 512; n += 256) ((float*)lrow)[n] = x[n];
    if (tid < 64) ((float*)rrow)[tid] = x[512 + tid];
  } else if (kFmt == 1) {
    for (int n = tid; n < 512; n += 256) ((uint16_t*)lrow)[n] = f32_to_bf16_bits(x[n]);
    if (tid < 64) ((uint16_t*)rrow)[tid] = f32_to_bf16_bits(x[512 + tid]);
  } else {
    // per-token scale amax / 448 (1 for an all-zero latent), codes of c / scale
    float m = fmaxf(fabsf(x[tid]), fabsf(x[tid + 256]));
    m = wave_max(m);
    if ((tid & 63) == 0) wmax[tid >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
    for (int n = tid; n < 512; n += 256) {
      const float q = fminf(fmaxf(x[n] / sc, -448.0f), 448.0f);
      lrow[n] = (uint8_t)e4m3_code(q);
    }
    if (tid == 0) a.scale[blk * a.scale_bs + row] = sc;
    if (tid < 64) ((uint16_t*)rrow)[tid] = f32_to_bf16_bits(x[512 + tid]);
  }
}

template __global__ void append_finish<0>(const AppendArgs);
template __global__ void append_finish<1>(const AppendArgs);
template __global__ void append_finish<2>(const AppendArgs);

}  // namespace mla
