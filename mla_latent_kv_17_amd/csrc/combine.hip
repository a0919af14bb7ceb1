// Split-KV merge: each KV chunk s of a query row produced a normalised latent
// output o_s and its log-sum-exp lse_s; the whole-context result is
//     lse = ln sum_s exp(lse_s),   o_lat = sum_s exp(lse_s - lse) o_s.
// This is the softmax over the union of the chunks' tokens, written out for
// chunks (deepforge.srivtx.xyz "DeepSeek-V2", section 1, "The bottleneck at
// inference time": attention over all earlier tokens).  Chunks that saw no
// token carry lse_s = -inf and weight 0.
//
// The partials are fp32 or fp16 (template argument); sums are fp32.  Lane
// l holds latent columns 8l .. 8l+7 of a row; a wave merges its chunks 16 per
// round, every load of a round issued before its arithmetic, so a round
// costs one memory latency.  Two shapes:
//  * kSolo (up to 16 chunks): one wave per query row, four rows per
//    workgroup, one round;
//  * otherwise one workgroup (4 waves) per query row: wave w merges chunks
//    w, w + 4, ..., and the four waves' running maxima, sums and rows then
//    combine through LDS (the same log-sum-exp update).
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

namespace {

constexpr int kRound = 16;  // chunks per wave per round

template <typename PT>
__device__ __forceinline__ void load8(const PT* p, f32x4& a, f32x4& b) {
  a = load4(p);
  b = load4(p + 4);
}

}  // namespace

template <typename PT, bool kSolo>
__global__ void __launch_bounds__(256) split_combine(const CombineArgs a) {
  __shared__ float xm[4], xz[4];
  __shared__ __attribute__((aligned(16))) float xo[4][512];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gr = kSolo ? 4 * blockIdx.x + wave : blockIdx.x;  // (sequence, row)
  if (kSolo && gr >= a.batch * a.rows) return;
  const int b = gr / a.rows, row = gr - b * a.rows;
  const int ns = a.num_splits;
  constexpr int kStride = kSolo ? 1 : 4;  // chunks between a wave's consecutive chunks
  const float* lp = a.lse_part + (int64_t)b * ns * a.rows + row;
  const PT* op = (const PT*)a.o_part + ((int64_t)b * ns * a.rows + row) * 512 + 8 * lane;
  const int64_t ostride = (int64_t)a.rows * 512;
  float m = -__builtin_inff(), z = 0.f;  // this wave's running maximum and sum of exp(lse_s - m)
  f32x4 acc0 = f32x4{}, acc1 = f32x4{};  // its running sum of exp(lse_s - m) o_s
  for (int s0 = kSolo ? 0 : wave; s0 < ns; s0 += kStride * kRound) {
    float ls[kRound];
    f32x4 v0[kRound], v1[kRound];
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      const int s = s0 + kStride * j;
      const bool in = s < ns;
      ls[j] = in ? lp[(int64_t)s * a.rows] : -__builtin_inff();
      if (in)
        load8(op + s * ostride, v0[j], v1[j]);
      else
        v0[j] = v1[j] = f32x4{};
    }
    float mb = m;
#pragma unroll
    for (int j = 0; j < kRound; ++j) mb = fmaxf(mb, ls[j]);
    if (mb == -__builtin_inff()) continue;  // no chunk so far saw a token
    const float alpha = m == -__builtin_inff() ? 0.f : expf(m - mb);
    z *= alpha;
    acc0 *= alpha;
    acc1 *= alpha;
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      if (ls[j] == -__builtin_inff()) continue;  // an empty chunk has weight 0 (its row may hold anything)
      const float e = expf(ls[j] - mb);
      z += e;
      acc0 += e * v0[j];
      acc1 += e * v1[j];
    }
    m = mb;
  }
  if (kSolo) {
    const float inv = z > 0.f ? 1.f / z : 0.f;
    float* orow = a.o_lat + ((int64_t)b * a.rows + row) * 512 + 8 * lane;
    *(f32x4*)orow = acc0 * inv;
    *(f32x4*)(orow + 4) = acc1 * inv;
    if (a.lse && lane == 0) a.lse[(int64_t)b * a.rows + row] = z > 0.f ? m + logf(z) : -__builtin_inff();
    return;
  }
  if (lane == 0) {
    xm[wave] = m;
    xz[wave] = z;
  }
  *(f32x4*)&xo[wave][8 * lane] = acc0;
  *(f32x4*)&xo[wave][8 * lane + 4] = acc1;
  __syncthreads();
  if (wave != 0) return;
  const float mm = fmaxf(fmaxf(xm[0], xm[1]), fmaxf(xm[2], xm[3]));
  float zt = 0.f;
  f32x4 o0 = f32x4{}, o1 = f32x4{};
  if (mm != -__builtin_inff()) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (xm[w] == -__builtin_inff()) continue;  // that wave's chunks were all empty
      const float e = expf(xm[w] - mm);
      zt += e * xz[w];
      o0 += e * *(const f32x4*)&xo[w][8 * lane];
      o1 += e * *(const f32x4*)&xo[w][8 * lane + 4];
    }
  }
  const float inv = zt > 0.f ? 1.f / zt : 0.f;
  float* orow = a.o_lat + ((int64_t)b * a.rows + row) * 512 + 8 * lane;
  *(f32x4*)orow = o0 * inv;
  *(f32x4*)(orow + 4) = o1 * inv;
  if (a.lse && lane == 0) a.lse[(int64_t)b * a.rows + row] = zt > 0.f ? mm + logf(zt) : -__builtin_inff();
}

template __global__ void split_combine<float, false>(const CombineArgs a);
template __global__ void split_combine<_Float16, false>(const CombineArgs a);
template __global__ void split_combine<float, true>(const CombineArgs a);
template __global__ void split_combine<_Float16, true>(const CombineArgs a);

}  // namespace mla
