// Split-KV merge: each KV chunk s of a query row produced a normalised latent
// output o_s and its log-sum-exp lse_s; the whole-context result is
//     lse = ln sum_s exp(lse_s),   o_lat = sum_s exp(lse_s - lse) o_s.
// This is the softmax over the union of the chunks' tokens, written out for
// chunks (deepforge.srivtx.xyz "DeepSeek-V2", section 1, "The bottleneck at
// inference time": attention over all earlier tokens).  Chunks that saw no
// token carry lse_s = -inf and weight 0.
//
// The partials are fp32 or fp16 (template argument); sums are fp32.
// 128 threads x 4 columns per query row, two rows per workgroup.  Up to
// kBatch chunks are handled per round with every load (log-sum-exps and
// partial rows) issued before any arithmetic, so a round costs one memory
// latency; the running merge across rounds is the same log-sum-exp update.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

template <typename PT>
__global__ void __launch_bounds__(256) split_combine(const CombineArgs a) {
  constexpr int kBatch = 8;
  const int gr = blockIdx.x * 2 + (threadIdx.x >> 7);
  if (gr >= a.batch * a.rows) return;
  const int b = gr / a.rows, row = gr - b * a.rows;
  const int ns = a.num_splits;
  const int c = (threadIdx.x & 127) * 4;
  const float* lp = a.lse_part + (int64_t)b * ns * a.rows + row;
  const PT* op = (const PT*)a.o_part + ((int64_t)b * ns * a.rows + row) * 512 + c;
  const int64_t ostride = (int64_t)a.rows * 512;
  float m = -__builtin_inff(), z = 0.f;  // running maximum and sum of exp(lse_s - m)
  f32x4 acc = f32x4{};                   // running sum of exp(lse_s - m) o_s
  for (int s0 = 0; s0 < ns; s0 += kBatch) {
    float ls[kBatch];
    f32x4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = s0 + j < ns;
      ls[j] = in ? lp[(int64_t)(s0 + j) * a.rows] : -__builtin_inff();
      v[j] = in ? load4(op + (s0 + j) * ostride) : f32x4{};
    }
    float mb = m;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, ls[j]);
    if (mb == -__builtin_inff()) continue;  // no chunk so far saw a token
    const float alpha = m == -__builtin_inff() ? 0.f : expf(m - mb);
    z *= alpha;
    acc *= alpha;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (ls[j] == -__builtin_inff()) continue;  // an empty chunk has weight 0
      const float e = expf(ls[j] - mb);
      z += e;
      acc += e * v[j];
    }
    m = mb;
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  *(f32x4*)(a.o_lat + ((int64_t)b * a.rows + row) * 512 + c) = acc * inv;
  if (a.lse && (threadIdx.x & 127) == 0)
    a.lse[(int64_t)b * a.rows + row] = z > 0.f ? m + logf(z) : -__builtin_inff();
}

template __global__ void split_combine<float>(const CombineArgs a);
template __global__ void split_combine<_Float16>(const CombineArgs a);

}  // namespace mla
