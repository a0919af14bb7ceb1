// Split-KV merge: each KV chunk s of a query row produced a normalised latent
// output o_s and its log-sum-exp lse_s; the whole-context result is
//     lse = ln sum_s exp(lse_s),   o_lat = sum_s exp(lse_s - lse) o_s.
// This is the softmax over the union of the chunks' tokens, written out for
// chunks (deepforge.srivtx.xyz "DeepSeek-V2", section 1, "The bottleneck at
// inference time": attention over all earlier tokens).  Chunks that saw no
// token carry lse_s = -inf and weight 0.
//
// One workgroup per query row, 128 threads x 4 columns; the ns partial rows
// are read once, coalesced.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

__global__ void __launch_bounds__(128) split_combine(const CombineArgs a) {
  __shared__ float wsh[1024];
  const int gr = blockIdx.x;
  const int b = gr / a.rows, row = gr - b * a.rows;
  const int ns = a.num_splits;
  const float* lp = a.lse_part + (int64_t)b * ns * a.rows + row;
  // max and normaliser over the chunks (every thread computes them; ns is small)
  float m = -__builtin_inff();
  for (int s = 0; s < ns; ++s) m = fmaxf(m, lp[(int64_t)s * a.rows]);
  float z = 0.f;
  if (m != -__builtin_inff()) {
    for (int s = threadIdx.x; s < ns; s += 128) {
      const float ls = lp[(int64_t)s * a.rows];
      const float e = ls == -__builtin_inff() ? 0.f : expf(ls - m);
      wsh[s] = e;
    }
    __syncthreads();
    for (int s = 0; s < ns; ++s) z += wsh[s];
  }
  const int c = threadIdx.x * 4;
  f32x4 acc = f32x4{};
  if (z > 0.f) {
    const float inv = 1.f / z;
    const float* op = a.o_part + ((int64_t)b * ns * a.rows + row) * 512 + c;
    for (int s = 0; s < ns; ++s) {
      const float ws = wsh[s] * inv;
      if (ws == 0.f) continue;
      const f32x4 v = *(const f32x4*)(op + (int64_t)s * a.rows * 512);
      acc += ws * v;
    }
  }
  *(f32x4*)(a.o_lat + ((int64_t)b * a.rows + row) * 512 + c) = acc;
  if (a.lse && threadIdx.x == 0) a.lse[(int64_t)b * a.rows + row] = z > 0.f ? m + logf(z) : -__builtin_inff();
}

}  // namespace mla
