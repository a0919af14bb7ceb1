// Query absorption: q_lat[r][h][:] = W_UK[h]^T q_nope[r][h][:]  (128 -> 512).
//
// deepforge.srivtx.xyz "DeepSeek-V2", section 1, formula box "MLA: compress
// once, reconstruct in attention": keys are k = W_UK c; because the map is
// linear it is folded into the query so scores can be taken against c.
// W_UK is stored per head as [d_head = 128][d_latent = 512].
//
// bf16 path: per head a [rows x 128] x [128 x 512] product on the matrix
// cores (v_mfma_f32_16x16x32_bf16, exact products, fp32 sums).  One
// workgroup covers one head and 64 latent columns (16 per wave) for every
// query row, so W_UK is streamed from HBM exactly once; it is the traffic
// that bounds this step.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

template <bool kOutBf16>
__global__ void __launch_bounds__(256) absorb_q_mfma(const AbsorbArgs a) {
  const int h = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c0 = blockIdx.y * 64 + wave * 16;
  const int n16 = lane & 15, kg = lane >> 4;
  const uint16_t* w = (const uint16_t*)a.w + (int64_t)h * 128 * 512;
  // B operand: W[d][c] for c = c0 + n16, d = ks*32 + 8*kg + j (a column read)
  bf16x8 bw[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = ks * 32 + 8 * kg + 2 * j;
      v[j] = (uint32_t)w[(int64_t)d * 512 + c0 + n16] | ((uint32_t)w[(int64_t)(d + 1) * 512 + c0 + n16] << 16);
    }
    bw[ks] = as_bf16x8(u32x4{v[0], v[1], v[2], v[3]});
  }
  const uint16_t* q = (const uint16_t*)a.q_nope;
  for (int m0 = 0; m0 < a.rows; m0 += 16) {
    const int r = m0 + n16;
    f32x4 acc = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 av = r < a.rows ? *(const u32x4*)(q + ((int64_t)r * a.heads + h) * 128 + ks * 32 + 8 * kg)
                                  : u32x4{0, 0, 0, 0};
      acc = mfma16x16x32(as_bf16x8(av), bw[ks], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 4 * kg + i;
      if (row < a.rows) {
        const int64_t off = ((int64_t)row * a.heads + h) * 512 + c0 + n16;
        if (kOutBf16)
          ((uint16_t*)a.q_lat)[off] = f32_to_bf16_bits(acc[i]);
        else
          ((float*)a.q_lat)[off] = acc[i];
      }
    }
  }
}

// fp32 inputs: one thread per latent column, fp32 FMA over d_head.
template <bool kOutBf16>
__global__ void __launch_bounds__(256) absorb_q_f32(const AbsorbArgs a) {
  __shared__ float qs[128];
  const int h = blockIdx.x, r = blockIdx.z;
  const int c = blockIdx.y * 256 + threadIdx.x;
  const float* q = (const float*)a.q_nope + ((int64_t)r * a.heads + h) * 128;
  if (threadIdx.x < 128) qs[threadIdx.x] = q[threadIdx.x];
  __syncthreads();
  const float* w = (const float*)a.w + (int64_t)h * 128 * 512 + c;
  float acc = 0.f;
  for (int d = 0; d < 128; ++d) acc = fmaf(w[(int64_t)d * 512], qs[d], acc);
  const int64_t off = ((int64_t)r * a.heads + h) * 512 + c;
  if (kOutBf16)
    ((uint16_t*)a.q_lat)[off] = f32_to_bf16_bits(acc);
  else
    ((float*)a.q_lat)[off] = acc;
}

template __global__ void absorb_q_mfma<true>(const AbsorbArgs);
template __global__ void absorb_q_mfma<false>(const AbsorbArgs);
template __global__ void absorb_q_f32<true>(const AbsorbArgs);
template __global__ void absorb_q_f32<false>(const AbsorbArgs);

}  // namespace mla
