// Output absorption: out[r][h][:] = W_UV[h] o_lat[r][h][:]  (512 -> 128).
//
// deepforge.srivtx.xyz "DeepSeek-V2", section 1, formula box "MLA: compress
// once, reconstruct in attention": values are v = W_UV c; since the map is
// linear, sum_t p_t v_t = W_UV sum_t p_t c_t and W_UV moves to the output side.
// W_UV is stored per head as [d_head = 128][d_latent = 512].
//
// bf16 weights: matrix cores (v_mfma_f32_16x16x32_bf16).  The fp32 o_lat is
// split into hi = bf16(x) and lo = bf16(x - hi), and both halves are
// multiplied by the exact bf16 weights with fp32 sums, which keeps about
// 16 significant bits of o_lat (fp32-level error for this product).
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

__global__ void __launch_bounds__(256) out_uv_mfma(const OutUvArgs a) {
  const int h = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d0 = blockIdx.y * 64 + wave * 16;
  const int n16 = lane & 15, kg = lane >> 4;
  // B operand: W[d][c] for d = d0 + n16, c = ks*32 + 8*kg + j (contiguous)
  const uint16_t* w = (const uint16_t*)a.w + ((int64_t)h * 128 + d0 + n16) * 512 + 8 * kg;
  bf16x8 bw[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) bw[ks] = as_bf16x8(*(const u32x4*)(w + ks * 32));
  for (int m0 = 0; m0 < a.rows; m0 += 16) {
    const int r = m0 + n16;
    const float* x = a.o_lat + ((int64_t)r * a.heads + h) * 512 + 8 * kg;
    f32x4 acc = f32x4{};
#pragma unroll 4
    for (int ks = 0; ks < 16; ++ks) {
      f32x4 v0 = f32x4{}, v1 = f32x4{};
      if (r < a.rows) {
        v0 = *(const f32x4*)(x + ks * 32);
        v1 = *(const f32x4*)(x + ks * 32 + 4);
      }
      const float xv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t hp = pack_bf16x2(xv[2 * j], xv[2 * j + 1]);
        const float h0 = __builtin_bit_cast(float, hp << 16);
        const float h1 = __builtin_bit_cast(float, hp & 0xFFFF0000u);
        hi[j] = hp;
        lo[j] = pack_bf16x2(xv[2 * j] - h0, xv[2 * j + 1] - h1);
      }
      acc = mfma16x16x32(as_bf16x8(u32x4{hi[0], hi[1], hi[2], hi[3]}), bw[ks], acc);
      acc = mfma16x16x32(as_bf16x8(u32x4{lo[0], lo[1], lo[2], lo[3]}), bw[ks], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 4 * kg + i;
      if (row < a.rows) a.out[((int64_t)row * a.heads + h) * 128 + d0 + n16] = acc[i];
    }
  }
}

// fp32 weights: one thread per output element, fp32 FMA over the latent.
__global__ void __launch_bounds__(128) out_uv_f32(const OutUvArgs a) {
  __shared__ float xs[512];
  const int h = blockIdx.x, r = blockIdx.y, d = threadIdx.x;
  const float* x = a.o_lat + ((int64_t)r * a.heads + h) * 512;
  for (int i = threadIdx.x; i < 512; i += 128) xs[i] = x[i];
  __syncthreads();
  const float* w = (const float*)a.w + ((int64_t)h * 128 + d) * 512;
  float acc = 0.f;
  for (int c = 0; c < 512; c += 4) {
    const f32x4 wv = *(const f32x4*)(w + c);
    acc = fmaf(wv[0], xs[c], acc);
    acc = fmaf(wv[1], xs[c + 1], acc);
    acc = fmaf(wv[2], xs[c + 2], acc);
    acc = fmaf(wv[3], xs[c + 3], acc);
  }
  a.out[((int64_t)r * a.heads + h) * 128 + d] = acc;
}

}  // namespace mla
