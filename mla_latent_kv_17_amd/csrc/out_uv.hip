// Output absorption: out[r][h][:] = W_UV[h] o_lat[r][h][:]  (512 -> 128).
//
// deepforge.srivtx.xyz "DeepSeek-V2", section 1, formula box "MLA: compress
// once, reconstruct in attention": values are v = W_UV c; since the map is
// linear, sum_t p_t v_t = W_UV sum_t p_t c_t and W_UV moves to the output side.
// W_UV is stored per head as [d_head = 128][d_latent = 512].
//
// bf16 weights: matrix cores (v_mfma_f32_32x32x16_bf16).  The fp32 o_lat is
// split into hi = bf16(x) and lo = bf16(x - hi), and both halves are
// multiplied by the exact bf16 weights with fp32 sums, which keeps about
// 16 significant bits of o_lat (fp32-level error for this product).
//
// Workgroup = (head, half of d_head): its 64 x 512 weight slice (64 KB) is
// read from HBM once into registers and reused for every 32-row tile.  The
// four waves split the latent (K) dimension, 128 columns each, so every wave
// issues all of its loads at once; the partial tiles are summed through LDS.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

__global__ void __launch_bounds__(256) out_uv_mfma(const OutUvArgs a) {
  constexpr int kPad = 33;  // LDS row stride (floats) of the partial tiles
  __shared__ float red[4][2][32 * kPad];
  const int h = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n32 = lane & 31, g = lane >> 5;
  const int c0 = wave * 128 + 8 * g;  // this lane's latent columns: c0 + 16 ks + 0..7
  // B operand: W[d][c], d = 64 half + 32 nt + n32, c = c0 + 16 ks + j
  bf16x8 bw[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint16_t* w = (const uint16_t*)a.w + ((int64_t)h * 128 + half * 64 + nt * 32 + n32) * 512 + c0;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bw[nt][ks] = as_bf16x8(*(const u32x4*)(w + ks * 16));
  }
  for (int m0 = 0; m0 < a.rows; m0 += 32) {
    const int r = m0 + n32;
    f32x4 x[8][2];
    if (r < a.rows) {
      const float* xp = a.o_lat + ((int64_t)r * a.heads + h) * 512 + c0;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        x[ks][0] = *(const f32x4*)(xp + ks * 16);
        x[ks][1] = *(const f32x4*)(xp + ks * 16 + 4);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) x[ks][0] = x[ks][1] = f32x4{};
    }
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const float xv[8] = {x[ks][0][0], x[ks][0][1], x[ks][0][2], x[ks][0][3],
                           x[ks][1][0], x[ks][1][1], x[ks][1][2], x[ks][1][3]};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t hp = pack_bf16x2(xv[2 * j], xv[2 * j + 1]);
        hi[j] = hp;
        lo[j] = pack_bf16x2(xv[2 * j] - __builtin_bit_cast(float, hp << 16),
                            xv[2 * j + 1] - __builtin_bit_cast(float, hp & 0xFFFF0000u));
      }
      const bf16x8 ah = as_bf16x8(u32x4{hi[0], hi[1], hi[2], hi[3]});
      const bf16x8 al = as_bf16x8(u32x4{lo[0], lo[1], lo[2], lo[3]});
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        acc[nt] = mfma32x32x16(ah, bw[nt][ks], acc[nt]);
        acc[nt] = mfma32x32x16(al, bw[nt][ks], acc[nt]);
      }
    }
    // partial tile of this wave's latent quarter: D row (r/4)*8 + 4g + r%4, column n32
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[wave][nt][((i >> 2) * 8 + 4 * g + (i & 3)) * kPad + n32] = acc[nt][i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = i * 256 + threadIdx.x;
      const int row = idx >> 6, d = idx & 63, nt = d >> 5, n = d & 31;
      const float v = red[0][nt][row * kPad + n] + red[1][nt][row * kPad + n] + red[2][nt][row * kPad + n] +
                      red[3][nt][row * kPad + n];
      if (m0 + row < a.rows) a.out[((int64_t)(m0 + row) * a.heads + h) * 128 + half * 64 + d] = v;
    }
    __syncthreads();
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
