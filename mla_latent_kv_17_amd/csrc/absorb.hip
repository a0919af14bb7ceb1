// Query absorption: q_lat[r][h][:] = W_UK[h]^T q_nope[r][h][:]  (128 -> 512).
//
// deepforge.srivtx.xyz "DeepSeek-V2", section 1, formula box "MLA: compress
// once, reconstruct in attention": keys are k = W_UK c; because the map is
// linear it is folded into the query so scores can be taken against c.
// W_UK is stored per head as [d_head = 128][d_latent = 512].
//
// bf16 path: per head a [rows x 128] x [128 x 512] product on the matrix
// cores (v_mfma_f32_32x32x16_bf16, exact products, fp32 sums).  The
// contraction runs over d_head, the row index of W_UK, so the weight operand
// needs a transpose: one workgroup stages its head's 128 x 256 half of W_UK
// in LDS with coalesced loads (W_UK is streamed from HBM exactly once, the
// traffic that bounds this step) and the matrix-core operand is read back
// with the transposing LDS load ds_read_b64_tr_b16.  Wave w covers latent
// columns 64w .. 64w+63 of the half for every 32-row tile of queries.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

template <bool kOutBf16>
__global__ void __launch_bounds__(256) absorb_q_mfma(const AbsorbArgs a) {
  // row d of the staged slice at d * kStride bytes; the 64-byte pad puts the
  // four rows of one transposing read in four distinct 16-bank groups
  constexpr int kStride = 512 + 64;
  __shared__ __attribute__((aligned(16))) uint8_t ws[128 * kStride];
  const int h = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  {
    const uint8_t* w = (const uint8_t*)a.w + ((int64_t)h * 128 * 512 + half * 256) * 2;
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = i * 256 + tid, d = idx >> 5, q = idx & 31;
      v[i] = *(const u32x4*)(w + (int64_t)d * 1024 + q * 16);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = i * 256 + tid, d = idx >> 5, q = idx & 31;
      *(MLA_LDS u32x4*)((MLA_LDS uint8_t*)ws + d * kStride + q * 16) = v[i];
    }
  }
  __syncthreads();
  // B operand of k-step ks, n-tile nt: lane l holds W[d = 16ks + 8(l/32) + j][c = 64w + 32nt + l%32].
  // Transposing read: in each 16-lane group, lane L reads row dbase + L/4,
  // columns cbase + 4(L%4) .. +3, and lane i receives column cbase + i.
  const int grp = lane >> 4, L = lane & 15;
  const int g = lane >> 5, n32 = lane & 31;
  const uint32_t boff = (uint32_t)((8 * (grp >> 1) + (L >> 2)) * kStride + (wave * 64 + 16 * (grp & 1) + 4 * (L & 3)) * 2);
  bf16x8 bw[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const MLA_LDS uint8_t* p = (const MLA_LDS uint8_t*)ws + boff + ks * 16 * kStride + nt * 64;
      const u32x2 lo = lds_read_tr16_b64(p);
      const u32x2 hi = lds_read_tr16_b64(p + 4 * kStride);
      bw[nt][ks] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  const uint16_t* q = (const uint16_t*)a.q_nope;
  for (int m0 = 0; m0 < a.rows; m0 += 32) {
    const int r = m0 + n32;
    u32x4 av[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      av[ks] = r < a.rows ? *(const u32x4*)(q + ((int64_t)r * a.heads + h) * 128 + ks * 16 + 8 * g)
                          : u32x4{0, 0, 0, 0};
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt] = mfma32x32x16(as_bf16x8(av[ks]), bw[nt][ks], acc[nt]);
    // D lane l, register i: row (i/4)*8 + 4g + i%4, column n32
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m0 + (i >> 2) * 8 + 4 * g + (i & 3);
        if (row < a.rows) {
          const int64_t off = ((int64_t)row * a.heads + h) * 512 + half * 256 + wave * 64 + nt * 32 + n32;
          if (kOutBf16)
            ((uint16_t*)a.q_lat)[off] = f32_to_bf16_bits(acc[nt][i]);
          else
            ((float*)a.q_lat)[off] = acc[nt][i];
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
