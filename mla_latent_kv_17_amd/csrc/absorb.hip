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
// needs a transpose: one workgroup stages its head's 128 x 128 quarter of
// W_UK in LDS with coalesced loads (W_UK is streamed from HBM exactly once,
// the traffic that bounds this step) and reads the matrix-core operand back
// with the transposing LDS load ds_read_b64_tr_b16.  The weight is the A
// operand (latent columns as the product's rows) and the queries the B
// operand, so each lane ends up with four consecutive latent columns of one
// query row: one 8-byte (bf16) or 16-byte (fp32) store each.  Wave w covers
// latent columns 32w .. 32w+31 of the quarter for every 32-row tile of
// queries; four workgroups per head leave room for two or more per compute
// unit, so one's loads overlap another's products and stores.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

template <bool kOutBf16>
__global__ void __launch_bounds__(256) absorb_q_mfma(const AbsorbArgs a) {
  // row d of the staged quarter at d * kStride bytes; the 64-byte pad puts
  // the four rows of one transposing read (and the two column halves of a
  // 32-lane half wave) in distinct bank groups
  constexpr int kStride = 256 + 64;
  __shared__ __attribute__((aligned(16))) uint8_t ws[128 * kStride];
  const int h = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  {
    // 128 rows x 256 bytes: thread t takes 16-byte chunk t % 16 of rows t / 16 + 16 i
    const uint8_t* w = (const uint8_t*)a.w + ((int64_t)h * 128 * 512 + quarter * 128) * 2;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = 16 * i + (tid >> 4), q = tid & 15;
      v[i] = *(const u32x4*)(w + (int64_t)d * 1024 + q * 16);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = 16 * i + (tid >> 4), q = tid & 15;
      *(MLA_LDS u32x4*)((MLA_LDS uint8_t*)ws + d * kStride + q * 16) = v[i];
    }
  }
  __syncthreads();
  // A operand of k-step ks: lane l holds W[d = 16ks + 8(l/32) + j][c = 32w + l%32].
  // Transposing read: in each 16-lane group, lane L reads row dbase + L/4,
  // columns cbase + 4(L%4) .. +3, and lane i receives column cbase + i.
  const int grp = lane >> 4, L = lane & 15;
  const int g = lane >> 5, n32 = lane & 31;
  const uint32_t woff = (uint32_t)((8 * (grp >> 1) + (L >> 2)) * kStride + (wave * 32 + 16 * (grp & 1) + 4 * (L & 3)) * 2);
  bf16x8 aw[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const MLA_LDS uint8_t* p = (const MLA_LDS uint8_t*)ws + woff + ks * 16 * kStride;
    const u32x2 lo = lds_read_tr16_b64(p);
    const u32x2 hi = lds_read_tr16_b64(p + 4 * kStride);
    aw[ks] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
  const uint16_t* q = (const uint16_t*)a.q_nope;
  for (int m0 = 0; m0 < a.rows; m0 += 32) {
    // B operand of k-step ks: lane l holds q_nope[row m0 + l%32][d = 16ks + 8(l/32) + j]
    const int r = m0 + n32;
    u32x4 bq[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      bq[ks] = r < a.rows ? *(const u32x4*)(q + ((int64_t)r * a.heads + h) * 128 + ks * 16 + 8 * g)
                          : u32x4{0, 0, 0, 0};
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) acc = mfma32x32x16(aw[ks], as_bf16x8(bq[ks]), acc);
    // D lane l, register i: latent column 32w + (i/4)*8 + 4g + i%4, query row m0 + l%32
    if (r < a.rows) {
      const int64_t base = ((int64_t)r * a.heads + h) * 512 + quarter * 128 + wave * 32 + 4 * g;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float x0 = acc[4 * i4], x1 = acc[4 * i4 + 1], x2 = acc[4 * i4 + 2], x3 = acc[4 * i4 + 3];
        if (kOutBf16)
          *(u32x2*)((uint16_t*)a.q_lat + base + 8 * i4) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        else
          *(f32x4*)((float*)a.q_lat + base + 8 * i4) = f32x4{x0, x1, x2, x3};
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
