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
// W_UK in LDS with coalesced loads (W_UK is streamed from HBM exactly once)
// and reads the matrix-core operand back with the transposing LDS load
// ds_read_b64_tr_b16.  The weight is the A operand (latent columns as the
// product's rows) and the queries the B operand: each 32-row query tile is
// loaded once per workgroup (16 lanes per 256-byte row) into LDS, where all
// four waves read it.  Each lane ends up with four consecutive latent
// columns of one query row; a tile's results pass through LDS so that 16
// lanes store each row's 128 columns as one contiguous segment.  Wave w
// covers latent columns 32w .. 32w+31 of the quarter for every tile.  Four
// workgroups per head leave room for several per compute unit.
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
  // two query tiles: row r at r * kQStride bytes (128 bf16 + 16 bytes of pad,
  // so 16 consecutive rows read at one chunk hit distinct bank groups)
  constexpr int kQStride = 256 + 16;
  __shared__ __attribute__((aligned(16))) uint8_t qs[2][32 * kQStride];
  // one tile's results: row r at r * kOutStride bytes (128 columns of the
  // output type, 16 bytes of pad)
  constexpr int kOutBytes = kOutBf16 ? 2 : 4;
  constexpr int kOutStride = 128 * kOutBytes + 16;
  __shared__ __attribute__((aligned(16))) uint8_t ot[32 * kOutStride];
  const int h = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, n32 = lane & 31;
  // a tile's 32 query rows (256 bytes each): thread t loads 16-byte chunk
  // t % 16 of rows t / 16 and t / 16 + 16 (rows past the end read zeros)
  const uint8_t* q = (const uint8_t*)a.q_nope;
  auto load_q = [&](int m0, u32x4 (&rq)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = m0 + (tid >> 4) + 16 * k;
      rq[k] = r < a.rows ? *(const u32x4*)(q + ((int64_t)r * a.heads + h) * 256 + (tid & 15) * 16) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_q = [&](int buf, const u32x4 (&rq)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
      *(MLA_LDS u32x4*)((MLA_LDS uint8_t*)qs[buf] + ((tid >> 4) + 16 * k) * kQStride + (tid & 15) * 16) = rq[k];
  };
  u32x4 rq[2];
  load_q(0, rq);  // before the weight, so the two latencies overlap
  {
    // 128 rows x 256 bytes: thread t takes 16-byte chunk t % 16 of rows t / 16 + 16 i
    const uint8_t* w = (const uint8_t*)a.w + ((int64_t)h * 128 * 512 + quarter * 128) * 2;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = 16 * i + (tid >> 4), qc = tid & 15;
      v[i] = *(const u32x4*)(w + (int64_t)d * 1024 + qc * 16);
    }
    store_q(0, rq);
    if (32 < a.rows) load_q(32, rq);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = 16 * i + (tid >> 4), qc = tid & 15;
      *(MLA_LDS u32x4*)((MLA_LDS uint8_t*)ws + d * kStride + qc * 16) = v[i];
    }
  }
  __syncthreads();
  // A operand of k-step ks: lane l holds W[d = 16ks + 8(l/32) + j][c = 32w + l%32].
  // Transposing read: in each 16-lane group, lane L reads row dbase + L/4,
  // columns cbase + 4(L%4) .. +3, and lane i receives column cbase + i.
  const int grp = lane >> 4, L = lane & 15;
  const uint32_t woff = (uint32_t)((8 * (grp >> 1) + (L >> 2)) * kStride + (wave * 32 + 16 * (grp & 1) + 4 * (L & 3)) * 2);
  bf16x8 aw[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const MLA_LDS uint8_t* p = (const MLA_LDS uint8_t*)ws + woff + ks * 16 * kStride;
    const u32x2 lo = lds_read_tr16_b64(p);
    const u32x2 hi = lds_read_tr16_b64(p + 4 * kStride);
    aw[ks] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
  // Tile t (rows m0 = 32 t ..) multiplies query tile buffer t % 2; tile t+1's
  // rows are in registers and go to the other buffer after the tile's first
  // barrier (its last reader, tile t-1, is done by then), and tile t+2's
  // loads are issued, a whole tile ahead of their store.
  for (int m0 = 0, t = 0; m0 < a.rows; m0 += 32, ++t) {
    const MLA_LDS uint8_t* qb = (const MLA_LDS uint8_t*)qs[t & 1];
    // B operand of k-step ks: lane l holds q_nope[row m0 + l%32][d = 16ks + 8(l/32) + j]
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      acc = mfma32x32x16(aw[ks], *(const MLA_LDS bf16x8*)(qb + n32 * kQStride + (2 * ks + g) * 16), acc);
    // D lane l, register i: latent column 32w + (i/4)*8 + 4g + i%4 of the
    // quarter, tile row l%32
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const float x0 = acc[4 * i4], x1 = acc[4 * i4 + 1], x2 = acc[4 * i4 + 2], x3 = acc[4 * i4 + 3];
      MLA_LDS uint8_t* o = (MLA_LDS uint8_t*)ot + n32 * kOutStride + (wave * 32 + 8 * i4 + 4 * g) * kOutBytes;
      if (kOutBf16)
        *(MLA_LDS u32x2*)o = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
      else
        *(MLA_LDS f32x4*)o = f32x4{x0, x1, x2, x3};
    }
    __syncthreads();
    if (m0 + 32 < a.rows) {
      store_q((t + 1) & 1, rq);
      if (m0 + 64 < a.rows) load_q(m0 + 64, rq);
    }
    // 32 rows x (128 x kOutBytes) bytes: thread t stores 16-byte chunk t % nc of rows t / nc + (256 / nc) k
    constexpr int nc = 128 * kOutBytes / 16;
#pragma unroll
    for (int k = 0; k < nc / 8; ++k) {
      const int rr = tid / nc + (256 / nc) * k, cc = tid % nc, r = m0 + rr;
      const u32x4 v = *(const MLA_LDS u32x4*)((const MLA_LDS uint8_t*)ot + rr * kOutStride + cc * 16);
      if (r < a.rows)
        *(u32x4*)((uint8_t*)a.q_lat + (((int64_t)r * a.heads + h) * 512 + quarter * 128) * kOutBytes + cc * 16) = v;
    }
    __syncthreads();  // ot and the query buffer are rewritten by the next tiles
  }
}

// fp32 inputs: one thread per latent column, fp32 FMA over d_head.
// fp32 inputs: workgroup = (head, block of 64 latent columns); wave w
// holds the weight rows d = 32w .. 32w+31 of the block in registers (lane l:
// column c0 + l, 32 coalesced loads issued together) and reuses them for
// every query row; the four waves' partial sums over their rows of d meet
// in LDS.
template <bool kOutBf16>
__global__ void __launch_bounds__(256) absorb_q_f32(const AbsorbArgs a) {
  __shared__ float qs[128];
  __shared__ float part[4][64];
  const int h = blockIdx.x >> 3, c0 = (blockIdx.x & 7) * 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* w = (const float*)a.w + ((int64_t)h * 128 + 32 * wave) * 512 + c0 + lane;
  float wr[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) wr[d] = w[(int64_t)d * 512];
  for (int r = 0; r < a.rows; ++r) {
    const float* q = (const float*)a.q_nope + ((int64_t)r * a.heads + h) * 128;
    if (threadIdx.x < 128) qs[threadIdx.x] = q[threadIdx.x];
    __syncthreads();
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < 32; ++d) acc = fmaf(wr[d], qs[32 * wave + d], acc);
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
      const float v = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
      const int64_t off = ((int64_t)r * a.heads + h) * 512 + c0 + lane;
      if (kOutBf16)
        ((uint16_t*)a.q_lat)[off] = f32_to_bf16_bits(v);
      else
        ((float*)a.q_lat)[off] = v;
    }
  }
}

template __global__ void absorb_q_mfma<true>(const AbsorbArgs);
template __global__ void absorb_q_mfma<false>(const AbsorbArgs);
template __global__ void absorb_q_f32<true>(const AbsorbArgs);
template __global__ void absorb_q_f32<false>(const AbsorbArgs);

}  // namespace mla
