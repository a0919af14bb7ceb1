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
// The two halves of a head run on one XCD (block ids 8 apart), where the
// second read of each o_lat row is an L2 hit.
//
// Merged form (merge_out_uv_mfma, out_uv_f32<true>): o_lat is not read but
// formed on the fly from the KV chunks' normalised partial outputs o_s and
// log-sum-exps lse_s (the split merge, same arithmetic as split_combine:
// weights exp(lse_s - max) over their sum, chunks with lse_s = -inf taking
// weight 0 whatever their o_s holds), so the merged rows never go through
// memory; the merged lse is written once per (row, head).
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {


__global__ void __launch_bounds__(256) out_uv_mfma(const OutUvArgs a) {
  constexpr int kPad = 33;  // LDS row stride (floats) of the partial tiles
  __shared__ float red[4][2][32 * kPad];
  // block ids: 8 consecutive heads, then their other halves
  const int h = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7), half = (blockIdx.x >> 3) & 1;
  if (h >= a.heads) return;
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
      if (m0 + row < a.rows) store_out(a.out, ((int64_t)(m0 + row) * a.heads + h) * 128 + half * 64 + d, v, a.out_bf16);
    }
    __syncthreads();
  }
}

// Merged form, bf16 weights.  Workgroup = (head, half of d_head), 4 waves
// (one per SIMD, so each holds up to 512 registers).  Per 32-row tile:
//  * every global load the tile needs is issued first: the weight slice, the
//    rows' chunk log-sum-exps and the first four chunks' partial rows
//    (thread t owns 16-byte column chunk t % 128 of rows t / 128 + 2 i, so a
//    wave's load covers 1 KB of one row);
//  * the merge weights exp(lse_s - max) / sum: 8 lanes per row, the lse held
//    in registers, reduced with lane shuffles, stored to LDS;
//  * the merged tile is summed in registers and stored to LDS as its bf16 hi
//    and lo terms, 16-byte chunk q of row r at slot q ^ r (32 rows read at
//    one chunk by the products then spread over the banks);
//  * wave w multiplies latent columns 128w .. 128w+127 (A from LDS, B = its
//    64 x 128 weight slice in registers); the four partial tiles are summed
//    through LDS.
// More than four chunks take further rounds of two; more than 64 recompute
// their weights from the row's max and sum.  The partials are fp32 or fp16
// (template argument; fp16 halves the bytes read), converted to fp32 on load.
template <typename PT>
__global__ void __launch_bounds__(256) merge_out_uv_mfma(const OutUvArgs a) {
  constexpr int kPad = 33;  // LDS row stride (floats) of the partial tiles
  constexpr int kW = 64;    // chunk weights held in LDS per round
  constexpr int kF = 4;     // chunks loaded with the first round
  __shared__ float red[4][2][32 * kPad];
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][32 * 1024];  // merged tile: hi, lo bf16
  __shared__ float wt[32][kW];
  __shared__ float rowm[32], rowinv[32];
  const int h = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7), half = (blockIdx.x >> 3) & 1;
  if (h >= a.heads) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n32 = lane & 31, g = lane >> 5;
  const int ns = a.num_splits;
  const int64_t rs = (int64_t)a.sq * a.heads;  // partial rows between consecutive chunks
  const int64_t cs = rs * 512;                 // floats between consecutive chunks
  // partial row of query row r (head h), chunk 0
  auto prow = [&](int r) -> int64_t {
    const int b = r / a.sq, q = r - b * a.sq;
    return (int64_t)b * ns * rs + (int64_t)q * a.heads + h;
  };
  // B operand: W[d][c], d = 64 half + 32 nt + n32, c = 128 wave + 16 ks + 8 g + j
  bf16x8 bw[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint16_t* w = (const uint16_t*)a.w + ((int64_t)h * 128 + half * 64 + nt * 32 + n32) * 512 + wave * 128 + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) bw[nt][ks] = as_bf16x8(*(const u32x4*)(w + ks * 16));
  }
  const int c = tid & 127, r0 = tid >> 7;
  for (int m0 = 0; m0 < a.rows; m0 += 32) {
    // ---- loads: the lse of row m0 + tid / 8 first (unconditional, clamped
    // indices), then the first chunks' partial rows: the weights wait only
    // for the former, the partial rows stay in flight meanwhile
    const int lr = tid >> 3, lj = tid & 7, r = m0 + lr;
    const float* lp = a.lse_part + prow(min(r, a.rows - 1));
    float lv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) lv[k] = lp[(int64_t)min(lj + 8 * k, ns - 1) * rs];
    asm volatile("" ::: "memory");  // keep the lse loads ahead of the partial rows
    const PT* vrow[16];  // chunk 0 of the thread's rows (clamped to a real row)
#pragma unroll
    for (int i = 0; i < 16; ++i) vrow[i] = (const PT*)a.o_part + prow(min(m0 + r0 + 2 * i, a.rows - 1)) * 512 + 4 * c;
    f32x4 v0[kF][16];
#pragma unroll
    for (int jj = 0; jj < kF; ++jj) {
      const int64_t so = (int64_t)min(jj, ns - 1) * cs;
#pragma unroll
      for (int i = 0; i < 16; ++i) v0[jj][i] = load4(vrow[i] + so);
    }
    // (an empty use of every lse value here keeps its load where it is, ahead
    // of the partial rows, instead of being moved into the branch below)
#pragma unroll
    for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(lv[k]));
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (!(r < a.rows && lj + 8 * k < ns)) lv[k] = -__builtin_inff();
    // ---- merge weights of row lr (8 lanes per row)
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, lv[k]);
    if (r < a.rows)
      for (int sk = lj + 64; sk < ns; sk += 8) m = fmaxf(m, lp[sk * rs]);
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float z = 0.f, ev[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ev[k] = lv[k] == -__builtin_inff() ? 0.f : expf(lv[k] - m);
      z += ev[k];
    }
    if (r < a.rows)
      for (int sk = lj + 64; sk < ns; sk += 8) {
        const float ls = lp[sk * rs];
        z += ls == -__builtin_inff() ? 0.f : expf(ls - m);
      }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) z += __shfl_xor(z, o, 64);
    const float inv = z > 0.f ? 1.f / z : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) wt[lr][lj + 8 * k] = ev[k] * inv;
    if (lj == 0) {
      rowm[lr] = m;
      rowinv[lr] = inv;
      if (a.lse && half == 0 && r < a.rows) a.lse[(int64_t)r * a.heads + h] = z > 0.f ? m + logf(z) : -__builtin_inff();
    }
    // LDS-only barrier: the weights are visible, the partial rows' loads stay
    // in flight (a full barrier would wait for every outstanding load)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // ---- merged tile in registers, chunk by chunk as the rows land; a chunk
    // past the end, or one whose weight is 0 (it saw no token: its data may
    // be anything), is dropped
    f32x4 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x4{};
#pragma unroll
    for (int jj = 0; jj < kF; ++jj)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = jj < ns ? wt[r0 + 2 * i][jj] : 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] = e > 0.f ? fmaf(e, v0[jj][i][k], acc[i][k]) : acc[i][k];
      }
    for (int s0 = kF; s0 < ns; s0 += 2) {
      if (s0 % kW == 0) {  // weights of chunks s0 .. s0 + kW - 1 from the rows' max and sum
        __syncthreads();
        for (int idx = tid; idx < 32 * kW; idx += 256) {
          const int rr = idx / kW, j = idx - rr * kW, rj = m0 + rr;
          float e = 0.f;
          if (rj < a.rows && s0 + j < ns && rowm[rr] != -__builtin_inff()) {
            const float ls = a.lse_part[prow(rj) + (int64_t)(s0 + j) * rs];
            e = ls == -__builtin_inff() ? 0.f : expf(ls - rowm[rr]) * rowinv[rr];
          }
          wt[rr][j] = e;
        }
        __syncthreads();
      }
      f32x4 v[2][16];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int64_t so = (int64_t)min(s0 + jj, ns - 1) * cs;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[jj][i] = load4(vrow[i] + so);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = s0 + jj < ns ? wt[r0 + 2 * i][(s0 + jj) % kW] : 0.f;
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[i][k] += e > 0.f ? e * v[jj][i][k] : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = r0 + 2 * i;
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float x0 = acc[i][2 * k], x1 = acc[i][2 * k + 1];
        hi[k] = pack_bf16x2(x0, x1);
        lo[k] = pack_bf16x2(x0 - __builtin_bit_cast(float, hi[k] << 16), x1 - __builtin_bit_cast(float, hi[k] & 0xFFFF0000u));
      }
      const int off = rr * 1024 + (((c >> 1) ^ rr) << 4) + (c & 1) * 8;
      *(u32x2*)(xs[0] + off) = u32x2{hi[0], hi[1]};
      *(u32x2*)(xs[1] + off) = u32x2{lo[0], lo[1]};
    }
    __syncthreads();
    // ---- products: A = merged rows n32, columns 128 wave + 16 ks + 8 g .. +7
    f32x16 acc2[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int q = 16 * wave + 2 * ks + g;
      const int off = n32 * 1024 + ((q ^ n32) << 4);
      const bf16x8 ah = *(const bf16x8*)(xs[0] + off);
      const bf16x8 al = *(const bf16x8*)(xs[1] + off);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        acc2[nt] = mfma32x32x16(ah, bw[nt][ks], acc2[nt]);
        acc2[nt] = mfma32x32x16(al, bw[nt][ks], acc2[nt]);
      }
    }
    // partial tile of this wave's latent quarter: D row (i/4)*8 + 4g + i%4, column n32
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[wave][nt][((i >> 2) * 8 + 4 * g + (i & 3)) * kPad + n32] = acc2[nt][i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = i * 256 + tid;
      const int row = idx >> 6, d = idx & 63, nt = d >> 5, n = d & 31;
      const float v = red[0][nt][row * kPad + n] + red[1][nt][row * kPad + n] + red[2][nt][row * kPad + n] +
                      red[3][nt][row * kPad + n];
      if (m0 + row < a.rows) store_out(a.out, ((int64_t)(m0 + row) * a.heads + h) * 128 + half * 64 + d, v, a.out_bf16);
    }
    __syncthreads();  // red, xs and wt are rewritten by the next tile
  }
}

// fp32 weights: workgroup = (head, block of 16 output dims d); wave w holds
// the weight rows d0 + 4w .. d0 + 4w + 3 in registers (lane l: columns
// 8l .. 8l+7 of each, a row read as 2 KB per wave) and reuses them for every
// query row: per row the wave's four dot products are reduced across the
// wave (DPP).  o_lat comes from memory, or (kMerge) is merged from the chunk
// partials into LDS first (weights exp(lse_s - max) over their sum, as in
// split_combine).
template <bool kMerge>
__global__ void __launch_bounds__(256) out_uv_f32(const OutUvArgs a) {
  __shared__ __attribute__((aligned(16))) float xs[512];
  const int h = blockIdx.x >> 3, d0 = (blockIdx.x & 7) * 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  f32x4 wr[4][2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float* w = (const float*)a.w + ((int64_t)h * 128 + d0 + 4 * wave + k) * 512 + 8 * lane;
    wr[k][0] = *(const f32x4*)w;
    wr[k][1] = *(const f32x4*)(w + 4);
  }
  for (int r = 0; r < a.rows; ++r) {
    __syncthreads();  // xs of the previous row is read
    if constexpr (kMerge) {
      if (tid < 128) {
        // thread t merges columns 4t .. 4t+3
        const int b = r / a.sq, q = r - b * a.sq;
        const int64_t rs = (int64_t)a.sq * a.heads;
        const int64_t base = (int64_t)b * a.num_splits * rs + (int64_t)q * a.heads + h;
        const float* lp = a.lse_part + base;
        const int64_t op = base * 512 + 4 * tid;  // element index of the chunk-0 partial
        float m = -__builtin_inff();
        for (int s = 0; s < a.num_splits; ++s) m = fmaxf(m, lp[s * rs]);
        f32x4 x = f32x4{};
        float z = 0.f;
        if (m != -__builtin_inff()) {
          for (int s = 0; s < a.num_splits; ++s) {
            const float ls = lp[s * rs];
            if (ls == -__builtin_inff()) continue;
            const float e = expf(ls - m);
            z += e;
            const int64_t i = op + s * rs * 512;
            x += e * (a.part_f16 ? load4((const _Float16*)a.o_part + i) : load4((const float*)a.o_part + i));
          }
        }
        *(f32x4*)&xs[4 * tid] = x * (z > 0.f ? 1.f / z : 0.f);
        if (a.lse && tid == 0 && (blockIdx.x & 7) == 0)
          a.lse[(int64_t)r * a.heads + h] = z > 0.f ? m + logf(z) : -__builtin_inff();
      }
    } else {
      if (tid < 128) *(f32x4*)&xs[4 * tid] = *(const f32x4*)(a.o_lat + ((int64_t)r * a.heads + h) * 512 + 4 * tid);
    }
    __syncthreads();
    const f32x4 x0 = *(const f32x4*)&xs[8 * lane], x1 = *(const f32x4*)&xs[8 * lane + 4];
    float acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) v = fmaf(wr[k][0][e], x0[e], fmaf(wr[k][1][e], x1[e], v));
      acc[k] = wave_sum_rows(v);
    }
    if (lane < 4) {
      const float v = lane == 0 ? acc[0] : lane == 1 ? acc[1] : lane == 2 ? acc[2] : acc[3];
      store_out(a.out, ((int64_t)r * a.heads + h) * 128 + d0 + 4 * wave + lane, v, a.out_bf16);
    }
  }
}

template __global__ void merge_out_uv_mfma<float>(const OutUvArgs);
template __global__ void merge_out_uv_mfma<_Float16>(const OutUvArgs);
template __global__ void out_uv_f32<false>(const OutUvArgs);
template __global__ void out_uv_f32<true>(const OutUvArgs);

}  // namespace mla
