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
// out_uv_mfma: workgroup = (head, half of d_head): its 64 x 512 weight
// slice (64 KB) is read from HBM once into registers and reused for every
// 32-row tile.  The
// four waves split the latent (K) dimension, 128 columns each, so every wave
// issues all of its loads at once; the partial tiles are summed through LDS.
// The two halves of a head run on one XCD (block ids 8 apart), where the
// second read of each o_lat row is an L2 hit.
//
// Merged form (merge_out_uv16, out_uv_f32<true>): o_lat is not read but
// formed on the fly from the KV chunks' normalised partial outputs o_s and
// log-sum-exps lse_s (the split merge, same arithmetic as split_combine:
// weights exp(lse_s - max) over their sum, chunks with lse_s = -inf taking
// weight 0 whatever their o_s holds), so the merged rows never go through
// memory; the merged lse is written once per (row, head).  merge_out_uv16
// gives each merged row to one workgroup, which holds its head's whole
// weight block (see the kernel).
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

// Eight consecutive chunk-partial values of one row (fp16 or fp32 storage,
// 16-byte aligned), converted to fp32 when used.
template <typename PT>
struct Piece8;
template <>
struct Piece8<_Float16> {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  f16x8 v;
  __device__ __forceinline__ void load(const _Float16* p) { v = *(const f16x8*)p; }
  __device__ __forceinline__ float operator[](int k) const { return (float)v[k]; }
};
template <>
struct Piece8<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *(const f32x4*)p;
    hi = *(const f32x4*)(p + 4);
  }
  __device__ __forceinline__ float operator[](int k) const { return k < 4 ? lo[k] : hi[k - 4]; }
};

// Merged form, bf16 weights, 16-row tiles.  Workgroup = (head, row group):
// the a.groups workgroups of a head take its 16-row tiles in turn (block
// ids 8 apart, so that they share an XCD and the head's weights in L2).
// Four waves, one per SIMD.  Wave w holds the weight rows (output dims)
// 32 w .. 32 w + 31 over all 512 latent columns in registers, so it
// multiplies the full K for its outputs and no partial sums are exchanged;
// each merged row is formed once, by one workgroup.  Per tile:
//  * thread t merges row t / 16, columns 8 (t % 16) + 128 j + 0..7 (j < 4):
//    the row's chunk log-sum-exps are loaded first, then the first four
//    chunks' pieces (16 bytes each, a wave load covering 256 contiguous
//    bytes of four rows);
//  * the 16 lanes of a row form its merge weights exp(lse_s - max) / sum
//    with lane shuffles while the pieces are in flight, and keep them in LDS;
//  * the merged pieces are summed in registers (a chunk whose weight is 0,
//    one that saw no token, is dropped whatever it holds) and stored to LDS
//    as bf16 hi and lo terms, 16-byte chunk q of row r at slot q ^ r;
//  * out^T[32 w + 16 db + 0..15][16 rows] with v_mfma_f32_16x16x32_bf16,
//    A = the weights (registers), B = the merged rows (LDS), hi then lo.
// More than four chunks take further rounds of two; more than 64 recompute
// their weights from the row's max and sum.  kF is the number of chunks the
// first round loads: 4, or 1 for a single chunk (num_splits == 1 only: the
// rounds after the first assume kF even).
template <typename PT, int kF>
__global__ void __launch_bounds__(256) merge_out_uv16(const OutUvArgs a) {
  static_assert(kF == 4 || kF == 1, "first round of four chunks, or the single chunk");
  const int groups = a.groups;
  constexpr int kW = 64;  // chunk weights held in LDS per round
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][16 * 1024];  // merged tile: hi, lo bf16
  __shared__ float wt[16][kW];
  __shared__ float rowm[16], rowinv[16];
  const int bid = blockIdx.x;
  const int h = bid / (8 * groups) * 8 + (bid & 7), grp = (bid >> 3) % groups;
  if (h >= a.heads) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i16 = lane & 15, q4 = lane >> 4;
  const int ns = a.num_splits;
  const int64_t rs = (int64_t)a.sq * a.heads;  // partial rows between consecutive chunks
  const int64_t cs = rs * 512;                 // elements between consecutive chunks
  auto prow = [&](int r) -> int64_t {          // partial row of query row r (head h), chunk 0
    const int b = r / a.sq, q = r - b * a.sq;
    return (int64_t)b * ns * rs + (int64_t)q * a.heads + h;
  };
  // A operand of k-step ks for block db: W[d][c], d = 32 wave + 16 db + i16,
  // c = 32 ks + 8 q4 .. +7
  bf16x8 aw[2][16];
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const uint16_t* w = (const uint16_t*)a.w + ((int64_t)h * 128 + 32 * wave + 16 * db + i16) * 512 + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) aw[db][ks] = as_bf16x8(*(const u32x4*)(w + 32 * ks));
  }
  const int lr = tid >> 4, cj = tid & 15;
  for (int m0 = 16 * grp; m0 < a.rows; m0 += 16 * groups) {
    const int r = m0 + lr;
    const int64_t pr = prow(min(r, a.rows - 1));
    const float* lp = a.lse_part + pr;
    float lv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) lv[k] = lp[(int64_t)min(cj + 16 * k, ns - 1) * rs];
    asm volatile("" ::: "memory");  // keep the lse loads ahead of the partial pieces
    const PT* vr = (const PT*)a.o_part + pr * 512 + 8 * cj;
    Piece8<PT> v0[kF][4];
#pragma unroll
    for (int jj = 0; jj < kF; ++jj) {
      const int64_t so = (int64_t)min(jj, ns - 1) * cs;
#pragma unroll
      for (int j = 0; j < 4; ++j) v0[jj][j].load(vr + so + 128 * j);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(lv[k]));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (!(r < a.rows && cj + 16 * k < ns)) lv[k] = -__builtin_inff();
    // ---- merge weights of row lr (its 16 lanes)
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < 4; ++k) m = fmaxf(m, lv[k]);
    if (r < a.rows)
      for (int sk = cj + 64; sk < ns; sk += 16) m = fmaxf(m, lp[(int64_t)sk * rs]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float z = 0.f, ev[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ev[k] = lv[k] == -__builtin_inff() ? 0.f : expf(lv[k] - m);
      z += ev[k];
    }
    if (r < a.rows)
      for (int sk = cj + 64; sk < ns; sk += 16) {
        const float ls = lp[(int64_t)sk * rs];
        z += ls == -__builtin_inff() ? 0.f : expf(ls - m);
      }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
    const float inv = z > 0.f ? 1.f / z : 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) wt[lr][cj + 16 * k] = ev[k] * inv;
    if (cj == 0) {
      rowm[lr] = m;
      rowinv[lr] = inv;
      if (a.lse && r < a.rows) a.lse[(int64_t)r * a.heads + h] = z > 0.f ? m + logf(z) : -__builtin_inff();
    }
    // LDS-only barrier: the weights are visible, the pieces stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float acc[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[j][k] = 0.f;
#pragma unroll
    for (int jj = 0; jj < kF; ++jj) {
      const float e = jj < ns ? wt[lr][jj] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[j][k] = e > 0.f ? fmaf(e, v0[jj][j][k], acc[j][k]) : acc[j][k];
    }
    for (int s0 = kF; s0 < ns; s0 += 2) {
      if (s0 % kW == 0) {  // weights of chunks s0 .. s0 + kW - 1 from the rows' max and sum
        __syncthreads();
        for (int idx = tid; idx < 16 * kW; idx += 256) {
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
      Piece8<PT> v[2][4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int64_t so = (int64_t)min(s0 + jj, ns - 1) * cs;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[jj][j].load(vr + so + 128 * j);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const float e = s0 + jj < ns ? wt[lr][(s0 + jj) % kW] : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[j][k] = e > 0.f ? fmaf(e, v[jj][j][k], acc[j][k]) : acc[j][k];
      }
    }
    // ---- the merged row as bf16 hi + lo: chunk cj + 16 j of row lr
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = acc[j][2 * k], x1 = acc[j][2 * k + 1];
        hi[k] = pack_bf16x2(x0, x1);
        lo[k] = pack_bf16x2(x0 - __builtin_bit_cast(float, hi[k] << 16), x1 - __builtin_bit_cast(float, hi[k] & 0xFFFF0000u));
      }
      const int off = lr * 1024 + (((cj + 16 * j) ^ lr) << 4);
      *(u32x4*)(xs[0] + off) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      *(u32x4*)(xs[1] + off) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
    __syncthreads();
    // ---- products: B = merged row i16, columns 32 ks + 8 q4 .. +7
    f32x4 acc2[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int off = i16 * 1024 + (((4 * ks + q4) ^ i16) << 4);
      const bf16x8 bh = *(const bf16x8*)(xs[0] + off);
      const bf16x8 bl = *(const bf16x8*)(xs[1] + off);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        acc2[db] = mfma16x16x32(aw[db][ks], bh, acc2[db]);
        acc2[db] = mfma16x16x32(aw[db][ks], bl, acc2[db]);
      }
    }
    // D: column i16 = row m0 + i16, rows 4 q4 + i = output dims of the block
    const int orow = m0 + i16;
    if (orow < a.rows) {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int64_t e = ((int64_t)orow * a.heads + h) * 128 + 32 * wave + 16 * db + 4 * q4;
        if (a.out_bf16)
          *(u32x2*)((uint16_t*)a.out + e) = u32x2{pack_bf16x2(acc2[db][0], acc2[db][1]), pack_bf16x2(acc2[db][2], acc2[db][3])};
        else
          *(f32x4*)((float*)a.out + e) = acc2[db];
      }
    }
    __syncthreads();  // xs and wt are rewritten by the next tile
  }
}

// Merged form, bf16 weights, for few query rows and many chunks (the fused
// kernel above spreads rows, not chunks, over its threads).  Workgroup =
// (head, half of d_head); per query row:
//  * the 256 threads merge the row: thread t takes columns 8 (t % 64) .. +7
//    of chunks g, g + 4, g + 8, ... (g = t / 64) in rounds of kR chunks,
//    every load of a round issued before any is used, each chunk group with
//    its own running maximum (a chunk with lse = -inf takes no part,
//    whatever its partial holds); the four groups are combined through LDS;
//  * wave w computes output dims d0 + 16 w .. + 15: lane l holds columns
//    8 l .. 8 l + 7 of those 16 weight rows in registers for every row, the
//    products (exact, bf16 x fp32) and sums are fp32, then summed across the
//    wave.
template <typename PT>
__global__ void __launch_bounds__(256) merge_out_uv_few(const OutUvArgs a) {
  constexpr int kR = sizeof(PT) == 2 ? 16 : 8;  // chunks per round and group
  __shared__ __attribute__((aligned(16))) float gx[4][512];
  __shared__ float gm[4], gz[4];
  __shared__ __attribute__((aligned(16))) float xs[512];
  const int h = blockIdx.x >> 1, d0 = (blockIdx.x & 1) * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  u32x4 wr[16];
#pragma unroll
  for (int k = 0; k < 16; ++k)
    wr[k] = *(const u32x4*)((const uint16_t*)a.w + ((int64_t)h * 128 + d0 + 16 * wave + k) * 512 + 8 * lane);
  const int ns = a.num_splits;
  const int64_t rs = (int64_t)a.sq * a.heads, cs = rs * 512;
  const int g = tid >> 6, c8 = tid & 63;
  for (int r = 0; r < a.rows; ++r) {
    const int b = r / a.sq, q = r - b * a.sq;
    const int64_t pr = (int64_t)b * ns * rs + (int64_t)q * a.heads + h;
    const float* lp = a.lse_part + pr;
    const PT* vp = (const PT*)a.o_part + pr * 512 + 8 * c8;
    float m = -__builtin_inff(), z = 0.f, x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.f;
    for (int s0 = g; s0 < ns; s0 += 4 * kR) {
      float l[kR];
      Piece8<PT> pv[kR];
#pragma unroll
      for (int k = 0; k < kR; ++k) {
        const int sc = min(s0 + 4 * k, ns - 1);  // past the last chunk: read it again, not counted
        l[k] = lp[sc * rs];
        pv[k].load(vp + sc * cs);
      }
      __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any result is used
#pragma unroll
      for (int k = 0; k < kR; ++k)
        if (s0 + 4 * k >= ns) l[k] = -__builtin_inff();
      float mr = m;
#pragma unroll
      for (int k = 0; k < kR; ++k) mr = fmaxf(mr, l[k]);
      // branch-free: while no chunk holds a token, m and mr are -inf and every weight is 0
      const float c = m == -__builtin_inff() ? 0.f : expf(m - mr);
      z *= c;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] *= c;
#pragma unroll
      for (int k = 0; k < kR; ++k) {
        const bool live = l[k] != -__builtin_inff();
        const float e = live ? expf(l[k] - mr) : 0.f;
        z += e;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = live ? fmaf(e, pv[k][j], x[j]) : x[j];
      }
      m = mr;
    }
    __syncthreads();  // xs of the previous row is read
    if (c8 == 0) {
      gm[g] = m;
      gz[g] = z;
    }
    *(f32x4*)&gx[g][8 * c8] = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4*)&gx[g][8 * c8 + 4] = f32x4{x[4], x[5], x[6], x[7]};
    __syncthreads();
    {
      const float mm = fmaxf(fmaxf(gm[0], gm[1]), fmaxf(gm[2], gm[3]));
      float wg[4], zz = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        wg[k] = gm[k] == -__builtin_inff() ? 0.f : expf(gm[k] - mm);
        zz += wg[k] * gz[k];
      }
      const float inv = zz > 0.f ? 1.f / zz : 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int col = tid + 256 * u;
        float v = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) v = fmaf(wg[k], gx[k][col], v);
        xs[col] = v * inv;
      }
      if (a.lse && tid == 0 && (blockIdx.x & 1) == 0)
        a.lse[(int64_t)r * a.heads + h] = zz > 0.f ? mm + logf(zz) : -__builtin_inff();
    }
    __syncthreads();
    const f32x4 x0 = *(const f32x4*)&xs[8 * lane], x1 = *(const f32x4*)&xs[8 * lane + 4];
    float mine = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w2 = wr[k][e];  // columns 8 lane + 2e, + 2e + 1
        v = fmaf(__uint_as_float(w2 << 16), e < 2 ? x0[2 * e] : x1[2 * e - 4], v);
        v = fmaf(__uint_as_float(w2 & 0xFFFF0000u), e < 2 ? x0[2 * e + 1] : x1[2 * e - 3], v);
      }
      v = wave_sum_rows(v);
      mine = lane == k ? v : mine;
    }
    if (lane < 16) store_out(a.out, ((int64_t)r * a.heads + h) * 128 + d0 + 16 * wave + lane, mine, a.out_bf16);
  }
}

// fp32 weights: workgroup = (head, block of 16 output dims d); wave w holds
// the weight rows d0 + 4w .. d0 + 4w + 3 in registers (lane l: columns
// 8l .. 8l+7 of each, a row read as 2 KB per wave) and reuses them for every
// query row: per row the wave's four dot products are reduced across the
// wave (DPP).  o_lat comes from memory, or (kMerge) is merged from the chunk
// partials into LDS first (weights exp(lse_s - max) over their sum, as in
// split_combine).

// Columns 4c .. 4c+3 of one row merged from its chunk partials (element
// index op of chunk 0, chunk s at op + s * cs; log-sum-exps at lp[s * ls]):
// rounds of 16 chunks with every load of a round issued before any is used
// (indices past the last chunk read the last one and are not counted); the
// running maximum rescales the sums between rounds.  A chunk with lse = -inf
// takes no part, whatever its partial holds.  Returns the normalised row
// piece and, through lse_out, ln of the weight sum plus the maximum.
template <typename PT>
__device__ __forceinline__ f32x4 merge_row4(const PT* part, int64_t op, int64_t cs, const float* lp, int64_t ls,
                                            int ns, float& lse_out) {
  constexpr int kR = 16;
  float m = -__builtin_inff(), z = 0.f;
  f32x4 x = f32x4{};
  for (int s0 = 0; s0 < ns; s0 += kR) {
    float l[kR];
    f32x4 pv[kR];
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const int sc = min(s0 + k, ns - 1);
      l[k] = lp[sc * ls];
      pv[k] = load4(part + op + sc * cs);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any result is used
#pragma unroll
    for (int k = 0; k < kR; ++k)
      if (s0 + k >= ns) l[k] = -__builtin_inff();
    float mr = m;
#pragma unroll
    for (int k = 0; k < kR; ++k) mr = fmaxf(mr, l[k]);
    // branch-free, so that the round's loads issue together: while no chunk
    // holds a token, m and mr are -inf and every weight below is 0
    const float c = m == -__builtin_inff() ? 0.f : expf(m - mr);
    z *= c;
    x *= c;
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const bool live = l[k] != -__builtin_inff();
      const float e = live ? expf(l[k] - mr) : 0.f;
      z += e;
      const f32x4 y = x + e * pv[k];
      x = live ? y : x;
    }
    m = mr;
  }
  lse_out = z > 0.f ? m + logf(z) : -__builtin_inff();
  return x * (z > 0.f ? 1.f / z : 0.f);
}

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
        const int64_t op = base * 512 + 4 * tid;  // element index of the chunk-0 partial
        float lse_r;
        const f32x4 x = a.part_f16
                            ? merge_row4((const _Float16*)a.o_part, op, rs * 512, a.lse_part + base, rs, a.num_splits, lse_r)
                            : merge_row4((const float*)a.o_part, op, rs * 512, a.lse_part + base, rs, a.num_splits, lse_r);
        *(f32x4*)&xs[4 * tid] = x;
        if (a.lse && tid == 0 && (blockIdx.x & 7) == 0) a.lse[(int64_t)r * a.heads + h] = lse_r;
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

template __global__ void merge_out_uv_few<float>(const OutUvArgs);
template __global__ void merge_out_uv_few<_Float16>(const OutUvArgs);
template __global__ void merge_out_uv16<float, 4>(const OutUvArgs);
template __global__ void merge_out_uv16<_Float16, 4>(const OutUvArgs);
template __global__ void merge_out_uv16<float, 1>(const OutUvArgs);
template __global__ void merge_out_uv16<_Float16, 1>(const OutUvArgs);
template __global__ void out_uv_f32<false>(const OutUvArgs);
template __global__ void out_uv_f32<true>(const OutUvArgs);

}  // namespace mla
