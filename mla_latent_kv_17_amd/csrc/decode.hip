// MLA absorbed decode attention over a paged latent cache, gfx950 (MI355X).
//
// Follows deepforge.srivtx.xyz "DeepSeek-V2", section 1: decode compares the
// newest query with the keys of all earlier tokens and mixes their values
// ("The bottleneck at inference time"); the cache holds only c_t (512) and
// k^R_t (64) and attention runs on it directly once W_UK is folded into the
// query and W_UV into the output ("Store a latent, rebuild the keys and
// values", "absorption").  Per query row r and cached token t:
//     s[r][t] = (q_lat[r] . c_t + q_rope[r] . k^R_t) * scale
//     o_lat[r] = sum_t softmax(s[r])_t c_t,   lse[r] = ln sum_t exp s[r][t]
//
// Two kernels:
//  * decode_mfma  (bf16 or fp8 cache): one workgroup = 4 waves owns one
//    (sequence, KV chunk, block of 128 query rows).  32-token tiles of the
//    576-wide rows are streamed HBM -> LDS (bf16: DMA loads that bypass
//    registers; fp8: register-staged with E4M3 -> bf16 conversion) into a
//    ring of tile buffers, and every tile is shared by all 128 rows.
//      - scores:  wave w computes S^T[32 tokens][its 32 rows] with
//        v_mfma_f32_32x32x16_bf16, A = cache rows from LDS, B = its queries
//        (held in registers for the whole kernel), K = 576.
//      - softmax: exp2-domain online softmax with a lazy reference max (the
//        accumulator is rescaled only when a row's max grows by more than
//        2^8), row sums kept per lane.
//      - values:  P is exchanged through LDS and wave w accumulates
//        O^T[its 128 latent columns][all 128 rows] += C^T P^T, A = cache
//        columns read with the gfx950 transposing LDS load, so each cache
//        element is read from LDS once per workgroup for this product.
//  * decode_scalar (fp32 cache, and any dtype as a plain second path):
//    one workgroup per (sequence, chunk, query row), fp32 VALU.
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

// Zero bytes standing in for cache rows past a sequence's length: their tile
// rows must hold zeros (not whatever is in memory) because the value product
// multiplies them by p = 0.
__device__ __attribute__((aligned(1024))) const uint32_t g_zero_row[256] = {0};

namespace {

constexpr int kTileTok = 32;                    // tokens per LDS tile
constexpr int kLatBytes = kTileTok * 64 * 16;   // latent part: 32 rows x 64 chunks of 16 B
constexpr int kRopeBytes = kTileTok * 8 * 16;   // RoPE part:   32 rows x 8 chunks
constexpr int kTileBytes = kLatBytes + kRopeBytes;  // 36,864
constexpr int kStageBytes = kTileTok * 512;     // fp8 latent codes of one tile
constexpr int kRowsPerWg = 64;
constexpr float kRefSlack = 64.0f;              // log2 headroom above a row's reference max

// LDS tile layout (64 banks x 4 B): chunk q of latent row r sits at slot
// r*64 + (q ^ s16(r)); chunk q of RoPE row r at r*8 + (q ^ s8(r)) after the
// latent part.  s16 makes 16 consecutive rows at one chunk hit 16 distinct
// bank groups (score operand reads) and 4 consecutive rows x 4 chunks hit 16
// distinct groups (transposing value-operand reads); s8 does the former for
// the 128-byte RoPE rows.
__device__ __forceinline__ int s16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int s8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lat_off(int r, int q) { return (r * 64 + (q ^ s16(r))) * 16; }
__device__ __forceinline__ int rope_off(int r, int q) { return kLatBytes + (r * 8 + (q ^ s8(r))) * 16; }

__device__ __forceinline__ uint32_t lds_addr(const MLA_LDS void* p) { return (uint32_t)(size_t)p; }

// Wave-wide HBM -> LDS copy of 16 bytes per lane: lane i's data lands at
// lds_base + 16 * i (the base travels in M0, which is saved and restored so
// the compiler's own use of M0 is untouched; one wait state separates the M0
// write from the load that reads it).  Issued through asm so that the
// compiler does not turn later LDS reads into waits for every outstanding
// copy; completion is tracked with explicit s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}

// Same copy with a wave-uniform 64-bit base in SGPRs plus a 32-bit per-lane
// byte offset (no per-lane address arithmetic).
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  // readfirstlane returns int: widen each half through uint32_t (a sign
  // extension of the low half would overwrite the high half of the address)
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  base = (const void*)(((uint64_t)hi << 32) | (uint64_t)lo);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds_base)
      : "memory");
}

// A wait the compiler sees (it updates its own counter model): all vector
// memory loads issued so far have completed.
__device__ __forceinline__ void wait_all_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Scalar (constant address space) load of a wave-uniform int: tracked by
// lgkmcnt, so it never waits on the outstanding HBM -> LDS copies.
__device__ __forceinline__ int load_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

struct Work {
  int b, split, rb;
  int len, tok0, tok1, ntiles;
};

// XCD-aware placement: workgroups are dispatched round-robin over the 8 XCDs,
// so the row blocks of one (sequence, chunk) get ids 8 apart and land on the
// same XCD, where the second read of each tile is an L2 hit.
__device__ __forceinline__ bool decode_work(const DecodeArgs& a, Work& w) {
  const int id = blockIdx.x;
  const int xcd = id & 7, k = id >> 3;
  w.rb = k % a.row_blocks;
  const int unit = (k / a.row_blocks) * 8 + xcd;
  if (unit >= a.units) return false;
  w.b = unit / a.num_splits;
  w.split = unit - w.b * a.num_splits;
  w.len = a.seq_lens[w.b];
  const int npages = (w.len + 63) >> 6;
  const int pps = (npages + a.num_splits - 1) / a.num_splits;
  const int p0 = w.split * pps;
  const int p1 = min(p0 + pps, npages);
  w.tok0 = p0 * 64;
  w.tok1 = min(p1 * 64, w.len);
  w.ntiles = w.tok1 > w.tok0 ? (w.tok1 - w.tok0 + kTileTok - 1) / kTileTok : 0;
  return true;
}

}  // namespace

// bf16 cache.  Workgroup = 4 waves = one (sequence, KV chunk, block of 64
// query rows).  The context is walked in 64-token steps (two 32-token tiles
// = one cache page).  Wave w: score rows 32*(w&1) .. +31 over the step's token
// half (w>>1), and value columns 128*w .. +127 for all 64 rows.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_mfma_bf16(const DecodeArgs a) {
  constexpr int kBuf = 4;                       // tile ring = 2 steps
  constexpr int kPBytes = 2 * 4 * 64 * 16;      // P^T fragments: 64 rows x 64 tokens
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kBuf * kTileBytes + kPBytes + 1024];
  MLA_LDS uint8_t* const tiles = (MLA_LDS uint8_t*)&smem[0];
  MLA_LDS uint8_t* const pl = tiles + kBuf * kTileBytes;
  MLA_LDS float* const xm = (MLA_LDS float*)(pl + kPBytes);   // [2 halves][64 rows] maxima
  MLA_LDS float* const xl = xm + 128;                         // [64] row sums
  MLA_LDS int* const xf = (MLA_LDS int*)(xl + 64);            // [4] overflow flags

  Work wk;
  if (!decode_work(a, wk)) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int g = lane >> 5;      // k-half of an MFMA operand
  const int n32 = lane & 31;
  const int rg = wave & 1;      // score row group
  const int th = wave >> 1;     // token half of a step
  const int rows = a.rows;
  const int row_base = wk.rb * kRowsPerWg;
  const int64_t slot = (int64_t)wk.b * a.num_splits + wk.split;
  const int ntiles = wk.ntiles;
  const int nsteps = (ntiles + 1) >> 1;
  const uint32_t tiles_lds = lds_addr(tiles);

  // ---- HBM -> LDS copies of one 32-token tile: 9 instructions per wave.
  // A step's two tiles are the halves of one 64-token page, so one block id
  // serves both; ids are fetched a step ahead with scalar loads.
  const int64_t bt_row = (int64_t)wk.b * a.max_blocks;
  auto page_block = [&](int st) __attribute__((always_inline)) -> int {
    return 2 * st < ntiles ? load_uniform(a.block_table, bt_row + (wk.tok0 >> 6) + st) : 0;
  };
  // RoPE part: rows wave*8 + lane/8, 8 chunks each (lane part of the address)
  const int rope_r = wave * 8 + (lane >> 3);
  const uint32_t rope_lane = (uint32_t)((lane >> 3) * a.rope_rs) + ((((lane & 7) ^ s8(rope_r))) << 4);
  // copy j of a full tile (all 32 rows hold tokens): j < 8 is latent row
  // wave*8 + j, j == 8 the wave's eight RoPE rows
  auto tile_chunk = [&](int t, int blk, int j) __attribute__((always_inline)) {
    const int tt = wk.tok0 + t * kTileTok;
    const int r0 = (tt & 63) + wave * 8;
    const uint32_t tl = tiles_lds + (t % kBuf) * kTileBytes;
    if (j < 8) {
      const uint8_t* rp = a.latent + blk * a.lat_bs + (int64_t)(r0 + j) * a.lat_rs;
      const int sw = ((j & 3) << 2) | ((2 * wave + (j >> 2)) & 3);  // s16(wave*8 + j)
      dma16s(rp, (uint32_t)(lane ^ sw) << 4, tl + (wave * 8 + j) * 1024);
    } else {
      const uint8_t* rr = a.rope + blk * a.rope_bs + (int64_t)r0 * a.rope_rs;
      dma16s(rr, rope_lane, tl + kLatBytes + wave * 1024);
    }
  };
  auto issue_tile = [&](int t, int blk) __attribute__((always_inline)) {
    const int tt = wk.tok0 + t * kTileTok;
    const int r0 = (tt & 63) + wave * 8;
    const uint32_t tl = tiles_lds + (t % kBuf) * kTileBytes;
    const uint8_t* rp = a.latent + blk * a.lat_bs + (int64_t)r0 * a.lat_rs;
    const uint8_t* rr = a.rope + blk * a.rope_bs + (int64_t)r0 * a.rope_rs;
    const int valid_rows = wk.len - tt - wave * 8;  // rows j < valid_rows hold tokens
    if (valid_rows >= 8) {
#pragma unroll
      for (int j = 0; j < 9; ++j) tile_chunk(t, blk, j);
    } else {  // last page of the sequence: rows past its length read zeros
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sw = ((j & 3) << 2) | ((2 * wave + (j >> 2)) & 3);
        if (j < valid_rows)
          dma16s(rp + (int64_t)j * a.lat_rs, (uint32_t)(lane ^ sw) << 4, tl + (wave * 8 + j) * 1024);
        else
          dma16s(g_zero_row, (uint32_t)lane << 4, tl + (wave * 8 + j) * 1024);
      }
      const uint8_t* src = (lane >> 3) < valid_rows ? rr + rope_lane : (const uint8_t*)g_zero_row + (lane << 4);
      dma16(src, tl + kLatBytes + wave * 1024);
    }
  };
  auto issue_step = [&](int st, int blk) __attribute__((always_inline)) {
    if (2 * st < ntiles) issue_tile(2 * st, blk);
    if (2 * st + 1 < ntiles) issue_tile(2 * st + 1, blk);
  };

  // first pass: the copies of step 0 overlap the query loads
  issue_step(0, page_block(0));

  // ---- queries of rows row_base + 32*rg + n32: B operand of the score product
  const int qrow = row_base + rg * 32 + n32;
  const bool qvalid = qrow < rows;
  bf16x8 qf[36];
  {
    const int qr = qvalid ? qrow : 0;
    const uint16_t* ql = a.q_lat + ((int64_t)wk.b * rows + qr) * 512 + 8 * g;
    const uint16_t* qp = a.q_rope + ((int64_t)wk.b * rows + qr) * 64 + 8 * g;
#pragma unroll
    for (int kb = 0; kb < 32; ++kb) qf[kb] = as_bf16x8(*(const u32x4*)(ql + kb * 16));
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qf[32 + kb] = as_bf16x8(*(const u32x4*)(qp + kb * 16));
    if (!qvalid)
#pragma unroll
      for (int kb = 0; kb < 36; ++kb) qf[kb] = as_bf16x8(u32x4{0, 0, 0, 0});
    // the query loads (and the step-0 copies) complete here, where the
    // compiler sees it, so it never waits on later copies when Q is used
    wait_all_vmem();
  }
  // a row's query sees tokens < its horizon; the chunk ends at tok1
  const int qi = qvalid ? qrow / a.heads : 0;
  const int hi_tok = min(wk.tok1, qvalid ? wk.len - (a.sq - 1 - qi) : 0);
  const int hi_min = min(wk.tok1, wk.len - (a.sq - 1));

  // ---- per-lane LDS offsets (the tile buffer adds a constant)
  // score operand: latent row n32, chunk 2kb+g; RoPE row n32, chunk 2(kb-32)+g
  const uint32_t c1_lat = n32 * 1024 + th * kTileBytes;
  const uint32_t lat_x = (16 * g) ^ (16 * s16(n32));
  const uint32_t c1_rope = kLatBytes + n32 * 128 + th * kTileBytes;
  const uint32_t rope_x = (16 * g) ^ (16 * s8(n32));
  // value operand (transposing reads): token row 16hb + 8j2 + 4g + i/4, columns
  // 128*wave + 32*mt + 16*(lane/16 % 2) + 4*(i%4), i = lane % 16
  const int i16 = lane & 15;
  const int vy = 2 * ((lane >> 4) & 1) + ((i16 >> 1) & 1);
  uint32_t voff[2][4];
#pragma unroll
  for (int j2 = 0; j2 < 2; ++j2) {
    const int sw = (((i16 >> 2) & 3) << 2) | ((2 * j2 + g) & 3);  // s16 of the row
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      voff[j2][mt] = (8 * j2 + 4 * g + (i16 >> 2)) * 1024 + wave * 256 + (((4 * mt) ^ vy ^ sw) << 4) + (i16 & 1) * 8;
  }

  // ---- accumulators.  A row's reference max m_ref is fixed at its first
  // finite step maximum, so P and O never need rescaling.  If a later score
  // exceeds it by more than 2^kRefSlack the pass is finished (its values are
  // discarded) and repeated with the row's chunk maximum as the reference:
  // exact either way, and never taken unless the scores of one row span more
  // than 44 nats.
  f32x16 oacc[4][2];
  float m_ref = -__builtin_inff();   // this lane's score row (log2 domain)
  float m_hi = -__builtin_inff();    // largest step maximum seen this pass
  float l_part = 0.f;                // this lane's share of the row sum
  bool ovf = false;

  auto run_step = [&](int st, int& blk_next, bool set_ref, auto parc) __attribute__((always_inline)) {
    constexpr int par = decltype(parc)::value;  // st & 1: which half of the tile ring
    // tiles of step st-1 are free (barrier 2 of the previous step): prefetch
    // step st+1.  When both of its tiles are full (every step but a
    // sequence's last page), the 18 copies are spread over the score
    // product below, one per two MFMAs, so that the wave never stalls on a
    // full memory queue with no matrix work in flight.
    const int blk_cur = blk_next;
    const bool spread = st + 1 < nsteps && wk.len - (wk.tok0 + (2 * st + 2) * kTileTok) >= 2 * kTileTok;
    if (st + 1 < nsteps && !spread) issue_step(st + 1, blk_cur);
    blk_next = page_block(st + 2);
    const bool own_valid = 2 * st + th < ntiles;
    const bool second_valid = 2 * st + 1 < ntiles;
    const int tt = wk.tok0 + (2 * st + th) * kTileTok;

    // ---- scores S^T[token][row] for this wave's token half, K = 576
    float p[16];
    if (own_valid) {
      const MLA_LDS uint8_t* tb = tiles + 2 * par * kTileBytes;
      auto ldA = [&](int kb) __attribute__((always_inline)) -> bf16x8 {
        if (kb < 32)
          return *(const MLA_LDS bf16x8*)(tb + c1_lat + (kb >> 3) * 256 + (((kb & 7) * 32) ^ lat_x));
        return *(const MLA_LDS bf16x8*)(tb + c1_rope + (((kb - 32) * 32) ^ rope_x));
      };
      constexpr int kDepth = 8;
      f32x16 sacc = f32x16{};
      bf16x8 ar[kDepth];
#pragma unroll
      for (int kb = 0; kb < kDepth; ++kb) ar[kb] = ldA(kb);
      if (spread) {
#pragma unroll
        for (int kb = 0; kb < 36; ++kb) {
          sacc = mfma32x32x16(ar[kb % kDepth], qf[kb], sacc);
          if (kb + kDepth < 36) ar[kb % kDepth] = ldA(kb + kDepth);
          if ((kb & 1) == 0) tile_chunk(2 * st + 2 + (kb >= 18), blk_cur, (kb >> 1) % 9);
          sched_fence();
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 36; ++kb) {
          sacc = mfma32x32x16(ar[kb % kDepth], qf[kb], sacc);
          if (kb + kDepth < 36) ar[kb % kDepth] = ldA(kb + kDepth);
          sched_fence();
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = sacc[r] * a.scale_log2;
      if (tt + kTileTok > hi_min) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = tt + (r >> 2) * 8 + 4 * g + (r & 3);
          if (tok >= hi_tok) p[r] = -__builtin_inff();
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = -__builtin_inff();
    }
    // value operand of the first 16-token block: issued now, used after barrier 1
    auto ldV = [&](int kb, bf16x8 (&av)[4]) __attribute__((always_inline)) {
      const MLA_LDS uint8_t* vt = tiles + (2 * par + (kb >> 1)) * kTileBytes + (kb & 1) * 16 * 1024;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const u32x2 lo = lds_read_tr16_b64(vt + voff[0][mt]);
        const u32x2 hi = lds_read_tr16_b64(vt + voff[1][mt]);
        av[mt] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
    };
    bf16x8 av[4];
    ldV(0, av);

    float mx = p[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, p[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (set_ref) {
      // first step of the first pass (workgroup-uniform): the two token halves
      // agree on each row's reference.  A row left at -inf here sees no token
      // of this chunk at all (a row's visible tokens are a prefix of it).
      if (lane < 32) xm[th * 64 + rg * 32 + lane] = mx;
      wg_barrier();
      mx = fmaxf(mx, xm[(th ^ 1) * 64 + rg * 32 + n32]);
      m_ref = mx;
    }
    m_hi = fmaxf(m_hi, mx);
    if (mx > m_ref + kRefSlack) ovf = true;
    const float mu = (m_ref == -__builtin_inff()) ? 0.f : m_ref;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = exp2f(p[r] - mu);
      l_part += p[r];
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const u32x4 pk = {pack_bf16x2(p[8 * hb + 0], p[8 * hb + 1]), pack_bf16x2(p[8 * hb + 2], p[8 * hb + 3]),
                        pack_bf16x2(p[8 * hb + 4], p[8 * hb + 5]), pack_bf16x2(p[8 * hb + 6], p[8 * hb + 7])};
      *(MLA_LDS u32x4*)(pl + ((rg * 4 + 2 * th + hb) * 64 + lane) * 16) = pk;
    }
    wg_barrier();  // ---- barrier 1: P visible

    // ---- values: O^T[columns 128w..][64 rows] += C^T[.., 64 tokens] P^T
    const int nkb = second_valid ? 4 : 2;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb >= nkb) break;
      const bf16x8 b0 = *(const MLA_LDS bf16x8*)(pl + ((0 * 4 + kb) * 64 + lane) * 16);
      const bf16x8 b1 = *(const MLA_LDS bf16x8*)(pl + ((1 * 4 + kb) * 64 + lane) * 16);
      bf16x8 an[4];
      if (kb + 1 < nkb) ldV(kb + 1, an);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        oacc[mt][0] = mfma32x32x16(av[mt], b0, oacc[mt][0]);
        oacc[mt][1] = mfma32x32x16(av[mt], b1, oacc[mt][1]);
      }
      sched_fence();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) av[mt] = an[mt];
    }
    // ---- barrier 2: P may be overwritten, step st's tiles are free, step st+1 resident
    wait_vmcnt<0>();
    wg_barrier();
  };

  for (bool first = true;; first = false) {  // one pass; repeated only after an overflow
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) oacc[i][j] = f32x16{};
    l_part = 0.f;
    ovf = false;
    if (!first) issue_step(0, page_block(0));
    wait_vmcnt<0>();
    wg_barrier();

    int blk_next = page_block(1);
    for (int st = 0; st < nsteps; st += 2) {
      run_step(st, blk_next, first && st == 0, std::integral_constant<int, 0>{});
      if (st + 1 < nsteps) run_step(st + 1, blk_next, false, std::integral_constant<int, 1>{});
    }
    // ---- did any row overflow its reference?  (its pair partner may not know)
    if (lane < 32) xm[th * 64 + rg * 32 + lane] = m_hi;
    // the vote runs in every lane (a ballot taken inside `if (lane == 0)`
    // would see lane 0's row alone)
    const bool wave_ovf = __builtin_amdgcn_ballot_w64(ovf) != 0;
    if (lane == 0) xf[wave] = wave_ovf;
    wg_barrier();
    const bool again = xf[0] | xf[1] | xf[2] | xf[3];
    if (!again) break;
    m_ref = fmaxf(m_hi, xm[(th ^ 1) * 64 + rg * 32 + n32]);  // the row's chunk maximum
    m_hi = -__builtin_inff();
    wg_barrier();
  }

  // ---- epilogue: complete row sums (two lane halves x two token halves)
  const float l_half = l_part + __shfl_xor(l_part, 32, 64);
  if (lane < 32) xm[th * 64 + rg * 32 + lane] = l_half;
  wg_barrier();
  if (lane < 32 && th == 0) {
    const float lt = l_half + xm[64 + rg * 32 + lane];
    xl[rg * 32 + lane] = lt;
    if (qvalid) a.lse[slot * rows + qrow] = lt > 0.f ? (m_ref + log2f(lt)) * kLn2 : -__builtin_inff();
  }
  wg_barrier();
  float* obase = a.o + slot * (int64_t)rows * 512;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int row = row_base + nt * 32 + n32;
    const float lt = xl[nt * 32 + n32];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* orow = obase + (int64_t)row * 512 + wave * 128;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = {oacc[mt][nt][4 * j] * inv, oacc[mt][nt][4 * j + 1] * inv,
                         oacc[mt][nt][4 * j + 2] * inv, oacc[mt][nt][4 * j + 3] * inv};
        if (row < rows) *(f32x4*)(orow + mt * 32 + j * 8 + 4 * g) = v;
      }
      sched_fence();
    }
  }
}

// ---------------------------------------------------------------------------
// Plain fp32 path: one workgroup per (sequence, chunk, query row).
// ---------------------------------------------------------------------------
template <int kFmt>  // 0 = f32 cache, 1 = bf16 cache, 2 = E4M3 + scale, bf16 k^R
__global__ void __launch_bounds__(256) decode_scalar(const DecodeArgs a) {
  __shared__ float q_s[576];
  __shared__ float sc_s[256];
  __shared__ float red[8];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row = blockIdx.x % a.rows;
  const int unit = blockIdx.x / a.rows;
  const int b = unit / a.num_splits, split = unit % a.num_splits;
  const int len = a.seq_lens[b];
  const int npages = (len + 63) >> 6;
  const int pps = (npages + a.num_splits - 1) / a.num_splits;
  const int p0 = split * pps, p1 = min(p0 + pps, npages);
  const int qi = row / a.heads;
  const int nvis = len - (a.sq - 1 - qi);
  const int tok0 = p0 * 64;
  const int tok1 = min(min(p1 * 64, len), max(nvis, 0));
  const int64_t qoff = (int64_t)b * a.rows + row;
  for (int i = tid; i < 576; i += 256) {
    if (kFmt == 0)
      q_s[i] = i < 512 ? ((const float*)a.q_lat)[qoff * 512 + i] : ((const float*)a.q_rope)[qoff * 64 + i - 512];
    else
      q_s[i] = i < 512 ? bf16_bits_to_f32(a.q_lat[qoff * 512 + i]) : bf16_bits_to_f32(a.q_rope[qoff * 64 + i - 512]);
  }
  __syncthreads();
  auto elem = [&](int tok, int c) -> float {
    const int blk = a.block_table[(int64_t)b * a.max_blocks + (tok >> 6)];
    const int r = tok & 63;
    if (c < 512) {
      const uint8_t* p = a.latent + blk * a.lat_bs + r * a.lat_rs;
      if (kFmt == 0) return ((const float*)p)[c];
      if (kFmt == 1) return bf16_bits_to_f32(((const uint16_t*)p)[c]);
      const uint32_t code = p[c];
      const float sc = *(const float*)(a.kv_scale_bytes + blk * a.scale_bs + r * 4);
      const uint32_t bits = ((code & 0x80u) << 24) | ((code & 0x7Fu) << 20);
      return __builtin_bit_cast(float, bits) * 0x1p120f * sc;  // E4M3 -> f32, exact
    }
    const uint8_t* p = a.rope + blk * a.rope_bs + r * a.rope_rs;
    if (kFmt == 0) return ((const float*)p)[c - 512];
    return bf16_bits_to_f32(((const uint16_t*)p)[c - 512]);
  };
  float m = -__builtin_inff(), l = 0.f;
  float o0 = 0.f, o1 = 0.f;  // columns tid, tid + 256
  for (int c0 = tok0; c0 < tok1; c0 += 256) {
    const int n = min(256, tok1 - c0);
    // scores: one wave per token, lanes split the 576-wide dot product
    for (int j = wave; j < n; j += 4) {
      float part = 0.f;
      for (int c = lane; c < 576; c += 64) part += q_s[c] * elem(c0 + j, c);
      part = wave_sum(part);
      if (lane == 0) sc_s[j] = part * a.softmax_scale;
    }
    __syncthreads();
    float cm = -__builtin_inff();
    for (int j = 0; j < n; ++j) cm = fmaxf(cm, sc_s[j]);
    const float mn = fmaxf(m, cm);
    const float alpha = expf(m - mn);
    l *= alpha; o0 *= alpha; o1 *= alpha;
    for (int j = 0; j < n; ++j) {
      const float pj = expf(sc_s[j] - mn);
      l += pj;
      o0 += pj * elem(c0 + j, tid);
      o1 += pj * elem(c0 + j, tid + 256);
    }
    m = mn;
    __syncthreads();
  }
  (void)red;
  const int64_t slot = (int64_t)b * a.num_splits + split;
  float* orow = a.o + (slot * a.rows + row) * 512;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  orow[tid] = o0 * inv;
  orow[tid + 256] = o1 * inv;
  if (tid == 0) a.lse[slot * a.rows + row] = l > 0.f ? m + logf(l) : -__builtin_inff();
}

template __global__ void decode_scalar<0>(const DecodeArgs);
template __global__ void decode_scalar<1>(const DecodeArgs);
template __global__ void decode_scalar<2>(const DecodeArgs);

}  // namespace mla
