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
// A KV chunk of a sequence (page-aligned split) yields its own normalised
// o_lat and lse, merged by split_combine.
//
// Three kernels:
//  * decode_mfma_bf16 (bf16 cache): eight waves per (sequence, chunk, block
//    of 64 query rows), 32-token tiles streamed HBM -> LDS by DMA, both
//    contractions on the matrix cores, fixed per-row softmax reference.
//  * decode_mfma_fp8 (E4M3 cache + fp32 token scales): the same pipeline with
//    register-staged tiles converted to bf16 and the scales applied in fp32.
//  * decode_f32 (fp32 cache): fp32 VALU, one workgroup per (chunk, query row)
//    over 16-token tiles copied to LDS by DMA, three tiles in flight.
#include <type_traits>

#include "mla_copy.h"
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

namespace {

constexpr int kTileTok = 32;                    // tokens per LDS tile
constexpr int kLatBytes = kTileTok * 64 * 16;   // latent part: 32 rows x 64 chunks of 16 B
constexpr int kRopeBytes = kTileTok * 8 * 16;   // RoPE part:   32 rows x 8 chunks
constexpr int kTileBytes = kLatBytes + kRopeBytes;  // 36,864
constexpr float kRefSlack = 64.0f;              // log2 headroom above a row's reference max

// LDS tile layout (64 banks x 4 B): chunk q of latent row r sits at slot
// r*64 + (q ^ s16(r)); chunk q of RoPE row r at r*8 + (q ^ s8(r)) after the
// latent part.  s16 makes 16 consecutive rows at one chunk hit 16 distinct
// bank groups (score operand reads) and 4 consecutive rows x 4 chunks hit 16
// distinct groups (transposing value-operand reads); s8 does the former for
// the 128-byte RoPE rows.
__device__ __forceinline__ int s16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int s8(int r) { return (r >> 1) & 7; }

struct Work {
  int b, split, rb;
  int len, tok0, tok1, ntiles;
};

// XCD-aware placement: workgroups are dispatched round-robin over the 8 XCDs
// (id % 8).  The (sequence, chunk, row block) items, unit-major, are cut into
// 8 contiguous ranges, one per XCD, so each XCD runs the row blocks of a
// unit back to back: a tile is fetched from HBM once and read from that
// XCD's L2 by the other row blocks, and the chunks of one sequence, which
// share its query block, mostly run on one XCD too.  With fewer units than
// XCDs a unit's row blocks spread over several XCDs (each fetches the tiles)
// rather than leaving XCDs idle.
__device__ __forceinline__ bool decode_work(const DecodeArgs& a, Work& w) {
  const int id = blockIdx.x;
  const int xcd = id & 7, k = id >> 3;
  const int total = a.units * a.row_blocks;
  const int per = (total + 7) >> 3;  // items per XCD
  const int item = xcd * per + k;
  if (k >= per || item >= total) return false;
  const int unit = item / a.row_blocks;
  w.rb = item - unit * a.row_blocks;
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

// A chunk that holds none of its sequence's tokens (the trailing chunks of a
// sequence shorter than num_splits pages): its rows get o = 0 and lse = -inf,
// as the pipeline would give them, without staging queries or tiles.
__device__ __forceinline__ void empty_chunk(const DecodeArgs& a, const Work& w, int nrows) {
  const int rows = a.rows, row_base = w.rb * nrows;
  const int64_t slot = (int64_t)w.b * a.num_splits + w.split;
  for (int i = threadIdx.x; i < nrows * 128; i += blockDim.x) {
    const int r = i >> 7, c4 = i & 127;
    if (row_base + r >= rows) continue;
    const int64_t e = (slot * rows + row_base + r) * 512 + 4 * c4;
    if (a.o_f16)
      *(f16x4*)((_Float16*)a.o + e) = f16x4{0, 0, 0, 0};
    else
      *(f32x4*)((float*)a.o + e) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if ((int)threadIdx.x < nrows && row_base + (int)threadIdx.x < rows)
    a.lse[slot * rows + row_base + threadIdx.x] = -__builtin_inff();
}

}  // namespace

// bf16 cache.  Workgroup = 8 waves = one (sequence, KV chunk, block of
// kRows = 64 or 32 query rows); the chunk is walked in 32-token tiles (half
// a cache page).  The description below is for 64 rows; with 32 rows each
// score wave holds one 16-row block and each value wave one 32-row block
// (half the products per tile, for launches with few (sequence, chunk)
// units: four row blocks per unit fill twice as many compute units).
// Two wave roles, one of each per SIMD:
//   score waves 0..3: wave w computes S^T[16 tokens (half w&1)][32 rows
//            (half w>>1)] with v_mfma_f32_16x16x32_bf16 over K = 576 (A = tile
//            rows from LDS, shared by the two 16-row blocks; B = the wave's
//            queries, held in registers), then the softmax of those scores
//            (log2 domain, fixed per-row reference) and writes P to LDS.
//   value waves 4..7: wave 4+v accumulates O^T[latent columns 128v..+127]
//            [64 rows] += C^T P^T with v_mfma_f32_32x32x16_bf16, C^T read by
//            the transposing LDS load, P^T from a double-buffered LDS array.
// Holding 32 query rows per score wave halves the LDS reads of the token
// operand against 16-row waves, and the two roles share each SIMD's matrix
// core: one wave's softmax arithmetic and LDS waits overlap the other's
// products.  Per tile s, with a ring of four LDS tile buffers, the score
// waves work on tile s, the value waves on tile s-1 (and refill their slices
// of its buffer with tile s+3 once read), tiles s+1 .. s+3 are in flight;
// one barrier per tile.
template <int kRows>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_mfma_bf16(const DecodeArgs a) {
  static_assert(kRows == 64 || kRows == 32, "64 or 32 query rows per workgroup");
  constexpr int kRB = kRows / 32;                 // 16-row blocks per score wave, 32-row blocks per value wave
  constexpr int kBuf = 4;                         // tile ring
  constexpr int kPBytes = kRows * 32 * 2;         // P of one tile: kRows rows x 32 tokens bf16
  constexpr int kQStride = 73;                    // staged query row: 72 chunks + 1 pad
  constexpr int kQBase = 2 * kTileBytes;          // queries are staged over tiles 2, 3 (+ P)
  constexpr int kXOff = kBuf * kTileBytes + 2 * kPBytes;
  static_assert(kQBase + (kRows * kQStride + 63) / 64 * 1024 <= kXOff, "query staging must fit before the exchange area");
  constexpr int kORow = 512 * 4 + 16;             // staged output row (epilogue)
  static_assert(64 * kORow <= kBuf * kTileBytes, "the output staging must fit in the tile ring");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kXOff + 1280];
  MLA_LDS uint8_t* const tiles = (MLA_LDS uint8_t*)&smem[0];
  MLA_LDS uint8_t* const pbuf = tiles + kBuf * kTileBytes;
  MLA_LDS float* const xm = (MLA_LDS float*)(tiles + kXOff);  // [2 token halves][64 rows]
  MLA_LDS float* const xl = xm + 128;                         // [2][64] row sums
  MLA_LDS int* const xf = (MLA_LDS int*)(xl + 128);           // [4] overflow flags of the score waves

  // the roles below assume exactly eight waves
  if (blockDim.x != 512) return;
  Work wk;
  if (!decode_work(a, wk)) return;
  if (wk.ntiles == 0) {
    empty_chunk(a, wk, kRows);
    return;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, 0..7
  const int lane = tid & 63;
  const int g = lane >> 5;        // k-half of a 32x32 operand
  const int n32 = lane & 31;
  const int q4 = lane >> 4;       // k-quarter of a 16x16 operand / token quad of its result
  const int i16 = lane & 15;
  const int rows = a.rows;
  const int row_base = wk.rb * kRows;
  const int64_t slot = (int64_t)wk.b * a.num_splits + wk.split;
  const int ntiles = wk.ntiles;
  const uint32_t tiles_lds = lds_addr(tiles);

  // ---- HBM -> LDS copies.  Tile layout here: the latent part is four 8 KB
  // slices, slice v holding latent columns 128 v .. 128 v + 127 of the 32 rows
  // (row r at 256 r in the slice, its 16-byte chunk q at slot q ^ s16(r)); the
  // RoPE part follows (row r at 128 r, chunk q at slot q ^ s8(r)).  Value wave
  // 4 + v copies slice v of every tile (eight copies of four 256-byte row
  // slices) and is the only wave that reads it in the value product; score
  // wave w copies RoPE rows 8w .. 8w+7 (one copy).  So in the iteration that
  // multiplies tile s-1, value wave 4 + v refills its slice of that buffer
  // with tile s+3 as soon as its own reads are done, and the score waves
  // refill the RoPE rows (free since the previous iteration): three tiles are
  // in flight while two are in use, in four buffers, with no extra barrier.
  // Copies take every row of the tile's half page as it is; rows past the
  // sequence's length (inside its last page, so still in the pool) are
  // zeroed by each wave in its own part once its copies have landed.  Tiles
  // past the chunk copy block 0 into a buffer nobody reads.
  constexpr int kSliceBytes = 32 * 256;
  const int64_t bt_row = (int64_t)wk.b * a.max_blocks;
  auto tile_block = [&](int t) __attribute__((always_inline)) -> int {
    return t < ntiles ? load_uniform(a.block_table, bt_row + ((wk.tok0 + t * kTileTok) >> 6)) : 0;
  };
  const bool valw = wave >= 4;
  const int v = wave & 3;      // slice of a value wave; RoPE rows 8 v .. of a score wave
  const int lrq = lane >> 4;   // row of a latent-copy lane among its copy's four
  // s16(4k + lrq) = (lrq << 2) | (k & 3): the lane part and the copy part
  const uint32_t lat_lc = (uint32_t)(((lane & 15) ^ (lrq << 2)) << 4);
  const uint32_t lat_lrow = (uint32_t)(lrq * a.lat_rs);
  const int rope_r = 8 * v + (lane >> 3);
  const uint32_t rope_lane = (uint32_t)((lane >> 3) * a.rope_rs) + ((((lane & 7) ^ s8(rope_r))) << 4);
  const int64_t lat_half = 32 * a.lat_rs, rope_half = 32 * a.rope_rs;
  struct TileSrc {
    const uint8_t* lat;   // latent row 0 of the tile
    const uint8_t* rope;  // RoPE row 8 v of the tile
    uint32_t lds;         // the tile's buffer
  };
  auto tile_src = [&](int t, int blk) __attribute__((always_inline)) -> TileSrc {
    const bool upper = (t & 1) != 0;  // chunks start on a page: odd tiles are upper half pages
    return TileSrc{a.latent + blk * a.lat_bs + (upper ? lat_half : 0),
                   a.rope + blk * a.rope_bs + (upper ? rope_half : 0) + (int64_t)(8 * v) * a.rope_rs,
                   tiles_lds + (uint32_t)((t % kBuf) * kTileBytes)};
  };
  // value wave: copy k = rows 4k .. 4k+3 of slice v
  auto lat_copy = [&](const TileSrc& src, int k) __attribute__((always_inline)) {
    dma16xy(src.lat, lat_lc, (uint32_t)(k & 3) << 4, lat_lrow, (uint32_t)(4 * k * a.lat_rs + 256 * v),
            src.lds + v * kSliceBytes + 1024 * k);
  };
  auto issue_tile = [&](int t, int blk) __attribute__((always_inline)) {  // this wave's copies of tile t
    const TileSrc src = tile_src(t, blk);
    if (valw) {
#pragma unroll
      for (int k = 0; k < 8; ++k) lat_copy(src, k);
    } else {
      dma16s(src.rope, rope_lane, src.lds + kLatBytes + 1024 * v);
    }
  };
  // A sequence's last tile may end inside it: once this wave's copies of
  // tile t have landed, zero its part of the rows at or past the length,
  // which the value product multiplies by P = 0 (an uninitialised row could
  // hold NaN).  Uniform: at most once per pass.
  auto fix_tail = [&](int t) __attribute__((always_inline)) {
    const int left = wk.len - (wk.tok0 + t * kTileTok);
    if (t < ntiles && left < kTileTok) {
      MLA_LDS uint8_t* tb = tiles + (t % kBuf) * kTileBytes;
      if (valw) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (4 * k + lrq >= left)
            *(MLA_LDS u32x4*)(tb + v * kSliceBytes + (4 * k + lrq) * 256 + (lane & 15) * 16) = u32x4{0, 0, 0, 0};
      } else if (rope_r >= left) {
        *(MLA_LDS u32x4*)(tb + kLatBytes + 1024 * v + lane * 16) = u32x4{0, 0, 0, 0};
      }
    }
  };

  // ---- prologue: stage the block's kRows query rows (q_lat | q_rope, 72
  // chunks of 16 bytes each, row stride 73 chunks) over tile buffers 2..3
  // with DMA (lanes past the last row copy a clamped row into the staging
  // area's tail, which nothing reads),
  // start tiles 0 and 1; the score waves then pull their queries into
  // registers.
  {
    const int64_t qbase = (int64_t)wk.b * rows;
    for (int i = wave; i < (kRows * kQStride + 63) / 64; i += 8) {
      const int sl = i * 64 + lane;
      const int r = sl / kQStride, c = sl - r * kQStride;
      const int qr = min(row_base + r, rows - 1);
      const uint8_t* src = c < 64 ? (const uint8_t*)(a.q_lat + (qbase + qr) * 512 + c * 8)
                                  : (const uint8_t*)(a.q_rope + (qbase + qr) * 64 + (c < 72 ? c - 64 : 0) * 8);
      dma16(src, tiles_lds + kQBase + i * 1024);
    }
  }
  const int blk_a = tile_block(0), blk_b = tile_block(1);
  issue_tile(0, blk_a);
  issue_tile(1, blk_b);
  // the queries (tiles 0 and 1 may still be in flight: 8 copies each for a
  // value wave, 1 for a score wave)
  if (valw)
    wait_vmcnt<16>();
  else
    wait_vmcnt<2>();
  wg_barrier();

  // The two roles run separate loops with the same sequence of barriers:
  // per pass, the pass start, the reference exchange (first pass, non-empty
  // chunk), tile 0's end, one per later tile, the overflow vote and (before a
  // repeat) the new reference; after the last pass the row sums.  A row's
  // reference max is fixed at its first tile, so P and O never need
  // rescaling.  If a later score exceeds it by more than 2^kRefSlack the pass
  // is finished (its values are discarded) and repeated with the row's chunk
  // maximum as the reference: exact either way, never taken unless the
  // scores of one row span more than 44 nats, and the repeat cannot
  // overflow, so there are two passes at most.
  if (wave < 4) {
    // ================= score waves =================
    const int th = wave & 1;  // token half of a tile
    const int rh = wave >> 1;  // row half of the block
    // B operand of k-step ks for row block rb: row 32 rh + 16 rb + i16; latent
    // chunk ks + 16 q4 for ks < 16 (each lane quarter walks its own quarter of
    // the row: with the tile swizzle this order keeps the tile reads free of
    // bank conflicts, measured), RoPE chunk 4 (ks - 16) + q4 after
    bf16x8 qf[kRB][18];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int r = (kRows / 2) * rh + 16 * rb + i16;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const int c = ks < 16 ? ks + 16 * q4 : 64 + 4 * (ks - 16) + q4;
        qf[rb][ks] = *(const MLA_LDS bf16x8*)(tiles + kQBase + (r * kQStride + c) * 16);
      }
    }
    wg_barrier();  // every score wave holds its queries: tiles 2, 3 and P are free

    // score operand: tile row 16 th + i16; latent chunk ks + 16 q4 sits in
    // slice q4 at byte 256 row + ((ks ^ s16(row)) << 4) = c1_lat ^ (ks << 4);
    // RoPE chunk 4 (ks - 16) + q4 after the latent part
    const int tr = 16 * th + i16;
    const uint32_t c1_lat = q4 * kSliceBytes + tr * 256 + (s16(tr) << 4);
    uint32_t c1_rope[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) c1_rope[k] = kLatBytes + tr * 128 + (((4 * k + q4) ^ s8(tr)) << 4);
    // this lane's score rows (block-relative), their causal limits and P
    // slots: tokens 16 th + 4 q4 + 0..3 of row R sit in 16-byte chunk
    // 2 th + (q4 & 1) (bytes 8 (q4 >> 1)..) at slot 4 R + (chunk ^ (R/4 % 4))
    int prow[2], hi_tok[2];
    uint32_t pwrite[2];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      prow[rb] = (kRows / 2) * rh + 16 * rb + i16;
      const int qrow = row_base + prow[rb];
      hi_tok[rb] = qrow < rows ? min(wk.tok1, wk.len - (a.sq - 1 - qrow / a.heads)) : 0;
      pwrite[rb] = (4 * prow[rb] + ((2 * th + (q4 & 1)) ^ ((prow[rb] >> 2) & 3))) * 16 + 8 * (q4 >> 1);
    }

    float m_ref[2] = {-__builtin_inff(), -__builtin_inff()};
    float m_hi[2], l_part[2];
    bool ovf;

    // scores of tile s: 18 k-steps, two 16x16x32 products each (one per row
    // block, same token operand).  `hook(ks)` runs after k-step ks.
    f32x4 sacc[kRB];
    auto scores = [&](int s, auto hook) __attribute__((always_inline)) {
      const MLA_LDS uint8_t* tb = tiles + (s % kBuf) * kTileBytes;
      auto ldA = [&](int ks) __attribute__((always_inline)) -> bf16x8 {
        if (ks < 16) return *(const MLA_LDS bf16x8*)(tb + (c1_lat ^ (uint32_t)(ks << 4)));
        return *(const MLA_LDS bf16x8*)(tb + c1_rope[ks - 16]);
      };
      constexpr int kDepth = 4;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sacc[rb] = f32x4{};
      bf16x8 ar[kDepth];
#pragma unroll
      for (int ks = 0; ks < kDepth; ++ks) ar[ks] = ldA(ks);
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) sacc[rb] = mfma16x16x32(ar[ks % kDepth], qf[rb][ks], sacc[rb]);
        if (ks + kDepth < 18) ar[ks % kDepth] = ldA(ks + kDepth);
        hook(ks);
        sched_fence();
      }
    };

    // softmax of tile s: lane holds tokens 16 th + 4 q4 + r of rows prow[rb]
    float p[2][4], mx[2];
    auto soft_scale = [&](int s) __attribute__((always_inline)) {
      const int tt = wk.tok0 + s * kTileTok + 16 * th + 4 * q4;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = sacc[rb][r] * a.scale_log2;
          p[rb][r] = tt + r < hi_tok[rb] ? x : -__builtin_inff();
        }
        mx[rb] = fmaxf(fmaxf(p[rb][0], p[rb][1]), fmaxf(p[rb][2], p[rb][3]));
      }
    };
    // hardware exp2 (v_exp_f32): results below 2^-126 flush to zero, which
    // cannot matter next to the row's largest weight (>= 1 after the first tile)
    auto soft_finish = [&](int s) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        m_hi[rb] = fmaxf(m_hi[rb], mx[rb]);
        ovf |= mx[rb] > m_ref[rb] + kRefSlack;
        const float mu = m_ref[rb] == -__builtin_inff() ? 0.f : m_ref[rb];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[rb][r] = __builtin_amdgcn_exp2f(p[rb][r] - mu);
          l_part[rb] += p[rb][r];
        }
        const u32x2 pk = {pack_bf16x2(p[rb][0], p[rb][1]), pack_bf16x2(p[rb][2], p[rb][3])};
        *(MLA_LDS u32x2*)(pbuf + (s & 1) * kPBytes + pwrite[rb]) = pk;
      }
    };

    for (int pass = 0; pass < 2; ++pass) {
      const bool first = pass == 0;
      l_part[0] = l_part[1] = 0.f;  // entry 1 unused with one row block
      m_hi[0] = m_hi[1] = -__builtin_inff();
      ovf = false;
      if (!first) {
        issue_tile(0, blk_a);
        issue_tile(1, blk_b);
      }
      wait_vmcnt<1>();  // tile 0 (tile 1 may still be in flight)
      fix_tail(0);
      wg_barrier();

      int blk_next = tile_block(4);
      if (ntiles > 0) {
        issue_tile(2, tile_block(2));  // buffers 2, 3 are free (queries held, or the last pass over)
        issue_tile(3, tile_block(3));
        scores(0, [](int) {});
        soft_scale(0);
        if (first) {
          // each row's maximum over the whole first tile (both token halves);
          // a row left at -inf sees no token of this chunk
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) {
            float m = fmaxf(mx[rb], __shfl_xor(mx[rb], 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            if (q4 == 0) xm[th * 64 + prow[rb]] = m;
            mx[rb] = m;
          }
          wg_barrier();
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) m_ref[rb] = fmaxf(mx[rb], xm[(th ^ 1) * 64 + prow[rb]]);
        }
        soft_finish(0);
        wait_vmcnt<2>();  // tile 1 (tiles 2, 3 may still be in flight)
        fix_tail(1);
        wg_barrier();
      }

      // tiles 1 ..: the RoPE rows of tile s+3 go into the buffer of tile s-1,
      // whose RoPE rows were read in the previous iteration
      for (int s = 1; s < ntiles; ++s) {
        issue_tile(s + 3, blk_next);
        scores(s, [](int) {});
        soft_scale(s);
        soft_finish(s);
        blk_next = tile_block(s + 4);  // a scalar load: read here, its wait joins the barrier's
        wait_vmcnt<2>();  // tile s+1 (tiles s+2, s+3 may still be in flight)
        fix_tail(s + 1);
        wg_barrier();
      }
      wait_vmcnt<0>();  // copies issued for tiles past the chunk have landed

      // ---- did any row overflow its reference?  (its partner lanes may not know)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float m = fmaxf(m_hi[rb], __shfl_xor(m_hi[rb], 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        m_hi[rb] = m;
        if (q4 == 0) xm[th * 64 + prow[rb]] = m;
      }
      // the vote runs in every lane (a ballot taken inside `if (lane == 0)`
      // would see lane 0's rows alone)
      const bool wave_ovf = __builtin_amdgcn_ballot_w64(ovf) != 0;
      if (lane == 0) xf[wave] = wave_ovf;
      wg_barrier();
      const bool again = (xf[0] | xf[1] | xf[2] | xf[3]) != 0;
      if (!again || !first) break;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) m_ref[rb] = fmaxf(m_hi[rb], xm[(th ^ 1) * 64 + prow[rb]]);
      wg_barrier();
    }

    // ---- row sums (4 token quads x 2 token halves) for the value waves; lse
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float l = l_part[rb] + __shfl_xor(l_part[rb], 16, 64);
      l += __shfl_xor(l, 32, 64);
      if (q4 == 0) xl[th * 64 + prow[rb]] = l;
    }
    wg_barrier();
    if (th == 0 && q4 == 0) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const int qrow = row_base + prow[rb];
        const float lt = xl[prow[rb]] + xl[64 + prow[rb]];
        if (qrow < rows) a.lse[slot * rows + qrow] = lt > 0.f ? (m_ref[rb] + log2f(lt)) * kLn2 : -__builtin_inff();
      }
    }
  } else {
    // ================= value waves =================
    wg_barrier();  // the score waves hold their queries
    // C^T operand (transposing reads, slice v): token row 16 ks + 8 j2 + 4 g +
    // i16/4 of the tile, latent columns 128 v + 32 mt + 16 (lane/16 % 2) + 4 (i16 % 4)
    const int vy = 2 * ((lane >> 4) & 1) + ((i16 >> 1) & 1);
    uint32_t voff[2][4];
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const int sw = (((i16 >> 2) & 3) << 2) | ((2 * j2 + g) & 3);  // s16 of the row
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        voff[j2][mt] = v * kSliceBytes + (8 * j2 + 4 * g + (i16 >> 2)) * 256 + (((4 * mt + vy) ^ sw) << 4) + (i16 & 1) * 8;
    }
    // P^T operand: row R = 32 nt + n32, 16-byte chunk 2 ks + g holding tokens
    // 16 ks + 4 g + 0..3 and 16 ks + 8 + 4 g + 0..3, at slot 4 R + (chunk ^
    // (R/4 % 4)) of the tile's P buffer (rows 32.. are 2048 bytes on)
    uint32_t pread[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pread[ks] = (4 * n32 + ((2 * ks + g) ^ ((n32 >> 2) & 3))) * 16;

    f32x16 oacc[4][kRB];
    // C^T operand of tile t, 16-token half ks, 32-column block mt
    auto av_load = [&](int t, int ks, int mt) __attribute__((always_inline)) -> bf16x8 {
      const MLA_LDS uint8_t* vt = tiles + (t % kBuf) * kTileBytes + ks * 16 * 256;
      const u32x2 lo = lds_read_tr16_b64(vt + voff[0][mt]);
      const u32x2 hi = lds_read_tr16_b64(vt + voff[1][mt]);
      return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    // the C^T operands of the next tile are read ahead, at the end of the
    // previous product (its tile has landed by then), so that a product
    // waits only for its P reads
    bf16x8 av[2][4];
    auto load_av = [&](int t) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) av[ks][mt] = av_load(t, ks, mt);
    };
    // value product of tile t (its C^T operands already in av): two 16-token
    // halves, eight 32x32x16 products each.  With `refill`, once every
    // operand read of slice v has completed, the slice is refilled with tile
    // nsrc: its eight copies go between the products, whose execution covers
    // their issue.  Then the operands of tile `next` (if >= 0) are read.
    auto values = [&](int t, bool refill, const TileSrc& nsrc, int next) __attribute__((always_inline)) {
      const MLA_LDS uint8_t* pb = pbuf + (t & 1) * kPBytes;
      bf16x8 bp[2][kRB];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nt = 0; nt < kRB; ++nt) bp[ks][nt] = *(const MLA_LDS bf16x8*)(pb + pread[ks] + 2048 * nt);
      if (refill) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads of slice v are done
#pragma unroll
      for (int i = 0; i < 8 * kRB; ++i) {
        const int ks = i / (4 * kRB), mt = (i / kRB) & 3, nt = i % kRB;
        oacc[mt][nt] = mfma32x32x16(av[ks][mt], bp[ks][nt], oacc[mt][nt]);
        if (refill && nt == 0) lat_copy(nsrc, i / kRB);
        sched_fence();
      }
      if (next >= 0) load_av(next);
    };

    for (int pass = 0; pass < 2; ++pass) {
      const bool first = pass == 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < kRB; ++nt) oacc[mt][nt] = f32x16{};
      if (!first) {
        issue_tile(0, blk_a);
        issue_tile(1, blk_b);
      }
      wait_vmcnt<8>();  // tile 0 (tile 1 may still be in flight)
      fix_tail(0);
      wg_barrier();

      int blk_next = tile_block(4);
      if (ntiles > 0) {
        load_av(0);
        issue_tile(2, tile_block(2));
        issue_tile(3, tile_block(3));
        if (first) wg_barrier();  // the score waves' reference exchange
        wait_vmcnt<16>();  // tile 1 (tiles 2, 3 may still be in flight)
        fix_tail(1);
        wg_barrier();
      }
      for (int s = 1; s < ntiles; ++s) {
        const TileSrc nsrc = tile_src(s + 3, blk_next);
        values(s - 1, true, nsrc, s);  // slice v of tile s-1's buffer takes tile s+3
        blk_next = tile_block(s + 4);
        wait_vmcnt<16>();  // tile s+1 (tiles s+2, s+3 may still be in flight)
        fix_tail(s + 1);
        wg_barrier();
      }
      wait_vmcnt<0>();
      if (ntiles > 0) values(ntiles - 1, false, tile_src(0, 0), -1);
      wg_barrier();  // overflow vote
      const bool again = (xf[0] | xf[1] | xf[2] | xf[3]) != 0;
      if (!again || !first) break;
      wg_barrier();  // new reference
    }

    // ---- epilogue: normalise by the row sums and stage this chunk's o_lat
    // in the tile ring (free now: every copy has landed, no tile is read),
    // rows of 512 fp32 plus 16 bytes of pad
    wg_barrier();  // row sums
#pragma unroll
    for (int nt = 0; nt < kRB; ++nt) {
      const int r = nt * 32 + n32;
      const float lt = xl[r] + xl[64 + r];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      MLA_LDS uint8_t* orow = tiles + r * kORow + v * 512;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 o = {oacc[mt][nt][4 * j] * inv, oacc[mt][nt][4 * j + 1] * inv,
                           oacc[mt][nt][4 * j + 2] * inv, oacc[mt][nt][4 * j + 3] * inv};
          *(MLA_LDS f32x4*)(orow + (mt * 32 + j * 8 + 4 * g) * 4) = o;
        }
      }
    }
  }
  // all eight waves write the staged rows: a wave's store covers a row's 2
  // KB (fp32) or 1 KB (fp16 partials) (the accumulator layout would write 32
  // rows x 32 bytes per store)
  wg_barrier();
  {
    const int c16 = tid & 127;
    const int64_t obase = slot * (int64_t)rows * 512;
#pragma unroll
    for (int k = 0; k < kRows / 4; ++k) {
      const int r = (tid >> 7) + 4 * k;
      const f32x4 o = *(const MLA_LDS f32x4*)(tiles + r * kORow + c16 * 16);
      const int64_t e = obase + (int64_t)(row_base + r) * 512 + 4 * c16;  // first element of the piece
      if (row_base + r < rows) {
        if (a.o_f16)
          *(f16x4*)((_Float16*)a.o + e) = to_f16x4(o);
        else
          *(f32x4*)((float*)a.o + e) = o;
      }
    }
  }
}

// E4M3 cache (fp8 codes + fp32 per-token scale, bf16 k^R).  The workgroup,
// wave roles, tile ring and slice-major tile layout of decode_mfma_bf16, with
// three differences.  Value wave 4+v stages slice v of each tile through
// registers: it loads the tile's codes of its 128 latent columns, converts
// them exactly to bf16 (a 3-bit mantissa and the E4M3 exponent range fit
// bf16; rows past the sequence's length become zeros there) and writes them
// into its slice once its own reads of the buffer's previous tile are done.
// The score waves copy the RoPE rows by DMA and score wave 0 the tile's 32
// token scales.  The per-token scale is applied in fp32 to the latent part of
// each score (kept in its own accumulator) and folded into P for the value
// product, so no dequantized value is rounded.
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_mfma_fp8(const DecodeArgs a) {
  constexpr int kBuf = 4;                         // tile ring
  constexpr int kPBytes = 64 * 32 * 2;            // P of one tile: 64 rows x 32 tokens bf16
  constexpr int kQStride = 73;                    // staged query row: 72 chunks + 1 pad
  constexpr int kQBase = 2 * kTileBytes;          // queries are staged over tiles 2, 3 (+ P)
  constexpr int kXOff = kBuf * kTileBytes + 2 * kPBytes;
  static_assert(kQBase + 64 * kQStride * 16 <= kXOff, "query staging must fit before the exchange area");
  constexpr int kORow = 512 * 4 + 16;             // staged output row (epilogue)
  static_assert(64 * kORow <= kBuf * kTileBytes, "the output staging must fit in the tile ring");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kXOff + 1280 + kBuf * 128];
  MLA_LDS uint8_t* const tiles = (MLA_LDS uint8_t*)&smem[0];
  MLA_LDS uint8_t* const pbuf = tiles + kBuf * kTileBytes;
  MLA_LDS float* const xm = (MLA_LDS float*)(tiles + kXOff);  // [2 token halves][64 rows]
  MLA_LDS float* const xl = xm + 128;                         // [2][64] row sums
  MLA_LDS int* const xf = (MLA_LDS int*)(xl + 128);           // [4] overflow flags of the score waves
  MLA_LDS float* const scl = (MLA_LDS float*)(tiles + kXOff + 1280);  // [kBuf][32] token scales

  // the roles below assume exactly eight waves
  if (blockDim.x != 512) return;
  Work wk;
  if (!decode_work(a, wk)) return;
  if (wk.ntiles == 0) {
    empty_chunk(a, wk, kDecodeRowsPerWg);
    return;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, 0..7
  const int lane = tid & 63;
  const int g = lane >> 5;        // k-half of a 32x32 operand
  const int n32 = lane & 31;
  const int q4 = lane >> 4;       // k-quarter of a 16x16 operand / token quad of its result
  const int i16 = lane & 15;
  const int rows = a.rows;
  const int row_base = wk.rb * kDecodeRowsPerWg;
  const int64_t slot = (int64_t)wk.b * a.num_splits + wk.split;
  const int ntiles = wk.ntiles;
  const uint32_t tiles_lds = lds_addr(tiles);

  // ---- copies.  Tile layout as in decode_mfma_bf16 (four 8 KB latent
  // slices, then the RoPE rows); the tile's token scales go to scl.
  // Value wave 4+v stages slice v (four 16-byte loads per lane, ordinary
  // loads tracked by the compiler); rows at or past the sequence's length,
  // and tiles past the chunk (whose loads read block 0), are stored as
  // zeros.  Score wave w copies RoPE rows 8w .. 8w+7 (one DMA copy) and score
  // wave 0 also the 128 bytes of token scales (one copy on 8 lanes); RoPE
  // rows past the length are zeroed by fix_tail once landed.
  constexpr int kSliceBytes = 32 * 256;
  const int64_t bt_row = (int64_t)wk.b * a.max_blocks;
  auto tile_block = [&](int t) __attribute__((always_inline)) -> int {
    return t < ntiles ? load_uniform(a.block_table, bt_row + ((wk.tok0 + t * kTileTok) >> 6)) : 0;
  };
  const bool valw = wave >= 4;
  const int v = wave & 3;      // slice of a value wave; RoPE rows 8 v .. of a score wave
  const int rope_r = 8 * v + (lane >> 3);
  const uint32_t rope_lane = (uint32_t)((lane >> 3) * a.rope_rs) + ((((lane & 7) ^ s8(rope_r))) << 4);
  const int64_t rope_half = 32 * a.rope_rs;
  const uint32_t scl_lds = tiles_lds + (kXOff + 1280);
  // score waves: this wave's DMA copies of tile t (1, or 2 for wave 0)
  auto issue_tile = [&](int t, int blk) __attribute__((always_inline)) {
    const bool upper = (t & 1) != 0;  // chunks start on a page: odd tiles are upper half pages
    const uint32_t buf = tiles_lds + (uint32_t)((t % kBuf) * kTileBytes);
    dma16s(a.rope + blk * a.rope_bs + (upper ? rope_half : 0) + (int64_t)(8 * v) * a.rope_rs, rope_lane,
           buf + kLatBytes + 1024 * v);
    if (wave == 0 && lane < 8)
      dma16(a.kv_scale_bytes + blk * a.scale_bs + (upper ? 128 : 0) + 16 * lane, scl_lds + (t % kBuf) * 128);
  };
  // score waves: wait until at most n tiles' copies are in flight
  auto wait_tiles2 = [&]() __attribute__((always_inline)) {
    if (wave == 0)
      wait_vmcnt<4>();
    else
      wait_vmcnt<2>();
  };
  auto wait_tiles1 = [&]() __attribute__((always_inline)) {
    if (wave == 0)
      wait_vmcnt<2>();
    else
      wait_vmcnt<1>();
  };
  // value waves: slice v of tile t staged in registers
  // Piece j of a lane is row 8 j + srow, codes 16 sc .. +15 of the slice
  // (local chunks 2 sc, 2 sc + 1).  The eight lanes of a row read its 128
  // contiguous codes; the rows of lanes 0-7 and 8-15 (and so on) differ in
  // bit 2, which flips the parity of the row's swizzle, so the 16 lanes of a
  // store hit 16 distinct bank groups.
  const int srow = ((lane >> 3) & 1) * 4 + (lane >> 4), sc = lane & 7;
  struct Staged {
    u32x4 c[4];
  };
  // wave-uniform base of tile t's rows, plus a per-lane 32-bit offset (a
  // block's 64 rows span well under 4 GB)
  uint32_t soff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) soff[j] = (uint32_t)((8 * j + srow) * a.lat_rs) + 128 * v + 16 * sc;
  auto stage_src = [&](int t, int blk) __attribute__((always_inline)) -> const uint8_t* {
    const bool upper = (t & 1) != 0;
    return a.latent + blk * a.lat_bs + (upper ? 32 * a.lat_rs : 0);
  };
  auto stage_load = [&](int t, int blk, Staged& st) __attribute__((always_inline)) {
    const uint8_t* lp = stage_src(t, blk);
#pragma unroll
    for (int j = 0; j < 4; ++j) st.c[j] = *(const u32x4*)(lp + soff[j]);
  };
  // piece j -> two 16-byte chunks (8 bf16 each) of row 8 j + srow, at slots
  // (2 sc + e) ^ s16(row) of slice v; a row at or past the length (or a tile
  // past the chunk) is stored as zeros.  The test sits here, not after the
  // loads, so that nothing waits for them before this point.
  auto stage_piece = [&](int t, const Staged& st, int j, int e) __attribute__((always_inline)) {
    const int row = 8 * j + srow;
    MLA_LDS uint8_t* sb = tiles + (t % kBuf) * kTileBytes + v * kSliceBytes + row * 256;
    const bool ok = t < ntiles && wk.tok0 + t * kTileTok + row < wk.len;
    const uint32_t w0 = ok ? st.c[j][2 * e] : 0u, w1 = ok ? st.c[j][2 * e + 1] : 0u;
    const u32x4 bf = {e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0), e4m3x2_to_bf16x2<false>(w1),
                      e4m3x2_to_bf16x2<true>(w1)};
    *(MLA_LDS u32x4*)(sb + (((2 * sc + e) ^ s16(row)) << 4)) = bf;
  };
  auto stage_store = [&](int t, const Staged& st) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      stage_piece(t, st, j, 0);
      stage_piece(t, st, j, 1);
    }
  };
  // A sequence's last tile may end inside it: once this score wave's RoPE
  // copy of tile t has landed, zero the RoPE rows at or past the length
  // (uninitialised pool rows could hold NaN; the latent part was staged as
  // zeros).  Uniform: at most once per pass.
  auto fix_tail = [&](int t) __attribute__((always_inline)) {
    const int left = wk.len - (wk.tok0 + t * kTileTok);
    if (t < ntiles && left < kTileTok && rope_r >= left)
      *(MLA_LDS u32x4*)(tiles + (t % kBuf) * kTileBytes + kLatBytes + 1024 * v + lane * 16) = u32x4{0, 0, 0, 0};
  };

  // ---- prologue: stage the block's 64 query rows (q_lat | q_rope, 72 chunks
  // of 16 bytes each, row stride 73 chunks) over tile buffers 2..3 with DMA,
  // start tiles 0 and 1; the score waves then pull their queries into
  // registers.
  {
    const int64_t qbase = (int64_t)wk.b * rows;
    for (int i = wave; i < (64 * kQStride) / 64; i += 8) {
      const int sl = i * 64 + lane;
      const int r = sl / kQStride, c = sl - r * kQStride;
      const int qr = min(row_base + r, rows - 1);
      const uint8_t* src = c < 64 ? (const uint8_t*)(a.q_lat + (qbase + qr) * 512 + c * 8)
                                  : (const uint8_t*)(a.q_rope + (qbase + qr) * 64 + (c < 72 ? c - 64 : 0) * 8);
      dma16(src, tiles_lds + kQBase + i * 1024);
    }
  }
  const int blk_a = tile_block(0), blk_b = tile_block(1);
  if (valw) {
    Staged st;
    stage_load(0, blk_a, st);
    stage_store(0, st);
    stage_load(1, blk_b, st);
    stage_store(1, st);
    wait_vmcnt<0>();  // the queries
  } else {
    issue_tile(0, blk_a);
    issue_tile(1, blk_b);
    wait_tiles2();  // the queries (tiles 0 and 1 may still be in flight)
  }
  wg_barrier();

  // The two roles run separate loops with the same sequence of barriers:
  // per pass, the pass start, the reference exchange (first pass, non-empty
  // chunk), tile 0's end, one per later tile, the overflow vote and (before a
  // repeat) the new reference; after the last pass the row sums.  A row's
  // reference max is fixed at its first tile, so P and O never need
  // rescaling.  If a later score exceeds it by more than 2^kRefSlack the pass
  // is finished (its values are discarded) and repeated with the row's chunk
  // maximum as the reference: exact either way, never taken unless the
  // scores of one row span more than 44 nats, and the repeat cannot
  // overflow, so there are two passes at most.
  if (wave < 4) {
    // ================= score waves =================
    const int th = wave & 1;  // token half of a tile
    const int rh = wave >> 1;  // row half of the block
    // B operand of k-step ks for row block rb: row 32 rh + 16 rb + i16; latent
    // chunk ks + 16 q4 for ks < 16 (each lane quarter walks its own quarter of
    // the row: with the tile swizzle this order keeps the tile reads free of
    // bank conflicts, measured), RoPE chunk 4 (ks - 16) + q4 after
    bf16x8 qf[2][18];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = 32 * rh + 16 * rb + i16;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const int c = ks < 16 ? ks + 16 * q4 : 64 + 4 * (ks - 16) + q4;
        qf[rb][ks] = *(const MLA_LDS bf16x8*)(tiles + kQBase + (r * kQStride + c) * 16);
      }
    }
    wg_barrier();  // every score wave holds its queries: tiles 2, 3 and P are free

    // score operand: tile row 16 th + i16; latent chunk ks + 16 q4 sits in
    // slice q4 at byte 256 row + ((ks ^ s16(row)) << 4) = c1_lat ^ (ks << 4);
    // RoPE chunk 4 (ks - 16) + q4 after the latent part
    const int tr = 16 * th + i16;
    const uint32_t c1_lat = q4 * kSliceBytes + tr * 256 + (s16(tr) << 4);
    uint32_t c1_rope[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) c1_rope[k] = kLatBytes + tr * 128 + (((4 * k + q4) ^ s8(tr)) << 4);
    // this lane's score rows (block-relative), their causal limits and P
    // slots: tokens 16 th + 4 q4 + 0..3 of row R sit in 16-byte chunk
    // 2 th + (q4 & 1) (bytes 8 (q4 >> 1)..) at slot 4 R + (chunk ^ (R/4 % 4))
    int prow[2], hi_tok[2];
    uint32_t pwrite[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      prow[rb] = 32 * rh + 16 * rb + i16;
      const int qrow = row_base + prow[rb];
      hi_tok[rb] = qrow < rows ? min(wk.tok1, wk.len - (a.sq - 1 - qrow / a.heads)) : 0;
      pwrite[rb] = (4 * prow[rb] + ((2 * th + (q4 & 1)) ^ ((prow[rb] >> 2) & 3))) * 16 + 8 * (q4 >> 1);
    }

    float m_ref[2] = {-__builtin_inff(), -__builtin_inff()};
    float m_hi[2], l_part[2];
    bool ovf;

    // scores of tile s: 18 k-steps, two 16x16x32 products each (one per row
    // block, same token operand); the latent part (k-steps 0..15) and the
    // RoPE part (16, 17) accumulate separately because only the former is
    // scaled.  `hook(ks)` runs after k-step ks.
    f32x4 sacc[2], sacc_r[2];
    auto scores = [&](int s, auto hook) __attribute__((always_inline)) {
      const MLA_LDS uint8_t* tb = tiles + (s % kBuf) * kTileBytes;
      auto ldA = [&](int ks) __attribute__((always_inline)) -> bf16x8 {
        if (ks < 16) return *(const MLA_LDS bf16x8*)(tb + (c1_lat ^ (uint32_t)(ks << 4)));
        return *(const MLA_LDS bf16x8*)(tb + c1_rope[ks - 16]);
      };
      constexpr int kDepth = 4;
      sacc[0] = sacc[1] = sacc_r[0] = sacc_r[1] = f32x4{};
      bf16x8 ar[kDepth];
#pragma unroll
      for (int ks = 0; ks < kDepth; ++ks) ar[ks] = ldA(ks);
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        if (ks < 16) {
          sacc[0] = mfma16x16x32(ar[ks % kDepth], qf[0][ks], sacc[0]);
          sacc[1] = mfma16x16x32(ar[ks % kDepth], qf[1][ks], sacc[1]);
        } else {
          sacc_r[0] = mfma16x16x32(ar[ks % kDepth], qf[0][ks], sacc_r[0]);
          sacc_r[1] = mfma16x16x32(ar[ks % kDepth], qf[1][ks], sacc_r[1]);
        }
        if (ks + kDepth < 18) ar[ks % kDepth] = ldA(ks + kDepth);
        hook(ks);
        sched_fence();
      }
    };

    // softmax of tile s: lane holds tokens 16 th + 4 q4 + r of rows prow[rb].
    // Score = scale_t (q_lat . code_t) + q_rope . k^R_t; the value product
    // takes p_t scale_t against the codes, the row sum p_t.
    float p[2][4], mx[2];
    f32x4 tsc[2];  // the lane's four token scales per row block (0 past the row's horizon)
    auto soft_scale = [&](int s) __attribute__((always_inline)) {
      const int tt = wk.tok0 + s * kTileTok + 16 * th + 4 * q4;
      const f32x4 sc = *(const MLA_LDS f32x4*)(scl + (s % kBuf) * 32 + 16 * th + 4 * q4);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool vis = tt + r < hi_tok[rb];
          tsc[rb][r] = vis ? sc[r] : 0.f;
          const float x = (sacc[rb][r] * sc[r] + sacc_r[rb][r]) * a.scale_log2;
          p[rb][r] = vis ? x : -__builtin_inff();
        }
        mx[rb] = fmaxf(fmaxf(p[rb][0], p[rb][1]), fmaxf(p[rb][2], p[rb][3]));
      }
    };
    // hardware exp2 (v_exp_f32): results below 2^-126 flush to zero, which
    // cannot matter next to the row's largest weight (>= 1 after the first tile)
    auto soft_finish = [&](int s) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        m_hi[rb] = fmaxf(m_hi[rb], mx[rb]);
        ovf |= mx[rb] > m_ref[rb] + kRefSlack;
        const float mu = m_ref[rb] == -__builtin_inff() ? 0.f : m_ref[rb];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[rb][r] = __builtin_amdgcn_exp2f(p[rb][r] - mu);
          l_part[rb] += p[rb][r];
        }
        const u32x2 pk = {pack_bf16x2(p[rb][0] * tsc[rb][0], p[rb][1] * tsc[rb][1]),
                          pack_bf16x2(p[rb][2] * tsc[rb][2], p[rb][3] * tsc[rb][3])};
        *(MLA_LDS u32x2*)(pbuf + (s & 1) * kPBytes + pwrite[rb]) = pk;
      }
    };

    for (int pass = 0; pass < 2; ++pass) {
      const bool first = pass == 0;
      l_part[0] = l_part[1] = 0.f;
      m_hi[0] = m_hi[1] = -__builtin_inff();
      ovf = false;
      if (!first) {
        issue_tile(0, blk_a);
        issue_tile(1, blk_b);
      }
      wait_tiles1();  // tile 0 (tile 1 may still be in flight)
      fix_tail(0);
      wg_barrier();

      int blk_next = tile_block(4);
      if (ntiles > 0) {
        issue_tile(2, tile_block(2));  // buffers 2, 3 are free (queries held, or the last pass over)
        issue_tile(3, tile_block(3));
        scores(0, [](int) {});
        soft_scale(0);
        if (first) {
          // each row's maximum over the whole first tile (both token halves);
          // a row left at -inf sees no token of this chunk
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            float m = fmaxf(mx[rb], __shfl_xor(mx[rb], 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            if (q4 == 0) xm[th * 64 + prow[rb]] = m;
            mx[rb] = m;
          }
          wg_barrier();
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) m_ref[rb] = fmaxf(mx[rb], xm[(th ^ 1) * 64 + prow[rb]]);
        }
        soft_finish(0);
        wait_tiles2();  // tile 1 (tiles 2, 3 may still be in flight)
        fix_tail(1);
        wg_barrier();
      }

      // tiles 1 ..: the RoPE rows and scales of tile s+3 go into the buffer of
      // tile s-1, whose RoPE rows and scales were read in the previous iteration
      for (int s = 1; s < ntiles; ++s) {
        issue_tile(s + 3, blk_next);
        scores(s, [](int) {});
        soft_scale(s);
        soft_finish(s);
        blk_next = tile_block(s + 4);  // a scalar load: read here, its wait joins the barrier's
        wait_tiles2();  // tile s+1 (tiles s+2, s+3 may still be in flight)
        fix_tail(s + 1);
        wg_barrier();
      }
      wait_vmcnt<0>();  // copies issued for tiles past the chunk have landed

      // ---- did any row overflow its reference?  (its partner lanes may not know)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float m = fmaxf(m_hi[rb], __shfl_xor(m_hi[rb], 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        m_hi[rb] = m;
        if (q4 == 0) xm[th * 64 + prow[rb]] = m;
      }
      // the vote runs in every lane (a ballot taken inside `if (lane == 0)`
      // would see lane 0's rows alone)
      const bool wave_ovf = __builtin_amdgcn_ballot_w64(ovf) != 0;
      if (lane == 0) xf[wave] = wave_ovf;
      wg_barrier();
      const bool again = (xf[0] | xf[1] | xf[2] | xf[3]) != 0;
      if (!again || !first) break;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) m_ref[rb] = fmaxf(m_hi[rb], xm[(th ^ 1) * 64 + prow[rb]]);
      wg_barrier();
    }

    // ---- row sums (4 token quads x 2 token halves) for the value waves; lse
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float l = l_part[rb] + __shfl_xor(l_part[rb], 16, 64);
      l += __shfl_xor(l, 32, 64);
      if (q4 == 0) xl[th * 64 + prow[rb]] = l;
    }
    wg_barrier();
    if (th == 0 && q4 == 0) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int qrow = row_base + prow[rb];
        const float lt = xl[prow[rb]] + xl[64 + prow[rb]];
        if (qrow < rows) a.lse[slot * rows + qrow] = lt > 0.f ? (m_ref[rb] + log2f(lt)) * kLn2 : -__builtin_inff();
      }
    }
  } else {
    // ================= value waves =================
    wg_barrier();  // the score waves hold their queries
    // C^T operand (transposing reads, slice v): token row 16 ks + 8 j2 + 4 g +
    // i16/4 of the tile, latent columns 128 v + 32 mt + 16 (lane/16 % 2) + 4 (i16 % 4)
    const int vy = 2 * ((lane >> 4) & 1) + ((i16 >> 1) & 1);
    uint32_t voff[2][4];
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const int sw = (((i16 >> 2) & 3) << 2) | ((2 * j2 + g) & 3);  // s16 of the row
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        voff[j2][mt] = v * kSliceBytes + (8 * j2 + 4 * g + (i16 >> 2)) * 256 + (((4 * mt + vy) ^ sw) << 4) + (i16 & 1) * 8;
    }
    // P^T operand: row R = 32 nt + n32, 16-byte chunk 2 ks + g holding tokens
    // 16 ks + 4 g + 0..3 and 16 ks + 8 + 4 g + 0..3, at slot 4 R + (chunk ^
    // (R/4 % 4)) of the tile's P buffer (rows 32.. are 2048 bytes on)
    uint32_t pread[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pread[ks] = (4 * n32 + ((2 * ks + g) ^ ((n32 >> 2) & 3))) * 16;

    f32x16 oacc[4][2];
    // C^T operand of tile t, 16-token half ks, 32-column block mt
    auto av_load = [&](int t, int ks, int mt) __attribute__((always_inline)) -> bf16x8 {
      const MLA_LDS uint8_t* vt = tiles + (t % kBuf) * kTileBytes + ks * 16 * 256;
      const u32x2 lo = lds_read_tr16_b64(vt + voff[0][mt]);
      const u32x2 hi = lds_read_tr16_b64(vt + voff[1][mt]);
      return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    // value product of tile t: two 16-token halves, eight 32x32x16 products
    // each.  With `refill`, once every operand read of slice v has completed,
    // the staged tile t+4 is converted into the slice and tile t+5 staged,
    // one 16-byte piece after each of the first eight products.
    // Its C^T operands are read ahead, at the end of the previous product,
    // as in decode_mfma_bf16; then the operands of tile `next` (if >= 0).
    Staged st;
    bf16x8 av[2][4];
    auto load_av = [&](int t) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) av[ks][mt] = av_load(t, ks, mt);
    };
    auto values = [&](int t, bool refill, int nblk, int next) __attribute__((always_inline)) {
      const MLA_LDS uint8_t* pb = pbuf + (t & 1) * kPBytes;
      bf16x8 bp[2][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bp[ks][0] = *(const MLA_LDS bf16x8*)(pb + pread[ks]);
        bp[ks][1] = *(const MLA_LDS bf16x8*)(pb + pread[ks] + 2048);
      }
      if (refill) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads of slice v are done
      const uint8_t* lp = stage_src(t + 5, nblk);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ks = i >> 3, mt = (i >> 1) & 3, nt = i & 1;
        oacc[mt][nt] = mfma32x32x16(av[ks][mt], bp[ks][nt], oacc[mt][nt]);
        if (refill && i < 8) {
          stage_piece(t + 4, st, i >> 1, i & 1);
          if (i & 1) st.c[i >> 1] = *(const u32x4*)(lp + soff[i >> 1]);
        }
        sched_fence();
      }
      if (next >= 0) load_av(next);
    };

    for (int pass = 0; pass < 2; ++pass) {
      const bool first = pass == 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) oacc[mt][nt] = f32x16{};
      if (!first) {
        stage_load(0, blk_a, st);
        stage_store(0, st);
        stage_load(1, blk_b, st);
        stage_store(1, st);
      }
      wg_barrier();

      if (ntiles > 0) {
        load_av(0);
        stage_load(2, tile_block(2), st);  // buffers 2, 3 are free (queries held, or the last pass over)
        stage_store(2, st);
        stage_load(3, tile_block(3), st);
        stage_store(3, st);
        stage_load(4, tile_block(4), st);
        if (first) wg_barrier();  // the score waves' reference exchange
        wg_barrier();
      }
      for (int s = 1; s < ntiles; ++s) {
        // slice v of tile s-1's buffer takes tile s+3 (staged last iteration); tile s+4 is staged
        values(s - 1, true, tile_block(s + 4), s);
        wg_barrier();
      }
      if (ntiles > 0) values(ntiles - 1, false, 0, -1);
      wg_barrier();  // overflow vote
      const bool again = (xf[0] | xf[1] | xf[2] | xf[3]) != 0;
      if (!again || !first) break;
      wg_barrier();  // new reference
    }

    // ---- epilogue: normalise by the row sums and stage this chunk's o_lat
    // in the tile ring (free now: every copy has landed, no tile is read),
    // rows of 512 fp32 plus 16 bytes of pad
    wg_barrier();  // row sums
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int r = nt * 32 + n32;
      const float lt = xl[r] + xl[64 + r];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      MLA_LDS uint8_t* orow = tiles + r * kORow + v * 512;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 o = {oacc[mt][nt][4 * j] * inv, oacc[mt][nt][4 * j + 1] * inv,
                           oacc[mt][nt][4 * j + 2] * inv, oacc[mt][nt][4 * j + 3] * inv};
          *(MLA_LDS f32x4*)(orow + (mt * 32 + j * 8 + 4 * g) * 4) = o;
        }
      }
    }
  }
  // all eight waves write the staged rows: a wave's store covers a row's 2
  // KB (fp32) or 1 KB (fp16 partials) (the accumulator layout would write 32
  // rows x 32 bytes per store)
  wg_barrier();
  {
    const int c16 = tid & 127;
    const int64_t obase = slot * (int64_t)rows * 512;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = (tid >> 7) + 4 * k;
      const f32x4 o = *(const MLA_LDS f32x4*)(tiles + r * kORow + c16 * 16);
      const int64_t e = obase + (int64_t)(row_base + r) * 512 + 4 * c16;  // first element of the piece
      if (row_base + r < rows) {
        if (a.o_f16)
          *(f16x4*)((_Float16*)a.o + e) = to_f16x4(o);
        else
          *(f32x4*)((float*)a.o + e) = o;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// fp32 cache and queries: one workgroup (512 threads) per (sequence, KV chunk,
// query row), fp32 arithmetic throughout.  The chunk is walked in 16-token
// tiles copied HBM -> LDS by DMA into a ring of four buffers (latent rows and
// RoPE keys in separate arrays, so every 1 KB copy reads from one
// wave-uniform base; two or three tiles in flight).  Two roles of four waves:
//   score waves 0..3: wave w forms the scores of tokens 4w .. 4w+3, lane l
//       summing q . c_t over latent floats 4l..4l+3 and 256+4l..+3 and RoPE
//       float l (16-byte LDS reads against the query held in registers); the
//       four tokens' sums are reduced within each row of 16 lanes (DPP) and
//       the four row sums of each token go to LDS;
//   value waves 4..7 issue the copies, and fold tile t into the output: lane
//       l of every 16-lane row takes token l of the tile (the sum of its four
//       row sums), the row maximum updates the running one (online softmax in
//       the log2 domain, hardware exp2), and thread i accumulates latent
//       columns 2i, 2i+1 with the 16 weights read from their lanes.
// One barrier per tile: after barrier t the score waves form the scores of
// tile t+1 while the value waves fold in tile t (scores double-buffered).
// Rows past the row's visible range are zeroed in LDS by the waves that
// copied them once their copies have landed (an uninitialised pool row may
// hold NaN; its weight is 0).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(512) decode_f32(const DecodeArgs a) {
  constexpr int kT = 16;          // tokens per tile
  constexpr int kRowF = 576;      // floats of a token row: latent, then RoPE key
  constexpr int kBufN = 4;        // tile ring
  constexpr int kCopies = kT * kRowF * 4 / 1024 / 4;  // 1 KB copies per value wave per tile (9)
  static_assert(kT * kRowF * 4 == 4 * kCopies * 1024, "whole copies per wave");
  // a tile's latent rows [16][512] and RoPE keys [16][64], each ring slot
  __shared__ __attribute__((aligned(1024))) float tlat[kBufN][kT * 512];
  __shared__ __attribute__((aligned(1024))) float trope[kBufN][kT * 64];
  __shared__ __attribute__((aligned(16))) float sp[2][kT * 4];  // [token][16-lane row] score sums
  if (blockDim.x != 512) return;  // the roles below assume eight waves
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool valw = wave >= 4;
  const int cw = wave & 3;
  // XCD-aware placement: workgroup ids are dealt round-robin over the 8
  // XCDs, so XCD x takes a contiguous range of (unit, row) pairs and the rows
  // of a chunk, which read the same pages, share that XCD's L2
  const int total = a.units * a.rows;
  const int per_xcd = (total + 7) >> 3;
  const int lin = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (lin >= total) return;
  const int row = lin % a.rows;
  const int unit = lin / a.rows;
  const int b = unit / a.num_splits, split = unit % a.num_splits;
  const int len = a.seq_lens[b];
  const int npages = (len + 63) >> 6;
  const int pps = (npages + a.num_splits - 1) / a.num_splits;
  const int p0 = split * pps, p1 = min(p0 + pps, npages);
  const int qi = row / a.heads;
  const int nvis = len - (a.sq - 1 - qi);
  const int tok0 = p0 * 64;
  const int tok1 = min(min(p1 * 64, len), max(nvis, 0));  // this row's tokens of the chunk: [tok0, tok1)
  const int ntiles = tok1 > tok0 ? (tok1 - tok0 + kT - 1) / kT : 0;
  const uint32_t lat_lds = lds_addr((MLA_LDS float*)&tlat[0][0]);
  const uint32_t rope_lds = lds_addr((MLA_LDS float*)&trope[0][0]);

  // The 36 1 KB copies of a tile, g = 9 cw + k for value wave 4 + cw: g < 32
  // brings half g & 1 of latent row g / 2, g >= 32 the RoPE keys of rows
  // 4 (g - 32) .. +3 (lane i: row + i / 16, bytes 16 (i % 16)).  Every copy
  // reads one 64-row page from a wave-uniform base; rows past the range are
  // read from the page (a whole block) and zeroed once landed.
  int blk = 0;
  auto tile_block = [&](int t) __attribute__((always_inline)) -> int {
    const int t0 = min(tok0 + t * kT, tok1 - 1);
    // scalar load: a vector one would make the compiler wait for the copies
    return load_uniform(a.block_table, (int64_t)b * a.max_blocks + (t0 >> 6));
  };
  const uint32_t rope_off = (uint32_t)((lane >> 4) * a.rope_rs + 16 * (lane & 15));
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int prow0 = (tok0 + t * kT) & 63;  // t < ntiles; tiles never cross a page
    const uint8_t* lat = a.latent + blk * a.lat_bs + prow0 * a.lat_rs;
    const uint8_t* rope = a.rope + blk * a.rope_bs + prow0 * a.rope_rs;
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
      const int g = kCopies * cw + k;
      if (g < 32)
        dma16s(lat + (g >> 1) * a.lat_rs + (g & 1) * 1024, 16 * lane,
               lat_lds + (uint32_t)(((t % kBufN) * kT * 512) * 4 + g * 1024));
      else
        dma16s(rope + 4 * (g - 32) * a.rope_rs, rope_off,
               rope_lds + (uint32_t)(((t % kBufN) * kT * 64) * 4 + (g - 32) * 1024));
    }
  };
  // zero this wave's copied pieces of tile t that lie past the range
  auto fix_tile = [&](int t) __attribute__((always_inline)) {
    const int t0 = tok0 + t * kT;
    if (t < ntiles && t0 + kT > tok1) {
#pragma unroll
      for (int k = 0; k < kCopies; ++k) {
        const int g = kCopies * cw + k;
        const int tr = g < 32 ? g >> 1 : 4 * (g - 32) + (lane >> 4);
        MLA_LDS float* dst = g < 32 ? (MLA_LDS float*)&tlat[t % kBufN][g * 256 + 4 * lane]
                                    : (MLA_LDS float*)&trope[t % kBufN][(g - 32) * 256 + 4 * lane];
        if (t0 + tr >= tok1) *(MLA_LDS f32x4*)dst = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  // The value waves' copy duties.  Barrier A0 needs tile 0, B_t tile t+1;
  // after B_t the buffer of tile t-1 (read for the last time before B_t)
  // takes tile t+3.
  auto copy_start = [&]() __attribute__((always_inline)) {
    blk = tile_block(0);
    issue(0);
    if (ntiles > 1) {
      blk = tile_block(1);
      issue(1);
    }
    wait_groups<kCopies, 1>(ntiles > 1 ? 1 : 0);  // tile 0 (tile 1 may still be in flight)
    fix_tile(0);
  };
  auto copy_first = [&]() __attribute__((always_inline)) {
    if (ntiles > 2) {
      blk = tile_block(2);
      issue(2);
    }
    blk = tile_block(3);
  };
  auto copy_land_first = [&]() __attribute__((always_inline)) {
    wait_groups<kCopies, 1>(ntiles > 2 ? 1 : 0);  // tile 1 (tile 2 may still be in flight)
    fix_tile(1);
  };
  auto copy_issue = [&](int t) __attribute__((always_inline)) {
    if (t + 3 < ntiles) {
      issue(t + 3);
      blk = tile_block(t + 4);
    }
  };
  auto copy_land = [&](int t) __attribute__((always_inline)) {
    wait_groups<kCopies, 1>(t + 3 < ntiles ? 1 : 0);  // tile t+2 (tile t+3 may still be in flight)
    fix_tile(t + 2);
  };

  if (!valw) {
    // ================= score waves =================
    const int64_t qoff = (int64_t)b * a.rows + row;
    const float* ql = (const float*)a.q_lat + qoff * 512;
    const f32x4 qa = *(const f32x4*)(ql + 4 * lane);
    const f32x4 qb = *(const f32x4*)(ql + 256 + 4 * lane);
    const float qr = ((const float*)a.q_rope + qoff * 64)[lane];
    // scores of tile t: wave w takes tokens 4w .. 4w+3; sp[t & 1][4 u + r]
    // receives row r's share of token u
    auto scores = [&](int t) __attribute__((always_inline)) {
      float part[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const MLA_LDS float* tr = (const MLA_LDS float*)&tlat[t % kBufN][(4 * cw + u) * 512];
        const f32x4 x = *(const MLA_LDS f32x4*)(tr + 4 * lane);
        const f32x4 y = *(const MLA_LDS f32x4*)(tr + 256 + 4 * lane);
        const float kr = trope[t % kBufN][(4 * cw + u) * 64 + lane];
        const float ax = fmaf(x[0], qa[0], fmaf(x[1], qa[1], fmaf(x[2], qa[2], x[3] * qa[3])));
        const float ay = fmaf(y[0], qb[0], fmaf(y[1], qb[1], fmaf(y[2], qb[2], fmaf(y[3], qb[3], kr * qr))));
        part[u] = ax + ay;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) part[u] = row_sum(part[u]);
      const int u = lane & 15;
      if (u < 4) {
        const float v = u == 0 ? part[0] : u == 1 ? part[1] : u == 2 ? part[2] : part[3];
        sp[t & 1][4 * (4 * cw + u) + (lane >> 4)] = v;
      }
    };
    if (ntiles > 0) {
      __syncthreads();  // A0: tile 0 has landed
      scores(0);
      __syncthreads();  // B_0: the scores of tile 0 are complete, tile 1 has landed
      for (int t = 0; t + 1 < ntiles; ++t) {
        scores(t + 1);
        __syncthreads();  // B_{t+1}
      }
    }
    return;
  }

  // ================= value waves =================
  const int c2 = 2 * (cw * 64 + lane);  // this thread's latent columns c2, c2 + 1
  float m = -__builtin_inff(), l = 0.f, o0 = 0.f, o1 = 0.f;
  // online softmax and values of tile t (its scores complete in sp[t & 1])
  auto values = [&](int t) __attribute__((always_inline)) {
    const MLA_LDS float* tl = (const MLA_LDS float*)&tlat[t % kBufN][0];
    const int u = lane & 15;
    const f32x4 pr = *(const MLA_LDS f32x4*)&sp[t & 1][4 * u];
    const float s = tok0 + t * kT + u < tok1 ? ((pr[0] + pr[1]) + (pr[2] + pr[3])) * a.scale_log2
                                             : -__builtin_inff();
    // every tile holds at least one token of the range, so mt is finite
    const float mt = fmaxf(m, row_max(s));
    const float alpha = __builtin_amdgcn_exp2f(m - mt);  // 0 on the first tile (m = -inf)
    const float p = __builtin_amdgcn_exp2f(s - mt);      // lane u: token u's weight
    l = l * alpha + row_sum(p);
    o0 *= alpha;
    o1 *= alpha;
#pragma unroll
    for (int v = 0; v < kT; ++v) {
      const float pv = lane_f(p, v);
      const float c0 = tl[v * 512 + c2], c1 = tl[v * 512 + c2 + 1];  // one 8-byte read
      o0 = fmaf(pv, c0, o0);
      o1 = fmaf(pv, c1, o1);
    }
    m = mt;
  };
  if (ntiles > 0) {
    copy_start();
    __syncthreads();  // A0
    copy_first();
    copy_land_first();
    __syncthreads();  // B_0
    for (int t = 0; t < ntiles; ++t) {
      copy_issue(t);
      values(t);
      if (t + 1 < ntiles) {
        copy_land(t);
        __syncthreads();  // B_{t+1}
      }
    }
  }
  wait_vmcnt<0>();
  const int64_t slot = (int64_t)b * a.num_splits + split;
  float* orow = (float*)a.o + (slot * a.rows + row) * 512;  // fp32 only (the launcher refuses fp16 here)
  const float inv = l > 0.f ? 1.f / l : 0.f;
  orow[c2] = o0 * inv;
  orow[c2 + 1] = o1 * inv;
  if (wave == 4 && lane == 0) a.lse[slot * a.rows + row] = l > 0.f ? (m + log2f(l)) * kLn2 : -__builtin_inff();
}

template __global__ void decode_mfma_bf16<64>(const DecodeArgs a);
template __global__ void decode_mfma_bf16<32>(const DecodeArgs a);

}  // namespace mla
