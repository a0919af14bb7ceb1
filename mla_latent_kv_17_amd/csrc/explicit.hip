// MLA attention in the explicit form, for many query tokens per sequence
// (chunked prefill, long speculative runs).
//
// deepforge.srivtx.xyz "DeepSeek-V2", section 1, "Store a latent, rebuild the
// keys and values" and the formula box "MLA: compress once, reconstruct in
// attention": keys and values are rebuilt from the cached latent, k = [W_UK c ;
// k^R] and v = W_UV c per head, and attention runs on them.  The absorbed form
// (mla_decode) instead folds W_UK into every query and W_UV into every output:
// per (query token, cached token, head) it costs 2 (576 + 512) flops against
// 2 (192 + 128) here, while rebuilding costs 2 x 2 x 128 x 512 per (cached
// token, head) once, whatever the number of query tokens.
//
// Two launches, bf16 on the matrix cores (v_mfma_f32_16x16x32_bf16) with fp32
// sums, every tile streamed HBM -> LDS by DMA:
//  * rebuild_kv: a GEMM per (sequence, head): [tokens x 512] latent rows times
//    the head's 256 weight rows (W_UK then W_UV), 256 tokens x 256 outputs per
//    workgroup, 32 latent columns per step, three steps in flight.  Eight
//    waves: (token quarter) x (keys or values).  Keys are written token-major,
//    values transposed per 32-token group (each group's 128 x 32 block
//    contiguous, the tokens of a value dimension adjacent), both rounded to
//    bf16, into the caller's workspace.
//  * attend_explicit: workgroup = (sequence, head, 256 query tokens), eight
//    waves; wave w holds query tokens 32w .. 32w+31 as the 192-wide
//    [q_nope ; q_rope] in registers.  Per 32 cached tokens (keys, RoPE keys
//    from the cache, values; copied to LDS by waves 0..3, four tiles in the
//    ring): S^T = K Q^T over the 192 key dimensions, causal mask (query i
//    sees the first len - (S_q - 1 - i) tokens), online softmax in the log2
//    domain (running max and per-lane partial sums, the output rescaled),
//    O^T += V^T P^T.  The scores' accumulator layout is the value product's
//    operand layout (the values are stored in the matching token order), so
//    probabilities never leave registers.
#include "mla_copy.h"
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

namespace {

// ---- rebuild ----
constexpr int kRbSteps = 16;                 // 512 latent columns / 32
constexpr int kRbHalf = kRebuildTok * 64;    // one operand: 256 rows x 32 columns bf16 = 16 KB
constexpr int kRbStage = 2 * kRbHalf;        // latent rows, then weight rows
constexpr int kRbStages = 4;

// Operand tiles are [rows][32 columns] bf16, 64 B = four 16-byte chunks per
// row; chunk c of row r sits at slot 4 r + (c ^ rb_sw(r)), so the 16 rows one
// quarter-wave reads at one chunk fall in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int rb_sw(int r) { return (r >> 2) & 3; }

// ---- attention ----
constexpr int kAtTok = 32;                         // cached tokens per tile
constexpr int kAtK = 0;                            // keys: 32 rows x 256 B
constexpr int kAtRope = kAtTok * 256;              // RoPE keys: 32 rows x 128 B
constexpr int kAtV = kAtRope + kAtTok * 128;       // values: 128 dims x 64 B
constexpr int kAtTile = kAtV + 128 * kAtTok * 2;   // 20 KB
constexpr int kAtBufs = 4;
constexpr float kSlack = 8.0f;                     // log2 headroom above a query's reference max

// Bank swizzles of the attention tile (16-byte chunk index XOR): key rows
// (16 chunks), RoPE rows (8 chunks), value rows (4 chunks).
__device__ __forceinline__ int k_sw(int r) { return r & 15; }
__device__ __forceinline__ int r_sw(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int v_sw(int d) { return (d >> 2) & 3; }

__device__ __forceinline__ bf16x8 ld_lds(const MLA_LDS uint8_t* p) { return *(const MLA_LDS bf16x8*)p; }

// Four fp32 values rounded to bf16 (nearest-even) and packed into 8 bytes.
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  return u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

}  // namespace

__global__ void __launch_bounds__(512) rebuild_kv(const ExplicitArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRbStage * kRbStages];
  MLA_LDS uint8_t* const lds = (MLA_LDS uint8_t*)&smem[0];
  // placement: the (token tile, head) items are grouped in blocks of
  // kRbBlockT tiles x kRbBlockH heads (one XCD's worth of workgroups at a
  // time: 1 MB of latent rows and 2 MB of weights, read from HBM once into
  // that XCD's L2 and shared there), the blocks cut into 8 contiguous
  // ranges, one per XCD (workgroups are dispatched round-robin over the XCDs)
  const int nt = a.batch * a.tiles;  // (sequence, token tile) pairs
  const int nbt = (nt + kRbBlockT - 1) / kRbBlockT;
  const int total = nbt * ((a.heads + kRbBlockH - 1) / kRbBlockH) * kRbBlockT * kRbBlockH;
  const int per = (total + 7) >> 3;
  const int id = blockIdx.x;
  const int k = id >> 3, item = (id & 7) * per + k;
  if (k >= per || item >= total) return;
  const int blkid = item / (kRbBlockT * kRbBlockH), w = item - blkid * (kRbBlockT * kRbBlockH);
  const int u = (blkid % nbt) * kRbBlockT + w % kRbBlockT, h = (blkid / nbt) * kRbBlockH + w / kRbBlockT;
  if (u >= nt || h >= a.heads) return;
  const int b = u / a.tiles, t0 = (u - b * a.tiles) * kRebuildTok;
  const int len = load_uniform(a.seq_lens, b);
  if (t0 >= len) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tq = wave & 3, nh = wave >> 2;  // token quarter; 0: keys (W_UK), 1: values (W_UV)
  const int i16 = lane & 15, q4 = lane >> 4;

  // copies: wave w moves latent instructions 2w, 2w+1 and weight
  // instructions 2w, 2w+1 of every step; instruction i covers rows
  // 16 i .. 16 i + 15 (lane: row 16 i + lane / 4, slot chunk lane % 4)
  const uint8_t* cbase[2];
  const uint8_t* wbase[2];
  uint32_t coff[2], woff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = 2 * wave + j;
    const int r = 16 * i + (lane >> 2);
    const int c = (lane & 3) ^ rb_sw(r);
    // tokens past the sequence read its last row (their outputs are never
    // used unmasked); the instruction's 16 rows share one page
    const int ts = min(t0 + r, len - 1);
    const int page = min(t0 + 16 * i, len - 1) >> 6;
    const int blk = load_uniform(a.block_table, (int64_t)b * a.max_blocks + page);
    cbase[j] = a.latent + (int64_t)blk * a.lat_bs;
    coff[j] = (uint32_t)((ts & 63) * a.lat_rs) + 16 * c;
    wbase[j] = (const uint8_t*)((i < 8 ? a.w_uk : a.w_uv) + (int64_t)h * 128 * 512);
    woff[j] = (uint32_t)((r & 127) * 1024 + 16 * c);
  }
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int ks) {
    const uint32_t sb = lds0 + (ks % kRbStages) * kRbStage;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16s(cbase[j] + 64 * ks, coff[j], sb + 1024 * (2 * wave + j));
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16s(wbase[j] + 64 * ks, woff[j], sb + kRbHalf + 1024 * (2 * wave + j));
  };

  // fragment offsets: rows 64 tq + 16 tb + i16 of the latent part, rows
  // 128 nh + 16 mb + i16 of the weight part, chunk q4
  const int sw = rb_sw(i16);
  const uint32_t cread = 16 * (4 * (64 * tq + i16) + (q4 ^ sw));
  const uint32_t wread = kRbHalf + 16 * (4 * (128 * nh + i16) + (q4 ^ sw));

  f32x4 acc[4][8];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) acc[tb][mb] = f32x4{};

#pragma unroll
  for (int ks = 0; ks < kRbStages - 1; ++ks) issue(ks);
  for (int ks = 0; ks < kRbSteps; ++ks) {
    // step ks has landed once at most the later steps' copies (4 per step) are in flight
    wait_groups<4, kRbStages - 2>(min(kRbStages - 2, kRbSteps - 1 - ks));
    wg_barrier();  // every wave's share landed; step ks - 1's buffer is free
    if (ks + kRbStages - 1 < kRbSteps) issue(ks + kRbStages - 1);
    const MLA_LDS uint8_t* sb = lds + (ks % kRbStages) * kRbStage;
    bf16x8 cf[4], wf[8];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) cf[tb] = ld_lds(sb + cread + 16 * 4 * 16 * tb);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) wf[mb] = ld_lds(sb + wread + 16 * 4 * 16 * mb);
    if (nh == 0) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) acc[tb][mb] = mfma16x16x32(wf[mb], cf[tb], acc[tb][mb]);  // [dim][token]
    } else {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) acc[tb][mb] = mfma16x16x32(cf[tb], wf[mb], acc[tb][mb]);  // [token][dim]
    }
  }

  const int64_t bh = (int64_t)b * a.heads + h;
  if (nh == 0) {
    // K[bh][t][d]: lane holds token 64 tq + 16 tb + i16, dims 16 mb + 4 q4 .. +3
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      uint16_t* kp = a.k + (bh * a.tokens + t0 + 64 * tq + 16 * tb + i16) * 128 + 4 * q4;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const f32x4 v = acc[tb][mb];
        *(u32x2*)(kp + 16 * mb) = pack4(v[0], v[1], v[2], v[3]);
      }
    }
  } else {
    // V^T[bh][group][d][pos]: lane holds dim 16 mb + i16, tokens
    // 64 tq + 16 tb + 4 q4 + i (i < 4), which sit at positions
    // 8 q4 + 4 (tb % 2) + i of their 32-token group; tokens past the sequence
    // are stored as 0 (weight 0 must not meet a NaN there)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int tok = t0 + 64 * tq + 16 * tb + 4 * q4;
      const int64_t grp = bh * (a.tokens / 32) + (t0 + 64 * tq + 32 * (tb >> 1)) / 32;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const f32x4 v = acc[tb][mb];
        uint16_t* vp = a.vt + (grp * 128 + 16 * mb + i16) * 32 + 8 * q4 + 4 * (tb & 1);
        *(u32x2*)vp = pack4(tok < len ? v[0] : 0.f, tok + 1 < len ? v[1] : 0.f, tok + 2 < len ? v[2] : 0.f,
                            tok + 3 < len ? v[3] : 0.f);
      }
    }
  }
}

__global__ void __launch_bounds__(64 * kAtWaves) attend_explicit(const ExplicitArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kAtTile * kAtBufs];
  MLA_LDS uint8_t* const lds = (MLA_LDS uint8_t*)&smem[0];
  // placement: the query blocks of one (sequence, head) run on one XCD, back
  // to back (its rebuilt keys and values are read from that XCD's L2)
  const int id = blockIdx.x;
  const int xcd = id & 7, k = id >> 3;
  const int ug = k / a.qblocks, qb = k - ug * a.qblocks;
  const int unit = 8 * ug + xcd;  // (sequence, head)
  if (unit >= a.batch * a.heads) return;
  const int b = unit / a.heads, h = unit - b * a.heads;
  const int len = load_uniform(a.seq_lens, b);
  const int q0 = qb * kExplicitQ;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i16 = lane & 15, q4 = lane >> 4;
  // tokens the workgroup's last query sees bound its loop; its first
  // query's bound the tiles that need no mask
  const int qlast = min(q0 + kExplicitQ, a.sq) - 1;
  const int wg_vis = max(0, len - (a.sq - 1 - qlast));
  const int ntiles = (wg_vis + kAtTok - 1) / kAtTok;
  const int full_vis = max(0, len - (a.sq - 1 - q0));
  // this wave's queries
  const int wq0 = q0 + 32 * wave;
  const int wave_vis = wq0 < a.sq ? max(0, len - (a.sq - 1 - min(wq0 + 31, a.sq - 1))) : 0;

  // copies: tile = 20 instructions of 64 x 16 B (8 key, 4 RoPE, 8 value),
  // wave w issues 5w .. 5w+4; lane's source offset relative to the
  // instruction's per-tile base, its LDS slot = lane
  const int64_t bh = (int64_t)b * a.heads + h;
  const uint8_t* kbase = (const uint8_t*)(a.k + bh * a.tokens * 128);
  const uint8_t* vbase = (const uint8_t*)(a.vt + bh * 128 * a.tokens);  // the sequence-head's first group
  int kind[5];
  uint32_t off[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int i = 5 * wave + j;
    if (i < 8) {
      const int r = 4 * i + (lane >> 4);
      kind[j] = 0;
      off[j] = (uint32_t)(r * 256 + 16 * ((lane & 15) ^ k_sw(r)));
    } else if (i < 12) {
      const int r = 8 * (i - 8) + (lane >> 3);
      kind[j] = 1;
      off[j] = (uint32_t)(r * a.rope_rs + 16 * ((lane & 7) ^ r_sw(r)));
    } else {
      const int d = 16 * (i - 12) + (lane >> 2);
      kind[j] = 2;
      off[j] = (uint32_t)(d * 64 + 16 * ((lane & 3) ^ v_sw(d)));
    }
  }
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int t) {
    if (wave >= 4) return;  // waves 0..3 copy the tiles
    const int j0 = t * kAtTok;
    const int blk = load_uniform(a.block_table, (int64_t)b * a.max_blocks + (j0 >> 6));
    const uint8_t* rbase = a.rope + (int64_t)blk * a.rope_bs + (int64_t)(j0 & 63) * a.rope_rs;
    const uint32_t tb = lds0 + (t % kAtBufs) * kAtTile;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const uint8_t* base = kind[j] == 0 ? kbase + (int64_t)j0 * 256 : kind[j] == 1 ? rbase : vbase + (int64_t)j0 * 256;
      dma16s(base, off[j], tb + 1024 * (5 * wave + j));
    }
  };

  // Q^T operands: lane (query i16 of block c, q4) holds dims 32 ks + 8 q4 .. +7
  // of [q_nope ; q_rope] (queries past S_q: zeros, and they see no token)
  bf16x8 qf[2][6];
  int vis[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int qi = wq0 + 16 * c + i16;
    const bool ok = qi < a.sq;
    vis[c] = ok ? len - (a.sq - 1 - qi) : 0;
    const int64_t r = ((int64_t)b * a.sq + min(qi, a.sq - 1)) * a.heads + h;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      const uint16_t* src = ks < 4 ? a.q_nope + r * 128 + 32 * ks + 8 * q4 : a.q_rope + r * 64 + 32 * (ks - 4) + 8 * q4;
      const u32x4 v = *(const u32x4*)src;
      qf[c][ks] = as_bf16x8(ok ? v : u32x4{0, 0, 0, 0});
    }
  }
  // the query loads complete before any copy is counted by the waits below
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int t = 0; t < kAtBufs - 1; ++t)
    if (t < ntiles) issue(t);

  // fragment offsets within a tile: key row 16 kb + i16 at chunk 4 ks + q4
  // (ks < 4), RoPE row 16 kb + i16 at chunk 4 (ks - 4) + q4, value row
  // 16 mb + i16 at chunk q4
  const uint32_t vread = kAtV + 16 * (4 * i16 + (q4 ^ v_sw(i16)));
  float m[2] = {-__builtin_inff(), -__builtin_inff()};  // reference max (log2 domain) per query
  float l[2] = {0.f, 0.f};                               // this lane's part of the sum of weights
  f32x4 o[8][2];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb][0] = o[mb][1] = f32x4{};

  for (int t = 0; t < ntiles; ++t) {
    // tile t has landed once at most the later tiles' copies (5 per tile) are in flight
    wait_groups<5, kAtBufs - 2>(min(kAtBufs - 2, ntiles - 1 - t));
    wg_barrier();  // tile t landed in every wave's share; tile t - 1's buffer is free
    if (t + kAtBufs - 1 < ntiles) issue(t + kAtBufs - 1);
    const int j0 = t * kAtTok;
    if (j0 >= wave_vis) continue;  // none of this wave's queries sees these tokens
    const MLA_LDS uint8_t* tb = lds + (t % kAtBufs) * kAtTile;
    // S^T[kb][c]: D[token 16 kb + 4 q4 + i][query 16 c + i16]
    f32x4 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb][0] = s[kb][1] = f32x4{};
      const int r = 16 * kb + i16;
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        const uint32_t ko = ks < 4 ? kAtK + r * 256 + 16 * ((4 * ks + q4) ^ k_sw(r))
                                   : kAtRope + r * 128 + 16 * ((4 * (ks - 4) + q4) ^ r_sw(r));
        const bf16x8 kf = ld_lds(tb + ko);
        s[kb][0] = mfma16x16x32(kf, qf[0][ks], s[kb][0]);
        s[kb][1] = mfma16x16x32(kf, qf[1][ks], s[kb][1]);
      }
    }
    const bool masked = j0 + kAtTok > full_vis;  // some query of the workgroup misses some token
    // scores in the log2 domain; a query's reference m stays fixed until a
    // score exceeds it by more than kSlack (weights stay below 2^kSlack),
    // then moves to the new maximum with O and l rescaled, for the four
    // lanes of the query together (in practice on a query's first tile)
    float x[2][8];
    bool up = false;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float mt = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = s[kb][c][i] * a.scale_log2;
          x[c][4 * kb + i] = !masked || j0 + 16 * kb + 4 * q4 + i < vis[c] ? v : -__builtin_inff();
          mt = fmaxf(mt, x[c][4 * kb + i]);
        }
      up |= mt > m[c] + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(up)) {  // wave-uniform
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float mt = m[c];
#pragma unroll
        for (int e = 0; e < 8; ++e) mt = fmaxf(mt, x[c][e]);
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        // 0 while the query has seen nothing (O and l are still 0)
        const float alpha = m[c] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m[c] - mt);
        l[c] *= alpha;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) o[mb][c] *= alpha;
        m[c] = mt;
      }
    }
    bf16x8 pf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float mref = m[c] == -__builtin_inff() ? 0.f : m[c];  // a query that has seen nothing keeps p = 0
      float p[8], ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(x[c][e] - mref);
        ps += p[e];
      }
      l[c] += ps;
      // P^T operand: k slots 8 q4 .. 8 q4 + 7 = tokens 4 q4 .. +3, 16 + 4 q4 .. +3
      pf[c] = as_bf16x8(u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                              pack_bf16x2(p[6], p[7])});
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const bf16x8 vf = ld_lds(tb + vread + 16 * 4 * 16 * mb);
#pragma unroll
      for (int c = 0; c < 2; ++c) o[mb][c] = mfma16x16x32(vf, pf[c], o[mb][c]);  // O^T[dim][query]
    }
  }

#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float lt = l[c] + __shfl_xor(l[c], 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int qi = wq0 + 16 * c + i16;
    if (qi >= a.sq) continue;
    const int64_t r = ((int64_t)b * a.sq + qi) * a.heads + h;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // lane holds dims 16 mb + 4 q4 .. +3 of its query
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const f32x4 v = o[mb][c] * inv;
      const int64_t e = r * 128 + 16 * mb + 4 * q4;
      if (a.out_bf16)
        *(u32x2*)((uint16_t*)a.out + e) = pack4(v[0], v[1], v[2], v[3]);
      else
        *(f32x4*)((float*)a.out + e) = v;
    }
    if (a.lse && q4 == 0) a.lse[r] = lt > 0.f ? (m[c] + log2f(lt)) * kLn2 : -__builtin_inff();
  }
}

}  // namespace mla
