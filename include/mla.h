/*
 * mla.h -- C ABI of the MLA absorbed-decode library for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  DeepSeek-V2 Multi-head Latent Attention caches, per token
 * per layer, a 512-wide latent c_t and one 64-wide decoupled RoPE key k^R_t
 * (deepforge.srivtx.xyz "DeepSeek-V2", section 1, "Store a latent, rebuild the
 * keys and values" and the formula box "MLA: compress once, reconstruct in
 * attention").  Keys and values are k = W_UK c and v = W_UV c per head; since
 * both maps are linear, W_UK is folded into the query and W_UV into the output
 * ("absorption", same passage), so decode attention runs on the cache itself:
 *
 *   q_lat[h]  = W_UK[h]^T q_nope[h]                          (mla_absorb_q)
 *   s_t[h]    = (q_lat[h] . c_t + q_rope[h] . k^R_t) * scale  (mla_decode)
 *   p[h]      = softmax_t(s[h]),  o_lat[h] = sum_t p_t[h] c_t
 *   o_lat     = log-sum-exp merge of per-chunk results          (mla_split_combine)
 *   o[h]      = W_UV[h] o_lat[h]                               (mla_out_uv)
 *
 * Decode compares the newest token's query with the keys of every earlier
 * token and mixes their values (same page, section 1, "The bottleneck at
 * inference time"); with S_q query tokens per sequence, query i (0-based,
 * oldest first) sees the first len - (S_q - 1 - i) cached tokens.
 *
 * Conventions for every entry point.
 *  - Every array argument is a DEVICE pointer owned by the caller; the library
 *    never allocates, frees, copies to the host or synchronizes.  Struct
 *    arguments (mla_dims, mla_paged_kv) are HOST pointers read during the call.
 *  - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream).  Calls return as soon as the work is enqueued.
 *  - Arrays are dense row-major unless a stride says otherwise; strides are
 *    in elements.  bf16 is stored as its 16-bit pattern, E4M3 as OCP E4M3FN
 *    bytes (the gfx950 fp8 format, max 448).
 *  - Arguments are validated on the host before any launch; an invalid call
 *    returns a negative mla_status and enqueues nothing.  Device-side data
 *    (block_table, seq_lens) is trusted: entries must name blocks below
 *    num_blocks and lengths must fit max_blocks_per_seq * block_size.  With
 *    the environment variable MLA_CHECK set to 1 at the call, mla_decode
 *    checks them too: it copies both arrays to the host on `stream`,
 *    synchronizes it (the one exception to the rule below), and returns
 *    MLA_ERR_SHAPE without launching if a length is negative or too long or
 *    a block id among a sequence's first ceil(len / block_size) entries is
 *    outside [0, num_blocks); MLA_ERR_DEVICE if the copy fails.
 *  - mla_decode with a bf16 cache runs 64 query rows per workgroup, or 32
 *    when 64-row workgroups would leave compute units idle (few sequence x
 *    chunk units); MLA_DECODE_ROWS=64 or 32 in the environment at the call
 *    fixes the choice (same results within rounding of the summation order).
 *  - Supported sizes: d_latent = 512, d_rope = 64, d_head = 128,
 *    block_size = 64, 1 <= q_per_seq <= MLA_MAX_Q_PER_SEQ; anything else is
 *    MLA_ERR_SHAPE.  The fp32 paths launch one grid row per query row, so
 *    there batch * q_per_seq is at most 65535 (mla_absorb_q, mla_out_uv and
 *    mla_combine_out_uv with F32 data, mla_cache_append with an F32 cache);
 *    mla_cache_append with bf16 inputs takes up to 65535 * 32 new tokens.
 *    Larger calls return MLA_ERR_SHAPE.
 *  - Thread-safe.  The library holds no mutable global state, with one
 *    exception: mla_cache_append_static keeps a fixed device array per GPU
 *    (its scratch) and that array's device address per device.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: adds mla_combine_out_uv; 3: adds the MLA_CHECK validation of mla_decode;
 * 4: adds out_dtype to mla_out_uv and mla_combine_out_uv; 5: adds mla_cache_append;
 * 6: q_per_seq up to 128 (was 2); 7: adds mla_moe_gate;
 * 8: adds mla_source_hash; 9: adds mla_cache_append_static and MLA_ERR_SCRATCH;
 * 10: the chunk partials of mla_decode may be fp16 (MLA_F16): o_dtype of
 * mla_decode, part_dtype of mla_split_combine and mla_combine_out_uv;
 * 11: q_per_seq up to 4096; adds the explicit form (mla_attend_explicit,
 * mla_attend_explicit_workspace_size) and mla_attention_form;
 * 12: adds mla_decode_num_splits_batch */
#define MLA_ABI_VERSION 12

typedef enum mla_dtype {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2, /* OCP E4M3FN, one fp32 scale per cached token */
  MLA_F16 = 3        /* IEEE binary16: mla_decode's chunk partials only */
} mla_dtype;

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,   /* a required pointer is NULL                         */
  MLA_ERR_SHAPE = -2,  /* a size is out of range or unsupported              */
  MLA_ERR_DTYPE = -3,  /* an unsupported dtype or dtype combination          */
  MLA_ERR_ALIGN = -4,  /* a pointer or stride breaks the 16-byte alignment   */
  MLA_ERR_SPLITS = -5, /* num_splits < 1 or > MLA_MAX_SPLITS                 */
  MLA_ERR_LAUNCH = -6, /* the HIP runtime refused the launch                 */
  MLA_ERR_DEVICE = -7, /* no usable gfx950 device is current                */
  MLA_ERR_SCRATCH = -8 /* the call needs more than the static scratch holds  */
} mla_status;

#define MLA_MAX_SPLITS 1024
/* Query tokens per sequence in one call (multi-token decode: speculative
 * tokens, prefill chunks). */
#define MLA_MAX_Q_PER_SEQ 4096

/* Static description of one decode batch. */
typedef struct mla_dims {
  int32_t batch;       /* B: sequences                                       */
  int32_t q_per_seq;   /* S_q: query tokens per sequence (1..4096)           */
  int32_t heads;       /* H: attention heads (1..1024)                       */
  int32_t d_latent;    /* 512                                                */
  int32_t d_rope;      /* 64                                                 */
  int32_t d_head;      /* 128                                                */
  float softmax_scale; /* multiplies q.k; DeepSeek-V2 head shape: 1/sqrt(192) */
} mla_dims;

/* Paged latent cache.  Token t of sequence b is row (t mod block_size) of
 * physical block block_table[b * max_blocks_per_seq + t / block_size].
 *
 *   latent row:  latent + block * latent_block_stride + row * latent_row_stride
 *                (d_latent values of latent_dtype)
 *   rope row:    rope   + block * rope_block_stride   + row * rope_row_stride
 *                (d_rope values of rope_dtype)
 *   fp8 scale:   scale[block * scale_block_stride + row]  (fp32; fp8 only;
 *                `scale` 16-byte aligned, scale_block_stride a multiple of 4)
 *
 * The 576-wide interleaved layout [c | k^R] is rope = latent + 512 with both
 * row strides 576 and both block strides 64 * 576.  Supported combinations:
 *   latent F32  + rope F32                  (use with F32 queries)
 *   latent BF16 + rope BF16                 (use with BF16 queries)
 *   latent FP8_E4M3 + scale + rope BF16     (use with BF16 queries)
 * Rows at or past a sequence's length may hold anything, NaN included: no
 * output depends on them. */
typedef struct mla_paged_kv {
  const void* latent;
  int32_t latent_dtype;
  int64_t latent_block_stride;
  int64_t latent_row_stride;
  const void* rope;
  int32_t rope_dtype;
  int64_t rope_block_stride;
  int64_t rope_row_stride;
  const float* scale; /* FP8_E4M3 latent only, else NULL */
  int64_t scale_block_stride;
  int32_t block_size;         /* 64 */
  int32_t num_blocks;         /* physical blocks in the pool */
  int32_t max_blocks_per_seq; /* row length of block_table */
  const int32_t* block_table; /* [batch][max_blocks_per_seq] int32 */
  const int32_t* seq_lens;    /* [batch] int32, cached tokens incl. the S_q query tokens */
} mla_paged_kv;

/* Human-readable name of a status code (static storage). */
const char* mla_status_str(int status);

/* MLA_ABI_VERSION of the built library. */
int mla_abi_version(void);

/* 16 lowercase hex digits identifying the sources the library was built from
 * (a hash over its kernel and header files, static storage).  Lets a caller
 * refuse a library built from other sources than the ones it expects. */
const char* mla_source_hash(void);

/* Query absorption (formula box "MLA: compress once, reconstruct in attention":
 * k = W_UK c, folded into the query side):
 *   q_lat[r][h][c] = sum_d w_uk[h][d][c] * q_nope[r][h][d],   r < batch*q_per_seq.
 * q_nope: [batch*q_per_seq][heads][d_head], in_dtype (F32 or BF16)
 * w_uk:   [heads][d_head][d_latent], in_dtype
 * q_lat:  [batch*q_per_seq][heads][d_latent], q_lat_dtype (F32, or BF16
 *         rounded to nearest-even from the fp32 sum)
 * Products are exact, sums are fp32. */
int mla_absorb_q(const mla_dims* dims, const void* q_nope, const void* w_uk, int32_t in_dtype,
                 void* q_lat, int32_t q_lat_dtype, void* stream);

/* Decode attention over the paged latent cache (same page, section 1, "The
 * bottleneck at inference time" and "Store a latent, rebuild the keys and
 * values"):
 *   s_t = (q_lat . c_t + q_rope . k^R_t) * softmax_scale,  t visible to the query,
 *   o_lat = sum_t softmax(s)_t c_t,   lse = ln sum_t exp(s_t).
 * q_lat:  [batch*q_per_seq][heads][d_latent], q_dtype
 * q_rope: [batch*q_per_seq][heads][d_rope],   q_dtype (F32 with an F32 cache, else BF16)
 * num_splits == 1: o = o_lat [batch*q_per_seq][heads][d_latent], lse [batch*q_per_seq][heads].
 * num_splits  > 1: each sequence's pages are cut into num_splits page-aligned
 *   chunks of ceil(pages / num_splits) pages; chunk s writes its own
 *   normalised result: o = [batch][num_splits][q_per_seq][heads][d_latent],
 *   lse = [batch][num_splits][q_per_seq][heads]; merge with mla_split_combine.
 * o_dtype: F32, or (num_splits > 1 with a BF16 or FP8 cache) F16: the
 *   normalised chunk result, accumulated in fp32, rounded to nearest-even
 *   binary16 (relative error below 2^-11; the merge reads half the bytes);
 *   lse is fp32 in every case.  Anything else is MLA_ERR_DTYPE.
 * A query (or chunk) that sees no token writes o = 0 and lse = -inf.
 * Arithmetic: bf16/fp8 caches use bf16 matrix cores with fp32 accumulation
 * (E4M3 codes are exact in bf16; the per-token scale is applied in fp32);
 * the F32 cache is computed in fp32 throughout. */
int mla_decode(const mla_dims* dims, const void* q_lat, const void* q_rope, int32_t q_dtype,
               const mla_paged_kv* kv, int32_t num_splits, void* o, int32_t o_dtype, float* lse, void* stream);

/* Log-sum-exp merge of mla_decode's per-chunk results:
 *   lse = ln sum_s exp(lse_s),   o_lat = sum_s exp(lse_s - lse) o_s.
 * Chunks with lse_s = -inf carry weight 0; if all do, o_lat = 0 and lse = -inf.
 * o_part: [batch][num_splits][q_per_seq][heads][d_latent], part_dtype (F32 or F16,
 *         as mla_decode wrote it); lse_part: [batch][num_splits][q_per_seq][heads] fp32
 * o_lat:  [batch*q_per_seq][heads][d_latent] fp32;  lse: same layout as
 *         mla_decode's, or NULL.  Sums are fp32. */
int mla_split_combine(const mla_dims* dims, int32_t num_splits, const void* o_part, int32_t part_dtype,
                      const float* lse_part, float* o_lat, float* lse, void* stream);

/* Output absorption (W_UV folded into the output side, same formula box):
 *   out[r][h][d] = sum_c w_uv[h][d][c] * o_lat[r][h][c].
 * o_lat: [batch*q_per_seq][heads][d_latent] fp32
 * w_uv:  [heads][d_head][d_latent], w_dtype (F32 or BF16)
 * out:   [batch*q_per_seq][heads][d_head], out_dtype: F32, or BF16 rounded to
 *        nearest-even from the fp32 sum; anything else is MLA_ERR_DTYPE
 * With BF16 weights the fp32 o_lat is split into two bf16 terms (hi + lo), so
 * the sum carries fp32-level accuracy at matrix-core speed. */
int mla_out_uv(const mla_dims* dims, const float* o_lat, const void* w_uv, int32_t w_dtype,
               void* out, int32_t out_dtype, void* stream);

/* The merge of mla_split_combine and the projection of mla_out_uv in one call,
 * for num_splits > 1 (same formulas, same passages): o_lat is formed on the fly
 * from the chunks' partials and never written,
 *   out[r][h][d] = sum_c w_uv[h][d][c] * (sum_s exp(lse_s - lse) o_s[r][h][c]),
 *   lse[r][h]    = ln sum_s exp(lse_s).
 * o_part, part_dtype, lse_part: mla_decode's outputs for num_splits > 1
 * (layouts and partial dtypes as for mla_split_combine);
 * w_uv, w_dtype, out, out_dtype: as for mla_out_uv; lse: [batch*q_per_seq][heads]
 * fp32, or NULL.
 * Chunks with lse_s = -inf carry weight 0 (their o_s may hold anything, NaN
 * included, and never reaches the result); a row whose chunks all do gets
 * out = 0 and lse = -inf.  Same accuracy as the two calls. */
int mla_combine_out_uv(const mla_dims* dims, int32_t num_splits, const void* o_part, int32_t part_dtype,
                       const float* lse_part, const void* w_uv, int32_t w_dtype, void* out, int32_t out_dtype,
                       float* lse, void* stream);

/* Cache append: the step that writes the S_q newest tokens of each sequence
 * into the paged cache before mla_decode reads them (same page, section 1,
 * "Store a latent, rebuild the keys and values": the down-projection
 * c_t = W_DKV h_t is where compression happens, and a separate 64-wide key
 * carries the position, because RoPE cannot pass through the absorbed
 * projections).  For token i of sequence b at position p = len_b - S_q + i
 * (skipped if p < 0), with h its hidden state:
 *   c_t    = W_DKV h                                   (512 values)
 *   k^R_t  = RoPE_p(W_KR h): pairs (2j, 2j+1) rotated by the angle
 *            p * rope_theta^(-2j/64), j = 0..31        (64 values)
 * and the token's cache row (kv's page table at position p) receives them:
 *   F32 cache:  c and k^R as fp32;
 *   BF16 cache: each rounded to nearest-even bf16;
 *   FP8 cache:  scale = amax_j |c_j| / 448 (fp32; 1 if c is all zero), codes
 *               = E4M3 of c_j / scale (fp32 division, nearest-even, clamped
 *               to +-448), k^R as bf16.
 * No other cache row is touched.
 * h:     [batch*q_per_seq][d_model], in_dtype (BF16 with a BF16 or FP8 cache,
 *        F32 with an F32 cache)
 * w_dkv: [d_latent][d_model], w_kr: [d_rope][d_model], in_dtype
 * kv:    the cache, written through its latent / rope / scale pointers
 *        (seq_lens: lengths including the new tokens)
 * d_model: a multiple of 64, 64 .. 65536
 * workspace: device memory of at least mla_cache_append_workspace_size() bytes
 *        (16-byte aligned; fp32 partial sums, contents on return unspecified)
 * Products are exact, sums fp32 over d_model; the rotation is computed in
 * fp64 from the fp32 sums. */
int mla_cache_append(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv, const void* w_kr,
                     int32_t in_dtype, float rope_theta, const mla_paged_kv* kv, void* workspace,
                     int64_t workspace_bytes, void* stream);

/* Bytes of workspace mla_cache_append needs for these sizes (host-only). */
int mla_cache_append_workspace_size(const mla_dims* dims, int32_t d_model, int64_t* bytes);

/* Device bytes of the scratch array mla_cache_append_static uses on each GPU. */
#define MLA_STATIC_SCRATCH_BYTES (16 << 20)

/* mla_cache_append for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, arguments, kernels and results as mla_cache_append
 * (bit-identical cache contents), with the fp32 partial sums kept in a fixed
 * array of MLA_STATIC_SCRATCH_BYTES that the library holds on each GPU from
 * its first call there until the process ends, instead of a workspace.
 * No device memory is allocated or freed by the call.
 * The partial sums need mla_cache_append_workspace_size() bytes; a call that
 * needs more than MLA_STATIC_SCRATCH_BYTES (at d_model 5120: more than 728
 * new tokens) returns MLA_ERR_SCRATCH and enqueues nothing.
 * Every call on one GPU shares that GPU's array (each call overwrites every
 * byte it reads before reading it): calls whose work overlaps on one GPU --
 * on different streams, or from different threads without ordering -- race
 * and give undefined results; calls ordered on one stream are safe.
 * MLA_ERR_DEVICE if the array's device address cannot be obtained. */
int mla_cache_append_static(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv,
                            const void* w_kr, int32_t in_dtype, float rope_theta, const mla_paged_kv* kv,
                            void* stream);

/* MoE gate: the routed experts each token uses and their gate values
 * (deepforge.srivtx.xyz "DeepSeek-V2", section 1, "Make the feed-forward
 * layer sparse" and its formula box "Top-K routed MoE layer"; DeepSeek-V2
 * routes over 160 experts and keeps 6, and its 2 shared experts take every
 * token without a gate).  For token t with hidden state u (row t of u) and
 * expert centroids e_i (rows of e):
 *   a_i = u^T e_i                      (exact products, fp32 sums over d_model)
 *   s_i = exp(a_i - max_j a_j) / sum_j exp(a_j - max_j a_j)    over the n_experts
 *   idx[t][0..top_k-1]: the top_k experts of largest s_i, largest first; the
 *        order compares the fp32 a_i (the softmax keeps it), and of equal a_i
 *        the lower expert index comes first
 *   weight[t][k] = s_(idx[t][k]): g_i = s_i, not renormalised over the kept
 *        experts (every expert not listed has g_i = 0)
 *   scores[t][i] = s_i if scores is not NULL.
 * u:      [tokens][d_model], e: [n_experts][d_model], both in_dtype (BF16 or
 *         F32), 16-byte aligned
 * idx:    [tokens][top_k] int32; weight: [tokens][top_k] fp32;
 *         scores: [tokens][n_experts] fp32 or NULL; caller-owned device memory
 * tokens: 0 .. 2097120 (fp32 inputs: 0 .. 65535); 0 launches nothing, and then
 *         the pointers are not read (NULL allowed) once the sizes are valid
 * d_model: a multiple of 64, 64 .. 65536; n_experts: 1 .. 256;
 * top_k: 1 .. min(n_experts, 16)
 * workspace: device memory of at least mla_moe_gate_workspace_size() bytes
 *         (16-byte aligned; fp32 partial sums, contents on return unspecified)
 * The affinities must be finite (a NaN or infinite one leaves the selection
 * unspecified).  Errors: MLA_ERR_NULL (a required pointer), MLA_ERR_SHAPE
 * (sizes, short workspace), MLA_ERR_DTYPE, MLA_ERR_ALIGN; nothing is
 * launched on an error. */
int mla_moe_gate(int32_t tokens, int32_t d_model, int32_t n_experts, int32_t top_k, const void* u, const void* e,
                 int32_t in_dtype, int32_t* idx, float* weight, float* scores, void* workspace,
                 int64_t workspace_bytes, void* stream);

/* Bytes of workspace mla_moe_gate needs for these sizes (host-only). */
int mla_moe_gate_workspace_size(int32_t tokens, int32_t d_model, int32_t n_experts, int32_t in_dtype,
                                int64_t* bytes);

/* Attention in the explicit form (same page, section 1, "Store a latent,
 * rebuild the keys and values" and the formula box "MLA: compress once,
 * reconstruct in attention"): per sequence and head the keys and values are
 * rebuilt from the cached latent,
 *   k_t = [W_UK[h] c_t ; k^R_t]  (192 values),   v_t = W_UV[h] c_t  (128 values),
 * and attention runs on them:
 *   s_t = ([q_nope ; q_rope] . k_t) * softmax_scale,  t visible to the query,
 *   out = sum_t softmax(s)_t v_t,   lse = ln sum_t exp(s_t).
 * The same result as mla_absorb_q + mla_decode + mla_split_combine +
 * mla_out_uv (the absorbed form is this algebra regrouped) at another cost:
 * the absorbed form spends 2 (576 + 512) flops per (query token, cached
 * token, head); this one 2 (192 + 128) per (query token, cached token, head)
 * plus 2 x 2 x 128 x 512 per (cached token, head) to rebuild K and V once.
 * With many query tokens per sequence (chunked prefill) this form is cheaper;
 * mla_attention_form says which to use.
 * q_nope: [batch*q_per_seq][heads][d_head] BF16 (in_dtype must be BF16)
 * q_rope: [batch*q_per_seq][heads][d_rope] BF16
 * kv:     a BF16 latent + BF16 rope cache (other caches: MLA_ERR_DTYPE)
 * w_uk, w_uv: [heads][d_head][d_latent] BF16
 * workspace: device memory of at least mla_attend_explicit_workspace_size()
 *         bytes (16-byte aligned): the rebuilt keys and values, bf16
 *         (contents on return unspecified)
 * out:    [batch*q_per_seq][heads][d_head], out_dtype F32 or BF16 (rounded to
 *         nearest-even from the fp32 result)
 * lse:    [batch*q_per_seq][heads] fp32, or NULL
 * Visibility as for mla_decode (query i sees the first len - (S_q - 1 - i)
 * tokens); a query that sees no token gets out = 0 and lse = -inf.
 * Arithmetic: keys and values are rebuilt with fp32 sums and rounded to bf16;
 * scores and the weighted sum of values run on bf16 matrix cores with fp32
 * accumulation (weights rounded to bf16), softmax in fp32.  Errors as for
 * mla_decode (MLA_ERR_SHAPE also for a short workspace); nothing is launched
 * on an error. */
int mla_attend_explicit(const mla_dims* dims, const void* q_nope, const void* q_rope, int32_t in_dtype,
                        const mla_paged_kv* kv, const void* w_uk, const void* w_uv, void* workspace,
                        int64_t workspace_bytes, void* out, int32_t out_dtype, float* lse, void* stream);

/* Bytes of workspace mla_attend_explicit needs for these sizes and a page
 * table of max_blocks_per_seq entries per sequence (host-only):
 * batch x heads x T x 512, T = max_blocks_per_seq x 64 rounded up to a
 * multiple of 256 (at most 2^24). */
int mla_attend_explicit_workspace_size(const mla_dims* dims, int32_t max_blocks_per_seq, int64_t* bytes);

/* The cheaper form for these sizes and cache (host-only): writes
 * MLA_FORM_EXPLICIT when the cache is BF16 and q_per_seq is at least
 * MLA_EXPLICIT_MIN_Q, else MLA_FORM_ABSORBED (FP8 and F32 caches always take
 * the absorbed form).  The flop counts above cross at 171 query tokens; on
 * MI355X (128 heads, a 4096-token context) the absorbed form measured faster
 * up to 256 and the explicit one from 320 on, since rebuilding K and V runs
 * further below the matrix-core peak than the absorbed decode does. */
#define MLA_FORM_ABSORBED 0
#define MLA_FORM_EXPLICIT 1
#define MLA_EXPLICIT_MIN_Q 288
int mla_attention_form(const mla_dims* dims, int32_t latent_dtype, int32_t* form);

/* A launch-shape helper: the num_splits mla_decode should use so that the
 * device's compute units are filled, given the longest sequence length the
 * caller expects.  Writes 1 when one chunk per sequence already fills the
 * device.  Host-only; reads the current device's compute-unit count. */
int mla_decode_num_splits(const mla_dims* dims, int32_t max_seq_len, int32_t* num_splits);

/* The same choice given also the sum of the batch's cached lengths (host-side
 * numbers the caller holds): for nearly uniform lengths (a sum of at least
 * 0.9 x batch x max_seq_len) the value mla_decode_num_splits writes; for
 * uneven ones at least enough chunks that a chunk holds about 16 pages on
 * average (the longest sequences then spread over many compute units and a
 * short sequence's chunks finish early; 64 sequences of 512 .. 16384 tokens:
 * 8 chunks), at most the longest sequence's pages and MLA_MAX_SPLITS.
 * MLA_ERR_SHAPE if total_tokens is negative or above batch * max_seq_len.
 * Host-only; reads the current device's compute-unit count. */
int mla_decode_num_splits_batch(const mla_dims* dims, int64_t total_tokens, int32_t max_seq_len,
                                int32_t* num_splits);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
