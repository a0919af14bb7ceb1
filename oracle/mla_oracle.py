"""Plain, slow, fp64 reference for MLA decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this module.  It shares no code with the HIP
path and imports nothing from it.

Sources (the pages this follows; the short names are used below):

* [DF-bottleneck]  deepforge.srivtx.xyz "DeepSeek-V2: A Strong, Economical, and
  Efficient Mixture-of-Experts Language Model", section 1 "Theory from first
  principles", part "The bottleneck at inference time": decode compares the new
  token's query with the keys of all earlier tokens and mixes their values; an
  MHA cache entry is one key and one value of width d_head per head per layer.
* [DF-latent]      same page, section 1, part "Store a latent, rebuild the keys
  and values" and its formula box "MLA: compress once, reconstruct in
  attention": the cache holds c_t (512 wide) and one 64-wide decoupled RoPE
  key per token per layer; keys and values are k = W_UK c and v = W_UV c, and
  because these maps are linear W_UK can be folded into the query side and
  W_UV into the output side ("absorption").
* [DF-snippet]     same page, section 1, the two cache-size helpers and the
  ratio they print for 128 heads x 128, 60 layers, 8192 context, 2 bytes.
* [DF-moe]         same page, section 1, part "Make the feed-forward layer
  sparse" and its formula box "Top-K routed MoE layer": the affinity of
  token u and expert centroid e_i is u^T e_i, s_i is its softmax over the
  routed experts, and g_i = s_i for the K_r largest s_i and 0 otherwise
  (160 routed experts, 6 active per token, 2 shared experts that every
  token uses and that need no gate).
* [CA-takeaways]   crackai.dev "DeepSeek-V2" card, "Key Takeaways for
  Interviews": MHA caches 2 x n_heads x d_head, GQA 2 x n_groups x d_head, MLA
  d_latent plus the small RoPE part, per token per layer.

The cache append (the step before decode) follows [DF-latent] too: the
latent is the down-projection c_t = W_DKV h_t, and a separate 64-wide key
carries the position because RoPE would break the absorbed projections.

What the pages leave open (read plainly, listed with reasons in the design
notes of the repository): the softmax scale is 1/sqrt(d_head + d_rope); one
k^R row per token is shared by all heads while q_rope is per head; inputs are
already RoPE-rotated; W_UK and W_UV are stored per head as [d_head][d_latent]
so that k = W_UK c; with S_q query tokens per sequence, query i sees the first
len - (S_q - 1 - i) cached tokens (its own included).  For the append: the
position key is k^R = RoPE_p(W_KR h) with the textbook rotation (pairs
(2j, 2j+1) turned by p * theta^(-2j/64), theta = 10000); the S_q new tokens
of a sequence sit at positions len - S_q + i; an fp8 cache row holds E4M3
codes of c / s with s = max |c| / 448.  For the MoE gate: the softmax runs
over the routed experts' affinities only; g_i is s_i itself (the formula does
not renormalise the K_r kept scores); the kept experts are listed by
decreasing s, and of equal scores the lower expert index ranks first.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
facts fixed outside this file -- numbers the pages print, closed forms, a
library attention routine, brute force in exact arithmetic, and planted
mistakes that must be caught.  No function is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_HEAD = 128

__all__ = [
    "decode_bf16", "decode_e4m3", "decode_f32",
    "gather_sequence", "reconstruct_keys", "reconstruct_values", "query_vector",
    "visible_tokens", "scores", "softmax_lse", "mix_values",
    "explicit_decode", "absorbed_decode", "absorbed_decode_batched", "split_ranges", "split_partials",
    "combine_partials", "cache_numbers_per_token_layer", "cache_bytes",
    "default_softmax_scale", "absorb_queries", "project_output",
    "down_project", "rope_angles", "rope_rotate", "e4m3_values", "e4m3_round_codes",
    "quantize_latent", "appended_tokens",
    "expert_affinities", "gate_softmax", "top_k", "moe_gate", "gate_dense",
]


# ----------------------------------------------------------------------------
# storage decoding (exact in fp64)
# ----------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64.  A bf16 value is the upper half of a
    float32, so shifting the 16 bits up and reinterpreting is exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def decode_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN bytes -> float64, from the format definition: sign bit 7,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
    subnormals m * 2^-9; 0x7F / 0xFF are NaN; there are no infinities.  The
    definition is evaluated once on the 256 byte values, which the codes then
    index (a large cache decodes in one gather)."""
    c = np.arange(256, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 0xF) & (c & 0x7 == 0x7), np.nan, mag)
    return (sign * mag)[np.asarray(codes, dtype=np.uint8)]


def _decoder(kind: str):
    return {"f32": decode_f32, "bf16": decode_bf16}[kind]


# ----------------------------------------------------------------------------
# the cached sequence
# ----------------------------------------------------------------------------

def gather_sequence(inp, b: int) -> Tuple[np.ndarray, np.ndarray]:
    """Logical cache of sequence b as (C [len][512], KR [len][64]) in fp64.

    Token t lives in row t mod P of physical block block_table[b][t div P]
    (P = 64).  Only the c_t latent and the k^R_t key are cached [DF-latent]."""
    n = int(inp.seq_lens[b])
    P = inp.latent.shape[1]
    t = np.arange(n)
    blocks = inp.block_table[b][t // P]
    rows = t % P
    kind = inp.wl.cache_dtype
    if kind == "fp8":
        C = decode_e4m3(inp.latent[blocks, rows]) * inp.scale[blocks, rows].astype(np.float64)[:, None]
        KR = decode_bf16(inp.rope[blocks, rows])
    else:
        full = _decoder(kind)(inp.latent[blocks, rows])
        C, KR = full[:, :D_LATENT], full[:, D_LATENT:D_LATENT + D_ROPE]
    return C, KR


def reconstruct_keys(C: np.ndarray, KR: np.ndarray, w_uk_h: np.ndarray) -> np.ndarray:
    """Per-head keys k_t = [W_UK c_t ; k^R_t]  ([DF-latent]: k = W_UK c, plus
    the decoupled RoPE key, shared by all heads).  W_UK is [d_head][d_latent]."""
    return np.concatenate([C @ w_uk_h.T, KR], axis=1)


def reconstruct_values(C: np.ndarray, w_uv_h: np.ndarray) -> np.ndarray:
    """Per-head values v_t = W_UV c_t  ([DF-latent])."""
    return C @ w_uv_h.T


def query_vector(q_nope: np.ndarray, q_rope: np.ndarray) -> np.ndarray:
    """The 192-wide query [q_nope ; q_rope] matching the key layout."""
    return np.concatenate([q_nope, q_rope])


def visible_tokens(seq_len: int, q_per_seq: int, i: int) -> int:
    """Query i of the S_q newest tokens sees every earlier token and itself
    ([DF-bottleneck]); the S_q query tokens are the last ones counted in len."""
    return max(0, int(seq_len) - (q_per_seq - 1 - i))


def scores(K: np.ndarray, q: np.ndarray, softmax_scale: float) -> np.ndarray:
    """s_t = (k_t . q) * scale."""
    return (K @ q) * softmax_scale


def softmax_lse(s: np.ndarray) -> Tuple[np.ndarray, float]:
    """Textbook softmax with the max subtracted; also ln(sum exp s)."""
    if s.size == 0:
        return s.copy(), -math.inf
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    return e / z, float(m + math.log(z))


def mix_values(p: np.ndarray, V: np.ndarray) -> np.ndarray:
    """o = sum_t p_t v_t  ([DF-bottleneck]: mix the values)."""
    if p.size == 0:
        return np.zeros(V.shape[1])
    return p @ V


def default_softmax_scale() -> float:
    return 1.0 / math.sqrt(D_HEAD + D_ROPE)


def _weights(inp):
    d = _decoder(inp.wl.w_dtype)
    return d, d


def _selection(inp, select: Optional[Iterable[Tuple[int, int, int]]]):
    """{b: {h: [i...]}} for the requested (b, i, h) rows, default all."""
    B, Sq, H = inp.wl.batch, inp.wl.q_per_seq, inp.wl.heads
    want = {}
    if select is None:
        for b in range(B):
            want[b] = {h: list(range(Sq)) for h in range(H)}
    else:
        for b, i, h in select:
            want.setdefault(int(b), {}).setdefault(int(h), []).append(int(i))
    return want


def explicit_decode(inp, select=None, softmax_scale: Optional[float] = None):
    """The definition: rebuild every head's keys and values from the latent
    cache and run softmax attention ([DF-latent], [DF-bottleneck]).

    Returns (o [B*S_q][H][128], lse [B*S_q][H]) in fp64; rows that were not
    selected are NaN."""
    wl = inp.wl
    B, Sq, H = wl.batch, wl.q_per_seq, wl.heads
    scale = inp.softmax_scale if softmax_scale is None else softmax_scale
    dq = _decoder(wl.q_dtype)
    dw = _decoder(wl.w_dtype)
    o = np.full((B * Sq, H, D_HEAD), np.nan)
    lse = np.full((B * Sq, H), np.nan)
    for b, heads in _selection(inp, select).items():
        C, KR = gather_sequence(inp, b)
        for h, rows in heads.items():
            K = reconstruct_keys(C, KR, dw(inp.w_uk[h]))
            V = reconstruct_values(C, dw(inp.w_uv[h]))
            for i in rows:
                r = b * Sq + i
                n = visible_tokens(inp.seq_lens[b], Sq, i)
                q = query_vector(dq(inp.q_nope[r, h]), dq(inp.q_rope[r, h]))
                p, l = softmax_lse(scores(K[:n], q, scale))
                o[r, h] = mix_values(p, V[:n])
                lse[r, h] = l
    return o, lse


def absorbed_decode(inp, select=None, softmax_scale: Optional[float] = None):
    """The absorbed form, written separately ([DF-latent] "absorption"):
    q_lat = W_UK^T q_nope, s_t = (q_lat . c_t + q_rope . k^R_t) * scale,
    o_lat = sum_t p_t c_t, o = W_UV o_lat.

    Returns (q_lat, o_lat, lse, o), fp64, NaN for unselected rows."""
    wl = inp.wl
    B, Sq, H = wl.batch, wl.q_per_seq, wl.heads
    scale = inp.softmax_scale if softmax_scale is None else softmax_scale
    dq = _decoder(wl.q_dtype)
    dw = _decoder(wl.w_dtype)
    q_lat = np.full((B * Sq, H, D_LATENT), np.nan)
    o_lat = np.full((B * Sq, H, D_LATENT), np.nan)
    o = np.full((B * Sq, H, D_HEAD), np.nan)
    lse = np.full((B * Sq, H), np.nan)
    for b, heads in _selection(inp, select).items():
        C, KR = gather_sequence(inp, b)
        for h, rows in heads.items():
            w_uk, w_uv = dw(inp.w_uk[h]), dw(inp.w_uv[h])
            for i in rows:
                r = b * Sq + i
                n = visible_tokens(inp.seq_lens[b], Sq, i)
                ql = w_uk.T @ dq(inp.q_nope[r, h])
                s = (C[:n] @ ql + KR[:n] @ dq(inp.q_rope[r, h])) * scale
                p, l = softmax_lse(s)
                ol = mix_values(p, C[:n])
                q_lat[r, h], o_lat[r, h], lse[r, h] = ql, ol, l
                o[r, h] = w_uv @ ol
    return q_lat, o_lat, lse, o


def absorbed_decode_batched(inp, softmax_scale: Optional[float] = None, batches: Optional[Iterable[int]] = None):
    """The absorbed form again, with every (query token, head) row of one
    sequence in a single matrix product.  All heads read the same cached rows
    ([DF-latent]: one c_t and one k^R_t per token), so the scores of the
    sequence are the [len x S_q*H] product [C | K^R] [q_lat | q_rope]^T times
    the scale; column (i, h) keeps its first len - (S_q - 1 - i) tokens; the
    softmax runs down each column (max subtracted); o_lat = P^T C and
    o[i][h] = W_UV[h] o_lat[i][h].  No blocking along the tokens.  It gives
    every output of a full-size workload in seconds, so that a whole output
    can be compared element by element.

    Returns (o_lat [B*S_q][H][512], lse [B*S_q][H], o [B*S_q][H][128]) in
    fp64; a column that sees no token gets o_lat = o = 0 and lse = -inf.  With
    `batches`, only those sequences are computed (the other rows are NaN)."""
    wl = inp.wl
    B, Sq, H = wl.batch, wl.q_per_seq, wl.heads
    scale = inp.softmax_scale if softmax_scale is None else softmax_scale
    dq = _decoder(wl.q_dtype)
    dw = _decoder(wl.w_dtype)
    w_uk = dw(inp.w_uk)                         # [H][128][512]
    w_uv_t = dw(inp.w_uv).transpose(0, 2, 1)    # [H][512][128]
    o_lat = np.full((B * Sq, H, D_LATENT), np.nan)
    o = np.full((B * Sq, H, D_HEAD), np.nan)
    lse = np.full((B * Sq, H), np.nan)
    for b in (range(B) if batches is None else batches):
        C, KR = gather_sequence(inp, b)
        n = C.shape[0]
        r0 = b * Sq
        # q_lat[i][h] = W_UK[h]^T q_nope[i][h], as a batch over heads
        qn = dq(inp.q_nope[r0:r0 + Sq]).transpose(1, 0, 2)          # [H][Sq][128]
        ql = np.matmul(qn, w_uk).transpose(1, 0, 2).reshape(Sq * H, D_LATENT)
        qr = dq(inp.q_rope[r0:r0 + Sq]).reshape(Sq * H, D_ROPE)
        S = (C @ ql.T + KR @ qr.T) * scale                           # [n][Sq*H], column i*H + h
        vis = np.repeat([visible_tokens(n, Sq, i) for i in range(Sq)], H)
        S[np.arange(n)[:, None] >= vis[None, :]] = -np.inf
        seen = vis > 0
        m = np.where(seen, S.max(axis=0, initial=-np.inf), 0.0)
        E = np.exp(S - m)
        z = E.sum(axis=0)
        P = E / np.where(seen, z, 1.0)
        ol = P.T @ C                                                 # [Sq*H][512]
        o_lat[r0:r0 + Sq] = ol.reshape(Sq, H, D_LATENT)
        lse[r0:r0 + Sq] = np.where(seen, m + np.log(np.where(seen, z, 1.0)), -np.inf).reshape(Sq, H)
        oo = np.matmul(ol.reshape(Sq, H, D_LATENT).transpose(1, 0, 2), w_uv_t)  # [H][Sq][128]
        o[r0:r0 + Sq] = oo.transpose(1, 0, 2)
    return o_lat, lse, o


def absorb_queries(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """Query-side absorption ([DF-latent]): q_lat[r][h] = W_UK[h]^T q_nope[r][h],
    so that q_lat . c_t equals q_nope . (W_UK c_t), the score against the
    rebuilt key.  q_nope [R][H][128], w_uk [H][128][512], fp64 -> [R][H][512]."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    out = np.empty((q_nope.shape[0], q_nope.shape[1], w_uk.shape[2]))
    for h in range(q_nope.shape[1]):
        out[:, h] = q_nope[:, h] @ w_uk[h]
    return out


def project_output(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Output-side absorption ([DF-latent]): o[r][h] = W_UV[h] o_lat[r][h];
    for o_lat = sum_t p_t c_t this is sum_t p_t (W_UV c_t), the mix of rebuilt
    values.  o_lat [R][H][512], w_uv [H][128][512], fp64 -> [R][H][128]."""
    o_lat = np.asarray(o_lat, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    out = np.empty((o_lat.shape[0], o_lat.shape[1], w_uv.shape[1]))
    for h in range(o_lat.shape[1]):
        out[:, h] = o_lat[:, h] @ w_uv[h].T
    return out


# ----------------------------------------------------------------------------
# split-KV and its log-sum-exp merge
# ----------------------------------------------------------------------------

def split_ranges(seq_len: int, num_splits: int, block: int = 64):
    """Cut a sequence's pages into num_splits page-aligned chunks of
    ceil(pages / num_splits) pages each; trailing chunks may be empty."""
    pages = -(-int(seq_len) // block)
    per = -(-pages // num_splits) if pages else 0
    out = []
    for s in range(num_splits):
        lo = min(s * per * block, seq_len)
        hi = min((s + 1) * per * block, seq_len)
        out.append((lo, hi))
    return out


def split_partials(inp, num_splits: int, select=None, softmax_scale=None):
    """Per chunk: normalised latent output and log-sum-exp over that chunk's
    visible tokens; an empty chunk gives zeros and -inf.

    Returns (o_part [B][ns][S_q][H][512], lse_part [B][ns][S_q][H])."""
    wl = inp.wl
    B, Sq, H = wl.batch, wl.q_per_seq, wl.heads
    scale = inp.softmax_scale if softmax_scale is None else softmax_scale
    dq = _decoder(wl.q_dtype)
    dw = _decoder(wl.w_dtype)
    o_part = np.full((B, num_splits, Sq, H, D_LATENT), np.nan)
    lse_part = np.full((B, num_splits, Sq, H), np.nan)
    for b, heads in _selection(inp, select).items():
        C, KR = gather_sequence(inp, b)
        ranges = split_ranges(inp.seq_lens[b], num_splits, inp.latent.shape[1])
        for h, rows in heads.items():
            w_uk = dw(inp.w_uk[h])
            for i in rows:
                r = b * Sq + i
                n = visible_tokens(inp.seq_lens[b], Sq, i)
                ql = w_uk.T @ dq(inp.q_nope[r, h])
                s_all = (C[:n] @ ql + KR[:n] @ dq(inp.q_rope[r, h])) * scale
                for sidx, (lo, hi) in enumerate(ranges):
                    hi = min(hi, n)
                    lo = min(lo, hi)
                    p, l = softmax_lse(s_all[lo:hi])
                    o_part[b, sidx, i, h] = mix_values(p, C[lo:hi])
                    lse_part[b, sidx, i, h] = l
    return o_part, lse_part


def combine_partials(o_part: np.ndarray, lse_part: np.ndarray):
    """Merge chunk results: lse = ln sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s.
    Chunks with lse = -inf carry weight 0; if every chunk is empty the result
    is o = 0, lse = -inf.  The split axis is axis 1 of o_part [B][ns][...][d]."""
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    m = lse_part.max(axis=1, keepdims=True)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_part), np.exp(lse_part - m_safe), 0.0)
    z = w.sum(axis=1, keepdims=True)
    lse = np.where(finite, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)[:, 0]
    wn = np.where(z > 0, w / np.where(z > 0, z, 1.0), 0.0)
    o = (wn[..., None] * np.where(wn[..., None] > 0, o_part, 0.0)).sum(axis=1)
    return o, lse


# ----------------------------------------------------------------------------
# cache accounting ([DF-bottleneck], [DF-snippet], [CA-takeaways])
# ----------------------------------------------------------------------------

def cache_numbers_per_token_layer(scheme: str, *, heads: int = 0, d_head: int = 0,
                                  groups: float = 0, d_latent: int = 0, d_rope: int = 0) -> float:
    """Numbers cached per token per layer.  MHA: a key and a value of width
    d_head for each head; GQA: the same per group; MLA: the latent plus the
    decoupled RoPE key."""
    if scheme == "mha":
        return 2 * heads * d_head
    if scheme == "gqa":
        return 2 * groups * d_head
    if scheme == "mla":
        return d_latent + d_rope
    raise ValueError(scheme)


def cache_bytes(numbers_per_token_layer: float, layers: int, context: int, bytes_per: int = 2):
    """Whole-cache bytes for one sequence."""
    return numbers_per_token_layer * layers * context * bytes_per


# ----------------------------------------------------------------------------
# cache append ([DF-latent]: c_t = W_DKV h_t, and a separate 64-wide key that
# carries the position)
# ----------------------------------------------------------------------------

def down_project(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Rows of h times W^T in fp64: c[r][n] = sum_k w[n][k] h[r][k]
    (c_t = W_DKV h_t for each token; the same map gives W_KR h_t)."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def rope_angles(pos: int, theta: float = 10000.0, d: int = D_ROPE) -> np.ndarray:
    """Rotation angle of each pair (2j, 2j+1) of a d-wide key at position pos:
    pos * theta^(-2j/d)."""
    j = np.arange(d // 2, dtype=np.float64)
    return float(pos) * np.power(float(theta), -2.0 * j / d)


def rope_rotate(x: np.ndarray, pos: int, theta: float = 10000.0) -> np.ndarray:
    """Turn each pair (x[2j], x[2j+1]) of the last axis by its angle at pos."""
    x = np.asarray(x, dtype=np.float64)
    a = rope_angles(pos, theta, x.shape[-1])
    c, s = np.cos(a), np.sin(a)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def e4m3_values() -> np.ndarray:
    """Values of the finite non-negative OCP E4M3FN codes 0x00 .. 0x7E (the
    decoding definition above applied to each code)."""
    return decode_e4m3(np.arange(0x7F, dtype=np.uint8))


def e4m3_round_codes(x: np.ndarray) -> np.ndarray:
    """E4M3FN code bytes of finite values with |x| <= 448: the nearest code
    value by exhaustive comparison, a tie going to the even code; the sign
    goes to bit 7 (also for zero, from the sign bit)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x).reshape(-1)
    vals = e4m3_values()
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes (at most two, adjacent) take the even one
    even = cand & (np.arange(vals.size)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1)).astype(np.uint8)
    return np.where(np.signbit(x.reshape(-1)), pick | np.uint8(0x80), pick).reshape(x.shape)


def quantize_latent(c: np.ndarray):
    """One token's fp8 cache row, the decisions taken in float32 as the
    encoder that writes the cache takes them: s = max|c| / 448 (1 for an
    all-zero c), q = c / s clamped to +-448, codes = E4M3 of q.
    Returns (codes uint8, s float32)."""
    c = np.asarray(c, dtype=np.float32)
    amax = np.float32(np.abs(c).max())
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    q = np.clip(c / s, np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    return e4m3_round_codes(q.astype(np.float64)), s


def appended_tokens(h: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray, seq_lens, q_per_seq: int,
                    theta: float = 10000.0):
    """The rows the append writes: for token i of sequence b (row b*S_q + i of
    h) at position p = len_b - S_q + i >= 0, c = W_DKV h and
    k^R = RoPE_p(W_KR h) in fp64.  Returns a list of (b, p, c, k^R)."""
    out = []
    c_all = down_project(h, w_dkv)
    k_all = down_project(h, w_kr)
    for b, ln in enumerate(np.asarray(seq_lens)):
        for i in range(q_per_seq):
            p = int(ln) - q_per_seq + i
            if p < 0:
                continue
            r = b * q_per_seq + i
            out.append((b, p, c_all[r], rope_rotate(k_all[r], p, theta)))
    return out



# ----------------------------------------------------------------------------
# MoE gate ([DF-moe]: s_i = softmax_i(u^T e_i); g_i = s_i for the K_r largest
# s_i, else 0)
# ----------------------------------------------------------------------------

def expert_affinities(u: np.ndarray, e: np.ndarray) -> np.ndarray:
    """u^T e_i for every token (rows of u) and every expert centroid (rows of
    e), in fp64: a [tokens x experts] array."""
    return np.asarray(u, dtype=np.float64) @ np.asarray(e, dtype=np.float64).T


def gate_softmax(a: np.ndarray) -> np.ndarray:
    """s_i = exp(a_i) / sum_j exp(a_j) over the last axis (the largest
    affinity subtracted first, which leaves the quotient unchanged)."""
    a = np.asarray(a, dtype=np.float64)
    z = np.exp(a - a.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def top_k(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of each row, largest first; of equal
    entries the lower index comes first (a stable sort of -s)."""
    s = np.asarray(s, dtype=np.float64)
    return np.argsort(-s, axis=-1, kind="stable")[..., :k]


def moe_gate(u: np.ndarray, e: np.ndarray, k: int):
    """The routed gate of each token: (idx [tokens x k] int64, the kept
    experts by decreasing score; g [tokens x k], their gate values g_i = s_i;
    s [tokens x experts], every score)."""
    s = gate_softmax(expert_affinities(u, e))
    idx = top_k(s, k)
    return idx, np.take_along_axis(s, idx, axis=-1), s


def gate_dense(u: np.ndarray, e: np.ndarray, k: int) -> np.ndarray:
    """g over all experts as the formula writes it: s_i where expert i is
    among the k kept, 0 elsewhere ([tokens x experts])."""
    idx, g, s = moe_gate(u, e, k)
    out = np.zeros_like(s)
    np.put_along_axis(out, idx, g, axis=-1)
    return out
