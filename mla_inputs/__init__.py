"""Seeded synthetic workloads for MLA absorbed decode.

This module only *makes inputs*: shapes, random draws, storage encodings
(bf16 round-to-nearest-even, OCP E4M3FN with a per-token scale), the paged
block pool with its page table, and NaN poison in memory that no output may
read.  It performs none of the attention arithmetic, so both the CPU oracle
and the HIP path can use it without sharing any of the method.

Shapes follow the DeepSeek-V2 explainer (deepforge "DeepSeek-V2", section 1,
"Store a latent, rebuild the keys and values"): per token per layer the cache
holds a 512-wide latent c_t plus a 64-wide decoupled RoPE key k^R_t; heads are
128 wide.  The five workloads below are the synthetic configurations the
library is measured on; their value distributions are stated in each docstring
field.

Storage formats (all little-endian, row-major):

* ``f32``  : latent pool  float32 [num_blocks][block][576]  (c | k^R interleaved)
* ``bf16`` : latent pool  uint16  [num_blocks][block][576]  (bf16 bit patterns)
* ``fp8``  : c8  uint8 [num_blocks][block][512] (E4M3FN codes),
             kR  uint16 [num_blocks][block][64] (bf16), scale float32 [num_blocks][block]

Draw order for a seed (numpy ``default_rng(seed)``): lengths (ragged only),
block permutation (paged only), c, k^R, q_nope, q_rope, W_UK, W_UV.  c and
k^R are drawn for every pool row (spare blocks and page tails included) and
then overwritten with NaN where no sequence owns the row.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_HEAD = 128
BLOCK = 64
ROW = D_LATENT + D_ROPE  # 576 numbers per token per layer

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_per_seq: int
    heads: int
    cache_dtype: str                 # "f32" | "bf16" | "fp8"
    seq_len: Optional[int] = None    # uniform context length
    len_range: Optional[Tuple[int, int]] = None  # inclusive uniform draw
    paged: bool = False              # permuted shared block pool
    spare_blocks: int = 0            # NaN-poisoned blocks no sequence owns
    num_splits: int = 1              # KV splits the workload prescribes (0 = launcher's choice)
    seed: int = 0
    weight_std: float = 1.0 / math.sqrt(D_LATENT)
    lens: Optional[Tuple[int, ...]] = None  # explicit per-sequence lengths (edge cases)

    @property
    def q_dtype(self) -> str:
        return "f32" if self.cache_dtype == "f32" else "bf16"

    @property
    def w_dtype(self) -> str:
        return "f32" if self.cache_dtype == "f32" else "bf16"

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five measured configurations.  Seeds are 1000 + position.
WORKLOADS = {
    # fp32 everywhere; B=1, H=16, T=1024, contiguous.
    "fp32_b1_h16_t1k": Workload("fp32_b1_h16_t1k", batch=1, q_per_seq=1, heads=16,
                                cache_dtype="f32", seq_len=1024, num_splits=0, seed=1000),
    # DeepSeek-V2 head shape, bf16 cache/q/weights; B=32, T=4096, contiguous.
    "bf16_b32_h128_t4k": Workload("bf16_b32_h128_t4k", batch=32, q_per_seq=1, heads=128,
                                  cache_dtype="bf16", seq_len=4096, num_splits=0, seed=1001),
    # Paged ragged batch: B=64, lengths ~ U[512, 16384], permuted shared pool.
    "bf16_paged_b64_ragged": Workload("bf16_paged_b64_ragged", batch=64, q_per_seq=1, heads=128,
                                      cache_dtype="bf16", len_range=(512, 16384), paged=True,
                                      spare_blocks=64, num_splits=0, seed=1002),
    # Long context: B=1, T=131072 split into 64 chunks, paged permuted.
    "bf16_long_t128k_s64": Workload("bf16_long_t128k_s64", batch=1, q_per_seq=1, heads=128,
                                    cache_dtype="bf16", seq_len=131072, paged=True,
                                    spare_blocks=64, num_splits=64, seed=1003),
    # fp8 E4M3 latent + fp32 per-token scale, bf16 k^R; B=128, T=8192, 2 causal query tokens.
    "fp8_b128_t8k_sq2": Workload("fp8_b128_t8k_sq2", batch=128, q_per_seq=2, heads=128,
                                 cache_dtype="fp8", seq_len=8192, paged=True,
                                 spare_blocks=64, num_splits=0, seed=1004),
}
WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "bf16_b32_h128_t4k"


def small_variants():
    """Reduced copies of each workload that the fp64 oracle finishes in
    seconds: several 64-token pages, ragged tails, every dtype and S_q."""
    w = WORKLOADS
    return {
        "fp32_b1_h16_t1k": w["fp32_b1_h16_t1k"],
        "bf16_small_contig": w["bf16_b32_h128_t4k"].scaled(
            name="bf16_small_contig", batch=3, seq_len=300, num_splits=1, seed=2001),
        "bf16_small_paged": w["bf16_paged_b64_ragged"].scaled(
            name="bf16_small_paged", batch=5, len_range=(1, 700), spare_blocks=5,
            num_splits=1, seed=2002),
        "bf16_small_split": w["bf16_long_t128k_s64"].scaled(
            name="bf16_small_split", seq_len=2500, spare_blocks=3, num_splits=7, seed=2003),
        "fp8_small_sq2": w["fp8_b128_t8k_sq2"].scaled(
            name="fp8_small_sq2", batch=3, len_range=(2, 333), spare_blocks=2,
            num_splits=1, seed=2004),
    }


# ----------------------------------------------------------------------------
# storage encodings
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray, chunk: int = 1 << 22) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the
    16-bit patterns.  Inputs here are finite draws, so no NaN handling.
    Works in chunks so the 32-bit temporaries stay small."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).reshape(-1)
    out = np.empty(u.shape, dtype=np.uint16)
    for lo in range(0, u.size, chunk):
        v = u[lo: lo + chunk]
        r = (v >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += v
        r >>= np.uint32(16)
        out[lo: lo + chunk] = r
    return out.reshape(np.shape(x))


def _e4m3_positive_table() -> np.ndarray:
    """Values of the 127 finite non-negative OCP E4M3FN codes 0x00..0x7E,
    from the format's definition: bias 7, 3 mantissa bits, subnormals at
    exponent field 0, code 0x7F is NaN, no infinities."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


_E4M3_POS = _e4m3_positive_table()
# midpoints of neighbouring codes have at most 5 significant bits: exact in float32
_E4M3_MID = ((_E4M3_POS[:-1] + _E4M3_POS[1:]) / 2.0).astype(np.float32)


def e4m3_codes_by_table(x: np.ndarray) -> np.ndarray:
    """Encode finite float32 values as OCP E4M3FN bytes by search among the
    127 finite code values: nearest, ties to the even code, saturating at
    +-448.  Slow; kept as the definition the fast encoder is checked against."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    v = x.reshape(-1)
    n_mid = _E4M3_MID.size
    a = np.minimum(np.abs(v), np.float32(E4M3_MAX))
    idx = np.searchsorted(_E4M3_MID, a, side="left")
    hit = np.minimum(idx, n_mid - 1)
    tie = (idx < n_mid) & (a == _E4M3_MID[hit])
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx).astype(np.uint8)
    return np.where(np.signbit(v), idx | np.uint8(0x80), idx).reshape(x.shape)


def e4m3_codes(x: np.ndarray, chunk: int = 1 << 22) -> np.ndarray:
    """Encode finite float32 values as OCP E4M3FN bytes, round to nearest with
    ties to the even code, saturating at +-448.  Normal range: the float32
    pattern rounded to 3 mantissa bits (nearest-even on the bits, a carry
    moves into the exponent as it should) and re-biased from 127 to 7;
    below 2^-6 the code is the nearest-even multiple of 2^-9.  Identical to
    ``e4m3_codes_by_table``; works in chunks."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for lo in range(0, flat.size, chunk):
        v = flat[lo: lo + chunk]
        a = np.minimum(np.abs(v), np.float32(E4M3_MAX))
        u = a.view(np.uint32)
        r = (u >> np.uint32(20)) & np.uint32(1)
        r += np.uint32(0x7FFFF)
        r += u
        r >>= np.uint32(20)
        normal = a >= np.float32(2.0 ** -6)
        code = np.where(normal, r.astype(np.int64) - (120 << 3),
                        np.rint(a * np.float32(512.0)).astype(np.int64)).astype(np.uint8)
        out[lo: lo + chunk] = np.where(np.signbit(v), code | np.uint8(0x80), code)
    return out.reshape(x.shape)


# ----------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    wl: Workload
    seq_lens: np.ndarray          # int32 [B]   cached tokens incl. the S_q query tokens
    block_table: np.ndarray       # int32 [B][max_blocks]
    num_blocks: int
    # cache storage (see module docstring)
    latent: np.ndarray            # f32/bf16: pool [nb][64][576]; fp8: c8 [nb][64][512]
    rope: Optional[np.ndarray]    # fp8 only: bf16 [nb][64][64]; else None (interleaved)
    scale: Optional[np.ndarray]   # fp8 only: float32 [nb][64]
    q_nope: np.ndarray            # [B*S_q][H][128]   f32 or bf16 bits
    q_rope: np.ndarray            # [B*S_q][H][64]
    w_uk: np.ndarray              # [H][128][512]
    w_uv: np.ndarray              # [H][128][512]
    softmax_scale: float

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def kv_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x)
    raise ValueError(dtype)


def draw_lengths(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    """Per-sequence cached-token counts.  A length below q_per_seq is legal:
    the queries that see no token give o = 0 and lse = -inf."""
    if wl.lens is not None:
        lens = np.asarray(wl.lens)
        if lens.size != wl.batch:
            raise ValueError("lens must give one length per sequence")
    elif wl.len_range is not None:
        lo, hi = wl.len_range
        lens = rng.integers(lo, hi + 1, size=wl.batch)
    else:
        lens = np.full(wl.batch, wl.seq_len)
    if (lens < 0).any():
        raise ValueError("negative sequence length")
    return lens.astype(np.int32)


def generate(wl: Workload, seed: Optional[int] = None, poison: bool = True) -> Inputs:
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, Sq, H = wl.batch, wl.q_per_seq, wl.heads
    lens = draw_lengths(wl, rng)
    pages = (lens.astype(np.int64) + BLOCK - 1) // BLOCK
    max_blocks = max(1, int(pages.max(initial=0)))
    used = int(pages.sum())
    nb = used + wl.spare_blocks
    if (pages == 0).any() and wl.spare_blocks < 1:
        raise ValueError("an empty sequence needs a spare block for its page-table row")
    if wl.paged:
        perm = rng.permutation(nb).astype(np.int32)
    else:
        perm = np.arange(nb, dtype=np.int32)
    table = np.zeros((B, max_blocks), dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, : pages[b]] = perm[off: off + pages[b]]
        # entries past the sequence's last page name a poisoned spare block
        # (or, without spares, the sequence's first block): no kernel may read them
        table[b, pages[b]:] = perm[used] if wl.spare_blocks > 0 else perm[off]
        off += pages[b]
    owned = np.zeros((nb, BLOCK), dtype=bool)
    for b in range(B):
        for j in range(pages[b]):
            rows = min(BLOCK, int(lens[b]) - j * BLOCK)
            owned[table[b, j], :rows] = True

    # Draw order: every block's c, then every block's k^R, then q_nope, q_rope,
    # W_UK, W_UV.  The cache is drawn and encoded a few blocks at a time (the
    # generator's stream does not depend on how a draw is cut into calls).
    step = max(1, (1 << 22) // (BLOCK * D_LATENT))
    scale = None
    rope = None
    if wl.cache_dtype == "fp8":
        latent = np.empty((nb, BLOCK, D_LATENT), dtype=np.uint8)
        scale = np.empty((nb, BLOCK), dtype=np.float32)
        for lo in range(0, nb, step):
            n = min(step, nb - lo)
            c = rng.standard_normal((n, BLOCK, D_LATENT), dtype=np.float32)
            sc = (np.abs(c).max(axis=2) / np.float32(E4M3_MAX)).astype(np.float32)
            safe = np.where(sc > 0, sc, np.float32(1.0))
            latent[lo: lo + n] = e4m3_codes(c / safe[..., None])
            scale[lo: lo + n] = sc
        rope = np.empty((nb, BLOCK, D_ROPE), dtype=np.uint16)
        for lo in range(0, nb, step):
            n = min(step, nb - lo)
            rope[lo: lo + n] = bf16_bits(rng.standard_normal((n, BLOCK, D_ROPE), dtype=np.float32))
    else:
        latent = np.empty((nb, BLOCK, ROW), dtype=np.float32 if wl.cache_dtype == "f32" else np.uint16)
        for lo in range(0, nb, step):
            n = min(step, nb - lo)
            latent[lo: lo + n, :, :D_LATENT] = _encode(
                rng.standard_normal((n, BLOCK, D_LATENT), dtype=np.float32), wl.cache_dtype)
        for lo in range(0, nb, step):
            n = min(step, nb - lo)
            latent[lo: lo + n, :, D_LATENT:] = _encode(
                rng.standard_normal((n, BLOCK, D_ROPE), dtype=np.float32), wl.cache_dtype)
    q_nope = rng.standard_normal((B * Sq, H, D_HEAD), dtype=np.float32)
    q_rope = rng.standard_normal((B * Sq, H, D_ROPE), dtype=np.float32)
    w_uk = rng.standard_normal((H, D_HEAD, D_LATENT), dtype=np.float32) * np.float32(wl.weight_std)
    w_uv = rng.standard_normal((H, D_HEAD, D_LATENT), dtype=np.float32) * np.float32(wl.weight_std)
    if poison:
        if wl.cache_dtype == "fp8":
            latent[~owned] = E4M3_NAN
            rope[~owned] = BF16_NAN
            scale[~owned] = np.float32("nan")
        else:
            latent[~owned] = np.float32("nan") if wl.cache_dtype == "f32" else BF16_NAN
    return Inputs(
        wl=wl, seq_lens=lens, block_table=table, num_blocks=nb,
        latent=latent, rope=rope, scale=scale,
        q_nope=_encode(q_nope, wl.q_dtype), q_rope=_encode(q_rope, wl.q_dtype),
        w_uk=_encode(w_uk, wl.w_dtype), w_uv=_encode(w_uv, wl.w_dtype),
        softmax_scale=1.0 / math.sqrt(D_HEAD + D_ROPE),
    )


# ----------------------------------------------------------------------------
# cache-append inputs (the step that writes the S_q new tokens of a sequence)
# ----------------------------------------------------------------------------

# Hidden width of the tokens entering the cache.  The pages do not state it;
# 5120 is DeepSeek-V2's published model width, used as the measured size
# (the append takes any multiple of 64).
APPEND_D_MODEL = 5120


@dataclasses.dataclass
class AppendInputs:
    d_model: int
    h: np.ndarray        # [B*S_q][d_model]   hidden states of the new tokens
    w_dkv: np.ndarray    # [512][d_model]     latent down-projection
    w_kr: np.ndarray     # [64][d_model]      position-key projection
    rope_theta: float


def generate_append(wl: Workload, d_model: int = APPEND_D_MODEL, seed: Optional[int] = None,
                    one_hot: bool = False) -> AppendInputs:
    """Draws h ~ N(0, 1) and both projections ~ N(0, std 1/sqrt(d_model)), so
    c and the position key come out near unit variance like the cached rows;
    encoded as the workload's weights (bf16, or fp32 for the fp32 cache).
    Draw order: h, W_DKV, W_KR, from seed + 500.  With `one_hot`, row r of h
    is instead the unit vector e_(r*7 mod d_model): each product is then a
    single weight, exact in every precision."""
    rng = np.random.default_rng((wl.seed if seed is None else seed) + 500)
    T = wl.batch * wl.q_per_seq
    h = rng.standard_normal((T, d_model), dtype=np.float32)
    std = np.float32(1.0 / math.sqrt(d_model))
    w_dkv = rng.standard_normal((D_LATENT, d_model), dtype=np.float32) * std
    w_kr = rng.standard_normal((D_ROPE, d_model), dtype=np.float32) * std
    if one_hot:
        h = np.zeros((T, d_model), dtype=np.float32)
        h[np.arange(T), (np.arange(T) * 7) % d_model] = 1.0
    return AppendInputs(d_model=d_model, h=_encode(h, wl.w_dtype), w_dkv=_encode(w_dkv, wl.w_dtype),
                        w_kr=_encode(w_kr, wl.w_dtype), rope_theta=10000.0)


GATE_EXPERTS, GATE_TOP_K = 160, 6


@dataclasses.dataclass
class GateInputs:
    u: np.ndarray   # [tokens][d_model]     hidden states entering the MoE layer
    e: np.ndarray   # [n_experts][d_model]  routed experts' centroids
    top_k: int


def generate_gate(tokens: int, d_model: int = APPEND_D_MODEL, n_experts: int = GATE_EXPERTS,
                  top_k: int = GATE_TOP_K, dtype: str = "bf16", seed: int = 0, one_hot: bool = False,
                  twins: bool = False) -> GateInputs:
    """Draws u ~ N(0, 1) and the centroids ~ N(0, std 1/sqrt(d_model)), so the
    affinities u^T e_i come out near unit variance; encoded as `dtype` (bf16
    or f32).  Draw order: u, e, from seed + 700.  With `one_hot`, row t of u
    is the unit vector e_((7t + 3) mod d_model): each affinity is then one
    centroid entry, exact in every precision.  With `twins`, centroid 2j+1
    is a copy of centroid 2j, so every affinity has an equal partner and
    every selection meets ties."""
    rng = np.random.default_rng(seed + 700)
    u = rng.standard_normal((tokens, d_model), dtype=np.float32)
    e = rng.standard_normal((n_experts, d_model), dtype=np.float32) * np.float32(1.0 / math.sqrt(d_model))
    if one_hot:
        u = np.zeros((tokens, d_model), dtype=np.float32)
        u[np.arange(tokens), (7 * np.arange(tokens) + 3) % d_model] = 1.0
    if twins:
        e[1::2] = e[0:n_experts - n_experts % 2:2]
    return GateInputs(u=_encode(u, dtype), e=_encode(e, dtype), top_k=top_k)


def depaged(inp: Inputs) -> Inputs:
    """Same logical cache, rewritten as a contiguous pool with an identity
    page table (sequence b owns blocks b*max_blocks ...).  Used to check that
    paging changes no output bit."""
    B, mb = inp.block_table.shape
    src = inp.block_table.reshape(-1)
    table = np.arange(B * mb, dtype=np.int32).reshape(B, mb)
    latent = np.ascontiguousarray(inp.latent[src])
    rope = None if inp.rope is None else np.ascontiguousarray(inp.rope[src])
    scale = None if inp.scale is None else np.ascontiguousarray(inp.scale[src])
    return dataclasses.replace(inp, block_table=table, num_blocks=B * mb,
                               latent=latent, rope=rope, scale=scale)


def cache_bytes_per_token(cache_dtype: str) -> int:
    """Bytes of one cached token as stored: 576 numbers (+ a 4-byte scale for fp8)."""
    return {"f32": ROW * 4, "bf16": ROW * 2, "fp8": D_LATENT + 4 + D_ROPE * 2}[cache_dtype]
