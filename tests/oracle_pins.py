"""Pin checks for the fp64 oracle.

Each ``check_*`` function raises AssertionError when the oracle disagrees with
something fixed outside it: a number the pages print, a closed form, a
library attention routine, brute force in exact arithmetic, or an invariant
the method guarantees.  ``test_oracle_pins.py`` runs them on the oracle as it
is; ``test_oracle_mutants.py`` plants plausible mistakes in the oracle and
requires at least one check to fail for each.
"""
from __future__ import annotations

import json
import math
import os
from types import SimpleNamespace

import numpy as np

import mla_inputs as MI

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DL, DR, DH = 512, 64, 128


def tiny_inputs(lens, heads=2, q_per_seq=1, seed=0, integer=False, block=64,
                permute=True, scale=None):
    """fp32-stored inputs of arbitrary small shape, built directly (no HIP
    code, no generator): random or small-integer values, an optionally
    permuted block pool, NaN in every row no sequence owns."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    B = lens.size
    pages = [max(1, -(-int(n) // block)) for n in lens]
    nb = sum(pages) + 1
    order = rng.permutation(nb) if permute else np.arange(nb)
    mb = max(pages)
    table = np.zeros((B, mb), dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :pages[b]] = order[off:off + pages[b]]
        table[b, pages[b]:] = order[-1]
        off += pages[b]
    draw = (lambda *s: rng.integers(-3, 4, size=s).astype(np.float32)) if integer else \
           (lambda *s: rng.standard_normal(s).astype(np.float32))
    latent = draw(nb, block, DL + DR)
    owned = np.zeros((nb, block), dtype=bool)
    for b in range(B):
        for t in range(int(lens[b])):
            owned[table[b, t // block], t % block] = True
    latent[~owned] = np.nan
    wscale = 1.0 if integer else 1.0 / math.sqrt(DL)
    wl = SimpleNamespace(batch=B, q_per_seq=q_per_seq, heads=heads, cache_dtype="f32",
                         q_dtype="f32", w_dtype="f32")
    return SimpleNamespace(
        wl=wl, seq_lens=lens, block_table=table, num_blocks=nb, latent=latent,
        rope=None, scale=None,
        q_nope=draw(B * q_per_seq, heads, DH), q_rope=draw(B * q_per_seq, heads, DR),
        w_uk=(draw(heads, DH, DL) * np.float32(wscale)).astype(np.float32),
        w_uv=(draw(heads, DH, DL) * np.float32(wscale)).astype(np.float32),
        softmax_scale=(1.0 / math.sqrt(DH + DR)) if scale is None else scale,
    )


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


# ----------------------------------------------------------------------------
# numbers the pages print
# ----------------------------------------------------------------------------

def check_cache_arithmetic():
    g = json.load(open(os.path.join(GOLDEN, "cache_arithmetic.json")))
    e = g["mha_numbers_per_token_60L_128H_128d"]
    per_layer = O.cache_numbers_per_token_layer("mha", heads=e["inputs"]["heads"],
                                                d_head=e["inputs"]["d_head"])
    total = per_layer * e["inputs"]["layers"]
    assert f"{total / 1e6:.2f}M" == e["value_printed"], total
    e = g["mla_numbers_per_token_layer"]
    assert O.cache_numbers_per_token_layer("mla", **e["inputs"]) == e["value_printed"]
    e = g["mha_numbers_per_token_layer_128H_128d"]
    assert O.cache_numbers_per_token_layer("mha", **e["inputs"]) == e["value_printed"]
    e = g["gqa_equivalent_groups"]
    mla = O.cache_numbers_per_token_layer("mla", d_latent=512, d_rope=64)
    assert O.cache_numbers_per_token_layer("gqa", groups=e["value_printed"],
                                           d_head=e["inputs"]["d_head"]) == mla
    e = g["dense_over_mla_bytes_integer_ratio"]
    i = e["inputs"]
    dense = O.cache_bytes(O.cache_numbers_per_token_layer("mha", heads=i["heads"], d_head=i["d_head"]),
                          i["layers"], i["context"], i["bytes_per"])
    mla = O.cache_bytes(O.cache_numbers_per_token_layer("mla", d_latent=i["d_latent"], d_rope=i["d_rope"]),
                        i["layers"], i["context"], i["bytes_per"])
    assert int(dense) // int(mla) == e["value_printed"]


# ----------------------------------------------------------------------------
# storage decoding vs the library's own casts
# ----------------------------------------------------------------------------

def check_decode_tables():
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_bf16(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


# ----------------------------------------------------------------------------
# softmax
# ----------------------------------------------------------------------------

def check_softmax():
    rng = np.random.default_rng(1)
    for n in (1, 2, 7, 1000):
        s = rng.standard_normal(n) * 5
        p, lse = O.softmax_lse(s)
        assert abs(p.sum() - 1.0) <= 1e-12
        assert (p >= 0).all()
        p2, lse2 = O.softmax_lse(s + 123.25)
        assert np.max(np.abs(p2 - p)) <= 1e-12
        assert abs((lse2 - 123.25) - lse) <= 1e-9
        assert abs(lse - math.log(math.fsum(math.exp(x) for x in s))) <= 1e-9
    p, lse = O.softmax_lse(np.array([0.0, math.log(3.0)]))
    assert abs(p[0] - 0.25) <= 1e-15 and abs(p[1] - 0.75) <= 1e-15
    assert abs(lse - math.log(4.0)) <= 1e-15


# ----------------------------------------------------------------------------
# reduction to a library attention routine
# ----------------------------------------------------------------------------

def check_textbook_reduction():
    """With W_UK = [I_128 | 0] the reconstructed key of token t is
    [c_t[:128] ; k^R_t]; MLA decode is then ordinary single-query softmax
    attention, which torch's scaled_dot_product_attention computes (CPU, fp64)."""
    import torch
    import torch.nn.functional as F
    inp = tiny_inputs([37, 130], heads=3, seed=5)
    wuk = np.zeros((DH, DL), dtype=np.float32)
    wuk[:, :DH] = np.eye(DH, dtype=np.float32)
    inp.w_uk = np.stack([wuk] * 3)
    o, lse = O.explicit_decode(inp)
    q_lat, o_lat, lse_a, o_a = O.absorbed_decode(inp)
    for b in range(2):
        n = int(inp.seq_lens[b])
        t = np.arange(n)
        rows = inp.latent[inp.block_table[b][t // 64], t % 64].astype(np.float64)
        for h in range(3):
            k = np.concatenate([rows[:, :DH], rows[:, DL:]], axis=1)
            v = rows[:, :DL] @ inp.w_uv[h].astype(np.float64).T
            q = np.concatenate([inp.q_nope[b, h], inp.q_rope[b, h]]).astype(np.float64)
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(q)[None, None, None], torch.from_numpy(k)[None, None],
                torch.from_numpy(v)[None, None], scale=1.0 / math.sqrt(192)).numpy()[0, 0, 0]
            assert np.max(np.abs(o[b, h] - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())
            assert np.max(np.abs(o_a[b, h] - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())
            s = (k @ q) / math.sqrt(192)
            ref_lse = float(torch.logsumexp(torch.from_numpy(s), 0))
            assert abs(lse[b, h] - ref_lse) <= 1e-12 and abs(lse_a[b, h] - ref_lse) <= 1e-12


# ----------------------------------------------------------------------------
# closed forms and special cases
# ----------------------------------------------------------------------------

def check_closed_forms():
    # one cached token: softmax weight 1, o = W_UV c_0, lse = s_0
    inp = tiny_inputs([1], heads=2, seed=2)
    o, lse = O.explicit_decode(inp)
    blk = inp.block_table[0, 0]
    c0 = inp.latent[blk, 0].astype(np.float64)
    for h in range(2):
        assert np.max(np.abs(o[0, h] - inp.w_uv[h].astype(np.float64) @ c0[:DL])) <= 1e-12
        k = np.concatenate([inp.w_uk[h].astype(np.float64) @ c0[:DL], c0[DL:]])
        q = np.concatenate([inp.q_nope[0, h], inp.q_rope[0, h]]).astype(np.float64)
        assert abs(lse[0, h] - (k @ q) / math.sqrt(192)) <= 1e-12
    # zero query: uniform weights, o = W_UV mean(c), lse = ln(len)
    inp = tiny_inputs([150], heads=2, seed=3)
    inp.q_nope[:] = 0
    inp.q_rope[:] = 0
    o, lse = O.explicit_decode(inp)
    t = np.arange(150)
    C = inp.latent[inp.block_table[0][t // 64], t % 64, :DL].astype(np.float64)
    for h in range(2):
        assert np.max(np.abs(o[0, h] - inp.w_uv[h].astype(np.float64) @ C.mean(axis=0))) <= 1e-12
        assert abs(lse[0, h] - math.log(150)) <= 1e-12
    # two tokens: p_0 = 1 / (1 + exp(s_1 - s_0))
    inp = tiny_inputs([2], heads=1, seed=4)
    o, lse = O.explicit_decode(inp)
    rows = inp.latent[inp.block_table[0, 0], :2].astype(np.float64)
    wuk, wuv = inp.w_uk[0].astype(np.float64), inp.w_uv[0].astype(np.float64)
    q = np.concatenate([inp.q_nope[0, 0], inp.q_rope[0, 0]]).astype(np.float64)
    s = [np.concatenate([wuk @ r[:DL], r[DL:]]) @ q / math.sqrt(192) for r in rows]
    p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    ref = p0 * (wuv @ rows[0, :DL]) + (1 - p0) * (wuv @ rows[1, :DL])
    assert np.max(np.abs(o[0, 0] - ref)) <= 1e-12
    # a token whose key dominates every other one takes all the weight
    inp = tiny_inputs([90], heads=1, seed=6)
    n = 90
    t = np.arange(n)
    blocks, rows_ = inp.block_table[0][t // 64], t % 64
    j = 41
    ql = inp.w_uk[0].astype(np.float64).T @ inp.q_nope[0, 0].astype(np.float64)
    inp.latent[blocks[j], rows_[j], :DL] = (60.0 * ql / np.linalg.norm(ql)).astype(np.float32)
    o, _ = O.explicit_decode(inp)
    cj = inp.latent[blocks[j], rows_[j], :DL].astype(np.float64)
    assert rel_l2(o[0, 0], inp.w_uv[0].astype(np.float64) @ cj) <= 1e-6


def check_brute_force_exact():
    """Small-integer inputs, every step written out with Python integers and
    math.fsum / math.exp, no numpy: scores are exact integers times the scale."""
    inp = tiny_inputs([3, 5], heads=2, q_per_seq=2, seed=7, integer=True)
    o, lse = O.explicit_decode(inp)
    Sq = 2
    for b in range(2):
        n_all = int(inp.seq_lens[b])
        toks = []
        for t in range(n_all):
            blk = int(inp.block_table[b][t // 64])
            toks.append([int(x) for x in inp.latent[blk, t % 64]])
        for h in range(2):
            wuk = [[int(x) for x in row] for row in inp.w_uk[h]]
            wuv = [[int(x) for x in row] for row in inp.w_uv[h]]
            keys = [[sum(wuk[d][k] * c[k] for k in range(DL)) for d in range(DH)] + c[DL:] for c in toks]
            vals = [[sum(wuv[d][k] * c[k] for k in range(DL)) for d in range(DH)] for c in toks]
            for i in range(Sq):
                r = b * Sq + i
                q = [int(x) for x in inp.q_nope[r, h]] + [int(x) for x in inp.q_rope[r, h]]
                n = n_all - (Sq - 1 - i)
                dots = [sum(kk * qq for kk, qq in zip(keys[t], q)) for t in range(n)]
                sc = 1.0 / math.sqrt(192)
                sf = [float(d) * sc for d in dots]
                m = max(sf)
                e = [math.exp(x - m) for x in sf]
                z = math.fsum(e)
                ref_o = [math.fsum(e[t] * vals[t][d] for t in range(n)) / z for d in range(DH)]
                ref_lse = m + math.log(z)
                scale_o = max(1.0, max(abs(x) for x in ref_o))
                assert max(abs(a - c) for a, c in zip(o[r, h], ref_o)) <= 1e-12 * scale_o
                assert abs(lse[r, h] - ref_lse) <= 1e-12 * max(1.0, abs(ref_lse))


# ----------------------------------------------------------------------------
# invariants the method guarantees
# ----------------------------------------------------------------------------

def check_absorbed_equals_explicit(inp, select=None, tol=1e-12):
    """Absorption is exact algebra ([DF-latent]): folding W_UK into the query
    and W_UV into the output changes nothing but rounding."""
    o, lse = O.explicit_decode(inp, select)
    _, _, lse_a, o_a = O.absorbed_decode(inp, select)
    m = ~np.isnan(lse)
    assert rel_l2(o_a[m], o[m]) <= tol, rel_l2(o_a[m], o[m])
    assert np.max(np.abs(lse_a[m] - lse[m])) <= tol * max(1.0, np.abs(lse[m]).max())


def check_batched_equals_explicit(inp, tol=1e-12):
    """The batched absorbed form (every head and query token of a sequence in
    one product) against the explicit definition: the same o and lse to
    rounding; rows that see no token give o = o_lat = 0 and lse = -inf in
    both."""
    o, lse = O.explicit_decode(inp)
    ol_b, lse_b, o_b = O.absorbed_decode_batched(inp)
    seen = np.isfinite(lse)
    assert np.array_equal(np.isneginf(lse_b), np.isneginf(lse))
    assert not np.isnan(o_b).any() and not np.isnan(lse_b).any()
    if seen.any():
        assert rel_l2(o_b[seen], o[seen]) <= tol, rel_l2(o_b[seen], o[seen])
        assert np.max(np.abs(lse_b[seen] - lse[seen])) <= tol * max(1.0, np.abs(lse[seen]).max())
    assert (o_b[~seen] == 0).all() and (ol_b[~seen] == 0).all()
    return ol_b


def check_batched_absorbed():
    """Batched absorbed form on paged inputs with three causal query tokens
    and three heads (so a mix-up of the query and head axes shows), a
    sequence shorter than S_q, an empty one and a page-aligned one; its
    latent output equals the per-row absorbed form's, and with one head and
    one query it reduces to the textbook softmax attention of a single row
    written out by hand."""
    inp = tiny_inputs([150, 2, 0, 64], heads=3, q_per_seq=3, seed=21)
    ol_b = check_batched_equals_explicit(inp)
    _, ol_a, lse_a, _ = O.absorbed_decode(inp)
    seen = np.isfinite(lse_a)
    assert rel_l2(ol_b[seen], ol_a[seen]) <= 1e-12
    # one row by hand: s_t = (q_lat . c_t + q_rope . k^R_t) * scale
    one = tiny_inputs([5], heads=1, q_per_seq=1, seed=22)
    ol1, lse1, o1 = O.absorbed_decode_batched(one)
    rows = one.latent[one.block_table[0, 0], :5].astype(np.float64)
    ql = one.w_uk[0].astype(np.float64).T @ one.q_nope[0, 0].astype(np.float64)
    s = [(sum(ql[j] * rows[t, j] for j in range(DL)) +
          sum(float(one.q_rope[0, 0, j]) * rows[t, DL + j] for j in range(DR))) * one.softmax_scale
         for t in range(5)]
    w = [math.exp(x - max(s)) for x in s]
    p = [x / sum(w) for x in w]
    assert abs(lse1[0, 0] - (max(s) + math.log(sum(w)))) <= 1e-12
    want = [sum(p[t] * rows[t, j] for t in range(5)) for j in range(DL)]
    assert np.max(np.abs(ol1[0, 0] - np.array(want))) <= 1e-12
    w_uv = one.w_uv[0].astype(np.float64)
    assert np.max(np.abs(o1[0, 0] - w_uv @ np.array(want))) <= 1e-12


def check_paging_invariance():
    inp = tiny_inputs([70, 200, 5], heads=2, seed=8, permute=True)
    flat = tiny_inputs([70, 200, 5], heads=2, seed=8, permute=True)
    # rebuild `flat` as the same logical cache in an identity-ordered pool
    B, mb = inp.block_table.shape
    src = inp.block_table.reshape(-1)
    flat.latent = np.ascontiguousarray(inp.latent[src])
    flat.block_table = np.arange(B * mb, dtype=np.int32).reshape(B, mb)
    a = O.explicit_decode(inp)
    b = O.explicit_decode(flat)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def check_causal_two_tokens():
    """With two query tokens, the older one sees one token fewer: it equals a
    single-query decode over the first len-1 tokens."""
    two = tiny_inputs([66, 131], heads=2, q_per_seq=2, seed=9)
    o2, l2 = O.explicit_decode(two)
    one = tiny_inputs([65, 130], heads=2, q_per_seq=1, seed=9)
    one.latent, one.block_table = two.latent, two.block_table
    one.w_uk, one.w_uv = two.w_uk, two.w_uv
    one.q_nope = np.ascontiguousarray(two.q_nope[0::2])
    one.q_rope = np.ascontiguousarray(two.q_rope[0::2])
    o1, l1 = O.explicit_decode(one)
    assert np.array_equal(o2[0::2], o1) and np.array_equal(l2[0::2], l1)
    # and the newer one sees the whole sequence
    full = tiny_inputs([66, 131], heads=2, q_per_seq=1, seed=9)
    full.latent, full.block_table = two.latent, two.block_table
    full.w_uk, full.w_uv = two.w_uk, two.w_uv
    full.q_nope = np.ascontiguousarray(two.q_nope[1::2])
    full.q_rope = np.ascontiguousarray(two.q_rope[1::2])
    of, lf = O.explicit_decode(full)
    assert np.array_equal(o2[1::2], of) and np.array_equal(l2[1::2], lf)


def check_split_combine():
    """Any page-aligned partition of the tokens, merged by log-sum-exp, equals
    the unsplit latent output (empty chunks included)."""
    inp = tiny_inputs([1, 64, 65, 300], heads=2, q_per_seq=2, seed=10)
    _, o_lat, lse, _ = O.absorbed_decode(inp)
    B, Sq, H = 4, 2, 2
    for ns in (1, 2, 3, 7):
        op, lp = O.split_partials(inp, ns)
        o, l = O.combine_partials(op, lp)
        o = o.reshape(B * Sq, H, DL)
        l = l.reshape(B * Sq, H)
        assert np.max(np.abs(o - o_lat)) <= 1e-12
        # a query that sees no token (len 1, older of two queries) has lse -inf
        assert np.array_equal(np.isneginf(l), np.isneginf(lse))
        fin = np.isfinite(lse)
        assert np.max(np.abs(l[fin] - lse[fin])) <= 1e-12
    # a chunking that cannot be page-aligned differently: each chunk alone
    assert O.split_ranges(300, 7) == [(0, 64), (64, 128), (128, 192), (192, 256),
                                      (256, 300), (300, 300), (300, 300)]
    assert O.split_ranges(300, 2) == [(0, 192), (192, 300)]
    # all-empty merge
    o, l = O.combine_partials(np.zeros((1, 3, 4)), np.full((1, 3), -np.inf))
    assert (o == 0).all() and np.isneginf(l).all()


def check_absorb_project_identities():
    """The two absorbed weight products against the rebuilt keys and values
    ([DF-latent]): q_lat . c = q_nope . (W_UK c) for every cached row c, and
    W_UV (sum_t p_t c_t) = sum_t p_t (W_UV c_t), per head; plus exact
    small-integer brute force for single elements."""
    inp = tiny_inputs([150], heads=3, seed=11)
    C, KR = O.gather_sequence(inp, 0)
    qn = inp.q_nope.astype(np.float64)
    q_lat = O.absorb_queries(qn, inp.w_uk)
    rng = np.random.default_rng(12)
    p = rng.random(C.shape[0])
    p /= p.sum()
    o_lat = np.broadcast_to(p @ C, (1, 3, DL))
    o = O.project_output(o_lat, inp.w_uv)
    for h in range(3):
        K = O.reconstruct_keys(C, KR, inp.w_uk[h].astype(np.float64))
        assert rel_l2(C @ q_lat[0, h], K[:, :DH] @ qn[0, h]) <= 1e-12
        V = O.reconstruct_values(C, inp.w_uv[h].astype(np.float64))
        assert rel_l2(o[0, h], p @ V) <= 1e-12
    # brute force, integers (exact): one element of each product
    t = tiny_inputs([3], heads=2, seed=13, integer=True)
    ql = O.absorb_queries(t.q_nope, t.w_uk)
    for h, c in ((0, 5), (1, 511)):
        assert ql[0, h, c] == sum(float(t.w_uk[h, d, c]) * float(t.q_nope[0, h, d]) for d in range(DH))
    x = np.arange(2 * DL, dtype=np.float64).reshape(1, 2, DL) % 7 - 3
    ob = O.project_output(x, t.w_uv)
    for h, d in ((0, 0), (1, 127)):
        assert ob[0, h, d] == sum(float(t.w_uv[h, d, c]) * x[0, h, c] for c in range(DL))


def check_append_projection():
    """c_t = W_DKV h_t ([DF-latent], formula box): a one-hot h picks one column
    of W exactly, and a hand-computed case."""
    rng = np.random.default_rng(21)
    w = rng.standard_normal((DL, 320))
    for k in (0, 7, 319):
        h = np.zeros((1, 320))
        h[0, k] = 1.0
        assert np.array_equal(O.down_project(h, w)[0], w[:, k])
    # [[1, 2, 3], [4, 5, 6]] times (1, -1, 2): (1 - 2 + 6, 4 - 5 + 12)
    got = O.down_project(np.array([[1.0, -1.0, 2.0]]), np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]]))
    assert np.array_equal(got, np.array([[5.0, 11.0]]))


def check_rope():
    """The position key's rotation: textbook values (pair (2j, 2j+1) turned by
    p * 10000^(-2j/64)) and the properties that define it."""
    a = O.rope_angles(1)
    assert a.shape == (32,) and a[0] == 1.0
    assert abs(a[8] - 0.1) < 1e-15 and abs(a[16] - 0.01) < 1e-15     # 10000^(-1/4), 10000^(-1/2)
    cos1, sin1 = 0.5403023058681398, 0.8414709848078965              # cos 1, sin 1
    x = np.zeros(64)
    x[0] = 1.0
    y = O.rope_rotate(x, 1)
    assert abs(y[0] - cos1) < 1e-15 and abs(y[1] - sin1) < 1e-15 and not y[2:].any()
    x = np.zeros(64)
    x[33] = 1.0                                                       # pair 16, second member
    y = O.rope_rotate(x, 100)                                         # angle 100 * 0.01 = 1
    assert abs(y[32] + sin1) < 1e-14 and abs(y[33] - cos1) < 1e-14
    assert not np.delete(y, [32, 33]).any()
    rng = np.random.default_rng(22)
    v, u = rng.standard_normal(64), rng.standard_normal(64)
    assert np.array_equal(O.rope_rotate(v, 0), v)
    r = O.rope_rotate(v, 12345)
    assert np.allclose(r[0::2] ** 2 + r[1::2] ** 2, v[0::2] ** 2 + v[1::2] ** 2, rtol=1e-12)
    assert rel_l2(O.rope_rotate(O.rope_rotate(v, 5), 7), O.rope_rotate(v, 12)) <= 1e-13
    # scores depend on the distance between positions only
    d1 = O.rope_rotate(v, 40) @ O.rope_rotate(u, 17)
    d2 = O.rope_rotate(v, 1040) @ O.rope_rotate(u, 1017)
    assert abs(d1 - d2) <= 1e-10 * max(1.0, abs(d1))


def check_e4m3_encoding():
    """Encoding to OCP E4M3FN: hand-derived codes (nearest code value, a tie
    going to the even code) and agreement with the input generator's
    bit-level encoder, a separate implementation."""
    cases = {1.0: 0x38, 1.0625: 0x38, 1.1875: 0x3A, -1.0: 0xB8, 448.0: 0x7E, 240.0: 0x77,
             0.1: 0x1D, 2.0 ** -6: 0x08, 2.0 ** -10: 0x00, 1.5 * 2.0 ** -9: 0x02, -0.0: 0x80}
    got = O.e4m3_round_codes(np.array(list(cases)))
    assert list(got) == list(cases.values()), list(got)
    rng = np.random.default_rng(23)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.standard_normal(4000) * 2.0 ** -7,
                        rng.standard_normal(2000)]).astype(np.float32)
    assert np.array_equal(O.e4m3_round_codes(x.astype(np.float64)), MI.e4m3_codes(x))


def check_fp8_row():
    """One token's fp8 cache row: the worked example by hand (scale 3/448;
    0.5/scale = 74.67 -> 72 = code 105, -3/scale = -448 -> 0xFE, 1/scale =
    149.3 -> 144 = code 113), the largest element at +-448 exactly, zeros."""
    codes, s = O.quantize_latent(np.array([0.5, -3.0, 1.0], dtype=np.float32))
    assert s == np.float32(3.0) / np.float32(448.0)
    assert list(codes) == [105, 254, 113]
    codes, s = O.quantize_latent(np.zeros(512, dtype=np.float32))
    assert s == 1.0 and not codes.any()
    rng = np.random.default_rng(24)
    c = rng.standard_normal(512).astype(np.float32)
    codes, s = O.quantize_latent(c)
    k = int(np.argmax(np.abs(c)))
    assert codes[k] & 0x7F == 0x7E
    back = O.decode_e4m3(codes) * float(s)
    # within half a code step (relative 1/16 at most) of the value
    assert np.all(np.abs(back - c) <= np.abs(c) / 16 + 2.0 ** -10 * float(s))


def check_append_positions():
    """The rows the append writes: token i of sequence b at position
    len_b - S_q + i, none where that is negative; the key of a position-0
    token is its plain projection."""
    rng = np.random.default_rng(25)
    h = rng.standard_normal((4, 64))
    w_dkv, w_kr = rng.standard_normal((DL, 64)), rng.standard_normal((64, 64))
    out = O.appended_tokens(h, w_dkv, w_kr, [5, 1], 2)
    assert [(b, p) for b, p, _, _ in out] == [(0, 3), (0, 4), (1, 0)]
    b, p, c, kr = out[2]
    assert np.allclose(c, w_dkv @ h[3], rtol=0, atol=1e-12) and np.allclose(kr, w_kr @ h[3], rtol=0, atol=1e-12)


def check_gate_worked_example():
    """[DF-moe] by hand: affinities (0, ln 2, ln 3) give s = (1/6, 1/3, 1/2);
    with K_r = 2 the kept experts are 2 then 1 with g = (1/2, 1/3), expert 0
    gets g = 0; and a hand product u^T e_i."""
    e = np.log(np.array([[1.0], [2.0], [3.0]]))
    idx, g, s = O.moe_gate(np.array([[1.0]]), e, 2)
    assert np.allclose(s, [[1 / 6, 1 / 3, 1 / 2]], rtol=0, atol=1e-15)
    assert idx.tolist() == [[2, 1]]
    assert np.allclose(g, [[0.5, 1 / 3]], rtol=0, atol=1e-15)
    assert np.allclose(O.gate_dense(np.array([[1.0]]), e, 2), [[0.0, 1 / 3, 0.5]], rtol=0, atol=1e-15)
    # u = (2, 1) against centroids (1, 2), (3, 4), (-1, 0): 4, 10, -2
    a = O.expert_affinities(np.array([[2.0, 1.0]]), np.array([[1.0, 2.0], [3.0, 4.0], [-1.0, 0.0]]))
    assert np.array_equal(a, [[4.0, 10.0, -2.0]])
    rng = np.random.default_rng(31)
    ee = rng.standard_normal((160, 96))
    for m in (0, 95):                      # a one-hot token reads one coordinate of every centroid
        u = np.zeros((1, 96))
        u[0, m] = 1.0
        assert np.array_equal(O.expert_affinities(u, ee)[0], ee[:, m])


def check_gate_softmax():
    """The scores are a softmax: agreement with scipy's routine, invariance
    to a common shift of the affinities, and the sum of all 160 scores 1."""
    from scipy.special import softmax
    rng = np.random.default_rng(32)
    a = rng.standard_normal((5, 160)) * 4
    s = O.gate_softmax(a)
    assert np.allclose(s, softmax(a, axis=-1), rtol=1e-13, atol=0)
    assert np.allclose(O.gate_softmax(a + 700.0), s, rtol=1e-12, atol=0)
    assert np.allclose(s.sum(axis=-1), 1.0, rtol=0, atol=1e-14)


def _rank_ok(s, idx, k):
    """Brute force, pure Python: idx lists k distinct experts by decreasing
    score (equal scores by increasing index), and every expert left out
    ranks below every one kept."""
    n = len(s)
    idx = [int(i) for i in idx]
    if len(idx) != k or len(set(idx)) != k:
        return False
    before = lambda i, j: s[i] > s[j] or (s[i] == s[j] and i < j)  # noqa: E731
    if any(not before(idx[t], idx[t + 1]) for t in range(k - 1)):
        return False
    return all(before(i, j) for i in idx for j in range(n) if j not in idx)


def check_gate_top_k():
    """TopK keeps the K_r largest scores: hand cases with ties (the lower
    index first), brute force over random rows with planted ties, and
    K_r = N keeping every expert with g summing to 1."""
    s = np.array([[0.2, 0.3, 0.3, 0.2]])
    assert O.top_k(s, 2).tolist() == [[1, 2]]
    assert O.top_k(s, 3).tolist() == [[1, 2, 0]]
    assert O.top_k(np.array([[0.1, 0.4, 0.2, 0.3]]), 4).tolist() == [[1, 3, 2, 0]]
    rng = np.random.default_rng(33)
    for _ in range(40):
        row = np.round(rng.standard_normal(24), 1)          # many equal values
        for k in (1, 6, 24):
            assert _rank_ok(row, O.top_k(row[None], k)[0], k), (row, k)
    u, e = rng.standard_normal((3, 32)), rng.standard_normal((160, 32))
    idx, g, s = O.moe_gate(u, e, 160)
    assert all(sorted(r.tolist()) == list(range(160)) for r in idx)
    assert np.allclose(g.sum(axis=-1), 1.0, rtol=0, atol=1e-13)


def check_gate_deepseek_shape():
    """160 routed experts, 6 kept: exactly 6 nonzero gate values per token,
    each the token's score of that expert, every one at least as large as
    every score left out, and their sum below 1 (no renormalisation)."""
    rng = np.random.default_rng(34)
    u, e = rng.standard_normal((8, 64)), rng.standard_normal((160, 64)) / 8
    gd = O.gate_dense(u, e, 6)
    idx, g, s = O.moe_gate(u, e, 6)
    sp = O.gate_softmax(O.expert_affinities(u, e))
    for t in range(8):
        nz = np.flatnonzero(gd[t])
        assert sorted(nz.tolist()) == sorted(idx[t].tolist()) and len(nz) == 6
        assert np.array_equal(gd[t][nz], sp[t][nz])
        assert gd[t][nz].min() >= np.delete(sp[t], nz).max()
        assert gd[t].sum() < 1.0
        assert _rank_ok(sp[t].tolist(), idx[t], 6)
        assert np.array_equal(g[t], sp[t][idx[t]])


ALL_CHECKS = [check_cache_arithmetic, check_decode_tables, check_softmax,
              check_textbook_reduction, check_closed_forms, check_brute_force_exact,
              check_paging_invariance, check_causal_two_tokens, check_split_combine,
              check_absorb_project_identities, check_append_projection, check_rope,
              check_e4m3_encoding, check_fp8_row, check_append_positions,
              check_gate_worked_example, check_gate_softmax, check_gate_top_k, check_gate_deepseek_shape,
              check_batched_absorbed]
