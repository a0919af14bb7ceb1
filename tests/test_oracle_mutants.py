"""Plant plausible mistakes in the oracle (on the CPU) and require that the
pin checks catch each one.  This shows the pins constrain every step: a
dropped term, a wrong scale, an off-by-one mask, a wrong index or operand."""
import inspect
import math
import textwrap

import numpy as np
import pytest

import oracle
import oracle.mla_oracle as M
from oracle_pins import ALL_CHECKS

_orig = {name: getattr(M, name) for name in dir(M) if callable(getattr(M, name))}


def _keys_without_rope(C, KR, w):
    return np.concatenate([C @ w.T, np.zeros_like(KR)], axis=1)


def _keys_transposed_weight(C, KR, w):
    # uses W_UK's first 128 latent columns as if it were [d_latent][d_head]
    return np.concatenate([C @ w.T[:, ::-1], KR], axis=1)


def _values_skip_projection(C, w):
    return C[:, :w.shape[0]]


def _scores_wrong_scale(K, q, s):
    return (K @ q) / math.sqrt(128)


def _scores_sign(K, q, s):
    return -(K @ q) * s


def _visible_excludes_self(n, sq, i):
    return max(0, int(n) - (sq - i))


def _visible_ignores_causal(n, sq, i):
    return int(n)


def _gather_ignores_table(inp, b):
    n = int(inp.seq_lens[b])
    t = np.arange(n)
    start = int(inp.block_table[b][0])
    blocks = start + t // 64
    full = M.decode_f32(inp.latent[blocks % inp.latent.shape[0], t % 64])
    return full[:, :512], full[:, 512:]


def _gather_wrong_row(inp, b):
    n = int(inp.seq_lens[b])
    t = np.arange(n)
    blocks = inp.block_table[b][t // 64]
    full = M.decode_f32(inp.latent[blocks, (63 - t % 64) % 64])
    return full[:, :512], full[:, 512:]


def _softmax_no_norm(s):
    if s.size == 0:
        return s.copy(), -math.inf
    m = s.max()
    e = np.exp(s - m)
    return e, float(m + math.log(e.sum()))


def _softmax_lse_missing_max(s):
    if s.size == 0:
        return s.copy(), -math.inf
    m = s.max()
    e = np.exp(s - m)
    return e / e.sum(), float(math.log(e.sum()))


def _mix_reversed(p, V):
    return p[::-1] @ V if p.size else np.zeros(V.shape[1])


def _query_swapped(qn, qr):
    return np.concatenate([qr, qn])


def _e4m3_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * np.exp2(e - 8.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def _e4m3_no_subnormal(codes):
    out = _orig["decode_e4m3"](codes)
    c = np.asarray(codes, dtype=np.uint8)
    return np.where((c & 0x78) == 0, 0.0 * out, out)


def _bf16_truncated_mantissa(bits):
    u = (np.asarray(bits, dtype=np.uint16) & np.uint16(0xFFFE)).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _combine_no_max_weight(o_part, lse_part):
    w = np.where(np.isfinite(lse_part), 1.0, 0.0)
    z = w.sum(axis=1, keepdims=True)
    wn = np.where(z > 0, w / np.where(z > 0, z, 1), 0)
    lse = np.log(np.exp(np.where(np.isfinite(lse_part), lse_part, -np.inf)).sum(axis=1))
    return (wn[..., None] * np.nan_to_num(o_part)).sum(axis=1), lse


def _split_token_equal(seq_len, ns, block=64):
    per = -(-int(seq_len) // ns)
    return [(min(s * per, seq_len), min((s + 1) * per, seq_len)) for s in range(ns)]


def _cache_mha_one_vector(scheme, **kw):
    if scheme == "mha":
        return kw["heads"] * kw["d_head"]
    return _orig["cache_numbers_per_token_layer"](scheme, **kw)


def _absorb_first_head(q_nope, w_uk):
    q_nope = np.asarray(q_nope, dtype=np.float64)
    return np.stack([q_nope[:, h] @ np.asarray(w_uk[0], dtype=np.float64) for h in range(q_nope.shape[1])], axis=1)


def _project_first_head(o_lat, w_uv):
    o_lat = np.asarray(o_lat, dtype=np.float64)
    return np.stack([o_lat[:, h] @ np.asarray(w_uv[0], dtype=np.float64).T for h in range(o_lat.shape[1])], axis=1)


def _project_drops_last_column(o_lat, w_uv):
    o_lat = np.asarray(o_lat, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    return np.stack([o_lat[:, h, :-1] @ w[h, :, :-1].T for h in range(o_lat.shape[1])], axis=1)


def _down_project_drops_last(h, w):
    return np.asarray(h, dtype=np.float64)[:, :-1] @ np.asarray(w, dtype=np.float64)[:, :-1].T


def _rope_half_split(x, pos, theta=10000.0):
    # pairs (j, j + 32) instead of (2j, 2j + 1)
    x = np.asarray(x, dtype=np.float64)
    a = _orig["rope_angles"](pos, theta, x.shape[-1])
    h = x.shape[-1] // 2
    out = np.empty_like(x)
    out[..., :h] = x[..., :h] * np.cos(a) - x[..., h:] * np.sin(a)
    out[..., h:] = x[..., :h] * np.sin(a) + x[..., h:] * np.cos(a)
    return out


def _rope_wrong_sign(x, pos, theta=10000.0):
    return _orig["rope_rotate"](x, -pos, theta)


def _rope_angles_full_width(pos, theta=10000.0, d=64):
    j = np.arange(d // 2, dtype=np.float64)
    return float(pos) * np.power(float(theta), -j / d)


def _e4m3_ties_up(x):
    x = np.asarray(x, dtype=np.float64)
    vals = _orig["e4m3_values"]()
    a = np.abs(x).reshape(-1)
    d = np.abs(a[:, None] - vals[None, :])
    pick = (d.shape[1] - 1 - np.argmin(d[:, ::-1], axis=1)).astype(np.uint8)   # the larger of two equally near
    return np.where(np.signbit(x.reshape(-1)), pick | np.uint8(0x80), pick).reshape(x.shape)


def _e4m3_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    vals = _orig["e4m3_values"]()
    a = np.abs(x).reshape(-1)
    pick = (np.searchsorted(vals, a, side="right") - 1).astype(np.uint8)
    return np.where(np.signbit(x.reshape(-1)), pick | np.uint8(0x80), pick).reshape(x.shape)


def _quantize_scale_480(c):
    c = np.asarray(c, dtype=np.float32)
    amax = np.float32(np.abs(c).max())
    s = np.float32(amax / np.float32(480.0)) if amax > 0 else np.float32(1.0)
    q = np.clip(c / s, np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    return _orig["e4m3_round_codes"](q.astype(np.float64)), s


def _appended_off_by_one(h, w_dkv, w_kr, seq_lens, q_per_seq, theta=10000.0):
    out = []
    for b, ln in enumerate(np.asarray(seq_lens)):
        for i in range(q_per_seq):
            p = int(ln) - q_per_seq + i + 1
            if p < 0:
                continue
            r = b * q_per_seq + i
            out.append((b, p, M.down_project(h[r:r + 1], w_dkv)[0],
                        M.rope_rotate(M.down_project(h[r:r + 1], w_kr)[0], p, theta)))
    return out


def _affinity_reversed_dim(u, e):
    return np.asarray(u, dtype=np.float64) @ np.asarray(e, dtype=np.float64)[:, ::-1].T


def _gate_softmax_no_norm(a):
    a = np.asarray(a, dtype=np.float64)
    return np.exp(a - a.max(axis=-1, keepdims=True))


def _gate_softmax_wrong_axis(a):
    a = np.asarray(a, dtype=np.float64)
    z = np.exp(a - a.max(axis=0, keepdims=True))
    return z / z.sum(axis=0, keepdims=True)


def _top_k_ascending(s, k):
    return np.argsort(np.asarray(s), axis=-1, kind="stable")[..., :k]


def _top_k_ties_high(s, k):
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[-1]
    return (n - 1 - np.argsort(-s[..., ::-1], axis=-1, kind="stable"))[..., :k]


def _top_k_unsorted(s, k):
    s = np.asarray(s, dtype=np.float64)
    return np.sort(np.argsort(-s, axis=-1, kind="stable")[..., :k], axis=-1)


def _moe_gate_renormalised(u, e, k):
    s = M.gate_softmax(M.expert_affinities(u, e))
    idx = M.top_k(s, k)
    g = np.take_along_axis(s, idx, axis=-1)
    return idx, g / g.sum(axis=-1, keepdims=True), s


def _moe_gate_raw_affinity(u, e, k):
    a = M.expert_affinities(u, e)
    s = M.gate_softmax(a)
    idx = M.top_k(s, k)
    return idx, np.take_along_axis(a, idx, axis=-1), s


def _gate_dense_keeps_all(u, e, k):
    return M.gate_softmax(M.expert_affinities(u, e))


def _mutated(name, label, old, new):
    """A copy of oracle function `name` with one piece of its source replaced."""
    src = textwrap.dedent(inspect.getsource(_orig[name]))
    assert src.count(old) == 1, (name, old)
    ns = dict(vars(M))
    exec(compile(src.replace(old, new), f"<{label}>", "exec"), ns)
    f = ns[name]
    f.__name__ = label
    return f


_BATCHED_MUTANTS = [
    _mutated("absorbed_decode_batched", "_batched_causal_reversed",
             "visible_tokens(n, Sq, i) for i in range(Sq)", "visible_tokens(n, Sq, Sq - 1 - i) for i in range(Sq)"),
    _mutated("absorbed_decode_batched", "_batched_query_head_axes_swapped",
             "o_lat[r0:r0 + Sq] = ol.reshape(Sq, H, D_LATENT)",
             "o_lat[r0:r0 + Sq] = ol.reshape(H, Sq, D_LATENT).transpose(1, 0, 2)"),
    _mutated("absorbed_decode_batched", "_batched_rope_unscaled",
             "S = (C @ ql.T + KR @ qr.T) * scale", "S = C @ ql.T * scale + KR @ qr.T"),
    _mutated("absorbed_decode_batched", "_batched_wrong_head_weight",
             "w_uv_t = dw(inp.w_uv).transpose(0, 2, 1)", "w_uv_t = dw(inp.w_uv)[::-1].transpose(0, 2, 1)"),
    _mutated("absorbed_decode_batched", "_batched_lse_missing_max",
             "m + np.log(np.where(seen, z, 1.0))", "np.log(np.where(seen, z, 1.0))"),
    _mutated("absorbed_decode_batched", "_batched_mask_off_by_one",
             "np.arange(n)[:, None] >= vis[None, :]", "np.arange(n)[:, None] > vis[None, :]"),
]

MUTANTS = {
    "absorbed_decode_batched": _BATCHED_MUTANTS,
    "down_project": [_down_project_drops_last],
    "rope_rotate": [_rope_half_split, _rope_wrong_sign],
    "rope_angles": [_rope_angles_full_width],
    "e4m3_round_codes": [_e4m3_ties_up, _e4m3_truncate],
    "quantize_latent": [_quantize_scale_480],
    "appended_tokens": [_appended_off_by_one],
    "reconstruct_keys": [_keys_without_rope, _keys_transposed_weight],
    "reconstruct_values": [_values_skip_projection],
    "scores": [_scores_wrong_scale, _scores_sign],
    "visible_tokens": [_visible_excludes_self, _visible_ignores_causal],
    "gather_sequence": [_gather_ignores_table, _gather_wrong_row],
    "softmax_lse": [_softmax_no_norm, _softmax_lse_missing_max],
    "mix_values": [_mix_reversed],
    "query_vector": [_query_swapped],
    "decode_e4m3": [_e4m3_bias8, _e4m3_no_subnormal],
    "decode_bf16": [_bf16_truncated_mantissa],
    "combine_partials": [_combine_no_max_weight],
    "split_ranges": [_split_token_equal],
    "cache_numbers_per_token_layer": [_cache_mha_one_vector],
    "absorb_queries": [_absorb_first_head],
    "project_output": [_project_first_head, _project_drops_last_column],
    "expert_affinities": [_affinity_reversed_dim],
    "gate_softmax": [_gate_softmax_no_norm, _gate_softmax_wrong_axis],
    "top_k": [_top_k_ascending, _top_k_ties_high, _top_k_unsorted],
    "moe_gate": [_moe_gate_renormalised, _moe_gate_raw_affinity],
    "gate_dense": [_gate_dense_keeps_all],
}

CASES = [(name, f) for name, fs in MUTANTS.items() for f in fs]


@pytest.mark.parametrize("name,mutant", CASES, ids=[f.__name__ for _, f in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(M, name, mutant)
    monkeypatch.setattr(oracle, name, mutant, raising=False)
    caught = []
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"planted mistake {mutant.__name__} in {name} went unnoticed"
