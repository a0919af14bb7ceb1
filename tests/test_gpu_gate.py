"""mla_moe_gate against the oracle (s_i = softmax of u^T e_i over the routed
experts; the top_k largest kept, largest first, equal scores by lower index;
g_i = s_i).

What is compared:
* scores and gate values: within the decode tolerances of the fp64 scores
  (fp32 sums of exact products; bf16 or fp32 inputs);
* the selection, where floating point decides it: the kernel ranks the fp32
  affinities, the oracle the fp64 ones, so where two affinities lie within
  the fp32 summation error of each other either order is correct.  The
  check: every kept expert's fp64 affinity is at least every left-out one's
  minus tau, consecutive kept ones do not rise by more than tau, and where
  the oracle's gaps all exceed tau the lists are identical.  tau for a pair
  is 2^-16 times the sum of both affinities' sums of |u_k e_ik|: the
  error of a blocked fp32 sum of d_model exact products is below about
  (block lengths + log2 chunks) * 2^-24 = 62 * 2^-24 of that magnitude (16-long
  matrix-core steps, 32-step waves, 4 waves, 10 chunks), four times margin;
* with one-hot tokens every affinity is one centroid entry, exact in fp32, so
  the selection must equal the oracle's bit for bit; with twin centroids
  every affinity has an equal partner and the lower index must win each tie.
"""
import numpy as np
import pytest

import mla_inputs as MI
import oracle as O
from parity import check

pytestmark = pytest.mark.gpu


def _decode(x, dtype):
    return O.decode_bf16(x) if dtype == "bf16" else O.decode_f32(x)


def _run(gi, dtype, with_scores=True):
    import torch
    import mla_latent_kv_17_amd as M
    dev = torch.device("cuda", 0)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    code = M.MLA_BF16 if dtype == "bf16" else M.MLA_F32
    tokens, d_model = gi.u.shape
    n = gi.e.shape[0]

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.int16).to(dev).view(torch.bfloat16) if dtype == "bf16" else t.to(dev)).view(td)
    u, e = up(gi.u), up(gi.e)
    ws = torch.empty(max(M.mla_moe_gate_workspace_size(tokens, d_model, n, code) // 4, 1), dtype=torch.float32,
                     device=dev)
    idx = torch.full((tokens, gi.top_k), -7, dtype=torch.int32, device=dev)
    w = torch.full((tokens, gi.top_k), float("nan"), dtype=torch.float32, device=dev)
    sc = torch.full((tokens, n), float("nan"), dtype=torch.float32, device=dev) if with_scores else None
    M.mla_moe_gate(u, e, gi.top_k, idx, w, ws, scores=sc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), None if sc is None else sc.cpu().numpy()


def _tau(u, e):
    mag = np.abs(u) @ np.abs(e).T          # [tokens][experts] sums of |u_k e_ik|
    return 2.0 ** -16 * mag


def _check_selection(name, idx, u, e, k, exact=False):
    a = O.expert_affinities(u, e)
    want_idx, _, _ = O.moe_gate(u, e, k)
    tau = _tau(u, e)
    n = e.shape[0]
    assert idx.shape == want_idx.shape
    assert np.all((idx >= 0) & (idx < n)), name
    same = 0
    for t in range(idx.shape[0]):
        row = idx[t].tolist()
        assert len(set(row)) == k, (name, t, row)
        if exact:
            assert row == want_idx[t].tolist(), (name, t, row, want_idx[t].tolist())
            continue
        out = np.setdiff1d(np.arange(n), row)
        for i in row:
            if out.size:
                assert np.all(a[t, i] >= a[t, out] - (tau[t, i] + tau[t, out])), (name, t, i)
        for p in range(k - 1):
            i, j = row[p], row[p + 1]
            assert a[t, j] <= a[t, i] + tau[t, i] + tau[t, j], (name, t, p)
        order = want_idx[t]
        ranked = np.concatenate([order, np.setdiff1d(np.argsort(-a[t], kind="stable"), order)])[:k + 1]
        gaps = a[t, ranked[:-1]] - a[t, ranked[1:]] if k < n else a[t, order[:-1]] - a[t, order[1:]]
        gtau = tau[t, ranked[:-1]] + tau[t, ranked[1:]] if k < n else tau[t, order[:-1]] + tau[t, order[1:]]
        if np.all(gaps > gtau):
            assert row == order.tolist(), (name, t, row, order.tolist())
            same += 1
    print(f"[parity] {name}: selection valid for {idx.shape[0]} tokens "
          f"({'exact' if exact else f'{same} with clear gaps identical'})", flush=True)


def _check_values(name, idx, w, sc, u, e, kind):
    s = O.gate_softmax(O.expert_affinities(u, e))
    check(f"{name} weights", w, np.take_along_axis(s, idx.astype(np.int64), axis=-1), kind)
    if sc is not None:
        check(f"{name} scores", sc, s, kind)
        # the gate value is the kernel's own score of that expert
        assert np.array_equal(w, np.take_along_axis(sc, idx.astype(np.int64), axis=-1)), name
        # kept scores are the largest (one fp32 rounding of slack: exp is monotone up to rounding)
        for t in range(idx.shape[0]):
            kept = sc[t, idx[t]]
            rest = np.delete(sc[t], idx[t])
            if rest.size:
                assert kept.min() >= rest.max() * (1 - 2.0 ** -21), (name, t)
            assert np.all(np.diff(kept) <= np.abs(kept[:-1]) * 2.0 ** -21), (name, t)


CASES = {
    # tokens, d_model, experts, top_k, dtype
    "bf16_deepseek_ragged": (37, 640, 160, 6, "bf16"),      # two 512-wide chunks (second partial), ragged tile
    "bf16_deepseek_d5120": (64, 5120, 160, 6, "bf16"),
    "bf16_max": (33, 1024, 256, 16, "bf16"),
    "bf16_one_expert": (5, 64, 1, 1, "bf16"),
    "bf16_keep_all": (9, 192, 24, 16, "bf16"),
    # from 768 tokens on the tall projection kernel (128 tokens x every expert per workgroup);
    # from 2048 tokens on four tokens per wave in the finish
    "bf16_tall_ragged": (800, 640, 160, 6, "bf16"),
    "bf16_tall_max": (771, 1024, 256, 16, "bf16"),
    "bf16_tall_few_experts": (777, 5120, 20, 4, "bf16"),
    "bf16_tall_n100": (1000, 1536, 100, 8, "bf16"),
    "bf16_rows_n101": (2100, 640, 101, 5, "bf16"),
    "bf16_rows_n250": (2053, 640, 250, 7, "bf16"),
    "bf16_rows_one_expert": (2050, 128, 1, 1, "bf16"),
    "bf16_rows_n3": (2049, 192, 3, 2, "bf16"),
    "f32_small": (11, 192, 64, 8, "f32"),
    "f32_deepseek": (6, 5120, 160, 6, "f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gate_vs_oracle(name):
    T, D, N, K, dt = CASES[name]
    print(f"[case] gate {name} tokens={T} d_model={D} experts={N} top_k={K} {dt}", flush=True)
    gi = MI.generate_gate(T, d_model=D, n_experts=N, top_k=K, dtype=dt, seed=len(name))
    idx, w, sc = _run(gi, dt)
    u, e = _decode(gi.u, dt), _decode(gi.e, dt)
    _check_selection(f"gate {name}", idx, u, e, K)
    _check_values(f"gate {name}", idx, w, sc, u, e, dt)
    if N == 1:
        assert np.all(w == 1.0) and np.all(idx == 0)


@pytest.mark.parametrize("twins", [False, True], ids=["distinct", "twins"])
@pytest.mark.parametrize("dt,tokens", [("bf16", 40), ("bf16", 800), ("bf16", 2050), ("f32", 7)])
def test_gate_one_hot_exact(dt, tokens, twins):
    """Exact affinities: the selection (ties included) equals the oracle's."""
    print(f"[case] gate one-hot {dt} tokens={tokens} twins={twins}", flush=True)
    gi = MI.generate_gate(tokens, d_model=640, n_experts=160, top_k=6, dtype=dt, seed=3, one_hot=True, twins=twins)
    idx, w, sc = _run(gi, dt)
    u, e = _decode(gi.u, dt), _decode(gi.e, dt)
    _check_selection(f"gate one-hot {dt} twins={twins}", idx, u, e, 6, exact=True)
    _check_values(f"gate one-hot {dt}", idx, w, sc, u, e, dt)
    if twins:
        # each kept pair lists the even expert first
        assert all(r.tolist()[0] % 2 == 0 for r in idx)


def test_gate_without_scores_and_empty():
    import torch
    import mla_latent_kv_17_amd as M
    print("[case] gate scores=None, tokens=0", flush=True)
    gi = MI.generate_gate(20, d_model=640, seed=9)
    idx_a, w_a, _ = _run(gi, "bf16", with_scores=True)
    idx_b, w_b, _ = _run(gi, "bf16", with_scores=False)
    assert np.array_equal(idx_a, idx_b) and np.array_equal(w_a, w_b)
    dev = torch.device("cuda", 0)
    u = torch.zeros((0, 640), dtype=torch.bfloat16, device=dev)
    e = torch.zeros((160, 640), dtype=torch.bfloat16, device=dev)
    idx = torch.full((1, 6), -7, dtype=torch.int32, device=dev)
    w = torch.zeros((1, 6), dtype=torch.float32, device=dev)
    ws = torch.zeros(4, dtype=torch.float32, device=dev)
    M.mla_moe_gate(u, e, 6, idx, w, ws)
    torch.cuda.synchronize()
    assert (idx.cpu() == -7).all()


def test_gate_full_size():
    """4096 tokens of DeepSeek-V2's router (d_model 5120, 160 experts, top 6),
    the size the benchmark times; every token checked."""
    print("[case] gate full size tokens=4096", flush=True)
    gi = MI.generate_gate(4096, d_model=MI.APPEND_D_MODEL, seed=11)
    idx, w, sc = _run(gi, "bf16")
    u, e = O.decode_bf16(gi.u), O.decode_bf16(gi.e)
    _check_selection("gate full size", idx, u, e, 6)
    _check_values("gate full size", idx, w, sc, u, e, "bf16")
