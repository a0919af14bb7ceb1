"""The five measured workloads at their full sizes, in the launch
configuration the benchmark times (the workload's split count, or the
library's choice when it names none).  The fp64 oracle recomputes sampled
(sequence, query, head) rows one by one -- corners, the longest and shortest
sequences and random picks -- and every row is checked for properties that
hold at any size: finite outputs, finite log-sum-exps, and a latent output
inside the range of the cached latent values (a convex combination of them)."""
import numpy as np
import pytest

import mla_inputs as MI
import oracle as O
from parity import check

pytestmark = pytest.mark.gpu


def picks(inp, n_random, seed):
    wl = inp.wl
    B, Sq, H = wl.batch, wl.q_per_seq, wl.heads
    lens = inp.seq_lens
    sel = {(0, 0, 0), (B - 1, Sq - 1, H - 1), (int(np.argmax(lens)), Sq - 1, H // 2),
           (int(np.argmin(lens)), 0, 1 % H)}
    rng = np.random.default_rng(seed)
    while len(sel) < 4 + n_random:
        sel.add((int(rng.integers(B)), int(rng.integers(Sq)), int(rng.integers(H))))
    return sorted(sel)


def latent_range(inp):
    """Bounds on every cached latent value (NaN poison ignored)."""
    if inp.wl.cache_dtype == "fp8":
        # each token's largest magnitude is 448 times its scale
        m = 448.0 * float(np.nanmax(inp.scale))
        return -m, m
    if inp.wl.cache_dtype == "f32":
        vals = inp.latent[:, :, :512]
    else:
        vals = (inp.latent[:, :, :512].astype(np.uint32) << np.uint32(16)).view(np.float32)
    return float(np.nanmin(vals)), float(np.nanmax(vals))


@pytest.mark.parametrize("name", MI.WORKLOAD_ORDER)
def test_full_size_sampled(name):
    import torch
    from mla_latent_kv_17_amd.runner import DecodeStep, DeviceInputs
    wl = MI.WORKLOADS[name]
    print(f"[case] {name}: generating", flush=True)
    inp = MI.generate(wl)
    dev = DeviceInputs(inp)
    step = DecodeStep(dev, wl.num_splits)
    print(f"[case] {name}: running, num_splits={step.num_splits}", flush=True)
    step.run()
    torch.cuda.synchronize()
    out = step.out.cpu().numpy()
    lse = step.lse.cpu().numpy()
    o_lat = step.latent_output().cpu().numpy()
    del dev, step

    # properties of every row
    assert np.isfinite(out).all() and np.isfinite(o_lat).all() and np.isfinite(lse).all()
    lo, hi = latent_range(inp)
    slack = 1e-3 * max(abs(lo), abs(hi))
    assert o_lat.min() >= lo - slack and o_lat.max() <= hi + slack

    # sampled rows against the oracle
    n_random = 2 if name == "bf16_long_t128k_s64" else 8
    sel = picks(inp, n_random, seed=6000 + MI.WORKLOAD_ORDER.index(name))
    if name == "fp32_b1_h16_t1k":
        sel = None  # small enough to compare every row
    o_ref, lse_ref = O.explicit_decode(inp, select=sel)
    mask = ~np.isnan(lse_ref)
    print(f"[case] {name}: {int(mask.sum())} rows compared", flush=True)
    check(f"{name}/o sampled", out[mask], o_ref[mask], wl.cache_dtype)
    assert np.max(np.abs(lse[mask] - lse_ref[mask])) < 1e-2
