"""Comparison helpers for GPU-vs-oracle parity (tolerances stated by the
workloads: bf16/fp8 inputs with fp32 accumulation -> max-abs <= 2e-2 and
relative L2 <= 5e-3 on the head output o; fp32 -> relative L2 <= 1e-5)."""
import sys

import numpy as np

TOL = {"bf16": dict(max_abs=2e-2, rel_l2=5e-3), "fp8": dict(max_abs=2e-2, rel_l2=5e-3),
       "f32": dict(max_abs=None, rel_l2=1e-5)}


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mask = ~np.isnan(ref)
    g, r = got[mask], ref[mask]
    if r.size == 0:
        return dict(max_abs=0.0, rel_l2=0.0, n=0)
    err = g - r
    return dict(max_abs=float(np.max(np.abs(err))), rel_l2=float(np.linalg.norm(err) / max(np.linalg.norm(r), 1e-300)),
                n=int(r.size), finite=bool(np.isfinite(g).all()))


def check(name, got, ref, kind):
    m = metrics(got, ref)
    tol = TOL[kind]
    print(f"[parity] {name}: max_abs={m['max_abs']:.3e} rel_l2={m['rel_l2']:.3e} n={m['n']}", flush=True)
    sys.stdout.flush()
    assert m["finite"], f"{name}: non-finite output"
    assert m["rel_l2"] <= tol["rel_l2"], (name, m)
    if tol["max_abs"] is not None:
        assert m["max_abs"] <= tol["max_abs"], (name, m)
    return m
