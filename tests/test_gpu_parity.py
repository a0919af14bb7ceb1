"""HIP path vs the fp64 oracle, element by element, through the C ABI."""
import numpy as np
import pytest

import mla_inputs as MI
import oracle as O
from parity import check, metrics

# every case runs at 64 and at 32 query rows per decode workgroup
pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("decode_rows")]


def run_gpu(inp, num_splits=None):
    import torch
    from mla_latent_kv_17_amd.runner import DecodeStep, DeviceInputs
    print(f"[case] {inp.wl.name} B={inp.wl.batch} Sq={inp.wl.q_per_seq} H={inp.wl.heads} "
          f"dtype={inp.wl.cache_dtype} splits={num_splits}", flush=True)
    dev = DeviceInputs(inp)
    ns = inp.wl.num_splits if num_splits is None else num_splits
    step = DecodeStep(dev, ns)
    step.run()  # merge fused into the projection when split
    torch.cuda.synchronize()
    out, lse = step.out.cpu().numpy(), step.lse.cpu().numpy()
    o_lat = step.latent_output().cpu().numpy()  # the merge on its own
    return out, o_lat, lse, step


@pytest.mark.parametrize("name", list(MI.small_variants()))
def test_small_variant_vs_oracle(name):
    wl = MI.small_variants()[name]
    inp = MI.generate(wl)
    out, o_lat, lse, _ = run_gpu(inp)
    o_ref, lse_ref = O.explicit_decode(inp)
    check(f"{name}/o", out, o_ref, wl.cache_dtype)
    _, olat_ref, lse_abs, _ = O.absorbed_decode(inp)
    m1, m2 = metrics(o_lat, olat_ref), metrics(lse, lse_ref)
    print(f"[report] {name}: o_lat rel_l2={m1['rel_l2']:.3e} lse max_abs={m2['max_abs']:.3e}", flush=True)
    assert m2["max_abs"] < 1e-2


@pytest.mark.parametrize("ns", [1, 2, 3, 7, 64])
def test_split_invariance(ns):
    wl = MI.small_variants()["bf16_small_split"]
    inp = MI.generate(wl)
    out, o_lat, lse, _ = run_gpu(inp, num_splits=ns)
    o_ref, lse_ref = O.explicit_decode(inp)
    check(f"split{ns}/o", out, o_ref, "bf16")
    assert np.max(np.abs(lse - lse_ref)) < 1e-2


@pytest.mark.parametrize("name", ["bf16_small_paged", "fp8_small_sq2"])
def test_paging_bit_exact(name):
    """A permuted pool and its de-paged contiguous copy give identical bits."""
    inp = MI.generate(MI.small_variants()[name])
    a = run_gpu(inp)
    b = run_gpu(MI.depaged(inp))
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_deterministic():
    inp = MI.generate(MI.small_variants()["bf16_small_contig"])
    a = run_gpu(inp)
    b = run_gpu(inp)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


# multi-token decode: S_q query tokens per sequence, each seeing the cache up
# to its own position (query i sees len - (S_q - 1 - i) tokens; the first
# queries of a sequence shorter than S_q see none)
MULTI = {
    "bf16_sq5": MI.small_variants()["bf16_small_paged"].scaled(name="bf16_sq5", q_per_seq=5, seed=2201),
    "bf16_sq16_split": MI.small_variants()["bf16_small_split"].scaled(name="bf16_sq16_split", q_per_seq=16,
                                                                      heads=16, seed=2202),
    "fp8_sq7": MI.small_variants()["fp8_small_sq2"].scaled(name="fp8_sq7", q_per_seq=7, lens=(3, 70, 200),
                                                           len_range=None, seed=2203),
    "fp32_sq3": MI.small_variants()["fp32_b1_h16_t1k"].scaled(name="fp32_sq3", q_per_seq=3, seq_len=130,
                                                              seed=2204),
    # many query tokens: a sequence shorter than S_q, splits on both sides
    # of the fused-merge limit (8)
    "bf16_sq128_split3": MI.small_variants()["bf16_small_paged"].scaled(
        name="bf16_sq128_split3", q_per_seq=128, heads=16, batch=3, lens=(100, 300, 700), len_range=None,
        num_splits=3, seed=2205),
    "bf16_sq128_h128_split12": MI.small_variants()["bf16_small_paged"].scaled(
        name="bf16_sq128_h128_split12", q_per_seq=128, heads=128, batch=2, lens=(90, 1500), len_range=None,
        num_splits=12, seed=2206),
    "fp8_sq65_split2": MI.small_variants()["fp8_small_sq2"].scaled(
        name="fp8_sq65_split2", q_per_seq=65, heads=8, batch=4, lens=(40, 64, 65, 300), len_range=None,
        num_splits=2, seed=2207),
    # past the absorbed/explicit crossover the absorbed form still runs
    "bf16_sq256_split2": MI.small_variants()["bf16_small_paged"].scaled(
        name="bf16_sq256_split2", q_per_seq=256, heads=8, batch=2, lens=(200, 1000), len_range=None,
        num_splits=2, seed=2208),
    "fp8_sq300": MI.small_variants()["fp8_small_sq2"].scaled(
        name="fp8_sq300", q_per_seq=300, heads=4, batch=2, lens=(333, 640), len_range=None, num_splits=1,
        seed=2209),
}
# cases with many rows: the batched absorbed form of the oracle (pinned to
# the explicit definition on the CPU) computes every row
MULTI_BATCHED = {"bf16_sq128_h128_split12"}


@pytest.mark.parametrize("name", list(MULTI))
def test_multi_token_vs_oracle(name):
    wl = MULTI[name]
    inp = MI.generate(wl)
    out, o_lat, lse, _ = run_gpu(inp)
    if name in MULTI_BATCHED:
        _, lse_ref, o_ref = O.absorbed_decode_batched(inp)
    else:
        o_ref, lse_ref = O.explicit_decode(inp)
    check(f"{name}/o", out, o_ref, wl.cache_dtype)
    none = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), none)
    assert np.max(np.abs(lse[~none] - lse_ref[~none])) < 1e-2
    assert (out[none] == 0).all()


# the library's split choice for an uneven batch (mla_decode_num_splits_batch):
# more chunks than the longest sequence alone would ask for, so a short
# sequence's trailing chunks are empty (they write o = 0, lse = -inf without
# running the pipeline and the merges give them weight 0)
def test_num_splits_batch_choice():
    import mla_latent_kv_17_amd as M
    d = M.make_dims(64, 1, 128)
    assert M.mla_decode_num_splits_batch(d, 64 * 8448, 16384) == 8        # 64 sequences of 512 .. 16384 tokens
    assert M.mla_decode_num_splits_batch(M.make_dims(32, 1, 128), 32 * 4096, 4096) == \
        M.mla_decode_num_splits(M.make_dims(32, 1, 128), 4096)            # uniform: unchanged
    assert M.mla_decode_num_splits_batch(M.make_dims(2, 1, 128), 300, 200) == \
        M.mla_decode_num_splits(M.make_dims(2, 1, 128), 200)              # few pages: at most the longest's


UNEVEN = {
    "bf16_uneven_ns16": (MI.small_variants()["bf16_small_paged"].scaled(
        name="bf16_uneven", batch=4, lens=(0, 70, 300, 1500), len_range=None, seed=2210), 16),
    "bf16_sq3_h16_ns8": (MI.small_variants()["bf16_small_paged"].scaled(
        name="bf16_sq3_h16", q_per_seq=3, heads=16, batch=4, lens=(2, 64, 300, 1000), len_range=None, seed=2211), 8),
    "fp8_ns6": (MI.small_variants()["fp8_small_sq2"], 6),
    "fp32_uneven_ns9": (MI.small_variants()["fp32_b1_h16_t1k"].scaled(
        name="fp32_uneven", batch=3, seq_len=None, lens=(100, 700, 1024), paged=True, spare_blocks=2, seed=2212), 9),
}


@pytest.mark.parametrize("name", list(UNEVEN))
def test_uneven_batch_many_chunks(name):
    wl, ns = UNEVEN[name]
    inp = MI.generate(wl)
    out, o_lat, lse, step = run_gpu(inp, num_splits=ns)
    assert step.num_splits == ns
    o_ref, lse_ref = O.explicit_decode(inp)
    check(f"{name}/o", out, o_ref, wl.cache_dtype)
    none = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), none)
    assert np.max(np.abs(lse[~none] - lse_ref[~none])) < 1e-2
    assert (out[none] == 0).all()
