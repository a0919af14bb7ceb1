"""Edge cases of the decode path against the fp64 oracle: sequences with no
or a single cached token (o = 0, lse = -inf for a query that sees nothing),
head counts that leave 64-row blocks partly empty, split counts far above the
page count (up to the largest allowed), scores whose running maximum jumps
far above the first page's, and an empty batch."""
import math

import numpy as np
import pytest

import mla_inputs as MI
import oracle as O
from parity import check, metrics

# every case runs at 64 and at 32 query rows per decode workgroup
pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("decode_rows")]


def run(inp, ns):
    import torch
    from mla_latent_kv_17_amd.runner import DecodeStep, DeviceInputs
    wl = inp.wl
    print(f"[case] {wl.name} B={wl.batch} Sq={wl.q_per_seq} H={wl.heads} {wl.cache_dtype} "
          f"lens={list(inp.seq_lens)[:8]} ns={ns}", flush=True)
    step = DecodeStep(DeviceInputs(inp), ns)
    step.run()  # merge fused into the projection when split
    torch.cuda.synchronize()
    out, lse = step.out.cpu().numpy(), step.lse.cpu().numpy()
    o_lat = step.latent_output().cpu().numpy()
    step.run_unfused()  # mla_split_combine + mla_out_uv
    torch.cuda.synchronize()
    out2, lse2 = step.out.cpu().numpy(), step.lse.cpu().numpy()
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse2))
    fin = ~np.isneginf(lse)
    assert np.max(np.abs(lse[fin] - lse2[fin]), initial=0.0) <= 1e-5 * max(1.0, np.abs(lse[fin]).max(initial=0.0))
    assert np.max(np.abs(out - out2), initial=0.0) <= 1e-5 * max(1.0, np.abs(out2).max(initial=0.0))
    return out, o_lat, lse


def compare(inp, ns):
    out, o_lat, lse = run(inp, ns)
    o_ref, lse_ref = O.explicit_decode(inp)
    none = np.isneginf(lse_ref)
    # a query that sees no token: exactly zero output and -inf log-sum-exp
    assert np.array_equal(np.isneginf(lse), none), "rows without visible tokens differ"
    assert (out[none] == 0).all() and (o_lat[none] == 0).all()
    assert np.isfinite(out).all() and np.isfinite(o_lat).all()
    check(f"{inp.wl.name}/ns{ns}/o", out, o_ref, inp.wl.cache_dtype)
    if (~none).any():
        assert np.max(np.abs(lse[~none] - lse_ref[~none])) < 1e-2
    return out, o_lat, lse


BASE = MI.WORKLOADS["bf16_paged_b64_ragged"]


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("sq", [1, 2])
def test_empty_and_single_token_sequences(dtype, sq):
    heads = 16 if dtype == "f32" else 100
    wl = BASE.scaled(name=f"edge_lens_{dtype}_sq{sq}", batch=7, q_per_seq=sq, heads=heads,
                     cache_dtype=dtype, len_range=None, lens=(0, 1, 2, 63, 64, 65, 130),
                     spare_blocks=3, seed=4000 + sq)
    inp = MI.generate(wl)
    for ns in (1, 3):
        compare(inp, ns)


def test_fp32_tile_boundaries():
    """fp32 cache: visible ranges ending on both sides of the kernel's 16-token
    tile edges (queries 0 and 1 of a sequence see len - 1 and len tokens), and
    chunks of one to thirteen tiles, so the four-slot tile ring is refilled."""
    wl = BASE.scaled(name="edge_f32_tiles", batch=12, q_per_seq=2, heads=16, cache_dtype="f32", len_range=None,
                     lens=(15, 16, 17, 31, 32, 33, 47, 48, 49, 80, 129, 200), spare_blocks=2, seed=4100)
    inp = MI.generate(wl)
    for ns in (1, 2, 4):
        compare(inp, ns)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("heads,sq", [(16, 1), (100, 1), (100, 2), (128, 2)])
def test_partial_row_blocks(heads, sq, dtype):
    wl = BASE.scaled(name=f"edge_rows_h{heads}_sq{sq}_{dtype}", batch=3, q_per_seq=sq, heads=heads, cache_dtype=dtype,
                     len_range=(100, 400), spare_blocks=2, seed=4100 + heads + sq)
    inp = MI.generate(wl)
    compare(inp, 2)


def test_max_splits_on_few_pages():
    """1024 chunks (the largest count) over sequences of 1-2 pages: almost
    every chunk is empty and must merge with weight 0."""
    wl = BASE.scaled(name="edge_max_splits", batch=2, heads=16, len_range=None, lens=(100, 64),
                     spare_blocks=1, seed=4200)
    inp = MI.generate(wl)
    compare(inp, 1024)


def _plant_token(inp, b, t, head, alpha):
    """Overwrite the RoPE key of cached token t of sequence b with
    alpha * sign(q_rope[b, head]): that head's score on the token rises by
    about 3.7 * alpha nats (other heads move by about +-0.6 * alpha), while
    the values, which come from the latent part alone, keep their size."""
    qr = O.decode_bf16(inp.q_rope[b * inp.wl.q_per_seq, head])
    row = np.where(qr >= 0, alpha, -alpha).astype(np.float32)
    blk = inp.block_table[b, t // 64]
    inp.latent[blk, t % 64, 512:] = MI.bf16_bits(row)


@pytest.mark.parametrize("alpha", [20.0, 100.0])
def test_late_score_far_above_first_page(alpha):
    """A token in a later page whose score is tens to hundreds of nats above
    everything before it: the kernel's running reference must be replaced
    (alpha = 20 moves head 0 by about 74 nats; alpha = 100 moves head 0 by
    about 370 and many other heads by more than 44)."""
    wl = MI.WORKLOADS["bf16_b32_h128_t4k"].scaled(name=f"edge_jump_{alpha:g}", batch=2, seq_len=700,
                                                  num_splits=1, seed=4300)
    inp = MI.generate(wl)
    _plant_token(inp, 0, 300, 0, alpha)
    _plant_token(inp, 1, 650, 5, alpha)
    for ns in (1, 2):
        compare(inp, ns)


def _plant_token_f32(inp, b, t, head, alpha):
    """_plant_token for an fp32 cache."""
    qr = inp.q_rope[b * inp.wl.q_per_seq, head]
    blk = inp.block_table[b, t // 64]
    inp.latent[blk, t % 64, 512:] = np.where(qr >= 0, alpha, -alpha).astype(np.float32)


@pytest.mark.parametrize("alpha", [20.0, 100.0])
def test_late_score_far_above_first_page_fp32(alpha):
    """The same for the fp32 decode, whose weights are formed against tile 0's
    maximum: a later score far above it makes the chunk be walked again."""
    wl = MI.small_variants()["fp32_b1_h16_t1k"].scaled(name=f"edge_jump_f32_{alpha:g}", batch=2, seq_len=700,
                                                       num_splits=1, seed=4310)
    inp = MI.generate(wl)
    _plant_token_f32(inp, 0, 300, 0, alpha)
    _plant_token_f32(inp, 1, 650, 5, alpha)
    for ns in (1, 2):
        compare(inp, ns)


def test_empty_batch_launches_nothing():
    import torch
    import mla_latent_kv_17_amd as M
    from mla_latent_kv_17_amd.runner import DeviceInputs
    inp = MI.generate(MI.small_variants()["bf16_small_contig"])
    dev = DeviceInputs(inp)
    dims = M.make_dims(0, 1, 128)
    o = torch.full((4, 128, 512), 7.0, device="cuda")
    lse = torch.full((4, 128), 7.0, device="cuda")
    M.mla_decode(dims, dev.q_nope, dev.q_rope, dev.cache, 1, o, lse)
    M.mla_split_combine(dims, 3, o, lse, o, lse)
    torch.cuda.synchronize()
    assert (o == 7.0).all() and (lse == 7.0).all()
