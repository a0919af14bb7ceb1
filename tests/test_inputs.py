"""The seeded input generator: reproducible, valid paging, poison where no
sequence owns memory, encodings equal to the library's own casts."""
import numpy as np
import pytest
import torch

import mla_inputs as MI


def test_seed_reproducible():
    wl = MI.small_variants()["bf16_small_paged"]
    a, b = MI.generate(wl), MI.generate(wl)
    for f in ("seq_lens", "block_table", "latent", "q_nope", "q_rope", "w_uk", "w_uv"):
        x, y = getattr(a, f), getattr(b, f)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f
    c = MI.generate(wl, seed=wl.seed + 1)
    assert not np.array_equal(a.q_nope, c.q_nope)


@pytest.mark.parametrize("name", list(MI.small_variants()))
def test_paging_and_poison(name):
    wl = MI.small_variants()[name]
    inp = MI.generate(wl)
    B = wl.batch
    pages = -(-inp.seq_lens.astype(np.int64) // MI.BLOCK)
    used = [inp.block_table[b, :pages[b]] for b in range(B)]
    allb = np.concatenate(used)
    assert len(np.unique(allb)) == allb.size, "a block is owned twice"
    assert allb.min() >= 0 and allb.max() < inp.num_blocks
    owned = np.zeros((inp.num_blocks, MI.BLOCK), dtype=bool)
    for b in range(B):
        for t in range(int(inp.seq_lens[b])):
            owned[inp.block_table[b, t // MI.BLOCK], t % MI.BLOCK] = True
    if wl.cache_dtype == "fp8":
        assert (inp.latent[~owned] == MI.E4M3_NAN).all()
        assert (inp.rope[~owned] == MI.BF16_NAN).all()
        assert np.isnan(inp.scale[~owned]).all() and np.isfinite(inp.scale[owned]).all()
    elif wl.cache_dtype == "bf16":
        assert (inp.latent[~owned] == MI.BF16_NAN).all()
        assert (inp.latent[owned] != MI.BF16_NAN).all()
    else:
        assert np.isnan(inp.latent[~owned]).all() and np.isfinite(inp.latent[owned]).all()


def test_full_workloads_shapes():
    """The five configurations' metadata, without drawing the large ones."""
    w = MI.WORKLOADS
    assert [w[n].batch for n in MI.WORKLOAD_ORDER] == [1, 32, 64, 1, 128]
    assert [w[n].heads for n in MI.WORKLOAD_ORDER] == [16, 128, 128, 128, 128]
    assert [w[n].q_per_seq for n in MI.WORKLOAD_ORDER] == [1, 1, 1, 1, 2]
    assert w["bf16_long_t128k_s64"].num_splits == 64
    assert w["bf16_paged_b64_ragged"].len_range == (512, 16384)
    assert MI.cache_bytes_per_token("bf16") == 1152
    assert MI.cache_bytes_per_token("fp8") == 644


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        # exact halfway cases, both parities
                        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(MI.bf16_bits(x), ref)


def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 50,
                        MI._E4M3_MID, -MI._E4M3_MID, np.float32([0, -0.0, 448, -448, 1e-9])])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(MI.e4m3_codes(x), ref)


def test_e4m3_fast_encoder_equals_table_search():
    """Every float32 bit pattern in a dense sweep of [0, 448] (and its
    negative), the code midpoints and values just beside them: the bit-level
    encoder and the search over the 127 code values agree."""
    u = np.arange(0, 0x43E00001, 97, dtype=np.uint32)  # 0 .. 448, every 97th pattern
    mids = MI._E4M3_MID
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    x = np.concatenate([u.view(np.float32), near, np.float32([0.0, 448.0, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10])])
    x = np.concatenate([x, -x])
    assert np.array_equal(MI.e4m3_codes(x), MI.e4m3_codes_by_table(x))


def test_fp8_scale_is_row_max_over_448():
    inp = MI.generate(MI.small_variants()["fp8_small_sq2"])
    b0 = inp.block_table[0, 0]
    codes = inp.latent[b0, 0]
    assert (codes & 0x7F).max() == 0x7E  # the row's largest magnitude maps to 448


def test_depaged_same_logical_cache():
    inp = MI.generate(MI.small_variants()["bf16_small_paged"])
    flat = MI.depaged(inp)
    for b in range(inp.wl.batch):
        for t in range(int(inp.seq_lens[b])):
            a = inp.latent[inp.block_table[b, t // 64], t % 64]
            c = flat.latent[flat.block_table[b, t // 64], t % 64]
            assert np.array_equal(a, c)
