"""mla_cache_append against the oracle: the rows of the S_q new tokens of
every sequence (c = W_DKV h and the rotated position key, encoded as the
cache stores them) land at the right page row, within tolerance of the fp64
values, and no other byte of the cache changes (poisoned rows included).

Tolerances: bf16 and fp32 caches as for the decode outputs (the sums are
fp32; a bf16 cache rounds once more, relative 2^-9).  fp8 rows: each
dequantized value within half an E4M3 step of the fp64 value (relative 1/16,
plus the subnormal step), the scale within fp32 rounding of max|c| / 448; and
with one-hot hidden states, which make every product and sum exact, the codes
and scales are bit-exact against the oracle's encoder."""
import numpy as np
import pytest

import mla_inputs as MI
import oracle as O
from parity import check

pytestmark = pytest.mark.gpu

D_MODEL = 640  # two 512-wide chunks, the second partial


def _host_cache(cache):
    """The device cache as host numpy arrays in storage format."""
    import torch
    out = {}
    for name in ("latent", "rope", "scale"):
        t = getattr(cache, name)
        if t is None:
            continue
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        out[name] = t.numpy().copy()
    return out


def _raw(a):
    """Bytes of an array, so NaN poison compares equal to itself."""
    return np.ascontiguousarray(a).view(np.uint8)


def _decode_in(x, kind):
    return O.decode_bf16(x) if kind == "bf16" else O.decode_f32(x)


def _run(wl, d_model=D_MODEL, one_hot=False):
    import torch
    from mla_latent_kv_17_amd.runner import CacheAppend, DeviceInputs
    inp = MI.generate(wl)
    dev = DeviceInputs(inp)
    app = MI.generate_append(wl, d_model=d_model, one_hot=one_hot)
    before = _host_cache(dev.cache)
    CacheAppend(dev, app).run()
    torch.cuda.synchronize()
    after = _host_cache(dev.cache)
    kind = wl.w_dtype
    rows = O.appended_tokens(_decode_in(app.h, kind), _decode_in(app.w_dkv, kind), _decode_in(app.w_kr, kind),
                             inp.seq_lens, wl.q_per_seq, app.rope_theta)
    return inp, before, after, rows


def _untouched(inp, before, after, rows):
    """Every cache row the append does not own is bit-identical."""
    mask = np.ones(inp.latent.shape[:2], dtype=bool)
    for b, p, _, _ in rows:
        mask[inp.block_table[b][p // 64], p % 64] = False
    for name in before:
        assert np.array_equal(_raw(before[name][mask]), _raw(after[name][mask])), name
    return mask


@pytest.mark.parametrize("name", ["bf16_small_paged", "bf16_small_contig", "fp32_b1_h16_t1k"])
def test_append_bf16_f32(name):
    wl = MI.small_variants()[name]
    print(f"[case] append {name} d_model={D_MODEL}", flush=True)
    inp, before, after, rows = _run(wl)
    assert rows
    _untouched(inp, before, after, rows)
    lat = after["latent"]
    got = np.stack([lat[inp.block_table[b][p // 64], p % 64] for b, p, _, _ in rows])
    got = O.decode_bf16(got) if wl.cache_dtype == "bf16" else O.decode_f32(got)
    want = np.stack([np.concatenate([c, kr]) for _, _, c, kr in rows])
    check(f"append {name} c", got[:, :512], want[:, :512], wl.cache_dtype)
    check(f"append {name} k^R", got[:, 512:], want[:, 512:], wl.cache_dtype)


def _fp8_rows(inp, after, rows):
    codes = np.stack([after["latent"][inp.block_table[b][p // 64], p % 64] for b, p, _, _ in rows])
    scale = np.array([after["scale"][inp.block_table[b][p // 64], p % 64] for b, p, _, _ in rows])
    kr = np.stack([after["rope"][inp.block_table[b][p // 64], p % 64] for b, p, _, _ in rows])
    return codes, scale, kr


@pytest.mark.parametrize("name,lens", [("fp8_small_sq2", None), ("fp8_append_edge", (1, 70, 64, 2))])
def test_append_fp8(name, lens):
    wl = MI.small_variants()["fp8_small_sq2"]
    if lens is not None:  # a sequence shorter than S_q: its first new token has no position
        wl = wl.scaled(name=name, batch=len(lens), lens=lens, len_range=None, seed=2100)
    print(f"[case] append {name} d_model={D_MODEL}", flush=True)
    inp, before, after, rows = _run(wl)
    if lens is not None:
        assert len(rows) == 2 * len(lens) - 1
    _untouched(inp, before, after, rows)
    codes, scale, kr = _fp8_rows(inp, after, rows)
    c = np.stack([r[2] for r in rows])
    amax = np.abs(c).max(axis=1)
    assert np.all(np.abs(scale.astype(np.float64) - amax / 448) <= 1e-5 * amax / 448), "scales"
    back = O.decode_e4m3(codes) * scale[:, None].astype(np.float64)
    bound = np.abs(c) / 16 + 2.0 ** -10 * scale[:, None] + 1e-6 * np.abs(c)
    assert np.all(np.abs(back - c) <= bound), float(np.max(np.abs(back - c) - bound))
    check(f"append {name} k^R", O.decode_bf16(kr), np.stack([r[3] for r in rows]), "bf16")


def test_append_fp8_exact_codes():
    """One-hot hidden states: every sum is a single weight (exact in fp32), so
    the encoder's inputs are the oracle's and codes and scales match bit for
    bit."""
    wl = MI.small_variants()["fp8_small_sq2"]
    print("[case] append fp8 one-hot", flush=True)
    inp, before, after, rows = _run(wl, one_hot=True)
    _untouched(inp, before, after, rows)
    codes, scale, _ = _fp8_rows(inp, after, rows)
    for k, (_, _, c, _) in enumerate(rows):
        want_codes, want_scale = O.quantize_latent(c.astype(np.float32))
        assert scale[k] == want_scale, (k, scale[k], want_scale)
        assert np.array_equal(codes[k], want_codes), k


def test_append_headline_full_size():
    """B = 32, d_model = 5120 (ten chunks), the headline cache (bf16); every token."""
    wl = MI.WORKLOADS[MI.HEADLINE]
    print(f"[case] append headline d_model={MI.APPEND_D_MODEL}", flush=True)
    inp, before, after, rows = _run(wl, d_model=MI.APPEND_D_MODEL)
    assert len(rows) == wl.batch
    _untouched(inp, before, after, rows)
    lat = after["latent"]
    got = O.decode_bf16(np.stack([lat[inp.block_table[b][p // 64], p % 64] for b, p, _, _ in rows]))
    want = np.stack([np.concatenate([c, kr]) for _, _, c, kr in rows])
    check("append headline c", got[:, :512], want[:, :512], "bf16")
    check("append headline k^R", got[:, 512:], want[:, 512:], "bf16")
