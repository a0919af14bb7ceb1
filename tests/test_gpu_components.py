"""Each C-ABI entry point on its own against the oracle's definition of that
step: mla_absorb_q, mla_out_uv, mla_split_combine and mla_combine_out_uv, at
row counts that span several row tiles with a ragged tail, and at the largest
split count."""
import math

import numpy as np
import pytest

import mla_inputs as MI
import oracle as O
from parity import check, metrics

pytestmark = pytest.mark.gpu

H = 128


def _bf16_tensor(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.int16).view(torch.bfloat16).to(device)


def _weights(rng, std=1.0 / math.sqrt(512)):
    return MI.bf16_bits(rng.standard_normal((H, 128, 512), dtype=np.float32) * np.float32(std))


@pytest.mark.parametrize("rows", [1, 37, 256])
def test_absorb_q_bf16(rows):
    import torch
    import mla_latent_kv_17_amd as M
    print(f"[case] absorb_q bf16 rows={rows}", flush=True)
    rng = np.random.default_rng(3000 + rows)
    qn = MI.bf16_bits(rng.standard_normal((rows, H, 128), dtype=np.float32))
    w = _weights(rng)
    q_lat = torch.empty((rows, H, 512), dtype=torch.bfloat16, device="cuda")
    M.mla_absorb_q(M.make_dims(rows, 1, H), _bf16_tensor(qn), _bf16_tensor(w), q_lat)
    got = q_lat.float().cpu().numpy().astype(np.float64)
    ref = O.absorb_queries(O.decode_bf16(qn), O.decode_bf16(w))
    # fp32 sums of exact products, rounded once to bf16 (nearest-even):
    # within half a bf16 step of the value, plus fp32 summation error
    bound = np.abs(ref) * 2.0 ** -8 + 1e-6
    worst = float(np.max(np.abs(got - ref) - bound))
    print(f"[parity] absorb rows={rows}: max excess over bf16 rounding bound {worst:.3e}", flush=True)
    assert worst <= 0.0


def test_absorb_q_f32_out():
    import torch
    import mla_latent_kv_17_amd as M
    rows = 33
    rng = np.random.default_rng(3100)
    qn = MI.bf16_bits(rng.standard_normal((rows, H, 128), dtype=np.float32))
    w = _weights(rng)
    q_lat = torch.empty((rows, H, 512), dtype=torch.float32, device="cuda")
    M.mla_absorb_q(M.make_dims(rows, 1, H), _bf16_tensor(qn), _bf16_tensor(w), q_lat)
    ref = O.absorb_queries(O.decode_bf16(qn), O.decode_bf16(w))
    check("absorb f32 out", q_lat.cpu().numpy(), ref, "f32")


@pytest.mark.parametrize("rows", [1, 37, 256])
def test_out_uv_bf16_weights(rows):
    import torch
    import mla_latent_kv_17_amd as M
    print(f"[case] out_uv bf16 rows={rows}", flush=True)
    rng = np.random.default_rng(3200 + rows)
    o_lat = rng.standard_normal((rows, H, 512)).astype(np.float32) * np.float32(0.05)
    w = _weights(rng)
    out = torch.empty((rows, H, 128), dtype=torch.float32, device="cuda")
    M.mla_out_uv(M.make_dims(rows, 1, H), torch.from_numpy(o_lat).cuda(), _bf16_tensor(w), out)
    ref = O.project_output(o_lat, O.decode_bf16(w))
    # o_lat enters as two bf16 halves (about 16 significant bits): fp32-level
    check(f"out_uv rows={rows}", out.cpu().numpy(), ref, "f32")


@pytest.mark.parametrize("rows,wdt,ns", [(37, "bf16", 1), (5, "f32", 1), (6, "bf16", 3), (3, "f32", 3),
                                         (2, "bf16", 12), (3, "f32", 20)])
def test_projection_bf16_output(rows, wdt, ns):
    """A bf16 output is the round-to-nearest-even of the same call's fp32
    output, bit for bit (the sums are the same; only the store differs)."""
    import torch
    import mla_latent_kv_17_amd as M
    print(f"[case] projection bf16 out rows={rows} w={wdt} ns={ns}", flush=True)
    rng = np.random.default_rng(3600 + rows)
    wf = rng.standard_normal((H, 128, 512), dtype=np.float32) * np.float32(1.0 / math.sqrt(512))
    w_dev = _bf16_tensor(MI.bf16_bits(wf)) if wdt == "bf16" else torch.from_numpy(wf).cuda()
    dims = M.make_dims(rows, 1, H)
    out32 = torch.empty((rows, H, 128), dtype=torch.float32, device="cuda")
    out16 = torch.empty((rows, H, 128), dtype=torch.bfloat16, device="cuda")
    if ns == 1:
        o_lat = torch.from_numpy(rng.standard_normal((rows, H, 512)).astype(np.float32) * np.float32(0.05)).cuda()
        M.mla_out_uv(dims, o_lat, w_dev, out32)
        M.mla_out_uv(dims, o_lat, w_dev, out16)
    else:
        o_part, lse_part = _combine_case(rows, ns, 1, H, 3700 + rows)
        op, lp = torch.from_numpy(o_part * np.float32(0.05)).cuda(), torch.from_numpy(lse_part).cuda()
        M.mla_combine_out_uv(dims, ns, op, lp, w_dev, out32)
        M.mla_combine_out_uv(dims, ns, op, lp, w_dev, out16)
    got = out16.cpu().view(torch.int16).numpy().view(np.uint16)
    want = MI.bf16_bits(out32.cpu().numpy())
    assert np.array_equal(got, want)


def _combine_case(B, ns, Sq, heads, seed):
    rng = np.random.default_rng(seed)
    o_part = rng.standard_normal((B, ns, Sq, heads, 512)).astype(np.float32)
    lse_part = (rng.standard_normal((B, ns, Sq, heads)) * 3.0).astype(np.float32)
    # empty chunks: lse -inf and garbage partial rows that must get weight 0
    empty = rng.random((B, ns, Sq, heads)) < 0.3
    lse_part[empty] = -np.inf
    o_part[empty] = np.nan
    # one query row that no chunk saw
    lse_part[0, :, 0, 0] = -np.inf
    o_part[0, :, 0, 0] = np.nan
    return o_part, lse_part


def _as_part(o_part, part):
    """The partials in the storage dtype of the case: fp32 as drawn, or their
    fp16 rounding (the oracle then merges exactly those fp16 values)."""
    return o_part if part == "f32" else o_part.astype(np.float16)


@pytest.mark.parametrize("part", ["f32", "f16"])
@pytest.mark.parametrize("B,ns,Sq,heads", [(3, 5, 2, 128), (2, 64, 1, 128), (1, 1024, 1, 16), (4, 1, 1, 16)])
def test_split_combine(B, ns, Sq, heads, part):
    import torch
    import mla_latent_kv_17_amd as M
    print(f"[case] split_combine B={B} ns={ns} Sq={Sq} H={heads} partials {part}", flush=True)
    o_part, lse_part = _combine_case(B, ns, Sq, heads, 3300 + ns)
    o_part = _as_part(o_part, part)
    o_lat = torch.empty((B * Sq, heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B * Sq, heads), dtype=torch.float32, device="cuda")
    M.mla_split_combine(M.make_dims(B, Sq, heads), ns, torch.from_numpy(o_part).cuda(),
                        torch.from_numpy(lse_part).cuda(), o_lat, lse)
    o_ref, lse_ref = O.combine_partials(o_part.astype(np.float64), lse_part)
    got = o_lat.cpu().numpy().reshape(B, Sq, heads, 512)
    gl = lse.cpu().numpy().reshape(B, Sq, heads)
    assert np.isfinite(got).all()
    check(f"combine ns={ns}", got, o_ref, "f32")
    none = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(gl), none)
    assert (got[none] == 0).all()
    assert np.max(np.abs(gl[~none] - lse_ref[~none])) <= 1e-5 * max(1.0, np.abs(lse_ref[~none]).max())


@pytest.mark.parametrize("part", ["f32", "f16"])
@pytest.mark.parametrize("B,ns,Sq,heads,wdt", [(3, 5, 2, 128, "bf16"), (37, 3, 1, 100, "bf16"),
                                               (2, 64, 1, 128, "bf16"), (5, 7, 2, 16, "f32"),
                                               # several 16-row tiles per workgroup; chunks past the first 64
                                               (40, 4, 2, 128, "bf16"), (2, 130, 1, 128, "bf16"),
                                               # fp32 weights: one full round of 16 chunks, and three
                                               # rounds with a partial last one
                                               (1, 16, 1, 16, "f32"), (2, 40, 2, 16, "f32"),
                                               # bf16 beyond 8 chunks: at most 8 query rows (chunks spread
                                               # over the workgroup; the 64- and 130-chunk cases above too),
                                               # and more rows (16-row tiles, rounds of two chunks)
                                               (1, 64, 1, 128, "bf16"), (4, 12, 2, 64, "bf16"),
                                               (3, 9, 1, 16, "bf16"), (5, 20, 2, 128, "bf16"),
                                               # a single chunk (the one-chunk instance; rows with no token)
                                               (40, 1, 2, 128, "bf16"), (3, 1, 1, 16, "f32")])
def test_combine_out_uv(B, ns, Sq, heads, wdt, part):
    """The merge fused into the projection against the fp64 merge followed by
    the fp64 projection, and against mla_split_combine + mla_out_uv."""
    import torch
    import mla_latent_kv_17_amd as M
    print(f"[case] combine_out_uv B={B} ns={ns} Sq={Sq} H={heads} w={wdt} partials {part}", flush=True)
    o_part, lse_part = _combine_case(B, ns, Sq, heads, 3400 + ns)
    o_part = _as_part(o_part * np.float32(0.05), part)
    rng = np.random.default_rng(3500 + heads)
    wf = rng.standard_normal((heads, 128, 512), dtype=np.float32) * np.float32(1.0 / math.sqrt(512))
    if wdt == "bf16":
        wb = MI.bf16_bits(wf)
        w_dev, w64 = _bf16_tensor(wb), O.decode_bf16(wb)
    else:
        w_dev, w64 = torch.from_numpy(wf).cuda(), wf.astype(np.float64)
    dims = M.make_dims(B, Sq, heads)
    op, lp = torch.from_numpy(o_part).cuda(), torch.from_numpy(lse_part).cuda()
    out = torch.empty((B * Sq, heads, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B * Sq, heads), dtype=torch.float32, device="cuda")
    M.mla_combine_out_uv(dims, ns, op, lp, w_dev, out, lse)
    o_ref, lse_ref = O.combine_partials(o_part.astype(np.float64), lse_part)
    ref = O.project_output(o_ref.reshape(B * Sq, heads, 512), w64)
    got, gl = out.cpu().numpy(), lse.cpu().numpy().reshape(B, Sq, heads)
    assert np.isfinite(got).all()
    check(f"combine_out_uv ns={ns} H={heads} {wdt}", got, ref, "f32")
    none = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(gl), none)
    assert (got.reshape(B, Sq, heads, 128)[none] == 0).all()
    assert np.max(np.abs(gl[~none] - lse_ref[~none])) <= 1e-5 * max(1.0, np.abs(lse_ref[~none]).max())
    # the two-call form of the same step
    o_lat = torch.empty((B * Sq, heads, 512), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    M.mla_split_combine(dims, ns, op, lp, o_lat, None)
    M.mla_out_uv(dims, o_lat, w_dev, out2)
    m = metrics(got, out2.cpu().numpy())
    print(f"[parity] fused vs two calls: rel_l2 {m['rel_l2']:.2e} max_abs {m['max_abs']:.2e}", flush=True)
    assert m["rel_l2"] <= 1e-5  # both are fp32 merges, summed in different orders
