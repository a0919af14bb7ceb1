"""The C-ABI library loads and exports what include/mla.h declares, and host
validation rejects bad calls with the documented status before any launch
(no GPU needed: every call here fails validation)."""
import ctypes
import os
import re

import pytest

import mla_latent_kv_17_amd as M

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mla.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mla_\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    syms = declared_symbols()
    assert len(syms) == 18, syms
    lib = ctypes.CDLL(M.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s
    assert sorted(M.EXPORTS) == syms


def test_source_hash_matches_the_sources():
    """The loaded library was built from the sources in the tree."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_mla_build", os.path.join(os.path.dirname(M.LIB_PATH), "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert re.fullmatch(r"[0-9a-f]{16}", M.source_hash())
    assert M.source_hash() == mod.source_hash() == mod.built_hash()


def test_version_and_status_strings():
    assert M.abi_version() == 12
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert M.status_str(code).startswith("MLA_")
    assert "UNKNOWN" in M.status_str(-99)


def _call_decode(dims, kv, ns=1, q=0x1000, qr=0x2000, o=0x3000, lse=0x4000, qdt=M.MLA_BF16, odt=M.MLA_F32):
    return M._lib.mla_decode(ctypes.byref(dims), q, qr, qdt, ctypes.byref(kv) if kv is not None else None,
                             ns, o, odt, lse, None)


def _kv(latent=0x10000, rope=0x10000 + 1024, ldt=M.MLA_BF16, rdt=M.MLA_BF16, scale=None, bs=64):
    return M.MlaPagedKV(latent, ldt, 64 * 576, 576, rope, rdt, 64 * 576, 576, scale, 64 if scale else 0,
                        bs, 10, 4, 0x20000, 0x30000)


def test_decode_validation():
    d = M.make_dims(2, 1, 128)
    assert _call_decode(d, None) == M.MLA_ERR_NULL
    assert _call_decode(d, _kv(), q=0) == M.MLA_ERR_NULL
    assert _call_decode(d, _kv(), ns=0) == M.MLA_ERR_SPLITS
    assert _call_decode(d, _kv(), ns=M.MLA_MAX_SPLITS + 1) == M.MLA_ERR_SPLITS
    assert _call_decode(d, _kv(bs=32)) == M.MLA_ERR_SHAPE
    assert _call_decode(d, _kv(), qdt=M.MLA_F32) == M.MLA_ERR_DTYPE
    assert _call_decode(d, _kv(ldt=M.MLA_FP8_E4M3)) == M.MLA_ERR_NULL           # fp8 needs a scale
    assert _call_decode(d, _kv(scale=0x50000)) == M.MLA_ERR_DTYPE               # scale only with fp8
    assert _call_decode(d, _kv(latent=0x10008)) == M.MLA_ERR_ALIGN
    assert _call_decode(d, _kv(), q=0x1004) == M.MLA_ERR_ALIGN
    bad = M.make_dims(2, M.MLA_MAX_Q_PER_SEQ + 1, 128)
    assert _call_decode(bad, _kv()) == M.MLA_ERR_SHAPE
    # fp16 partials: only for split decodes of bf16 / fp8 caches
    assert _call_decode(d, _kv(), ns=1, odt=M.MLA_F16) == M.MLA_ERR_DTYPE
    assert _call_decode(d, _kv(), ns=4, odt=M.MLA_BF16) == M.MLA_ERR_DTYPE
    assert _call_decode(d, _kv(ldt=M.MLA_F32, rdt=M.MLA_F32), ns=4, qdt=M.MLA_F32, odt=M.MLA_F16) == M.MLA_ERR_DTYPE
    bad = M.make_dims(2, 0, 128)
    assert _call_decode(bad, _kv()) == M.MLA_ERR_SHAPE
    bad = M.MlaDims(2, 1, 128, 256, 64, 128, 0.1)
    assert _call_decode(bad, _kv()) == M.MLA_ERR_SHAPE
    bad = M.MlaDims(2, 1, 128, 512, 64, 128, float("nan"))
    assert _call_decode(bad, _kv()) == M.MLA_ERR_SHAPE
    bad = M.make_dims(2, 1, 0)
    assert _call_decode(bad, _kv()) == M.MLA_ERR_SHAPE
    # batch 0: nothing to do, nothing launched
    assert _call_decode(M.make_dims(0, 1, 128), _kv()) == M.MLA_OK


def test_other_entry_points_validation():
    d = M.make_dims(2, 1, 128)
    L = M._lib
    assert L.mla_absorb_q(ctypes.byref(d), None, 0x1000, M.MLA_BF16, 0x2000, M.MLA_BF16, None) == M.MLA_ERR_NULL
    assert L.mla_absorb_q(ctypes.byref(d), 0x1000, 0x1000, M.MLA_FP8_E4M3, 0x2000, M.MLA_BF16, None) == M.MLA_ERR_DTYPE
    assert L.mla_absorb_q(ctypes.byref(d), 0x1002, 0x1000, M.MLA_BF16, 0x2000, M.MLA_BF16, None) == M.MLA_ERR_ALIGN
    assert L.mla_absorb_q(None, 0x1000, 0x1000, M.MLA_BF16, 0x2000, M.MLA_BF16, None) == M.MLA_ERR_NULL
    F32, F16 = M.MLA_F32, M.MLA_F16
    assert L.mla_split_combine(ctypes.byref(d), 0, 0x1000, F32, 0x2000, 0x3000, None, None) == M.MLA_ERR_SPLITS
    assert L.mla_split_combine(ctypes.byref(d), 4, None, F32, 0x2000, 0x3000, None, None) == M.MLA_ERR_NULL
    assert L.mla_split_combine(ctypes.byref(d), 4, 0x1004, F16, 0x2000, 0x3000, None, None) == M.MLA_ERR_ALIGN
    assert L.mla_split_combine(ctypes.byref(d), 4, 0x1000, M.MLA_BF16, 0x2000, 0x3000, None, None) == M.MLA_ERR_DTYPE
    assert L.mla_out_uv(ctypes.byref(d), 0x1000, 0x2000, M.MLA_FP8_E4M3, 0x3000, M.MLA_F32, None) == M.MLA_ERR_DTYPE
    assert L.mla_out_uv(ctypes.byref(d), 0x1000, 0x2000, M.MLA_BF16, 0x3000, M.MLA_FP8_E4M3, None) == M.MLA_ERR_DTYPE
    assert L.mla_out_uv(ctypes.byref(d), None, 0x2000, M.MLA_BF16, 0x3000, M.MLA_F32, None) == M.MLA_ERR_NULL
    assert L.mla_out_uv(ctypes.byref(d), 0x1000, 0x2000, M.MLA_BF16, 0x3008, M.MLA_BF16, None) == M.MLA_ERR_ALIGN
    assert L.mla_combine_out_uv(ctypes.byref(d), 4, 0x1000, F32, 0x2000, 0x3000, M.MLA_BF16, 0x4000, 7, None,
                                None) == M.MLA_ERR_DTYPE
    assert L.mla_combine_out_uv(ctypes.byref(d), 4, 0x1000, M.MLA_FP8_E4M3, 0x2000, 0x3000, M.MLA_BF16, 0x4000,
                                M.MLA_F32, None, None) == M.MLA_ERR_DTYPE
    assert L.mla_combine_out_uv(ctypes.byref(d), 0, 0x1000, F16, 0x2000, 0x3000, M.MLA_BF16, 0x4000, M.MLA_F32, None,
                                None) == M.MLA_ERR_SPLITS
    out = ctypes.c_int32(0)
    assert L.mla_decode_num_splits(ctypes.byref(d), 100, None) == M.MLA_ERR_NULL
    assert L.mla_decode_num_splits(ctypes.byref(d), -1, ctypes.byref(out)) == M.MLA_ERR_SHAPE


def test_cache_append_validation():
    d = M.make_dims(2, 1, 128)
    L = M._lib
    n = ctypes.c_int64(0)
    assert L.mla_cache_append_workspace_size(ctypes.byref(d), 5120, ctypes.byref(n)) == M.MLA_OK
    assert n.value == 10 * 2 * 576 * 4
    assert L.mla_cache_append_workspace_size(ctypes.byref(d), 100, ctypes.byref(n)) == M.MLA_ERR_SHAPE
    assert L.mla_cache_append_workspace_size(ctypes.byref(d), 5120, None) == M.MLA_ERR_NULL

    def call(d_model=640, h=0x1000, dt=M.MLA_BF16, theta=10000.0, kv=None, ws=0x9000, wsb=1 << 20):
        kv = kv if kv is not None else _kv()
        return L.mla_cache_append(ctypes.byref(d), d_model, h, 0x2000, 0x3000, dt, theta, ctypes.byref(kv), ws,
                                  wsb, None)
    assert call(h=0) == M.MLA_ERR_NULL
    assert call(ws=0) == M.MLA_ERR_NULL
    assert call(d_model=96) == M.MLA_ERR_SHAPE
    assert call(d_model=65536 + 64) == M.MLA_ERR_SHAPE
    assert call(theta=0.0) == M.MLA_ERR_SHAPE
    assert call(theta=float("inf")) == M.MLA_ERR_SHAPE
    assert call(dt=M.MLA_F32) == M.MLA_ERR_DTYPE                      # fp32 inputs need an fp32 cache
    assert call(kv=_kv(ldt=M.MLA_FP8_E4M3)) == M.MLA_ERR_NULL          # fp8 needs a scale
    assert call(h=0x1008) == M.MLA_ERR_ALIGN
    assert call(wsb=2 * 2 * 576 * 4 - 4) == M.MLA_ERR_SHAPE             # 640 wide: two chunks
    assert call(kv=_kv(bs=32)) == M.MLA_ERR_SHAPE
    assert L.mla_cache_append(ctypes.byref(M.make_dims(0, 1, 128)), 640, 0x1000, 0x2000, 0x3000, M.MLA_BF16,
                              10000.0, ctypes.byref(_kv()), 0x9000, 0, None) == M.MLA_OK  # nothing to do


def test_cache_append_static_validation():
    """The no-allocation append validates like mla_cache_append and refuses a
    call whose partial sums exceed its fixed scratch before touching any
    device (every call here returns before a launch)."""
    L = M._lib

    def call(batch=2, sq=1, d_model=640, h=0x1000, dt=M.MLA_BF16, kv=None):
        kv = kv if kv is not None else _kv()
        return L.mla_cache_append_static(ctypes.byref(M.make_dims(batch, sq, 128)), d_model, h, 0x2000, 0x3000, dt,
                                         10000.0, ctypes.byref(kv), None)
    assert call(h=0) == M.MLA_ERR_NULL
    assert call(d_model=96) == M.MLA_ERR_SHAPE
    assert call(dt=M.MLA_F32) == M.MLA_ERR_DTYPE
    assert call(h=0x1008) == M.MLA_ERR_ALIGN
    # d_model 5120: 10 chunks x 576 x 4 bytes per token; 728 tokens fit in 16 MiB, 729 do not
    assert 728 * 10 * 576 * 4 <= M.MLA_STATIC_SCRATCH_BYTES < 729 * 10 * 576 * 4
    assert call(batch=729, d_model=5120) == M.MLA_ERR_SCRATCH
    assert call(batch=243, sq=3, d_model=5120) == M.MLA_ERR_SCRATCH
    assert call(batch=0) == M.MLA_OK  # nothing to do, no device touched
    assert "scratch" in M.status_str(M.MLA_ERR_SCRATCH)



def test_moe_gate_validation():
    L = M._lib
    n = ctypes.c_int64(0)
    assert L.mla_moe_gate_workspace_size(32, 5120, 160, M.MLA_BF16, ctypes.byref(n)) == M.MLA_OK
    assert n.value == 10 * 32 * 160 * 4
    assert L.mla_moe_gate_workspace_size(32, 5120, 160, M.MLA_F32, ctypes.byref(n)) == M.MLA_OK
    assert n.value == 32 * 160 * 4
    # from 768 tokens on: slices cut for about 256 workgroups of 128 tokens (4096 tokens: 8 slices of 640)
    assert L.mla_moe_gate_workspace_size(4096, 5120, 160, M.MLA_BF16, ctypes.byref(n)) == M.MLA_OK
    assert n.value == 8 * 4096 * 160 * 4
    # partial rows padded to a multiple of 4 experts
    assert L.mla_moe_gate_workspace_size(800, 640, 101, M.MLA_BF16, ctypes.byref(n)) == M.MLA_OK
    assert n.value == 1 * 800 * 104 * 4
    assert L.mla_moe_gate_workspace_size(800, 640, 160, M.MLA_BF16, ctypes.byref(n)) == M.MLA_OK
    assert n.value == 1 * 800 * 160 * 4
    assert L.mla_moe_gate_workspace_size(700, 640, 160, M.MLA_BF16, ctypes.byref(n)) == M.MLA_OK
    assert n.value == 2 * 700 * 160 * 4                                 # below 768 tokens: 512-wide slices
    assert L.mla_moe_gate_workspace_size(32, 5120, 257, M.MLA_BF16, ctypes.byref(n)) == M.MLA_ERR_SHAPE
    assert L.mla_moe_gate_workspace_size(32, 5120, 160, M.MLA_FP8_E4M3, ctypes.byref(n)) == M.MLA_ERR_DTYPE
    assert L.mla_moe_gate_workspace_size(32, 5120, 160, M.MLA_BF16, None) == M.MLA_ERR_NULL

    def call(T=32, D=640, N=160, K=6, u=0x1000, e=0x2000, dt=M.MLA_BF16, idx=0x3000, w=0x4000, sc=None,
             ws=0x9000, wsb=1 << 20):
        return L.mla_moe_gate(T, D, N, K, u, e, dt, idx, w, sc, ws, wsb, None)
    assert call(u=0) == M.MLA_ERR_NULL
    assert call(idx=0) == M.MLA_ERR_NULL
    assert call(ws=0) == M.MLA_ERR_NULL
    assert call(D=100) == M.MLA_ERR_SHAPE
    assert call(D=65536 + 64) == M.MLA_ERR_SHAPE
    assert call(N=0) == M.MLA_ERR_SHAPE
    assert call(N=257) == M.MLA_ERR_SHAPE
    assert call(K=0) == M.MLA_ERR_SHAPE
    assert call(K=17, N=160) == M.MLA_ERR_SHAPE
    assert call(K=5, N=4) == M.MLA_ERR_SHAPE
    assert call(T=-1) == M.MLA_ERR_SHAPE
    assert call(T=65536, dt=M.MLA_F32) == M.MLA_ERR_SHAPE
    assert call(T=65535 * 32 + 1) == M.MLA_ERR_SHAPE                   # the largest bf16 token count is 2097120
    assert call(dt=M.MLA_FP8_E4M3) == M.MLA_ERR_DTYPE
    assert call(u=0x1008) == M.MLA_ERR_ALIGN
    assert call(w=0x4002) == M.MLA_ERR_ALIGN
    assert call(sc=0x5001) == M.MLA_ERR_ALIGN
    assert call(wsb=2 * 32 * 160 * 4 - 4) == M.MLA_ERR_SHAPE          # 640 wide: two chunks
    assert call(T=0, wsb=0) == M.MLA_OK                                 # nothing to do
    assert call(T=0, u=0, idx=0, w=0, ws=0, wsb=0) == M.MLA_OK          # ... and no pointer read
    assert call(T=0, K=0) == M.MLA_ERR_SHAPE                            # sizes still checked


def _call_explicit(dims, kv, qn=0x1000, qr=0x2000, wk=0x3000, wv=0x4000, ws=0x5000, ws_bytes=1 << 40, out=0x6000,
                   idt=M.MLA_BF16, odt=M.MLA_F32):
    return M._lib.mla_attend_explicit(ctypes.byref(dims), qn, qr, idt, ctypes.byref(kv) if kv is not None else None,
                                      wk, wv, ws, ws_bytes, out, odt, None, None)


def test_explicit_validation():
    d = M.make_dims(2, 300, 16)
    n = ctypes.c_int64(0)
    assert M._lib.mla_attend_explicit_workspace_size(ctypes.byref(d), 4, ctypes.byref(n)) == M.MLA_OK
    assert n.value == 2 * 16 * 256 * 128 * 2 * 2          # 4 pages = 256 tokens
    assert M._lib.mla_attend_explicit_workspace_size(ctypes.byref(d), 5, ctypes.byref(n)) == M.MLA_OK
    assert n.value == 2 * 16 * 512 * 128 * 2 * 2          # 320 tokens round up to 512
    assert M._lib.mla_attend_explicit_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == M.MLA_ERR_SHAPE
    assert M._lib.mla_attend_explicit_workspace_size(ctypes.byref(d), 4, None) == M.MLA_ERR_NULL
    assert M._lib.mla_attend_explicit_workspace_size(ctypes.byref(d), (1 << 18) + 1, ctypes.byref(n)) == \
        M.MLA_ERR_SHAPE                                     # more than 2^24 tokens
    assert _call_explicit(d, None) == M.MLA_ERR_NULL
    assert _call_explicit(d, _kv(), ws=0) == M.MLA_ERR_NULL
    assert _call_explicit(d, _kv(), wv=0) == M.MLA_ERR_NULL
    assert _call_explicit(d, _kv(), idt=M.MLA_F32) == M.MLA_ERR_DTYPE
    assert _call_explicit(d, _kv(ldt=M.MLA_FP8_E4M3, scale=0x50000)) == M.MLA_ERR_DTYPE
    assert _call_explicit(d, _kv(ldt=M.MLA_F32, rdt=M.MLA_F32)) == M.MLA_ERR_DTYPE
    assert _call_explicit(d, _kv(), odt=M.MLA_F16) == M.MLA_ERR_DTYPE
    assert _call_explicit(d, _kv(bs=32)) == M.MLA_ERR_SHAPE
    assert _call_explicit(d, _kv(), wk=0x3008) == M.MLA_ERR_ALIGN
    assert _call_explicit(d, _kv(), ws=0x5004) == M.MLA_ERR_ALIGN
    need = 2 * 16 * 256 * 128 * 2 * 2                      # _kv(): 4 blocks per sequence
    assert _call_explicit(d, _kv(), ws_bytes=need - 1) == M.MLA_ERR_SHAPE
    assert _call_explicit(M.make_dims(2, M.MLA_MAX_Q_PER_SEQ + 1, 16), _kv()) == M.MLA_ERR_SHAPE
    # batch 0: nothing to do, nothing launched
    assert _call_explicit(M.make_dims(0, 300, 16), _kv(), ws_bytes=0) == M.MLA_OK


def test_attention_form():
    """The explicit form from MLA_EXPLICIT_MIN_Q query tokens per sequence on,
    for a bf16 cache only."""
    form = ctypes.c_int32(-1)
    L = M._lib
    for sq, ldt, want in [(1, M.MLA_BF16, M.MLA_FORM_ABSORBED), (M.MLA_EXPLICIT_MIN_Q - 1, M.MLA_BF16,
                                                                 M.MLA_FORM_ABSORBED),
                          (M.MLA_EXPLICIT_MIN_Q, M.MLA_BF16, M.MLA_FORM_EXPLICIT),
                          (4096, M.MLA_BF16, M.MLA_FORM_EXPLICIT), (4096, M.MLA_FP8_E4M3, M.MLA_FORM_ABSORBED),
                          (4096, M.MLA_F32, M.MLA_FORM_ABSORBED)]:
        assert L.mla_attention_form(ctypes.byref(M.make_dims(4, sq, 128)), ldt, ctypes.byref(form)) == M.MLA_OK
        assert form.value == want, (sq, ldt)
    assert L.mla_attention_form(ctypes.byref(M.make_dims(4, 8, 128)), 7, ctypes.byref(form)) == M.MLA_ERR_DTYPE
    assert L.mla_attention_form(ctypes.byref(M.make_dims(4, 8, 128)), M.MLA_BF16, None) == M.MLA_ERR_NULL


def test_num_splits_batch_validation():
    """Validation of mla_decode_num_splits_batch (the choice itself reads the
    device's compute units: covered by the GPU tests)."""
    d = M.make_dims(2, 1, 128)
    L = M._lib
    ns = ctypes.c_int32(-1)
    assert L.mla_decode_num_splits_batch(ctypes.byref(d), 10, 4, ctypes.byref(ns)) == M.MLA_ERR_SHAPE  # above 2 x 4
    assert L.mla_decode_num_splits_batch(ctypes.byref(d), -1, 4, ctypes.byref(ns)) == M.MLA_ERR_SHAPE
    assert L.mla_decode_num_splits_batch(ctypes.byref(d), 8, -1, ctypes.byref(ns)) == M.MLA_ERR_SHAPE
    assert L.mla_decode_num_splits_batch(ctypes.byref(d), 4, 4, None) == M.MLA_ERR_NULL
    assert L.mla_decode_num_splits_batch(None, 4, 4, ctypes.byref(ns)) == M.MLA_ERR_NULL
