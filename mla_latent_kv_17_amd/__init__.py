"""Python binding of libmla.so, the C-ABI MLA absorbed-decode library for
MI355X (gfx950).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C entry point of the same name and raises on a
non-zero status.  All arithmetic runs in the library's HIP kernels; PyTorch
provides device memory and streams.  The library must have been built
(``python mla_latent_kv_17_amd/build.py``); importing fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_F32, MLA_BF16, MLA_FP8_E4M3, MLA_F16 = 0, 1, 2, 3
MLA_OK = 0
MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DTYPE, MLA_ERR_ALIGN = -1, -2, -3, -4
MLA_ERR_SPLITS, MLA_ERR_LAUNCH, MLA_ERR_DEVICE, MLA_ERR_SCRATCH = -5, -6, -7, -8
MLA_STATIC_SCRATCH_BYTES = 16 << 20
MLA_MAX_SPLITS = 1024
MLA_MAX_Q_PER_SEQ = 4096
MLA_FORM_ABSORBED, MLA_FORM_EXPLICIT = 0, 1
MLA_EXPLICIT_MIN_Q = 288
D_LATENT, D_ROPE, D_HEAD, BLOCK = 512, 64, 128, 64

# the C entry points this binding exposes (also checked by the tests)
EXPORTS = ["mla_status_str", "mla_abi_version", "mla_source_hash", "mla_absorb_q", "mla_decode",
           "mla_split_combine", "mla_out_uv", "mla_combine_out_uv", "mla_decode_num_splits",
           "mla_cache_append", "mla_cache_append_workspace_size", "mla_cache_append_static", "mla_moe_gate",
           "mla_moe_gate_workspace_size", "mla_attend_explicit", "mla_attend_explicit_workspace_size",
           "mla_attention_form", "mla_decode_num_splits_batch"]
MLA_GATE_MAX_EXPERTS, MLA_GATE_MAX_TOP_K = 256, 16


class MlaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_per_seq", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class MlaPagedKV(ctypes.Structure):
    _fields_ = [("latent", ctypes.c_void_p), ("latent_dtype", ctypes.c_int32),
                ("latent_block_stride", ctypes.c_int64), ("latent_row_stride", ctypes.c_int64),
                ("rope", ctypes.c_void_p), ("rope_dtype", ctypes.c_int32),
                ("rope_block_stride", ctypes.c_int64), ("rope_row_stride", ctypes.c_int64),
                ("scale", ctypes.c_void_p), ("scale_block_stride", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p)]


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


def _hip_runtimes():
    try:
        maps = open("/proc/self/maps").read().splitlines()
    except OSError:
        return set()
    return {ln.split()[-1] for ln in maps if "libamdhip64" in ln}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python mla_latent_kv_17_amd/build.py`")
    # torch brings its own HIP runtime; load it first so that libmla.so binds to
    # the same runtime (same soname) instead of a second copy whose streams and
    # allocations would be foreign to torch's.
    import torch  # noqa: F401
    torch.cuda.is_available  # the HIP runtime is loaded with torch's extension
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped ({sorted(runtimes)}); import torch before loading "
                          f"{LIB_PATH} by any other route")
    vp, i32, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    dp, kvp = ctypes.POINTER(MlaDims), ctypes.POINTER(MlaPagedKV)
    sig = {
        "mla_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "mla_abi_version": ([], ctypes.c_int),
        "mla_source_hash": ([], ctypes.c_char_p),
        "mla_absorb_q": ([dp, vp, vp, i32, vp, i32, vp], ctypes.c_int),
        "mla_decode": ([dp, vp, vp, i32, kvp, i32, vp, i32, f32p, vp], ctypes.c_int),
        "mla_split_combine": ([dp, i32, vp, i32, f32p, f32p, f32p, vp], ctypes.c_int),
        "mla_out_uv": ([dp, f32p, vp, i32, vp, i32, vp], ctypes.c_int),
        "mla_combine_out_uv": ([dp, i32, vp, i32, f32p, vp, i32, vp, i32, f32p, vp], ctypes.c_int),
        "mla_decode_num_splits": ([dp, i32, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
        "mla_cache_append": ([dp, i32, vp, vp, vp, i32, ctypes.c_float, kvp, vp, ctypes.c_int64, vp], ctypes.c_int),
        "mla_cache_append_workspace_size": ([dp, i32, ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
        "mla_cache_append_static": ([dp, i32, vp, vp, vp, i32, ctypes.c_float, kvp, vp], ctypes.c_int),
        "mla_moe_gate": ([i32, i32, i32, i32, vp, vp, i32, vp, f32p, f32p, vp, ctypes.c_int64, vp], ctypes.c_int),
        "mla_moe_gate_workspace_size": ([i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
        "mla_attend_explicit": ([dp, vp, vp, i32, kvp, vp, vp, vp, ctypes.c_int64, vp, i32, f32p, vp], ctypes.c_int),
        "mla_attend_explicit_workspace_size": ([dp, i32, ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
        "mla_attention_form": ([dp, i32, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
        "mla_decode_num_splits_batch": ([dp, ctypes.c_int64, i32, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    # a library built from other sources than the ones beside it is refused
    built, want = lib.mla_source_hash().decode(), _build_script().source_hash()
    if built != want:
        raise ImportError(f"{LIB_PATH} was built from other sources (hash {built}, sources {want}); "
                          f"rebuild with `python mla_latent_kv_17_amd/build.py`")
    return lib


def _build_script():
    """build.py, loaded by path (it holds the source hash; importing it as a
    submodule would import this package first)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_mla_build", os.path.join(_HERE, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_lib = _load()


def status_str(status: int) -> str:
    return _lib.mla_status_str(int(status)).decode()


def abi_version() -> int:
    return int(_lib.mla_abi_version())


def source_hash() -> str:
    """Hash of the sources the loaded library was built from."""
    return _lib.mla_source_hash().decode()


def _check(fn: str, status: int):
    if status != MLA_OK:
        raise MlaError(fn, status)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: MLA_F32, torch.bfloat16: MLA_BF16, torch.float16: MLA_F16,
            torch.float8_e4m3fn: MLA_FP8_E4M3, torch.uint8: MLA_FP8_E4M3}[t.dtype]


def make_dims(batch: int, q_per_seq: int, heads: int, softmax_scale: Optional[float] = None) -> MlaDims:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D_HEAD + D_ROPE)
    return MlaDims(batch, q_per_seq, heads, D_LATENT, D_ROPE, D_HEAD, softmax_scale)


class PagedCache:
    """Describes a paged latent cache held in torch device tensors.

    ``latent``: [num_blocks][64][576] (f32/bf16, c | k^R interleaved) when
    ``rope`` is None; else the fp8 codes [num_blocks][64][512] with
    ``rope`` bf16 [num_blocks][64][64] and ``scale`` fp32 [num_blocks][64].
    ``block_table`` int32 [B][max_blocks], ``seq_lens`` int32 [B]."""

    def __init__(self, latent, block_table, seq_lens, rope=None, scale=None):
        self.latent, self.rope, self.scale = latent, rope, scale
        self.block_table, self.seq_lens = block_table, seq_lens
        nb = latent.shape[0]
        if rope is None:
            ld = _dtype_code(latent)
            row = latent.shape[2]
            self.kv = MlaPagedKV(latent.data_ptr(), ld, BLOCK * row, row,
                                 latent.data_ptr() + D_LATENT * latent.element_size(), ld, BLOCK * row, row,
                                 None, 0, BLOCK, nb, block_table.shape[1],
                                 block_table.data_ptr(), seq_lens.data_ptr())
        else:
            self.kv = MlaPagedKV(latent.data_ptr(), MLA_FP8_E4M3, BLOCK * D_LATENT, D_LATENT,
                                 rope.data_ptr(), _dtype_code(rope), BLOCK * D_ROPE, D_ROPE,
                                 _ptr(scale), BLOCK, BLOCK, nb, block_table.shape[1],
                                 block_table.data_ptr(), seq_lens.data_ptr())


def mla_absorb_q(dims: MlaDims, q_nope, w_uk, q_lat, stream=None):
    """q_lat[r][h][:] = W_UK[h]^T q_nope[r][h][:]."""
    _check("mla_absorb_q", _lib.mla_absorb_q(ctypes.byref(dims), _ptr(q_nope), _ptr(w_uk), _dtype_code(q_nope),
                                             _ptr(q_lat), _dtype_code(q_lat), _stream(stream)))


def mla_decode(dims: MlaDims, q_lat, q_rope, cache: PagedCache, num_splits: int, o, lse, stream=None):
    """Decode attention over the paged latent cache; o/lse are o_lat/lse
    (num_splits == 1) or the per-chunk partials (num_splits > 1; o fp32, or
    fp16 with a bf16 / fp8 cache)."""
    _check("mla_decode", _lib.mla_decode(ctypes.byref(dims), _ptr(q_lat), _ptr(q_rope), _dtype_code(q_lat),
                                         ctypes.byref(cache.kv), int(num_splits), _ptr(o), _dtype_code(o),
                                         _ptr(lse), _stream(stream)))


def mla_decode_num_splits_batch(dims: MlaDims, total_tokens: int, max_seq_len: int) -> int:
    """num_splits for mla_decode from the sum and the maximum of the cached lengths."""
    out = ctypes.c_int32(0)
    _check("mla_decode_num_splits_batch", _lib.mla_decode_num_splits_batch(ctypes.byref(dims), int(total_tokens),
                                                                           int(max_seq_len), ctypes.byref(out)))
    return int(out.value)


def mla_split_combine(dims: MlaDims, num_splits: int, o_part, lse_part, o_lat, lse=None, stream=None):
    """o_lat (fp32) and lse merged from the chunk partials (o_part fp32 or fp16)."""
    _check("mla_split_combine", _lib.mla_split_combine(ctypes.byref(dims), int(num_splits), _ptr(o_part),
                                                       _dtype_code(o_part), _ptr(lse_part), _ptr(o_lat), _ptr(lse),
                                                       _stream(stream)))


def mla_out_uv(dims: MlaDims, o_lat, w_uv, out, stream=None):
    """out[r][h][:] = W_UV[h] o_lat[r][h][:]; out is fp32 or bf16."""
    _check("mla_out_uv", _lib.mla_out_uv(ctypes.byref(dims), _ptr(o_lat), _ptr(w_uv), _dtype_code(w_uv),
                                         _ptr(out), _dtype_code(out), _stream(stream)))


def mla_combine_out_uv(dims: MlaDims, num_splits: int, o_part, lse_part, w_uv, out, lse=None, stream=None):
    """out[r][h][:] = W_UV[h] (log-sum-exp merge of the chunk partials), lse = merged lse; out is fp32 or bf16."""
    _check("mla_combine_out_uv", _lib.mla_combine_out_uv(ctypes.byref(dims), int(num_splits), _ptr(o_part),
                                                         _dtype_code(o_part), _ptr(lse_part), _ptr(w_uv),
                                                         _dtype_code(w_uv), _ptr(out), _dtype_code(out), _ptr(lse),
                                                         _stream(stream)))


def mla_decode_num_splits(dims: MlaDims, max_seq_len: int) -> int:
    out = ctypes.c_int32(0)
    _check("mla_decode_num_splits", _lib.mla_decode_num_splits(ctypes.byref(dims), int(max_seq_len),
                                                               ctypes.byref(out)))
    return int(out.value)


def mla_cache_append_workspace_size(dims: MlaDims, d_model: int) -> int:
    """Bytes of workspace mla_cache_append needs."""
    out = ctypes.c_int64(0)
    _check("mla_cache_append_workspace_size",
           _lib.mla_cache_append_workspace_size(ctypes.byref(dims), int(d_model), ctypes.byref(out)))
    return int(out.value)


def mla_cache_append(dims: MlaDims, d_model: int, h, w_dkv, w_kr, cache: PagedCache, workspace,
                     rope_theta: float = 10000.0, stream=None):
    """Write c = W_DKV h and k^R = RoPE_p(W_KR h) of the S_q newest tokens of each
    sequence (position p = len - S_q + i) into the paged cache."""
    _check("mla_cache_append", _lib.mla_cache_append(ctypes.byref(dims), int(d_model), _ptr(h), _ptr(w_dkv),
                                                     _ptr(w_kr), _dtype_code(h), float(rope_theta),
                                                     ctypes.byref(cache.kv), _ptr(workspace),
                                                     int(workspace.numel() * workspace.element_size()),
                                                     _stream(stream)))


def mla_cache_append_static(dims: MlaDims, d_model: int, h, w_dkv, w_kr, cache: PagedCache,
                            rope_theta: float = 10000.0, stream=None):
    """mla_cache_append with the partial sums in the library's fixed per-GPU
    scratch instead of a workspace (allocates nothing; calls that overlap on
    one GPU race)."""
    _check("mla_cache_append_static",
           _lib.mla_cache_append_static(ctypes.byref(dims), int(d_model), _ptr(h), _ptr(w_dkv), _ptr(w_kr),
                                        _dtype_code(h), float(rope_theta), ctypes.byref(cache.kv),
                                        _stream(stream)))


def mla_moe_gate_workspace_size(tokens: int, d_model: int, n_experts: int, in_dtype: int) -> int:
    """Bytes of workspace mla_moe_gate needs."""
    out = ctypes.c_int64(0)
    _check("mla_moe_gate_workspace_size",
           _lib.mla_moe_gate_workspace_size(int(tokens), int(d_model), int(n_experts), int(in_dtype),
                                            ctypes.byref(out)))
    return int(out.value)


def mla_moe_gate(u, e, top_k: int, idx, weight, workspace, scores=None, stream=None):
    """The routed experts of each token (rows of u [tokens][d_model]) over the
    centroids e [n_experts][d_model]: idx [tokens][top_k] int32 (largest score
    first), weight [tokens][top_k] fp32 = their softmax scores, and every
    score into scores [tokens][n_experts] if given."""
    tokens, d_model = u.shape
    if e.dtype != u.dtype or e.dim() != 2 or e.shape[1] != d_model:
        raise ValueError(f"centroids {tuple(e.shape)} {e.dtype} do not match tokens {tuple(u.shape)} {u.dtype}")
    _check("mla_moe_gate", _lib.mla_moe_gate(int(tokens), int(d_model), int(e.shape[0]), int(top_k), _ptr(u),
                                             _ptr(e), _dtype_code(u), _ptr(idx), _ptr(weight), _ptr(scores),
                                             _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                             _stream(stream)))


def mla_attend_explicit_workspace_size(dims: MlaDims, max_blocks_per_seq: int) -> int:
    """Bytes of workspace mla_attend_explicit needs."""
    out = ctypes.c_int64(0)
    _check("mla_attend_explicit_workspace_size",
           _lib.mla_attend_explicit_workspace_size(ctypes.byref(dims), int(max_blocks_per_seq), ctypes.byref(out)))
    return int(out.value)


def mla_attend_explicit(dims: MlaDims, q_nope, q_rope, cache: PagedCache, w_uk, w_uv, workspace, out, lse=None,
                        stream=None):
    """Attention in the explicit form: K = [W_UK c ; k^R] and V = W_UV c rebuilt
    per head into the workspace, then softmax attention on them; out is fp32
    or bf16 [B*S_q][H][128], lse [B*S_q][H] fp32 or None."""
    _check("mla_attend_explicit",
           _lib.mla_attend_explicit(ctypes.byref(dims), _ptr(q_nope), _ptr(q_rope), _dtype_code(q_nope),
                                    ctypes.byref(cache.kv), _ptr(w_uk), _ptr(w_uv), _ptr(workspace),
                                    int(workspace.numel() * workspace.element_size()), _ptr(out), _dtype_code(out),
                                    _ptr(lse), _stream(stream)))


def mla_attention_form(dims: MlaDims, latent_dtype: int) -> int:
    """MLA_FORM_EXPLICIT or MLA_FORM_ABSORBED: the cheaper form for these sizes."""
    out = ctypes.c_int32(0)
    _check("mla_attention_form", _lib.mla_attention_form(ctypes.byref(dims), int(latent_dtype), ctypes.byref(out)))
    return int(out.value)
