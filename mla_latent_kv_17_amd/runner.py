"""Drive the four library calls for one decode step on torch device tensors.

    absorb:  q_lat = W_UK^T q_nope              (mla_absorb_q)
    decode:  o_lat, lse over the paged cache     (mla_decode)
    output:  o = W_UV o_lat                      (mla_out_uv; with num_splits > 1
             the log-sum-exp merge of the KV chunks is done on the way, by
             mla_combine_out_uv, and o_lat itself is never written;
             latent_output() runs mla_split_combine to get it)

Host-side plumbing only: uploads arrays, allocates outputs and the split-KV
workspace with torch, and calls the binding.  Inputs are any object with the
fields of a generated workload (numpy arrays in storage format).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (PagedCache, make_dims, mla_absorb_q, mla_attend_explicit, mla_attend_explicit_workspace_size,
               mla_attention_form, mla_cache_append, mla_cache_append_workspace_size, mla_combine_out_uv, mla_decode,
               mla_decode_num_splits_batch, mla_moe_gate, mla_moe_gate_workspace_size, mla_out_uv, mla_split_combine,
               MLA_BF16, MLA_F32, MLA_FP8_E4M3, MLA_FORM_EXPLICIT)

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def _dev(x: np.ndarray, kind: str, device):
    """Upload a storage-format numpy array (bf16 as uint16 bits, fp8 as uint8)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if kind == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    elif kind == "fp8":
        t = t.view(torch.uint8)
    return t.to(device)


class DeviceInputs:
    def __init__(self, inp, device="cuda"):
        wl = inp.wl
        self.wl = wl
        self.batch, self.q_per_seq, self.heads = wl.batch, wl.q_per_seq, wl.heads
        self.softmax_scale = inp.softmax_scale
        self.seq_lens_host = np.asarray(inp.seq_lens)
        self.block_table = torch.from_numpy(np.ascontiguousarray(inp.block_table)).to(device)
        self.seq_lens = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to(device)
        if wl.cache_dtype == "fp8":
            latent = _dev(inp.latent, "fp8", device)
            rope = _dev(inp.rope, "bf16", device)
            scale = torch.from_numpy(np.ascontiguousarray(inp.scale)).to(device)
            self.cache = PagedCache(latent, self.block_table, self.seq_lens, rope=rope, scale=scale)
        else:
            latent = _dev(inp.latent, wl.cache_dtype, device)
            self.cache = PagedCache(latent, self.block_table, self.seq_lens)
        self.q_nope = _dev(inp.q_nope, wl.q_dtype, device)
        self.q_rope = _dev(inp.q_rope, wl.q_dtype, device)
        self.w_uk = _dev(inp.w_uk, wl.w_dtype, device)
        self.w_uv = _dev(inp.w_uv, wl.w_dtype, device)
        self.q_dtype = _TORCH[wl.q_dtype]
        self.dims = make_dims(self.batch, self.q_per_seq, self.heads, self.softmax_scale)

    @property
    def cache_bytes(self) -> int:
        c = self.cache
        n = c.latent.numel() * c.latent.element_size()
        if c.rope is not None:
            n += c.rope.numel() * c.rope.element_size() + c.scale.numel() * 4
        return n


class DecodeStep:
    """Owns the outputs and the split workspace of one decode step
    (num_splits <= 0: the library's choice, mla_decode_num_splits_batch)."""

    def __init__(self, dev: DeviceInputs, num_splits: int = 0):
        self.dev = dev
        if num_splits <= 0:
            lens = dev.seq_lens_host
            num_splits = mla_decode_num_splits_batch(dev.dims, int(lens.astype(np.int64).sum()),
                                                     int(lens.max(initial=0)))
        self.num_splits = num_splits
        R = dev.batch * dev.q_per_seq
        H = dev.heads
        device = dev.q_nope.device
        self.q_lat = torch.empty((R, H, 512), dtype=dev.q_dtype, device=device)
        self.o_lat = torch.empty((R, H, 512), dtype=torch.float32, device=device)
        self.lse = torch.empty((R, H), dtype=torch.float32, device=device)
        self.out = torch.empty((R, H, 128), dtype=torch.float32, device=device)
        if num_splits > 1:
            # chunk partials: fp16 for the bf16 / fp8 caches (half the bytes
            # written by the decode and read by the merge), fp32 for fp32
            part = torch.float32 if dev.wl.cache_dtype == "f32" else torch.float16
            self.o_part = torch.empty((dev.batch, num_splits, dev.q_per_seq, H, 512), dtype=part, device=device)
            self.lse_part = torch.empty((dev.batch, num_splits, dev.q_per_seq, H), dtype=torch.float32,
                                        device=device)
        else:
            self.o_part = self.lse_part = None

    def absorb(self, stream=None):
        mla_absorb_q(self.dev.dims, self.dev.q_nope, self.dev.w_uk, self.q_lat, stream)

    def decode(self, stream=None):
        d = self.dev
        if self.num_splits > 1:
            mla_decode(d.dims, self.q_lat, d.q_rope, d.cache, self.num_splits, self.o_part, self.lse_part, stream)
        else:
            mla_decode(d.dims, self.q_lat, d.q_rope, d.cache, 1, self.o_lat, self.lse, stream)

    def combine(self, stream=None):
        if self.num_splits > 1:
            mla_split_combine(self.dev.dims, self.num_splits, self.o_part, self.lse_part, self.o_lat, self.lse,
                              stream)

    def project(self, stream=None):
        mla_out_uv(self.dev.dims, self.o_lat, self.dev.w_uv, self.out, stream)

    # With bf16 weights the fused merge for many query rows walks the chunks
    # a few at a time per 16-row tile, paying one memory latency per round:
    # beyond FUSED_MERGE_MAX_SPLITS chunks the separate merge, which spreads
    # rows over workgroups, is faster, unless there are at most
    # FUSED_FEW_ROWS query rows (the library then spreads each row's chunks
    # over a workgroup).  The fp32 form issues 16 chunks' loads at once and
    # is fused at every chunk count.
    FUSED_MERGE_MAX_SPLITS = 8
    FUSED_FEW_ROWS = 8
    # one chunk: from this many query rows the merged kernel (one chunk of
    # weight 1) projects faster than mla_out_uv (256 rows of 128 heads: 33.0
    # against 37.1 us; 32 rows: 11.8 against 10.7 us)
    FUSED_ONE_CHUNK_ROWS = 64

    def merge_project(self, stream=None):
        """out and lse; with 1 < num_splits the merge is fused into the
        projection (mla_combine_out_uv), except with bf16 weights beyond
        FUSED_MERGE_MAX_SPLITS chunks and FUSED_FEW_ROWS query rows, where
        mla_split_combine then mla_out_uv run.  With one chunk, mla_out_uv,
        or from FUSED_ONE_CHUNK_ROWS query rows with bf16 weights
        mla_combine_out_uv on the single chunk."""
        rows = self.dev.batch * self.dev.q_per_seq
        if (self.num_splits > self.FUSED_MERGE_MAX_SPLITS and self.dev.w_uv.dtype != torch.float32
                and rows > self.FUSED_FEW_ROWS):
            self.combine(stream)
            self.project(stream)
        elif self.num_splits > 1:
            mla_combine_out_uv(self.dev.dims, self.num_splits, self.o_part, self.lse_part, self.dev.w_uv, self.out,
                               self.lse, stream)
        elif rows >= self.FUSED_ONE_CHUNK_ROWS and self.dev.w_uv.dtype != torch.float32:
            # one chunk, many query rows: o_lat and lse as a single chunk's
            # result (the layouts coincide); the merged kernel projects them
            # faster than mla_out_uv (lse is already written)
            mla_combine_out_uv(self.dev.dims, 1, self.o_lat, self.lse, self.dev.w_uv, self.out, None, stream)
        else:
            self.project(stream)

    def latent_output(self, stream=None):
        """o_lat of the last decode (merged by mla_split_combine when split; lse untouched)."""
        if self.num_splits > 1:
            mla_split_combine(self.dev.dims, self.num_splits, self.o_part, self.lse_part, self.o_lat, None, stream)
        return self.o_lat

    def run(self, stream=None):
        self.absorb(stream)
        self.decode(stream)
        self.merge_project(stream)
        return self.out

    def run_unfused(self, stream=None):
        """The same step through mla_split_combine and mla_out_uv."""
        self.absorb(stream)
        self.decode(stream)
        self.combine(stream)
        self.project(stream)
        return self.out


class ExplicitStep:
    """Owns the workspace (rebuilt keys and values) and the outputs of one
    attention call in the explicit form (mla_attend_explicit)."""

    def __init__(self, dev: DeviceInputs, out_dtype=torch.float32):
        self.dev = dev
        R, H = dev.batch * dev.q_per_seq, dev.heads
        device = dev.q_nope.device
        n = mla_attend_explicit_workspace_size(dev.dims, dev.cache.kv.max_blocks_per_seq)
        self.workspace = torch.empty(max(n // 2, 8), dtype=torch.bfloat16, device=device)
        self.out = torch.empty((R, H, 128), dtype=out_dtype, device=device)
        self.lse = torch.empty((R, H), dtype=torch.float32, device=device)

    def run(self, stream=None, with_lse: bool = True):
        d = self.dev
        mla_attend_explicit(d.dims, d.q_nope, d.q_rope, d.cache, d.w_uk, d.w_uv, self.workspace, self.out,
                            self.lse if with_lse else None, stream)
        return self.out


def attention_step(dev: DeviceInputs, num_splits: int = 0):
    """The step in the form the library calls cheaper for these sizes
    (mla_attention_form): an ExplicitStep or a DecodeStep."""
    code = {"f32": MLA_F32, "bf16": MLA_BF16, "fp8": MLA_FP8_E4M3}[dev.wl.cache_dtype]
    if mla_attention_form(dev.dims, code) == MLA_FORM_EXPLICIT:
        return ExplicitStep(dev)
    return DecodeStep(dev, num_splits)


class CacheAppend:
    """Device copies of the append inputs (h, W_DKV, W_KR) and the append's
    workspace; run() writes the S_q new tokens of every sequence into the
    device cache of `dev` (mla_cache_append)."""

    def __init__(self, dev: DeviceInputs, app):
        self.dev = dev
        self.d_model, self.rope_theta = app.d_model, app.rope_theta
        device = dev.q_nope.device
        kind = dev.wl.w_dtype
        self.h = _dev(app.h, kind, device)
        self.w_dkv = _dev(app.w_dkv, kind, device)
        self.w_kr = _dev(app.w_kr, kind, device)
        n = mla_cache_append_workspace_size(dev.dims, app.d_model)
        self.workspace = torch.empty(max(n // 4, 4), dtype=torch.float32, device=device)

    def run(self, stream=None):
        mla_cache_append(self.dev.dims, self.d_model, self.h, self.w_dkv, self.w_kr, self.dev.cache,
                         self.workspace, self.rope_theta, stream)



class MoeGate:
    """Device copies of the gate inputs (tokens u, centroids e), its outputs
    and workspace; run() selects the top_k experts of every token
    (mla_moe_gate)."""

    def __init__(self, gi, kind: str = "bf16", device=None, with_scores: bool = False):
        device = device or torch.device("cuda", 0)
        self.u = _dev(gi.u, kind, device)
        self.e = _dev(gi.e, kind, device)
        self.top_k = gi.top_k
        tokens, d_model = gi.u.shape
        n = gi.e.shape[0]
        self.idx = torch.empty((tokens, gi.top_k), dtype=torch.int32, device=device)
        self.weight = torch.empty((tokens, gi.top_k), dtype=torch.float32, device=device)
        self.scores = torch.empty((tokens, n), dtype=torch.float32, device=device) if with_scores else None
        ws = mla_moe_gate_workspace_size(tokens, d_model, n, MLA_BF16 if kind == "bf16" else MLA_F32)
        self.workspace = torch.empty(max(ws // 4, 4), dtype=torch.float32, device=device)

    def run(self, stream=None):
        mla_moe_gate(self.u, self.e, self.top_k, self.idx, self.weight, self.workspace, self.scores, stream)
