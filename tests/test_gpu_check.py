"""mla_decode with MLA_CHECK=1: valid paging data gives the unchecked result
bit for bit; a block id at or past num_blocks, or a length longer than a
table row covers, is refused with MLA_ERR_SHAPE and nothing is launched.

Each invalid case is built so that the memory it names is allocated (the
block past the declared num_blocks is a real pool block; the over-long
sequence is not the last one, so its extra table entries are the next row's
valid ids): the case would stay in bounds even if the check missed it."""
import ctypes

import numpy as np
import pytest

import mla_inputs as MI

pytestmark = pytest.mark.gpu


def test_check_mode(monkeypatch):
    import torch
    import mla_latent_kv_17_amd as M
    from mla_latent_kv_17_amd.runner import DecodeStep, DeviceInputs
    print("[case] MLA_CHECK bf16_small_paged", flush=True)
    inp = MI.generate(MI.small_variants()["bf16_small_paged"])
    dev = DeviceInputs(inp)
    step = DecodeStep(dev, 1)
    step.absorb()
    monkeypatch.delenv("MLA_CHECK", raising=False)
    step.decode()
    torch.cuda.synchronize()
    ref_o, ref_lse = step.o_lat.clone(), step.lse.clone()

    monkeypatch.setenv("MLA_CHECK", "1")
    step.o_lat.fill_(float("nan"))
    step.lse.fill_(float("nan"))
    step.decode()
    torch.cuda.synchronize()
    assert torch.equal(step.o_lat, ref_o) and torch.equal(step.lse, ref_lse)

    class Cache:  # what mla_decode reads of a PagedCache
        def __init__(self, kv):
            self.kv = kv

    def decode_status(kv):
        step.o_lat.fill_(-1.0)
        try:
            M.mla_decode(dev.dims, step.q_lat, dev.q_rope, Cache(kv), 1, step.o_lat, step.lse)
        except M.MlaError as e:
            return e.status
        return 0

    # the largest block id in use, declared out of range by shrinking num_blocks to it
    lens = np.asarray(inp.seq_lens)
    table = np.asarray(inp.block_table)
    used = [int(table[b, p]) for b in range(len(lens)) for p in range((int(lens[b]) + 63) // 64)]
    kv = M.MlaPagedKV.from_buffer_copy(dev.cache.kv)
    kv.num_blocks = max(used)
    assert decode_status(kv) == -2
    torch.cuda.synchronize()
    assert bool((step.o_lat == -1.0).all()), "a refused call must launch nothing"

    # sequence 0 one token longer than its table row
    assert len(lens) > 1
    bad_lens = dev.seq_lens.clone()
    bad_lens[0] = table.shape[1] * 64 + 1
    kv = M.MlaPagedKV.from_buffer_copy(dev.cache.kv)
    kv.seq_lens = ctypes.c_void_p(bad_lens.data_ptr()).value
    assert decode_status(kv) == -2
    torch.cuda.synchronize()
    assert bool((step.o_lat == -1.0).all())
