"""The four calls of a decode step captured as a HIP graph: every replay,
with eager work and synchronisation between replays, reproduces the eager
step bit for bit (the library allocates nothing and issues no memsets)."""
import numpy as np
import pytest

import mla_inputs as MI

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,ns", [("bf16_small_split", 7), ("bf16_small_paged", 1), ("fp8_small_sq2", 2),
                                     # merges fused beyond 8 chunks: one query row (bf16), fp32 weights
                                     ("bf16_small_split", 12), ("fp32_b1_h16_t1k", 16)])
def test_graph_replays_match_eager(name, ns):
    import torch
    from mla_latent_kv_17_amd.runner import DecodeStep, DeviceInputs
    print(f"[case] graph {name} ns={ns}", flush=True)
    inp = MI.generate(MI.small_variants()[name])
    step = DecodeStep(DeviceInputs(inp), ns)
    ref = step.run().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    scratch = torch.empty(1 << 22, device="cuda")
    for i in range(4):
        step.out.fill_(float("nan"))     # eager work between replays
        scratch.normal_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref), f"replay {i} differs"
