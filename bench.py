"""Benchmark: MLA absorbed decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = the whole decode path for one batch: mla_absorb_q, mla_decode,
mla_split_combine (when the context is split) and mla_out_uv, on the
synthetic workload B=32, H=128, T=4096, bf16 cache/queries/weights
(d_latent 512, d_rope 64, d_head 128), inputs resident in HBM.

Before every timed step an untimed read of a 1 GiB buffer evicts the 256 MB
Infinity Cache and the L2s, so the step streams its cache and weights from
HBM as it would with other layers' data in between.  HIP events on the
stream the library launches on (torch's current stream) bracket each step;
none sits between the step's four launches, because an event recorded
between two kernels delays the second by about 6 us.  The decode kernel on
its own (the roofline line) is timed as K launches back to back between two
events, each launch on its own copy of the cache, the copies together being
several times larger than the Infinity Cache, so every launch streams from
HBM.  --graph also times the step replayed from a HIP graph of the four
calls.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # dense bf16 FLOP/s
FP32_VECTOR_PEAK = 157.3e12  # fp32 vector FLOP/s
METRIC = "MLA decode KV-tokens/s + achieved TB/s & TFLOP/s vs roofline (H=128,B=32,T=4K)"
COUNTERS = os.path.join(ROOT, "profiles", "decode_bf16_b32_h128_t4k_counters.json")


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "mla_copy.h", "mla_device.h", "mla_kernels.h"):
        h.update(open(os.path.join(ROOT, "mla_latent_kv_17_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_peaks(torch, device="cuda"):
    """What this part reaches in practice, from the probes in libmla_peaks.so:
    a streaming read of 2 GiB (beyond the 256 MB Infinity Cache) and
    independent bf16 32x32x16 matrix products on every CU.  Best of five
    runs each, HIP events."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mla_latent_kv_17_amd", "libmla_peaks.so"))
    lib.mla_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.mla_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    blocks = 4096
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=device)

    def best(fn, reps=5):
        fn()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        return min(times)

    t_read = best(lambda: lib.mla_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream))
    iters = 4096
    mfma_blocks = 2048
    t_mfma = best(lambda: lib.mla_probe_mfma(sink.data_ptr(), mfma_blocks, iters, stream))
    flops = mfma_blocks * 4 * iters * 8 * 2 * 32 * 32 * 16
    del buf, sink
    return {"hbm_read_gbps": nbytes / t_read / 1e9, "mfma_bf16_tflops": flops / t_mfma / 1e12,
            "probes": "2 GiB streaming read, 4096 blocks each reading its own contiguous share; "
                      "8 independent bf16 32x32x16 products per wave, 2048 x 4 waves"}


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter runs,
    or None for another workload than theirs, or when the decode kernel
    source changed since they were taken."""
    try:
        c = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if not str(c.get("workload", "")).startswith(workload + " ") or c.get("decode_source_hash") != decode_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


DECODE_KERNEL = {"bf16": "decode_mfma_bf16", "fp8": "decode_mfma_fp8", "f32": "decode_f32"}


def rotation_caches(dev, gib: float):
    """The cache and enough copies of its pages that together they exceed
    `gib` GiB (at least two, at most sixteen): timing launches that rotate
    over them keeps every launch's cache reads cold."""
    import torch
    from mla_latent_kv_17_amd import PagedCache
    c = dev.cache
    n = max(2, min(16, math.ceil(gib * (1 << 30) / max(dev.cache_bytes, 1))))
    out = [c]
    for _ in range(n - 1):
        out.append(PagedCache(c.latent.clone(), c.block_table, c.seq_lens,
                              rope=None if c.rope is None else c.rope.clone(),
                              scale=None if c.scale is None else c.scale.clone()))
    torch.cuda.synchronize()
    return out


def cpu_baseline(inp, budget_s: float):
    """Time the fp64 oracle (explicit K/V reconstruction) on the first
    (sequence, head) rows of the same workload until `budget_s` elapses."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    wl = inp.wl
    done = []
    t0 = time.perf_counter()
    for b in range(wl.batch):
        for h in range(wl.heads):
            O.explicit_decode(inp, select=[(b, i, h) for i in range(wl.q_per_seq)])
            done.append((b, h))
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    # a (sequence, head) row covers len_b KV tokens for one of H heads
    kv_equiv = sum(int(inp.seq_lens[b]) for b, _ in done) / wl.heads
    return {"value": kv_equiv / el, "unit": "KV-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(done)} (sequence, head) rows of {wl.name} ({wl.batch * wl.heads} in a step), "
                      f"explicit fp64 K/V reconstruction, {el:.1f} s",
            "method": "measured in this run on the sample; value = the sample's KV-token equivalents / its time "
                      "(a whole step is not run on the host)",
            "cpu_model": cpu_model(), "blas": blas_vendor()}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def blas_vendor() -> str:
    import numpy as np
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # noqa: BLE001
        return "unknown"


def forms_sweep(args):
    """Both forms of the attention on the same prefill chunk, per S_q: the
    absorbed one (absorb_q + decode + merge / out_uv, splits chosen by the
    library) and the explicit one (rebuild_kv + attend_explicit).  Each step
    timed alone after an eviction read, median of --steps."""
    import numpy as np
    import torch
    import mla_inputs as MI
    from mla_latent_kv_17_amd import MLA_BF16, MLA_FORM_EXPLICIT, mla_attention_form
    from mla_latent_kv_17_amd.runner import DecodeStep, DeviceInputs, ExplicitStep

    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    flush.fill_(1.0)

    def timed(fn):
        for _ in range(max(args.warmup, 1)):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1 in ev:
            torch.sum(flush)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3

    for sq in args.forms:
        wl = MI.WORKLOADS["bf16_b32_h128_t4k"].scaled(name=f"prefill_b{args.forms_batch}_sq{sq}",
                                                      batch=args.forms_batch, q_per_seq=sq,
                                                      seq_len=args.forms_context, num_splits=0, seed=3000 + sq)
        print(f"[forms] generating {wl.name}", file=sys.stderr, flush=True)
        inp = MI.generate(wl)
        dev = DeviceInputs(inp)
        absorbed, explicit = DecodeStep(dev, 0), ExplicitStep(dev)
        a_us = timed(absorbed.run)
        e_us = timed(explicit.run)
        pairs = sum(max(0, int(L) - (sq - 1 - i)) for L in inp.seq_lens for i in range(sq))
        kv = int(inp.seq_lens.astype(np.int64).sum())
        H = wl.heads
        a_flops = pairs * H * 2 * (576 + 512) + 2 * wl.batch * sq * H * 2 * 128 * 512
        rebuild_flops = kv * H * 2 * 2 * 128 * 512
        e_flops = pairs * H * 2 * (192 + 128) + rebuild_flops
        diff = (explicit.out - absorbed.out).float().norm() / absorbed.out.float().norm()
        print(json.dumps({
            "forms": wl.name, "q_per_seq": sq, "batch": wl.batch, "context": args.forms_context, "heads": H,
            "absorbed_us": a_us, "explicit_us": e_us, "absorbed_splits": absorbed.num_splits,
            "absorbed_tflops": a_flops / (a_us * 1e-6) / 1e12, "explicit_tflops": e_flops / (e_us * 1e-6) / 1e12,
            "absorbed_gflop": a_flops / 1e9, "explicit_gflop": e_flops / 1e9, "rebuild_gflop": rebuild_flops / 1e9,
            "faster": "explicit" if e_us < a_us else "absorbed",
            "library_choice": "explicit" if mla_attention_form(dev.dims, MLA_BF16) == MLA_FORM_EXPLICIT
            else "absorbed",
            "rel_l2_explicit_vs_absorbed": float(diff),
            "timing": f"median of {args.steps} steps, each after a 1 GiB eviction read, HIP events"}), flush=True)
        del absorbed, explicit, dev, inp
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_b32_h128_t4k")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip timing the cache append")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak probes")
    ap.add_argument("--no-gate", action="store_true", help="skip timing the MoE gate")
    ap.add_argument("--gate-tokens", type=int, nargs="*", default=None,
                    help="token counts at which to time the MoE gate (default: the step's tokens and 4096)")
    ap.add_argument("--q-per-seq", type=int, default=0,
                    help="query tokens per sequence instead of the workload's (multi-token decode)")
    ap.add_argument("--append-d-model", type=int, default=5120,
                    help="hidden width of the tokens the cache append projects (not on the pages)")
    ap.add_argument("--warm", action="store_true", help="also time steps without cache eviction")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a HIP graph of the four calls (checked bit for bit "
                         "against the eager step; not the headline: eager launches are already queued behind "
                         "the eviction read, so a graph removes no gap and adds its own launch)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run three 256 MiB device-to-device copies and exit (the known-size reference "
                         "for rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--rotate-gib", type=float, default=1.5,
                    help="total size of the cache copies the decode timing rotates over")
    ap.add_argument("--forms", type=int, nargs="*", default=None,
                    help="time the absorbed and the explicit form (keys and values rebuilt) at these query "
                         "tokens per sequence on one bf16 prefill chunk (B=--forms-batch, H=128, a "
                         "--forms-context-token context incl. the chunk), one JSON line each, and exit")
    ap.add_argument("--forms-batch", type=int, default=1)
    ap.add_argument("--forms-context", type=int, default=4096)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported (the decode shards by "
              f"sequence with no exchange between GPUs, so the one-GPU rate is the per-GPU rate)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.copy_calibration:
        src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")  # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "copies": 3}), flush=True)
        return
    if args.forms is not None:
        forms_sweep(args)
        return
    import mla_inputs as MI
    from mla_latent_kv_17_amd import mla_decode
    from mla_latent_kv_17_amd.runner import CacheAppend, DecodeStep, DeviceInputs, MoeGate

    wl = MI.WORKLOADS[args.workload]
    if args.q_per_seq:  # multi-token decode on the workload's cache (context figure, not a configuration)
        wl = wl.scaled(name=f"{wl.name}_sq{args.q_per_seq}", q_per_seq=args.q_per_seq)
    print(f"[bench] generating {wl.name}", file=sys.stderr, flush=True)
    inp = MI.generate(wl)
    dev = DeviceInputs(inp)
    step = DecodeStep(dev, args.num_splits if args.num_splits > 0 else wl.num_splits)
    kv_tokens = int(inp.seq_lens.astype(np.int64).sum())
    rows = wl.q_per_seq * wl.heads
    per_tok = MI.cache_bytes_per_token(wl.cache_dtype)
    cache_bytes = kv_tokens * per_tok
    # score (2*576) + value (2*512) flops per (query row, visible token)
    pairs = sum(max(0, int(L) - (wl.q_per_seq - 1 - i)) for L in inp.seq_lens for i in range(wl.q_per_seq))
    decode_flops = pairs * wl.heads * 2 * (576 + 512)
    proj_flops = 2 * (wl.batch * wl.q_per_seq) * wl.heads * 2 * 128 * 512
    # queries read (q_lat | q_rope) and outputs written (o_lat, or the chunk
    # partials, and lse) by the decode
    q_bytes = wl.batch * rows * (512 + 64) * (4 if wl.q_dtype == "f32" else 2)
    io_bytes = q_bytes + wl.batch * step.num_splits * rows * (512 + 1) * 4

    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    flush.fill_(1.0)

    def do_flush():
        torch.sum(flush)

    for _ in range(args.warmup):
        do_flush()
        step.run()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(K):
        do_flush()
        e0, e3 = ev[i]
        e0.record()
        step.run()
        e3.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])

    # ---- the decode kernel alone: K launches back to back over rotating
    # copies of the cache (every launch cold), between two events
    caches = rotation_caches(dev, args.rotate_gib)
    o_dec = step.o_part if step.num_splits > 1 else step.o_lat
    l_dec = step.lse_part if step.num_splits > 1 else step.lse
    for c in caches:
        mla_decode(dev.dims, step.q_lat, dev.q_rope, c, step.num_splits, o_dec, l_dec)
    do_flush()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for i in range(K):
        mla_decode(dev.dims, step.q_lat, dev.q_rope, caches[i % len(caches)], step.num_splits, o_dec, l_dec)
    d1.record()
    torch.cuda.synchronize()
    dec_avg = d0.elapsed_time(d1) / K
    n_rot = len(caches)
    del caches

    # warm (no eviction between steps): context only, never the headline; off by
    # default so that every decode launch of a default run is a cold one
    warm_ms = None
    if args.warm:
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        for _ in range(K):
            step.run()
        w1.record()
        torch.cuda.synchronize()
        warm_ms = w0.elapsed_time(w1) / K

    # the same four calls captured once as a HIP graph and replayed: the
    # library allocates nothing and issues no memsets, so the step captures
    # as is; the replay must reproduce the eager result bit for bit
    graph_ms = None
    if args.graph:
        ref_out = step.run().clone()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step.run()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step.run()
        for _ in range(2):
            do_flush()
            graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(step.out, ref_out):
            print("bench.py: graph replay differs from the eager step", file=sys.stderr)
            sys.exit(1)
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for i in range(K):
            do_flush()
            gev[i][0].record()
            graph.replay()
            gev[i][1].record()
        torch.cuda.synchronize()
        graph_ms = np.array([a.elapsed_time(b) for a, b in gev])

    # the cache append (the step before the decode path, not part of it):
    # c = W_DKV h and the rotated position key of the B*S_q new tokens,
    # written into their page rows; each launch timed alone after an eviction
    append = None
    if not args.no_append:
        app = CacheAppend(dev, MI.generate_append(wl, d_model=args.append_d_model))
        for _ in range(3):
            app.run()
        aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for e0, e1 in aev:
            do_flush()
            e0.record()
            app.run()
            e1.record()
        torch.cuda.synchronize()
        app_us = float(np.median([a.elapsed_time(b) for a, b in aev])) * 1e3
        T = wl.batch * wl.q_per_seq
        wbytes = 2 if wl.w_dtype == "bf16" else 4
        app_bytes = (576 + T) * args.append_d_model * wbytes + T * per_tok
        append = {"kernels": "append_proj_mfma + append_finish" if wl.w_dtype == "bf16"
                  else "append_proj_f32 + append_finish", "tokens": T, "d_model": args.append_d_model,
                  "us": app_us, "algorithmic_bytes": app_bytes,
                  "achieved_gbps": app_bytes / (app_us * 1e-6) / 1e9,
                  "frac_hbm": app_bytes / (app_us * 1e-6) / HBM_PEAK,
                  "timing": "median of 20 launches, each after an eviction read, HIP events around the two launches"}

    # the MoE gate of DeepSeek-V2's routed experts (160 centroids of width
    # 5120, top 6), a second workload beside the attention path: at the
    # step's token count and at a prefill-sized 4096 tokens
    gate = None
    if not args.no_gate:
        gate_runs = []
        for T in (args.gate_tokens if args.gate_tokens is not None else [wl.batch * wl.q_per_seq, 4096]):
            g = MoeGate(MI.generate_gate(T, d_model=MI.APPEND_D_MODEL), "bf16", torch.device("cuda", 0))
            for _ in range(3):
                g.run()
            gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
            for e0, e1 in gev:
                do_flush()
                e0.record()
                g.run()
                e1.record()
            torch.cuda.synchronize()
            g_us = float(np.median([a.elapsed_time(b) for a, b in gev])) * 1e3
            d, n, k = MI.APPEND_D_MODEL, MI.GATE_EXPERTS, MI.GATE_TOP_K
            g_bytes = (T + n) * d * 2 + T * k * 8
            gate_runs.append({"tokens": T, "us": g_us, "algorithmic_bytes": g_bytes,
                              "achieved_gbps": g_bytes / (g_us * 1e-6) / 1e9,
                              "frac_hbm": g_bytes / (g_us * 1e-6) / HBM_PEAK,
                              "tflops": 2.0 * T * n * d / (g_us * 1e-6) / 1e12})
            del g
        gate = {"kernels": "gate_proj_mfma + gate_finish", "d_model": MI.APPEND_D_MODEL,
                "n_experts": MI.GATE_EXPERTS, "top_k": MI.GATE_TOP_K, "dtype": "bf16", "runs": gate_runs,
                "timing": "median of 20 launches, each after an eviction read, HIP events around the two launches"}

    peaks = None if args.no_peaks else measured_peaks(torch)

    eager_ms_per_step = float(step_ms.mean())
    ms_per_step = eager_ms_per_step
    traffic = measured_traffic(wl.name)
    # which roof bounds the decode: its flops per cache byte against the ridge
    # of the peak it would run at (bf16 matrix cores, or fp32 vector ALUs for
    # the fp32 cache)
    flop_peak = FP32_VECTOR_PEAK if wl.cache_dtype == "f32" else MFMA_BF16_PEAK
    if decode_flops / cache_bytes > flop_peak / HBM_PEAK:
        roof = {"bound": "mfma" if wl.cache_dtype != "f32" else "alu",
                "achieved": decode_flops / (dec_avg * 1e-3) / 1e12, "peak": flop_peak / 1e12, "unit": "TFLOP/s",
                "frac": decode_flops / (dec_avg * 1e-3) / flop_peak, "algorithmic_flops": decode_flops}
    else:
        roof = {"bound": "hbm", "achieved": cache_bytes / (dec_avg * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": cache_bytes / (dec_avg * 1e-3) / HBM_PEAK}
    # the same rate against what the probes reach on this part
    frac_measured = None
    if peaks is not None and roof["bound"] == "hbm":
        frac_measured = roof["achieved"] / peaks["hbm_read_gbps"]
    elif peaks is not None and roof["bound"] == "mfma":
        frac_measured = roof["achieved"] / peaks["mfma_bf16_tflops"]
    out = {
        "metric": METRIC,
        "value": kv_tokens / (ms_per_step * 1e-3),
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.cache_dtype != "f32" else "f32",
        "data": "synthetic (seeded N(0,1) cache and queries, weights N(0, std 1/sqrt(512)))",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": int(inp.seq_lens.max()),
                   "q_per_seq": wl.q_per_seq, "heads": wl.heads, "d_latent": 512, "d_rope": 64, "d_head": 128,
                   "block_size": 64, "cache_dtype": wl.cache_dtype, "num_splits": step.num_splits,
                   "steps_timed": "absorb_q + decode + the split merge fused into out_uv (combine_out_uv; split_combine "
                                  "+ out_uv above 8 chunks with bf16 weights and more than 8 query rows, out_uv alone "
                                  "for one chunk), caches evicted before each"},
        "roofline": {**roof, "frac_of_measured": frac_measured, "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, "
                                     "calibrated on a 256 MiB copy)",
                     "traffic_source": "not measured in this run: read from profiles/decode_bf16_b32_h128_t4k_counters.json "
                                       "(rocprofv3 counter runs), reported only while the decode sources hash to the "
                                       "value recorded there; null otherwise",
                     "kernel": DECODE_KERNEL[wl.cache_dtype], "launch_ms": dec_avg,
                     "launch_timing": f"{K} back-to-back launches over {n_rot} cache copies, HIP events",
                     "algorithmic_bytes": cache_bytes},
        "decode_tflops": decode_flops / (dec_avg * 1e-3) / 1e12,
        "decode_mfma_frac": decode_flops / (dec_avg * 1e-3) / MFMA_BF16_PEAK,
        "kv_tokens_per_step": kv_tokens,
        # (query token, visible KV token) pairs: differs from KV tokens when S_q > 1
        "query_kv_pairs_per_step": pairs,
        "query_kv_pairs_per_s": pairs / (ms_per_step * 1e-3),
        # the decode's bytes with its queries read and its outputs written
        "decode_gbps_cache_q_o": (cache_bytes + io_bytes) / (dec_avg * 1e-3) / 1e9,
        "step_ms_p10_p50_p90": [float(np.percentile(step_ms, q)) for q in (10, 50, 90)],
        "graph_ms_per_step": float(graph_ms.mean()) if graph_ms is not None else None,
        "step_tflops": (decode_flops + proj_flops) / (ms_per_step * 1e-3) / 1e12,
        "warm_ms_per_step": warm_ms,
        "wall_s_timed_loop_incl_eviction": wall,
        "cache_append": append,
        "moe_gate": gate,
        "measured_peaks": peaks,
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
        out["cpu_baseline"]["cpu"] = platform.processor() or platform.machine()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
