"""Benchmark of the Llama-3.1-8B GQA attention block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_p1000]

Headline workload: one decode block-step at the pages' decode point (B = 1,
P = 1,000 cached positions, row 1,000 written, rows 0-1,000 read).  A step is
one gqa_block_decode call: QKV projection + RoPE + cache append, attention,
wo (one launch under the fused schedule the library picks for this shape;
the three-launch schedule is timed beside it).  Inputs are seeded synthetic
bf16 tensors already resident in HBM.  The
timed loop cycles through 8 independent weight + cache sets (8 x 84 MiB),
so the 256 MB Infinity Cache cannot hold what a step reads.

Printed: one JSON line with the step time, HBM throughput, the roofline of
the dominant kernel (under the one-launch schedule the step time itself,
measured with HIP events over the timed region on the stream the kernel runs
on; under the three-launch schedule HIP events around each kernel), the
oracle timed on this host's cores, and a prefill (B = 4, T = 2,048) record
with tokens/s and matrix-core utilisation.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode µs/block-step & HBM TB/s (% peak); prefill tokens/s & MFMA util"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS = 2500.0        # MI355X dense bf16/fp16
N_SETS = 8

D, NQKV, KVH, HD = 4096, 6144, 8, 128


def decode_bytes(B: int, P: int, kvh: int = KVH) -> dict:
    """Algorithmic HBM bytes of one decode block-step and of each kernel
    (kvh key/value heads; 8 for Llama 3.1 8B)."""
    w_qkv = (D + 2 * kvh * HD) * D * 2
    w_o = D * D * 2
    kv_read = B * (P + 1) * kvh * HD * 2 * 2      # rows 0..P of K and V (row P just written)
    kv_write = B * kvh * HD * 2 * 2
    qkv = w_qkv + B * D * 2 + kv_write + B * D * 4 + 64 * 8      # x in, Q fp32 out, rope row
    attn = kv_read + B * D * 4 + B * D * 2 * 2                     # K/V, Q in, O hi/lo out
    wo = w_o + B * D * 2 * 2 + B * D * 4                           # Wo, O hi/lo in, out fp32
    # whole step as the pages count it: weights + cache read + cache write + x + out + rope
    step = w_qkv + w_o + B * P * kvh * HD * 2 * 2 + kv_write + B * D * 2 + B * D * 4 + 64 * 8
    return {"qkv": qkv, "attn": attn, "wo": wo, "step": step}


def prefill_flops(B: int, T: int, start_pos: int = 0, kvh: int = KVH) -> dict:
    M = B * T
    qkv = 2.0 * M * (D + 2 * kvh * HD) * D
    causal_pairs = B * (T * start_pos + T * (T + 1) / 2)   # token i sees start_pos + i + 1 keys
    attn = 4.0 * causal_pairs * 32 * HD             # QK^T and PV over visible pairs, 32 heads
    wo = 2.0 * M * D * D
    return {"qkv": qkv, "attn": attn, "wo": wo, "total": qkv + attn + wo}


def counter_traffic(summary: str, kernel: str, source: str):
    """HBM bytes per launch of `kernel` measured by rocprofv3 (FETCH_SIZE +
    WRITE_SIZE, calibrated on a known-size copy), as recorded in a profile
    summary; None when the kernel source has changed since the counters were
    taken."""
    import hashlib
    try:
        fields = {}
        for line in open(os.path.join(ROOT, "profiles", summary)).read().splitlines():
            line = line.strip()
            if line.startswith(("traffic_bytes_per_launch[", "kernel_source_sha256:")):
                k, v = line.split(": ", 1)
                fields[k] = v
        digest = hashlib.sha256(open(os.path.join(ROOT, source), "rb").read()).hexdigest()
        if fields.get("kernel_source_sha256") != digest:
            return None
        return int(fields[f"traffic_bytes_per_launch[{kernel}]"])
    except (OSError, KeyError, ValueError):
        return None


def bench_decode(G, synth, steps: int, warmup: int, B=1, P=1000, T_max=1024, use_graph=True,
                 schedule=None, kvh=KVH):
    """Eager, graph-replay and per-kernel timings of decode steps under the
    given decode schedule (the library's choice when None)."""
    if schedule is not None:
        prev = G.set_decode_schedule(schedule)
        try:
            return bench_decode(G, synth, steps, warmup, B, P, T_max, use_graph, None, kvh)
        finally:
            G.set_decode_schedule(prev)
    dev = torch.device("cuda:0")
    # the one-launch schedule exists for 8 key/value heads only
    fused = kvh == KVH and G.decode_schedule(B, P, T_max) == G.DECODE_FUSED
    sets = []
    for s in range(N_SETS):
        x, w, kc_rows, vc_rows = synth.decode_workload(s, B, P, n_kv_heads=kvh)
        kc, vc = G.empty_caches(B, T_max, dev, kvh)
        kc.zero_()
        vc.zero_()
        G.kcache_by_position(kc)[:, :P] = kc_rows.to(dev)
        G.vcache_write(vc, 0, vc_rows.to(dev))
        sets.append(dict(x=x.to(dev), w=[t.to(dev) for t in w], kc=kc, vc=vc))
    rope = G.rope_table(T_max, device=dev)
    ws = G.workspace(B, 1, T_max, dev)
    out = torch.empty((B, D), dtype=torch.float32, device=dev)

    def step(i, events=None):
        st = sets[i % N_SETS]
        G.block_decode(st["x"], *st["w"], st["kc"], st["vc"], rope, P, out=out, ws=ws,
                       events=events)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # timed loop: plain calls
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    wall0 = time.perf_counter()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1)
    us_step = ms * 1000.0 / steps

    # the same steps replayed from a captured HIP graph (8 steps per graph,
    # one per weight set), which removes the host-side launch cost
    graph_us = None
    graph_spread = None
    if use_graph:
        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    step(i)
            return g
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(N_SETS):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        g8 = capture(N_SETS)
        rem = steps % N_SETS
        grem = capture(rem) if rem else None
        for _ in range(3):
            g8.replay()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps // N_SETS):
            g8.replay()
        if grem is not None:
            grem.replay()
        t1.record()
        torch.cuda.synchronize()
        graph_us = t0.elapsed_time(t1) * 1000.0 / steps
        # spread: 20 more timings of one 8-step replay each (one step per set)
        reps = []
        for _ in range(20):
            t0.record()
            g8.replay()
            t1.record()
            torch.cuda.synchronize()
            reps.append(t0.elapsed_time(t1) * 1000.0 / N_SETS)
        graph_spread = [float(np.percentile(reps, q)) for q in (10, 50, 90)]

    # hot-cache figure (not the headline): every step reuses set 0, so its
    # weights and cache stay in the 256 MB Infinity Cache between steps
    hot_us = None
    if use_graph:
        def step0(i):
            step(0)
        hot_us = _timed_steps(step0, steps, 3, True)

    # the same loop through the profiled entry point: HIP events recorded on
    # the library's stream around each kernel
    ev = G.HipEvents(G.DECODE_STAGES + 1)
    per = np.zeros((steps, G.DECODE_STAGES))
    for i in range(steps):
        step(i, events=ev)
        for k in range(G.DECODE_STAGES):
            per[i, k] = ev.elapsed_ms(k, k + 1)
    ev.close()
    kern_us = per.mean(axis=0) * 1000.0
    # the fused schedule is one kernel: stage 1 covers it, the others are empty
    names = ["decode_step"] if fused else ["qkv", "attn", "wo"]
    return dict(us_step=us_step, wall_us_step=wall * 1e6 / steps, graph_us_step=graph_us,
                hot_cache_us_step=hot_us, graph_spread_us=graph_spread,
                schedule="fused" if fused else "split",
                kern_us=dict(zip(names, kern_us.tolist())),
                profiled_us_step=float(per.sum(axis=1).mean() * 1000.0))


def bench_prefill(G, synth, steps: int, warmup: int, B=4, T=2048, kvh=KVH):
    dev = torch.device("cuda:0")
    x, w = synth.prefill_workload(0, B, T, n_kv_heads=kvh)
    x = x.to(dev)
    w = [t.to(dev) for t in w]
    kc, vc = G.empty_caches(B, T, dev, kvh)
    rope = G.rope_table(T, device=dev)
    ws = G.workspace(B, T, T, dev, n_kv_heads=kvh)
    out = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        G.block_prefill(x, *w, kc, vc, rope, out=out, ws=ws)
    torch.cuda.synchronize()
    ev = G.HipEvents(G.PREFILL_STAGES + 1)
    per = np.zeros((steps, G.PREFILL_STAGES))
    tot = []
    for i in range(steps):
        G.block_prefill(x, *w, kc, vc, rope, out=out, ws=ws, events=ev)
        for k in range(G.PREFILL_STAGES):
            per[i, k] = ev.elapsed_ms(k, k + 1)
        tot.append(ev.elapsed_ms(0, G.PREFILL_STAGES))
    ev.close()
    us_events = float(np.mean(tot) * 1000.0)
    # whole-call time: the same calls back to back with no events inside them
    # (each event recorded between kernels adds a few microseconds)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        G.block_prefill(x, *w, kc, vc, rope, out=out, ws=ws)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1000.0 / steps
    fl = prefill_flops(B, T, kvh=kvh)
    kern = dict(zip(["wo_fp16", "qkv", "attn", "wo"], (per.mean(axis=0) * 1000.0).tolist()))
    return dict(B=B, T=T, us_step=us, us_step_with_kernel_events=us_events,
                tokens_per_s=B * T / (us * 1e-6),
                mfma_util=fl["total"] / (us * 1e-6) / (MFMA_PEAK_TFLOPS * 1e12),
                algorithmic_gflop=fl["total"] / 1e9, kern_us=kern,
                kern_tflops={k: fl[k] / (kern[k] * 1e-6) / 1e12 for k in ("qkv", "attn", "wo")})


def bench_layer_decode(G, synth, steps: int, warmup: int, B=1, P=1000, T_max=1024):
    """Graph-replay time per step of the layer (RMSNorm, block, residual:
    gqa_layer_decode) and of the bare block on the same rotated inputs."""
    dev = torch.device("cuda:0")
    sets = []
    for s_ in range(N_SETS):
        x, w, kc_rows, vc_rows = synth.decode_workload(s_, B, P)
        kc, vc = G.empty_caches(B, T_max, dev)
        kc.zero_()
        vc.zero_()
        G.kcache_by_position(kc)[:, :P] = kc_rows.to(dev)
        G.vcache_write(vc, 0, vc_rows.to(dev))
        sets.append(dict(x=x.to(dev), w=[t.to(dev) for t in w], kc=kc, vc=vc,
                         g=synth.norm_gain(100 + s_).to(dev)))
    rope = G.rope_table(T_max, device=dev)
    ws = G.layer_workspace(B, 1, T_max, dev)
    h = torch.empty((B, D), dtype=torch.float32, device=dev)
    h16 = torch.empty((B, D), dtype=torch.bfloat16, device=dev)

    def layer(i):
        st = sets[i % N_SETS]
        G.layer_decode(st["x"], st["g"], *st["w"], st["kc"], st["vc"], rope, P, h=h, h_bf16=h16,
                       ws=ws)

    def block(i):
        st = sets[i % N_SETS]
        G.block_decode(st["x"], *st["w"], st["kc"], st["vc"], rope, P, out=h, ws=ws)

    n = max(N_SETS, steps // N_SETS * N_SETS)
    return _timed_steps(layer, n, warmup, True), _timed_steps(block, n, warmup, True)


def bench_chunked_prefill(G, synth, steps: int, warmup: int, B=4, P=2048, T=2048):
    """Whole-call timing of a prefill of T tokens after P cached rows per
    sequence (gqa_block_prefill_from), HIP events on the current stream."""
    dev = torch.device("cuda:0")
    x, w, kc_rows, vc_rows = synth.chunked_prefill_workload(0, B, P, T)
    x = x.to(dev)
    w = [t.to(dev) for t in w]
    T_max = P + T
    kc, vc = G.empty_caches(B, T_max, dev)
    G.kcache_by_position(kc)[:, :P] = kc_rows.to(dev)
    G.vcache_write(vc, 0, vc_rows.to(dev))
    del kc_rows, vc_rows
    rope = G.rope_table(T_max, device=dev)
    ws = G.workspace(B, T, T_max, dev, start_pos=P)
    out = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        G.block_prefill(x, *w, kc, vc, rope, out=out, ws=ws, start_pos=P)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        G.block_prefill(x, *w, kc, vc, rope, out=out, ws=ws, start_pos=P)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1000.0 / steps
    fl = prefill_flops(B, T, P)
    return us, fl


def _timed_steps(step, steps, warmup, use_graph):
    """Median-free whole-loop timing of `steps` calls of step(i) (graph replay
    of the whole loop when use_graph), HIP events on the current stream."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        t0.record()
        g.replay()
        t1.record()
    else:
        t0.record()
        for i in range(steps):
            step(i)
        t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1000.0 / steps


def bench_batched(G, synth, steps, warmup, B=64, P=8192, T_max=8224, kvh=KVH):
    """Batched decode: B=64 sequences, 8,192 cached positions each, kvh
    key/value heads (8 for Llama 3.1 8B)."""
    dev = torch.device("cuda:0")
    n_w = 4   # weight sets rotated (the 2.15 GB cache already defeats the MALL)
    gen = synth.generator(0)
    xs = [synth.randn_bf16(gen, (B, D)).to(dev) for _ in range(n_w)]
    ws_sets = [[t.to(dev) for t in synth.block_weights(gen, n_kv_heads=kvh)] for _ in range(n_w)]
    kc, vc = G.empty_caches(B, T_max, dev, kvh)
    dgen = synth.generator(1, dev)
    synth.fill_randn_bf16_(kc, dgen)
    synth.fill_randn_bf16_(vc, dgen)
    rope = G.rope_table(T_max, device=dev)
    ws = G.workspace(B, 1, T_max, dev)
    out = torch.empty((B, D), dtype=torch.float32, device=dev)

    def step(i, events=None):
        G.block_decode(xs[i % n_w], *ws_sets[i % n_w], kc, vc, rope, P, out=out, ws=ws,
                       events=events)

    us = _timed_steps(step, steps, warmup, True)
    ev = G.HipEvents(G.DECODE_STAGES + 1)
    per = np.zeros((steps, G.DECODE_STAGES))
    for i in range(steps):
        step(i, events=ev)
        for k in range(G.DECODE_STAGES):
            per[i, k] = ev.elapsed_ms(k, k + 1)
    ev.close()
    kern = dict(zip(["qkv", "attn", "wo"], (per.mean(axis=0) * 1000.0).tolist()))
    nb = decode_bytes(B, P, kvh)
    return us, kern, nb


def bench_stacked(G, synth, steps, warmup, B=8, P=131071, T_max=131072, L=32):
    """32 stacked blocks, B=8, 131,071 cached positions per sequence per
    block (128 GiB of cache), residual h <- h + Delta, no norms or FFN."""
    dev = torch.device("cuda:0")
    dgen = synth.generator(0, dev)
    x0 = synth.randn_bf16(dgen, (B, D), device=dev)
    blocks = []
    t_start = time.perf_counter()
    for l in range(L):
        w = synth.block_weights(dgen, device=dev)
        kc, vc = G.empty_caches(B, T_max, dev)
        synth.fill_randn_bf16_(kc, dgen)
        synth.fill_randn_bf16_(vc, dgen)
        blocks.append((w, kc, vc))
        torch.cuda.synchronize()
        print(f"stacked: block {l + 1}/{L} staged ({time.perf_counter() - t_start:.1f} s)",
              file=sys.stderr, flush=True)
    rope = G.rope_table(T_max, device=dev)
    ws = G.workspace(B, 1, T_max, dev)
    h = torch.empty((B, D), dtype=torch.float32, device=dev)
    xa = torch.empty_like(x0)
    xb = torch.empty_like(x0)

    def step(i):
        h.copy_(x0)
        xa.copy_(x0)
        a, b = xa, xb
        for w, kc, vc in blocks:
            G.block_decode(a, *w, kc, vc, rope, P, out=h, out_bf16=b, accumulate=True, ws=ws)
            a, b = b, a

    us_step = _timed_steps(step, steps, warmup, False)
    nb = decode_bytes(B, P)
    finite = bool(torch.isfinite(h).all())
    return us_step, nb, finite


def cpu_baseline(synth, B=1, P=1000, budget_s=12.0):
    """The oracle as it stands, timed on this host on a bounded sample of the
    same workload (whole decode block-steps, repeated until ~budget_s)."""
    from oracle import gqa_oracle as O
    x, w, kc, vc = synth.decode_workload(0, B, P)
    f = lambda t: t.float().numpy().astype(np.float64)
    xs, ws = f(x)[:, None, :], [f(t) for t in w]
    kcs, vcs = f(kc), f(vc)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    n = 0
    t0 = time.perf_counter()
    while True:
        O.gqa_block(xs, *ws, kcs, vcs, P)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 20000:
            break
    return {"value": el / n * 1e6, "unit": "us/block-step", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} whole decode block-steps (B={B}, P={P}) of the fp64 NumPy oracle, "
                      f"{el:.1f} s of CPU time on inputs already converted to fp64"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill record")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    ap.add_argument("--schedule", default="auto", choices=["auto", "split", "fused"],
                    help="decode schedule of the headline workloads (auto: the library's "
                         "choice, which is the one-launch schedule where it applies)")
    ap.add_argument("--workload", default="decode_p1000",
                    choices=["decode_p1000", "decode_p128", "batched", "mha_batched", "stacked_long",
                             "chunked_prefill", "layer_decode_p1000", "vocab_b1",
                             "mha_decode_p1000", "kv16_decode_p1000"],
                    help="decode_p1000 (headline), batched (B=64, P=8192) or "
                         "stacked_long (32 blocks, B=8, P=131071)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import grouped_query_attention_gemv_amd as G
    from grouped_query_attention_gemv_amd import synth
    G.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.workload in ("batched", "mha_batched"):
        kvh = 32 if args.workload == "mha_batched" else KVH
        us, kern, nb = bench_batched(G, synth, args.steps if args.steps != 400 else 50,
                                     min(args.warmup, 10), kvh=kvh)
        tbs = nb["step"] / (us * 1e-6) / 1e12
        attn_gbs = nb["attn"] / (kern["attn"] * 1e-6) / 1e9
        name = ("Llama-3.1-8B GQA block batched decode, B=64, P=8192" if kvh == KVH else
                "Llama-3.1-8B-shaped attention block batched decode, multi-head (n_kv = 32), "
                "B=64, P=8192")
        print(json.dumps({
            "metric": METRIC, "value": round(us, 3), "unit": "us/block-step", "n_gpus": 1,
            "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": name, "B": 64, "P": 8192, "T_max": 8224, "kv_heads": kvh,
                       "hip_graph": True},
            "hbm_tbs": round(tbs, 4), "hbm_frac_of_peak": round(tbs * 1000 / HBM_PEAK_GBS, 4),
            "tokens_per_s": 64 / (us * 1e-6), "kernels_us": {k: round(v, 3) for k, v in kern.items()},
            "roofline": {"kernel": f"decode_attn_kernel<{kvh}>", "bound": "hbm",
                         "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "algorithmic_bytes": nb["attn"]}}), flush=True)
        return
    if args.workload == "vocab_b1":
        dev = torch.device("cuda:0")
        V, B = G.VOCAB, 1
        w = torch.empty((V, D), dtype=torch.bfloat16, device=dev)
        synth.fill_randn_bf16_(w, synth.generator(60, dev), 0.02)
        h = synth.randn_bf16(synth.generator(61), (B, D)).to(dev)
        g = synth.norm_gain(62).to(dev)
        L = torch.empty((B, V), dtype=torch.float32, device=dev)
        steps = args.steps if args.steps != 400 else 50
        us = _timed_steps(lambda i: G.vocab_logits(h, w, g, logits=L), steps,
                          min(args.warmup, 5), True)
        nb = V * D * 2 + B * D * 2 + D * 2 + B * V * 4
        gbs = nb / (us * 1e-6) / 1e9
        print(json.dumps({
            "metric": METRIC, "value": round(us, 3), "unit": "us/call", "n_gpus": 1,
            "steps": steps, "warmup": min(args.warmup, 5), "ms_per_step": round(us / 1000, 5),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "Llama-3.1 vocabulary projection with final RMSNorm, "
                                   "B=1, 4096 x 128256 bf16 weights", "B": B, "V": V,
                       "hip_graph": True},
            "roofline": {"kernel": "vocab_gemv_kernel<1>", "bound": "hbm",
                         "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "algorithmic_bytes": nb}}), flush=True)
        return
    if args.workload == "layer_decode_p1000":
        steps = args.steps if args.steps != 400 else 200
        lay, blk = bench_layer_decode(G, synth, steps, min(args.warmup, 20))
        nb = decode_bytes(1, 1000)["step"] + 2 * 4096 * 2 + 2 * 4096 * 4   # + x, gain, h, h_bf16
        tbs = nb / (lay * 1e-6) / 1e12
        print(json.dumps({
            "metric": METRIC, "value": round(lay, 3), "unit": "us/layer-step", "n_gpus": 1,
            "steps": steps, "warmup": min(args.warmup, 20), "ms_per_step": round(lay / 1000, 5),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "Llama-3.1-8B attention layer decode (RMSNorm, block, residual), "
                                   "B=1, P=1000", "B": 1, "P": 1000, "T_max": 1024,
                       "hip_graph": True},
            "block_only_us": round(blk, 3), "norm_residual_overhead_us": round(lay - blk, 3),
            "hbm_tbs": round(tbs, 4), "hbm_frac_of_peak": round(tbs * 1000 / HBM_PEAK_GBS, 4)}),
            flush=True)
        return
    if args.workload == "chunked_prefill":
        B, P, T = 4, 2048, 2048
        steps = args.steps if args.steps != 400 else 10
        us, fl = bench_chunked_prefill(G, synth, steps, min(args.warmup, 3), B, P, T)
        tfs = fl["total"] / (us * 1e-6) / 1e12
        print(json.dumps({
            "metric": METRIC, "value": round(B * T / (us * 1e-6), 1), "unit": "tokens/s",
            "n_gpus": 1, "steps": steps, "warmup": min(args.warmup, 3),
            "ms_per_step": round(us / 1000, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "Llama-3.1-8B GQA block chunked prefill: B=4 sequences, "
                                   "2,048 new tokens after 2,048 cached rows each",
                       "B": B, "start_pos": P, "T": T, "T_max": P + T},
            "algorithmic_gflop": round(fl["total"] / 1e9, 3),
            "roofline": {"kernel": "whole call (prep, QKV GEMM, attention, wo GEMM)",
                         "bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tfs / MFMA_PEAK_TFLOPS, 4),
                         "traffic": None}}), flush=True)
        return
    if args.workload == "stacked_long":
        us, nb, finite = bench_stacked(G, synth, args.steps if args.steps != 400 else 5,
                                       min(args.warmup, 2))
        per_block = us / 32
        tbs = nb["step"] / (per_block * 1e-6) / 1e12
        print(json.dumps({
            "metric": METRIC, "value": round(per_block, 3), "unit": "us/block-step", "n_gpus": 1,
            "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "32 stacked Llama-3.1-8B GQA blocks, decode B=8, P=131071 "
                                   "(128 GiB cache), residual, no norms/FFN",
                       "B": 8, "P": 131071, "T_max": 131072, "blocks": 32, "hip_graph": False},
            "ms_per_32_block_step": round(us / 1000, 4), "hbm_tbs": round(tbs, 4),
            "hbm_frac_of_peak": round(tbs * 1000 / HBM_PEAK_GBS, 4),
            "tokens_per_s": 8 / (us * 1e-6), "outputs_finite": finite}), flush=True)
        return

    if args.workload in ("mha_decode_p1000", "kv16_decode_p1000"):
        kvh = 32 if args.workload.startswith("mha") else 16
        B, P, T_max = 1, 1000, 1024
        dec = bench_decode(G, synth, args.steps, args.warmup, B, P, T_max,
                           use_graph=not args.no_graph, kvh=kvh)
        us = dec["graph_us_step"] if dec["graph_us_step"] is not None else dec["us_step"]
        nb = decode_bytes(B, P, kvh)
        step_tbs = nb["step"] / (us * 1e-6) / 1e12
        qkv_gbs = nb["qkv"] / (dec["kern_us"]["qkv"] * 1e-6) / 1e9
        kind = "multi-head (n_kv = 32)" if kvh == 32 else "GQA with n_kv = 16"
        print(json.dumps({
            "metric": METRIC, "value": round(us, 3), "unit": "us/block-step", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": us / 1000.0,
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded bf16 N(0,1) x and cache, N(0,0.02) weights; 8 sets)",
            "config": {"workload": f"Llama-3.1-8B-shaped attention block decode, {kind}, "
                                   f"B=1, P={P}",
                       "B": B, "P": P, "T_max": T_max, "kv_heads": kvh,
                       "hip_graph": dec["graph_us_step"] is not None,
                       "schedule": dec["schedule"]},
            "hbm_tbs": round(step_tbs, 4),
            "hbm_frac_of_peak": round(step_tbs * 1000.0 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_step": nb["step"],
            "eager_us_step": round(dec["us_step"], 3),
            "kernels_us": {k: round(v, 3) for k, v in dec["kern_us"].items()},
            "roofline": {"kernel": f"decode_qkv_kernel<1, {kvh}> (QKV GEMV + RoPE + append)",
                         "bound": "hbm", "achieved": round(qkv_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(qkv_gbs / HBM_PEAK_GBS, 4),
                         "traffic": None, "algorithmic_bytes": nb["qkv"]},
            "prefill": None if args.no_prefill else bench_prefill(G, synth, steps=10, warmup=3,
                                                                  kvh=kvh)}), flush=True)
        return

    B, P, T_max = (1, 128, 256) if args.workload == "decode_p128" else (1, 1000, 1024)
    sched = {"auto": None, "split": G.DECODE_SPLIT, "fused": G.DECODE_FUSED}[args.schedule]
    dec = bench_decode(G, synth, args.steps, args.warmup, B, P, T_max,
                       use_graph=not args.no_graph, schedule=sched)
    # headline: HIP-graph replay when available (what a serving loop runs),
    # with the eager figure reported beside it
    headline_us = dec["graph_us_step"] if dec["graph_us_step"] is not None else dec["us_step"]
    nb = decode_bytes(B, P)
    step_tbs = nb["step"] / (headline_us * 1e-6) / 1e12
    src = "grouped_query_attention_gemv_amd/csrc/decode.hip"
    if dec["schedule"] == "fused":
        # one kernel carries the whole step, so the step time measured over
        # the timed region (HIP events on the stream the graph or the calls
        # run on) is that kernel's average duration
        dom_us = headline_us
        dom_bytes = nb["step"]
        roof_kernel = ("decode_step_kernel<1> (whole step in one launch: QKV + RoPE + append, "
                       "attention, wo)")
        traffic = counter_traffic("decode_p1000_hbm_traffic.md", "decode_step_kernel<1>", src)
    else:
        dom_us = dec["kern_us"]["qkv"]
        dom_bytes = nb["qkv"]
        roof_kernel = "decode_qkv_kernel<1, 8> (QKV GEMV + RoPE + cache append)"
        traffic = counter_traffic("decode_p1000_hbm_traffic.md", "decode_qkv_kernel<1, 8>", src)
    dom_gbs = dom_bytes / (dom_us * 1e-6) / 1e9
    other = None
    if dec["schedule"] == "fused":
        # the three-launch schedule on the same workload, for comparison
        alt = bench_decode(G, synth, args.steps, args.warmup, B, P, T_max,
                           use_graph=not args.no_graph, schedule=G.DECODE_SPLIT)
        alt_us = alt["graph_us_step"] if alt["graph_us_step"] is not None else alt["us_step"]
        other = {"schedule": "split", "us_step": round(alt_us, 3),
                 "kernels_us": {k: round(v, 3) for k, v in alt["kern_us"].items()}}

    record = {
        "metric": METRIC,
        "value": round(headline_us, 3),
        "unit": "us/block-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": headline_us / 1000.0,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,1) x and cache, N(0,0.02) weights; 8 rotated sets)",
        "config": {"workload": f"Llama-3.1-8B GQA block decode, B=1, P={P} (write row {P}, "
                               f"read rows 0-{P})",
                   "B": B, "P": P, "T_max": T_max, "d": 4096, "heads": 32, "kv_heads": 8,
                   "head_dim": 128, "rope": "scaled, theta=5e5",
                   "hip_graph": dec["graph_us_step"] is not None,
                   "schedule": dec["schedule"]},
        "hbm_tbs": round(step_tbs, 4),
        "hbm_frac_of_peak": round(step_tbs * 1000.0 / HBM_PEAK_GBS, 4),
        "tokens_per_s": B / (headline_us * 1e-6),
        "eager_us_step": round(dec["us_step"], 3),
        "host_us_per_eager_step": round(dec["wall_us_step"], 3),
        # one set reused every step, held by the Infinity Cache: not the headline
        "hot_cache_us_step": (round(dec["hot_cache_us_step"], 3)
                              if dec["hot_cache_us_step"] is not None else None),
        # p10 / median / p90 of 20 separately timed 8-step replays (per step)
        "us_step_p10_p50_p90": ([round(v, 3) for v in dec["graph_spread_us"]]
                                if dec["graph_spread_us"] is not None else None),
        "algorithmic_bytes_per_step": nb["step"],
        "kernels_us": {k: round(v, 3) for k, v in dec["kern_us"].items()},
        "profiled_us_step": round(dec["profiled_us_step"], 3),
        "roofline": {"kernel": roof_kernel,
                     "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": dom_bytes},
    }
    if other is not None:
        record["other_schedule"] = other
    if args.workload == "decode_p128":
        record["roofline"]["traffic"] = None    # counters were taken on the P=1000 run
    if not args.no_prefill:
        record["prefill"] = bench_prefill(G, synth, steps=10, warmup=3)
    if not args.no_cpu:
        record["cpu_baseline"] = cpu_baseline(synth, B, P)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
