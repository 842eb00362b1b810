"""Benchmark of the Llama-3.1-8B GQA attention block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all]

The default run measures every configuration of the block's benchmark on one
GPU and prints one JSON line:

  headline (``value``)  32 stacked blocks decoding B = 8 sequences at
                        P = 131,071 cached positions each (128 GiB of cache),
                        residual h <- h + Delta, no norms or FFN: microseconds
                        per block-step.  A step is one pass through all 32
                        blocks; K steps are timed after W warm-up steps.
  sub-records           decode B = 1 at start_pos 128 and at P = 1,000, the
                        causal prefill B = 4, T = 2,048, and the batched
                        decode B = 64, P = 8,192, each with its own roofline.

Every record carries a ``roofline`` object for its dominant kernel: the
algorithmic bytes (or FLOPs) of one launch divided by that kernel's average
duration, measured here with HIP events on the stream the library launches
on, and ``traffic``, the HBM bytes per launch from the rocprofv3
FETCH_SIZE/WRITE_SIZE summaries in profiles/ (null when the kernel's code
changed since they were taken).  Inputs are seeded synthetic bf16 tensors
already resident in HBM; decode workloads that read less than the 256 MB
Infinity Cache rotate 8 independent weight + cache sets.  After every timed
loop the workspace's error word is checked.

``cpu_baseline`` times the fp64 oracle on this host's cores on a bounded
sample of the headline workload (one block's decode step for one of its 8
sequences at P = 131,071, scaled to the block-step); the B = 1, P = 1,000
sub-record carries its own (whole block-steps).

Other workloads: --workload decode_p128 | decode_p1000 | prefill | batched |
stacked_long | mha_batched | mha_decode_p1000 | kv16_decode_p1000 |
chunked_prefill | layer_decode_p1000 | vocab_b1 (one record each), and
--pmc-summary to turn rocprofv3 counter runs into a profiles/ summary.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
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
# the decode kernels' whole source: decode.hip and the headers it includes
DECODE_SRC = tuple(f"grouped_query_attention_gemv_amd/csrc/{f}"
                   for f in ("decode.hip", "common.h", "gemv.h", "kernels.h"))

D, NQKV, KVH, HD = 4096, 6144, 8, 128


# ----------------------------------------------------------------------------
# algorithmic work
# ----------------------------------------------------------------------------

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


def roofline(kernel: str, bound: str, work: float, us: float, traffic=None) -> dict:
    """Roofline object of one kernel: work per launch (bytes or FLOPs) over
    its average launch duration in microseconds."""
    if bound == "hbm":
        ach = work / (us * 1e-6) / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": int(work), "kernel_us": round(us, 3)}
    ach = work / (us * 1e-6) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
            "algorithmic_flops": work, "kernel_us": round(us, 3)}


def code_digest(paths) -> str:
    """sha256 of C++ sources (one path or several, in order) with their
    comments and blank lines removed, so that a counter summary stays valid
    across edits that change only comments (string literals in these sources
    hold no comment markers)."""
    lines = []
    for path in ((paths,) if isinstance(paths, str) else paths):
        text = open(os.path.join(ROOT, path)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines += [ln.rstrip() for ln in text.splitlines() if ln.strip()]
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def counter_traffic(summary: str, kernel: str, source: str = DECODE_SRC):
    """HBM bytes per launch of `kernel` measured by rocprofv3 (FETCH_SIZE +
    WRITE_SIZE, calibrated on a known-size copy), as recorded in a profile
    summary; None when the kernel source has changed since the counters were
    taken, or when no summary holds the kernel."""
    try:
        fields = {}
        for line in open(os.path.join(ROOT, "profiles", summary)).read().splitlines():
            line = line.strip()
            if line.startswith(("traffic_bytes_per_launch[", "kernel_code_sha256:")):
                k, v = line.split(": ", 1)
                fields[k] = v
        if fields.get("kernel_code_sha256") != code_digest(source):
            return None
        return int(fields[f"traffic_bytes_per_launch[{kernel}]"])
    except (OSError, KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------
# timing helpers
# ----------------------------------------------------------------------------

def _sync_all():
    """Barrier of this one-process run: every queued GPU operation done."""
    torch.cuda.synchronize()


def _timed_steps(step, steps, warmup, use_graph):
    """Whole-loop timing of `steps` calls of step(i) (graph replay of the
    whole loop when use_graph), HIP events on the current stream; returns
    microseconds per step."""
    for i in range(warmup):
        step(i)
    _sync_all()
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
        _sync_all()
        t0.record()
        g.replay()
        t1.record()
    else:
        _sync_all()
        t0.record()
        for i in range(steps):
            step(i)
        t1.record()
    _sync_all()
    return t0.elapsed_time(t1) * 1000.0 / steps


def _stage_events(G, n_stages, steps, call):
    """Mean microseconds of each stage over `steps` calls of call(i, events),
    the library recording a HIP event on its stream between stages."""
    ev = G.HipEvents(n_stages + 1)
    per = np.zeros((steps, n_stages))
    for i in range(steps):
        call(i, ev)
        for k in range(n_stages):
            per[i, k] = ev.elapsed_ms(k, k + 1)
    ev.close()
    return (per.mean(axis=0) * 1000.0).tolist()


def _assert_clean(G, ws, where):
    err = G.workspace_errors(ws)
    if err:
        raise RuntimeError(f"{where}: workspace error word {err:#x} after the timed loop")


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def _decode_sets(G, synth, B, P, T_max, kvh, dev):
    sets = []
    for s in range(N_SETS):
        x, w, kc_rows, vc_rows = synth.decode_workload(s, B, P, n_kv_heads=kvh)
        kc, vc = G.empty_caches(B, T_max, dev, kvh)
        kc.zero_()
        vc.zero_()
        G.kcache_by_position(kc)[:, :P] = kc_rows.to(dev)
        G.vcache_write(vc, 0, vc_rows.to(dev))
        sets.append(dict(x=x.to(dev), w=[t.to(dev) for t in w], kc=kc, vc=vc))
    return sets


def bench_decode(G, synth, steps, warmup, B=1, P=1000, T_max=1024, schedule=None, kvh=KVH,
                 use_graph=True, spread=True):
    """Graph-replay, eager and per-kernel timings of decode steps over 8
    rotated weight + cache sets under `schedule` (the library's choice when
    None)."""
    dev = torch.device("cuda:0")
    schedule = G.DECODE_AUTO if schedule is None else schedule
    fused = G.decode_schedule(B, P, T_max, kvh, schedule) == G.DECODE_FUSED
    sets = _decode_sets(G, synth, B, P, T_max, kvh, dev)
    rope = G.rope_table(T_max, device=dev)
    ws = G.workspace(G.OP_DECODE, B, T_max, dev, n_kv_heads=kvh)
    out = torch.empty((B, D), dtype=torch.float32, device=dev)

    def step(i, events=None):
        st = sets[i % N_SETS]
        G.block_decode(st["x"], *st["w"], st["kc"], st["vc"], rope, P, out=out, ws=ws,
                       events=events, schedule=schedule)

    eager_us = _timed_steps(step, steps, warmup, False)
    graph_us = _timed_steps(step, steps, 0, True) if use_graph else None
    _assert_clean(G, ws, "decode")
    spread_us = None
    if use_graph and spread:
        # p10 / median / p90 of 20 separately timed replays of 8 steps (one per set)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        g8 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g8):
            for i in range(N_SETS):
                step(i)
        g8.replay()
        reps = []
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        for _ in range(20):
            _sync_all()
            t0.record()
            g8.replay()
            t1.record()
            _sync_all()
            reps.append(t0.elapsed_time(t1) * 1000.0 / N_SETS)
        spread_us = [round(float(np.percentile(reps, q)), 3) for q in (10, 50, 90)]
        _assert_clean(G, ws, "decode spread")
    # one set reused every step: held by the Infinity Cache, not a headline
    hot_us = _timed_steps(lambda i: step(0), steps, 3, True) if use_graph else None
    kern = _stage_events(G, G.DECODE_STAGES, min(steps, 100), lambda i, ev: step(i, ev))
    _assert_clean(G, ws, "decode stages")
    names = ["decode_step"] if fused else ["qkv", "attn", "wo"]
    return dict(us_step=graph_us if graph_us is not None else eager_us, eager_us=eager_us,
                graph=graph_us is not None, hot_cache_us=hot_us, spread_us=spread_us,
                fused=fused, kern_us=dict(zip(names, kern)),
                off_home_launches=G.workspace_off_home(ws))


def record_decode_b1(G, synth, P, T_max, steps, warmup, traffic_summary):
    """Sub-record of a B = 1 decode workload (configs 1 and 2)."""
    dec = bench_decode(G, synth, steps, warmup, 1, P, T_max)
    alt = bench_decode(G, synth, steps, warmup, 1, P, T_max, schedule=G.DECODE_SPLIT,
                       spread=False)
    nb = decode_bytes(1, P)
    us = dec["us_step"]
    if dec["fused"]:
        # one kernel per step: the step time over the timed region is that
        # kernel's average duration (HIP events on the stream the graph runs on)
        kname = "decode_step_kernel<1, 8>"
        roof = roofline(kname, "hbm", nb["step"], us, counter_traffic(traffic_summary, kname))
    else:
        kname = "decode_qkv_kernel<1, 8, 4>"
        roof = roofline(kname, "hbm", nb["qkv"], dec["kern_us"]["qkv"],
                        counter_traffic(traffic_summary, kname))
    tbs = nb["step"] / (us * 1e-6) / 1e12
    return {
        "config": {"workload": f"Llama-3.1-8B GQA block decode, B=1, start_pos={P} (cache rows "
                               f"0-{P - 1} filled, row {P} written, rows 0-{P} read)",
                   "B": 1, "P": P, "T_max": T_max, "schedule": "fused" if dec["fused"] else "split",
                   "hip_graph": dec["graph"], "rotated_sets": N_SETS},
        "value": round(us, 3), "unit": "us/block-step", "steps": steps,
        "ms_per_step": round(us / 1000.0, 6), "hbm_tbs": round(tbs, 4),
        "hbm_frac_of_peak": round(tbs * 1000.0 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": nb["step"],
        "eager_us_step": round(dec["eager_us"], 3),
        "hot_cache_us_step": None if dec["hot_cache_us"] is None else round(dec["hot_cache_us"], 3),
        "us_step_p10_p50_p90": dec["spread_us"],
        "kernels_us": {k: round(v, 3) for k, v in dec["kern_us"].items()},
        "fused_launches_placed_off_xcd": dec["off_home_launches"],
        "three_launch_schedule": {"us_step": round(alt["us_step"], 3),
                                  "kernels_us": {k: round(v, 3) for k, v in alt["kern_us"].items()}},
        "roofline": roof,
    }


def identity_check_p1000(G, synth):
    """Config 2's check against a full causal prefill over 1,001 tokens: the
    GPU decode of token 1,000 after a GPU prefill of 1,000 tokens against the
    last row of a GPU prefill of 1,001 tokens (normalised max / mean
    difference; the parity tests hold both against the oracle)."""
    dev = torch.device("cuda:0")
    T = 1000
    x, w = synth.prefill_workload(0, 1, T + 1)
    x, w = x.to(dev), [t.to(dev) for t in w]
    rope = G.rope_table(1024, device=dev)
    kc, vc = G.empty_caches(1, 1024, dev)
    full = G.block_prefill(x, *w, kc, vc, rope)
    kc2, vc2 = G.empty_caches(1, 1024, dev)
    G.block_prefill(x[:, :T].contiguous(), *w, kc2, vc2, rope)
    dec = G.block_decode(x[:, T].contiguous(), *w, kc2, vc2, rope, T)
    _sync_all()
    ref = full[:, T].double()
    d = (dec.double() - ref).abs()
    rms = float(ref.pow(2).mean().sqrt())
    return {"decode_after_prefill_1000_vs_prefill_1001_last_row":
            {"max_over_rms": float(d.max()) / rms, "mean_over_rms": float(d.mean()) / rms}}


def bench_prefill(G, synth, steps, warmup, B=4, T=2048, kvh=KVH, wo16=False):
    """Prefill timings: calls back to back (whole call), then a pass with HIP
    events between the kernels (per-kernel split)."""
    dev = torch.device("cuda:0")
    x, w = synth.prefill_workload(0, B, T, n_kv_heads=kvh)
    x = x.to(dev)
    w = [t.to(dev) for t in w]
    kc, vc = G.empty_caches(B, T, dev, kvh)
    rope = G.rope_table(T, device=dev)
    ws = G.workspace(G.OP_PREFILL, B, T, dev, T, 0, kvh)
    out = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    w16 = G.wo_to_fp16(w[3]) if wo16 else None

    def call(i, events=None):
        G.block_prefill(x, *w[:3], None if wo16 else w[3], kc, vc, rope, out=out, ws=ws,
                        events=events, wo16=w16)

    us = _timed_steps(call, steps, warmup, False)
    _assert_clean(G, ws, "prefill")
    kern = dict(zip(["prep", "qkv", "attn", "wo"],
                    _stage_events(G, G.PREFILL_STAGES, steps, call)))
    _assert_clean(G, ws, "prefill stages")
    fl = prefill_flops(B, T, kvh=kvh)
    return dict(B=B, T=T, us=us, fl=fl, kern=kern)


def record_prefill(G, synth):
    """Sub-record of config 3 (causal prefill B = 4, T = 2,048)."""
    steps = 10
    pf = bench_prefill(G, synth, steps, 3)
    pf16 = bench_prefill(G, synth, steps, 3, wo16=True)
    fl, us, kern = pf["fl"], pf["us"], pf["kern"]
    dom = max(("qkv", "attn", "wo"), key=lambda k: kern[k])
    kname = {"qkv": "gemm_kernel<GEMM_QKV>", "attn": "prefill_attn_kernel<8>",
             "wo": "gemm_kernel<GEMM_OUT>"}[dom]
    return {
        "config": {"workload": "Llama-3.1-8B GQA block causal prefill, B=4, T=2048 from "
                               "position 0 (cache rows 0-2047 written, Delta [4, 2048, 4096])",
                   "B": 4, "T": 2048, "start_pos": 0},
        "value": round(4 * 2048 / (us * 1e-6), 1), "unit": "tokens/s", "steps": steps,
        "ms_per_step": round(us / 1000.0, 5), "us_per_call": round(us, 2),
        "mfma_util": round(fl["total"] / (us * 1e-6) / (MFMA_PEAK_TFLOPS * 1e12), 4),
        "algorithmic_gflop": round(fl["total"] / 1e9, 3),
        "kernels_us_with_events": {k: round(v, 2) for k, v in kern.items()},
        "kernels_tflops": {k: round(fl[k] / (kern[k] * 1e-6) / 1e12, 1) for k in ("qkv", "attn", "wo")},
        "with_caller_fp16_wo": {"us_per_call": round(pf16["us"], 2),
                                "tokens_per_s": round(4 * 2048 / (pf16["us"] * 1e-6), 1),
                                "mfma_util": round(fl["total"] / (pf16["us"] * 1e-6) /
                                                   (MFMA_PEAK_TFLOPS * 1e12), 4)},
        "roofline": roofline(kname, "mfma", fl[dom], kern[dom]),
    }


def bench_batched(G, synth, steps, warmup, B=64, P=8192, T_max=8224, kvh=KVH):
    """Batched decode: B = 64 sequences with 8,192 cached positions each."""
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
    ws = G.workspace(G.OP_DECODE, B, T_max, dev, n_kv_heads=kvh)
    out = torch.empty((B, D), dtype=torch.float32, device=dev)

    def step(i, events=None):
        G.block_decode(xs[i % n_w], *ws_sets[i % n_w], kc, vc, rope, P, out=out, ws=ws,
                       events=events)

    us = _timed_steps(step, steps, warmup, True)
    _assert_clean(G, ws, "batched decode")
    kern = dict(zip(["qkv", "attn", "wo"], _stage_events(G, G.DECODE_STAGES, steps, step)))
    _assert_clean(G, ws, "batched decode stages")
    return us, kern, decode_bytes(B, P, kvh)


def record_batched(G, synth, kvh=KVH):
    """Sub-record of config 4 (batched decode B = 64, P = 8,192)."""
    steps = 50
    us, kern, nb = bench_batched(G, synth, steps, 10, kvh=kvh)
    tbs = nb["step"] / (us * 1e-6) / 1e12
    kname = f"decode_attn_kernel<{kvh}>"
    summary = "decode_b64_p8192_hbm_traffic.md" if kvh == KVH else "decode_mha_b64_p8192_hbm_traffic.md"
    kind = "GQA" if kvh == KVH else "multi-head (n_kv = 32)"
    return {
        "config": {"workload": f"Llama-3.1-8B-shaped attention block batched decode, {kind}, "
                               "B=64 sequences with P=8192 cached positions each",
                   "B": 64, "P": 8192, "T_max": 8224, "kv_heads": kvh, "hip_graph": True},
        "value": round(us, 3), "unit": "us/block-step", "steps": steps,
        "ms_per_step": round(us / 1000.0, 6), "hbm_tbs": round(tbs, 4),
        "hbm_frac_of_peak": round(tbs * 1000 / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(64 / (us * 1e-6), 1), "algorithmic_bytes_per_step": nb["step"],
        "kernels_us": {k: round(v, 3) for k, v in kern.items()},
        "roofline": roofline(kname, "hbm", nb["attn"], kern["attn"], counter_traffic(summary, kname)),
    }


def run_stacked(G, synth, steps, warmup, B=8, P=131071, T_max=131072, L=32, cpu_sample=False):
    """32 stacked blocks, B = 8, 131,071 cached positions per sequence per
    block (128 GiB of cache), residual h <- h + Delta, no norms or FFN.  One
    step runs all 32 blocks.  With cpu_sample, also returns a host copy of
    one block's inputs for one sequence (the oracle's sample)."""
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
        if (l + 1) % 8 == 0:
            _sync_all()
            print(f"stacked: {l + 1}/{L} blocks staged ({time.perf_counter() - t_start:.1f} s)",
                  file=sys.stderr, flush=True)
    rope = G.rope_table(T_max, device=dev)
    ws = G.workspace(G.OP_DECODE, B, T_max, dev)
    h = torch.empty((B, D), dtype=torch.float32, device=dev)
    xa = torch.empty_like(x0)
    xb = torch.empty_like(x0)

    def step(i, events=None):
        h.copy_(x0)
        xa.copy_(x0)
        a, b = xa, xb
        for k, (w, kc, vc) in enumerate(blocks):
            G.block_decode(a, *w, kc, vc, rope, P, out=h, out_bf16=b, accumulate=True, ws=ws,
                           events=None if events is None else events[k])
            a, b = b, a

    for i in range(warmup):
        step(i)
    _sync_all()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    _sync_all()
    us_step = t0.elapsed_time(t1) * 1000.0 / steps
    _assert_clean(G, ws, "stacked decode")
    finite = bool(torch.isfinite(h).all())
    # per-kernel split: one more 32-block step with events between the kernels
    evs = [G.HipEvents(G.DECODE_STAGES + 1) for _ in range(L)]
    step(0, evs)
    per = np.array([[e.elapsed_ms(k, k + 1) for k in range(G.DECODE_STAGES)] for e in evs])
    for e in evs:
        e.close()
    _assert_clean(G, ws, "stacked decode stages")
    kern = dict(zip(["qkv", "attn", "wo"], (per.mean(axis=0) * 1000.0).tolist()))
    sample = None
    if cpu_sample:
        # block 0, sequence 0: its input and cached rows 0 .. P-1 (decode
        # writes only row P, so these are the rows every step read)
        w, kc, vc = blocks[0]
        sample = dict(x=x0[0:1].cpu(), w=[t.cpu() for t in w], P=P, B=B,
                      k=G.kcache_by_position(kc[0:1])[:, :P].cpu(),
                      v=G.vcache_read(vc[0:1], 0, P).cpu())
    return us_step, kern, decode_bytes(B, P), finite, sample


def record_stacked(G, synth, steps, warmup, cpu_sample=False):
    us, kern, nb, finite, sample = run_stacked(G, synth, steps, warmup, cpu_sample=cpu_sample)
    per_block = us / 32
    tbs = nb["step"] / (per_block * 1e-6) / 1e12
    kname = "decode_attn_kernel<8>"
    return {
        "config": {"workload": "32 stacked Llama-3.1-8B GQA blocks decoding B=8 sequences at "
                               "P=131071 cached positions each (128 GiB cache), residual "
                               "h <- h + Delta, no norms/FFN",
                   "B": 8, "P": 131071, "T_max": 131072, "blocks": 32, "hip_graph": False},
        "value": round(per_block, 3), "unit": "us/block-step", "steps": steps,
        "blocks_per_step": 32, "ms_per_step": round(us / 1000.0, 4),
        "hbm_tbs": round(tbs, 4), "hbm_frac_of_peak": round(tbs * 1000 / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(8 / (us * 1e-6), 2), "algorithmic_bytes_per_block_step": nb["step"],
        "kernels_us_per_block": {k: round(v, 3) for k, v in kern.items()},
        "outputs_finite": finite,
        "roofline": roofline(kname, "hbm", nb["attn"], kern["attn"],
                             counter_traffic("stacked_b8_p131071_hbm_traffic.md", kname)),
    }, sample


def _blas_threads(cores):
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=cores)
    except Exception:
        return None


def cpu_baseline_stacked(sample, budget_s=15.0):
    """The oracle as it stands, timed on this host on a bounded sample of the
    32-block workload: one block's decode step for one of its B sequences at
    P = 131,071 (the same inputs the GPU read), repeated for about budget_s of
    wall time and scaled by B to the unit of the headline, microseconds per
    block-step (each block-step decodes B sequences)."""
    from oracle import gqa_oracle as O
    cores = len(os.sched_getaffinity(0))
    f = lambda t: t.float().numpy().astype(np.float64)
    x = f(sample["x"])[:, None, :]
    w = [f(t) for t in sample["w"]]
    kc, vc = f(sample["k"]), f(sample["v"])
    P, B = sample["P"], sample["B"]
    limiter = _blas_threads(cores)
    n = 0
    t0 = time.perf_counter()
    while True:
        O.gqa_block(x, *w, kc, vc, P)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": round(el / n * B * 1e6, 1), "unit": "us/block-step", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{n} single-sequence decode steps of one block at P={P} (block 0, "
                      f"sequence 0 of the workload's inputs) of the fp64 NumPy oracle, "
                      f"{el:.1f} s of wall time, scaled x{B} to a block-step of {B} sequences; "
                      f"BLAS threads = {cores} (the cores this process may run on); inputs "
                      f"already converted to fp64"}


def cpu_baseline(synth, B=1, P=1000, budget_s=12.0):
    """The oracle as it stands, timed on this host on a bounded sample of the
    same workload: whole decode block-steps repeated for about budget_s of
    wall time, with the BLAS thread pool set to the cores this process may
    run on."""
    from oracle import gqa_oracle as O
    cores = len(os.sched_getaffinity(0))
    x, w, kc, vc = synth.decode_workload(0, B, P)
    f = lambda t: t.float().numpy().astype(np.float64)
    xs, ws = f(x)[:, None, :], [f(t) for t in w]
    kcs, vcs = f(kc), f(vc)
    limiter = _blas_threads(cores)
    n = 0
    t0 = time.perf_counter()
    while True:
        O.gqa_block(xs, *ws, kcs, vcs, P)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 20000:
            break
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": round(el / n * 1e6, 1), "unit": "us/block-step", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{n} whole decode block-steps (B={B}, P={P}) of the fp64 NumPy oracle, "
                      f"{el:.1f} s of wall time, BLAS threads = {cores} (the cores this "
                      f"process may run on), inputs already converted to fp64"}


# ----------------------------------------------------------------------------
# extra workloads (one record each)
# ----------------------------------------------------------------------------

def bench_layer_decode(G, synth, steps, warmup, B=1, P=1000, T_max=1024):
    """Graph-replay time per step of the layer (RMSNorm, block, residual) and
    of the bare block on the same rotated inputs."""
    dev = torch.device("cuda:0")
    sets = _decode_sets(G, synth, B, P, T_max, KVH, dev)
    for s_, st in enumerate(sets):
        st["g"] = synth.norm_gain(100 + s_).to(dev)
    rope = G.rope_table(T_max, device=dev)
    ws = G.workspace(G.OP_LAYER_DECODE, B, T_max, dev)
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
    lay, blk = _timed_steps(layer, n, warmup, True), _timed_steps(block, n, warmup, True)
    _assert_clean(G, ws, "layer decode")
    return lay, blk


def bench_chunked_prefill(G, synth, steps, warmup, B=4, P=2048, T=2048):
    """Whole-call timing of a prefill of T tokens after P cached rows."""
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
    ws = G.workspace(G.OP_PREFILL, B, T_max, dev, T, P)
    out = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    us = _timed_steps(lambda i: G.block_prefill(x, *w, kc, vc, rope, out=out, ws=ws, start_pos=P),
                      steps, warmup, False)
    _assert_clean(G, ws, "chunked prefill")
    return us, prefill_flops(B, T, P)


def _base_record(args):
    return {"metric": METRIC, "n_gpus": 1, "warmup": args.warmup, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded bf16 N(0,1) x and cache, N(0,0.02) weights)"}


def extra_workload(G, synth, args):
    w = args.workload
    rec = _base_record(args)
    if w in ("batched", "mha_batched"):
        rec.update(record_batched(G, synth, 32 if w == "mha_batched" else KVH))
        rec["higher_is_better"] = False
    elif w in ("decode_p128", "decode_p1000"):
        P, T_max = (128, 256) if w == "decode_p128" else (1000, 1024)
        rec.update(record_decode_b1(G, synth, P, T_max, args.steps, args.warmup,
                                    f"decode_p{P}_hbm_traffic.md"))
        rec["higher_is_better"] = False
    elif w == "prefill":
        rec.update(record_prefill(G, synth))
        rec["higher_is_better"] = True
    elif w == "stacked_long":
        rec.update(record_stacked(G, synth, args.steps, args.warmup)[0])
        rec["higher_is_better"] = False
    elif w in ("mha_decode_p1000", "kv16_decode_p1000"):
        kvh = 32 if w.startswith("mha") else 16
        dec = bench_decode(G, synth, args.steps, args.warmup, 1, 1000, 1024, kvh=kvh)
        nb = decode_bytes(1, 1000, kvh)
        us = dec["us_step"]
        tbs = nb["step"] / (us * 1e-6) / 1e12
        if dec["fused"]:
            # one kernel per step, as for 8 kv heads
            roof = roofline(f"decode_step_kernel<1, {kvh}>", "hbm", nb["step"], us)
        else:
            roof = roofline(f"decode_qkv_kernel<1, {kvh}, 4>", "hbm", nb["qkv"], dec["kern_us"]["qkv"])
        pf = bench_prefill(G, synth, 10, 3, kvh=kvh)
        rec.update({
            "value": round(us, 3), "unit": "us/block-step", "steps": args.steps,
            "ms_per_step": round(us / 1000.0, 6), "higher_is_better": False,
            "config": {"workload": "Llama-3.1-8B-shaped attention block decode, "
                                   f"{'multi-head (n_kv = 32)' if kvh == 32 else 'n_kv = 16'}, "
                                   "B=1, P=1000", "B": 1, "P": 1000, "kv_heads": kvh,
                       "schedule": "fused" if dec["fused"] else "split", "hip_graph": dec["graph"]},
            "hbm_tbs": round(tbs, 4), "hbm_frac_of_peak": round(tbs * 1000 / HBM_PEAK_GBS, 4),
            "kernels_us": {k: round(v, 3) for k, v in dec["kern_us"].items()},
            "roofline": roof,
            "prefill_b4_t2048": {"us_per_call": round(pf["us"], 2),
                                 "mfma_util": round(pf["fl"]["total"] / (pf["us"] * 1e-6) /
                                                    (MFMA_PEAK_TFLOPS * 1e12), 4)},
        })
    elif w == "layer_decode_p1000":
        steps = args.steps
        lay, blk = bench_layer_decode(G, synth, steps, min(args.warmup, 20))
        nb = decode_bytes(1, 1000)["step"] + 2 * 4096 * 2 + 2 * 4096 * 4   # + x, gain, h, h_bf16
        tbs = nb / (lay * 1e-6) / 1e12
        rec.update({"value": round(lay, 3), "unit": "us/layer-step", "steps": steps,
                    "ms_per_step": round(lay / 1000, 6), "higher_is_better": False,
                    "config": {"workload": "Llama-3.1-8B attention layer decode (RMSNorm, block, "
                                           "residual), B=1, P=1000", "B": 1, "P": 1000,
                               "hip_graph": True},
                    "block_only_us": round(blk, 3), "norm_residual_overhead_us": round(lay - blk, 3),
                    "hbm_tbs": round(tbs, 4), "hbm_frac_of_peak": round(tbs * 1000 / HBM_PEAK_GBS, 4)})
    elif w == "chunked_prefill":
        B, P, T = 4, 2048, 2048
        us, fl = bench_chunked_prefill(G, synth, 10, 3, B, P, T)
        rec.update({"value": round(B * T / (us * 1e-6), 1), "unit": "tokens/s", "steps": 10,
                    "ms_per_step": round(us / 1000, 4), "higher_is_better": True,
                    "config": {"workload": "Llama-3.1-8B GQA block chunked prefill: B=4 "
                                           "sequences, 2,048 new tokens after 2,048 cached rows",
                               "B": B, "start_pos": P, "T": T, "T_max": P + T},
                    "roofline": roofline("whole call (prep, QKV GEMM, attention, wo GEMM)", "mfma",
                                         fl["total"], us)})
    elif w == "vocab_b1":
        dev = torch.device("cuda:0")
        V, B = G.VOCAB, 1
        wt = torch.empty((V, D), dtype=torch.bfloat16, device=dev)
        synth.fill_randn_bf16_(wt, synth.generator(60, dev), 0.02)
        h = synth.randn_bf16(synth.generator(61), (B, D)).to(dev)
        g = synth.norm_gain(62).to(dev)
        L = torch.empty((B, V), dtype=torch.float32, device=dev)
        steps = 50
        us = _timed_steps(lambda i: G.vocab_logits(h, wt, g, logits=L), steps, 5, True)
        nb = V * D * 2 + B * D * 2 + D * 2 + B * V * 4
        rec.update({"value": round(us, 3), "unit": "us/call", "steps": steps,
                    "ms_per_step": round(us / 1000, 5), "higher_is_better": False,
                    "config": {"workload": "Llama-3.1 vocabulary projection with final RMSNorm, "
                                           "B=1, 4096 x 128256 bf16 weights", "B": B, "V": V,
                               "hip_graph": True},
                    "roofline": roofline("vocab_gemv_kernel<1>", "hbm", nb, us)})
    return rec


# ----------------------------------------------------------------------------
# rocprofv3 counter summaries
# ----------------------------------------------------------------------------

def _short_kernel(name: str) -> str:
    n = re.sub(r"^void ", "", name)
    n = re.sub(r"^gqa::", "", n)
    depth, out = 0, []
    for ch in n:                    # drop the parameter list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).replace("gqa::", "")


def _counter_means(path: str, counter: str):
    sums, cnt, copies = {}, {}, []
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            k = _short_kernel(row["Kernel_Name"])
            v = float(row["Counter_Value"])
            if "copyBuffer" in k:
                copies.append(v)
                continue
            if "gqa::" not in row["Kernel_Name"]:      # the library's kernels only
                continue
            sums[k] = sums.get(k, 0.0) + v
            cnt[k] = cnt.get(k, 0) + 1
    return {k: (sums[k] / cnt[k], cnt[k]) for k in sums}, copies


def pmc_summary(fetch_csv: str, write_csv: str, copy_mib: int, title: str, commands, out: str):
    """Write a profiles/ summary of two counter runs (FETCH_SIZE, WRITE_SIZE,
    KiB per dispatch), each scaled by what the counter reads for the plain
    device copy of copy_mib MiB the runs begin with."""
    fetch, fcopies = _counter_means(fetch_csv, "FETCH_SIZE")
    write, wcopies = _counter_means(write_csv, "WRITE_SIZE")
    kib = copy_mib * 1024.0
    # the copy probe is the largest copy dispatch of each run
    ffac = kib / max(fcopies)
    wfac = kib / max(wcopies)
    digest = code_digest(DECODE_SRC)
    lines = [f"# {title} — HBM traffic per kernel (rocprofv3 counters)", "",
             "Commands (two passes, one counter each, repository root):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", f"Calibration: the runs begin with a {copy_mib} MiB device-to-device copy "
              f"({kib:,.0f} KiB read and written).  Its largest dispatch read FETCH_SIZE = "
              f"{max(fcopies):,.1f} KiB and WRITE_SIZE = {max(wcopies):,.1f} KiB, so FETCH_SIZE "
              f"is scaled by {ffac:.4f} and WRITE_SIZE by {wfac:.4f} below.", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |",
              "|---|---|---|---|---|"]
    traffic = {}
    for k in sorted(fetch):
        if k not in write:
            continue
        fb, n = fetch[k]
        wb, _ = write[k]
        t = int(round((fb * ffac + wb * wfac) * 1024))
        traffic[k] = t
        lines.append(f"| {k} | {n} | {fb:,.1f} | {wb:,.1f} | {t:,} |")
    lines += ["", "Figures read by bench.py (`roofline.traffic`; it reports null instead when "
              "the code of the decode kernels (decode.hip, common.h, gemv.h, kernels.h), "
              "comments aside, differs from the code these counters were taken on):", ""]
    lines += [f"    traffic_bytes_per_launch[{k}]: {v}" for k, v in traffic.items()]
    lines += [f"    kernel_code_sha256: {digest}", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out}")


def trace_summary(stats_csv: str, bench_log: str, title: str, command: str, out: str):
    """Write a profiles/ summary of a rocprofv3 --kernel-trace --stats run:
    its per-kernel statistics (run_kernel_stats.csv) and, beside them, the
    bench.py record the traced command printed (its own HIP-event timings)."""
    rows = list(csv.DictReader(open(stats_csv)))
    rec = None
    for line in open(bench_log):
        if line.startswith("{"):
            rec = json.loads(line)
    lines = [f"# {title} — rocprofv3 kernel trace", "", "Command (repository root):", "",
             f"    {command}", "",
             "Per-kernel statistics from `run_kernel_stats.csv` (every dispatch of the run: "
             "warm-up, timed steps and the per-stage event passes):", "",
             "| kernel | calls | mean µs | min µs | max µs | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("void gqa::", "").split("(")[0]
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    if rec is not None:
        keep = {k: rec[k] for k in ("value", "unit", "ms_per_step", "kernels_us", "roofline",
                                    "hbm_frac_of_peak", "mfma_frac_of_peak", "config")
                if k in rec}
        lines += ["", "The bench.py record of the same run (HIP events around the timed "
                  "steps; `kernels_us` from the per-stage event pass):", "",
                  "    " + json.dumps(keep)]
    lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out}")


def counter_summary(csvs, title: str, commands, out: str):
    """Write a profiles/ summary of rocprofv3 --pmc runs (one counter set per
    CSV): each counter's mean per dispatch for every kernel of this library,
    and the derived matrix-core and VALU figures.  SQ_VALU_MFMA_BUSY_CYCLES
    reads 16 cycles per 16x16x32 MFMA summed over the chip's 1024 SIMDs, and
    SQ_BUSY_CYCLES the busy cycles summed over its 32 shader engines (their
    ratio to a kernel's duration gives its shader clock), so
    busy / (SQ_BUSY_CYCLES / 32 * 1024) is the fraction of the kernel's
    cycles the matrix cores worked."""
    agg = {}
    for path in csvs:
        for r in csv.DictReader(open(path)):
            name = _short_kernel(r["Kernel_Name"])
            if not name or name.startswith("at::") or "rocclr" in name:
                continue
            agg.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for d in agg.values() for c in d})
    lines = [f"# {title} — rocprofv3 counters", "", "Commands (repository root):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "Mean per dispatch:", "", "| kernel | dispatches | " + " | ".join(names) + " |",
              "|---|---|" + "---|" * len(names)]
    for k in sorted(agg):
        d = agg[k]
        n = max(len(v) for v in d.values())
        lines.append(f"| {k} | {n} | " + " | ".join(
            f"{sum(d[c]) / len(d[c]):.4g}" if c in d else "" for c in names) + " |")
    simds, engines = 1024, 32
    lines += ["", f"Derived (MI355X: {simds} SIMDs, {engines} shader engines):", ""]
    for k in sorted(agg):
        d = {c: sum(v) / len(v) for c, v in agg[k].items()}
        if d.get("SQ_BUSY_CYCLES", 0) <= 0 or d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) <= 0:
            continue
        cycles = d["SQ_BUSY_CYCLES"] / engines
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * simds)
        parts = [f"matrix cores busy {busy:.1%} of {cycles:,.0f} cycles"]
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in d:
            parts.append(f"VALU co-executing in {d['SQ_VALU_MFMA_COEXEC_CYCLES'] / d['SQ_VALU_MFMA_BUSY_CYCLES']:.1%} of them")
        if d.get("SQ_INSTS_MFMA", 0) > 0 and "SQ_INSTS_VALU" in d:
            parts.append(f"{(d['SQ_INSTS_VALU'] - d['SQ_INSTS_MFMA']) / d['SQ_INSTS_MFMA']:.2f} other VALU instructions per MFMA")
        if d.get("SQ_LDS_IDX_ACTIVE", 0) > 0 and "SQ_LDS_BANK_CONFLICT" in d:
            parts.append(f"LDS bank conflicts in {d['SQ_LDS_BANK_CONFLICT'] / d['SQ_LDS_IDX_ACTIVE']:.1%} of LDS-active cycles")
        lines.append(f"- {k}: " + "; ".join(parts) + ".")
    lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out}")


# ----------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps of the record's headline workload (default: 10 for the "
                         "32-block stack, 400 for B = 1 decode)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    ap.add_argument("--workload", default="all",
                    choices=["all", "stacked_long", "decode_p128", "decode_p1000", "prefill",
                             "batched", "mha_batched", "mha_decode_p1000", "kv16_decode_p1000",
                             "chunked_prefill", "layer_decode_p1000", "vocab_b1"])
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "TITLE", "OUT"),
                    help="write a profiles/ summary from two rocprofv3 counter runs "
                         "(commands given with --pmc-commands, calibration copy with "
                         "--copy-probe-mib)")
    ap.add_argument("--pmc-commands", nargs="*", default=[])
    ap.add_argument("--counter-summary", nargs="+", metavar="ARG",
                    help="TITLE OUT CSV [CSV ...]: write a profiles/ summary of rocprofv3 --pmc "
                         "runs (commands given with --pmc-commands)")
    ap.add_argument("--trace-summary", nargs=5, metavar=("STATS_CSV", "BENCH_LOG", "TITLE", "COMMAND", "OUT"),
                    help="write a profiles/ summary of a kernel-trace run and exit")
    args = ap.parse_args()

    if args.counter_summary:
        title, out, *csvs = args.counter_summary
        counter_summary(csvs, title, args.pmc_commands, out)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.pmc_summary:
        fcsv, wcsv, title, out = args.pmc_summary
        pmc_summary(fcsv, wcsv, args.copy_probe_mib or 256, title, args.pmc_commands, out)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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
        _sync_all()
        for _ in range(3):
            b.copy_(a)
        _sync_all()
        del a, b

    if args.workload != "all":
        if args.steps is None:
            args.steps = 10 if args.workload == "stacked_long" else 400
        if args.warmup is None:
            args.warmup = 2 if args.workload == "stacked_long" else 50
        print(json.dumps(extra_workload(G, synth, args)), flush=True)
        return

    if args.steps is None:
        args.steps = 10
    if args.warmup is None:
        args.warmup = 2
    t_all = time.perf_counter()

    def note(msg):
        print(f"bench: {msg} ({time.perf_counter() - t_all:.0f} s)", file=sys.stderr, flush=True)

    # headline: config 5, then release its 128 GiB before the others
    head, sample = record_stacked(G, synth, args.steps, args.warmup, cpu_sample=not args.no_cpu)
    note("stacked decode done")
    torch.cuda.empty_cache()
    subs = {}
    subs["decode_b1_start_pos_128"] = record_decode_b1(G, synth, 128, 256, 400, 50,
                                                       "decode_p128_hbm_traffic.md")
    note("decode start_pos 128 done")
    subs["decode_b1_p1000"] = record_decode_b1(G, synth, 1000, 1024, 400, 50,
                                               "decode_p1000_hbm_traffic.md")
    subs["decode_b1_p1000"].update(identity_check_p1000(G, synth))
    note("decode P=1000 done")
    subs["prefill_b4_t2048"] = record_prefill(G, synth)
    note("prefill done")
    torch.cuda.empty_cache()
    subs["batched_decode_b64_p8192"] = record_batched(G, synth)
    note("batched decode done")
    torch.cuda.empty_cache()

    rec = _base_record(args)
    rec.update(head)
    rec["higher_is_better"] = False
    rec["sub_records"] = subs
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline_stacked(sample)
        del sample
        note("cpu baseline done")
        subs["decode_b1_p1000"]["cpu_baseline"] = cpu_baseline(synth)
        note("cpu baseline of the B=1 decode done")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
