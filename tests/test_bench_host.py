"""Host-side checks of bench.py's measurement logic (no GPU): the algorithmic
work it divides by, the roofline arithmetic, the code digest that keys the
counter summaries, the summaries' calibration, and the refusal of more than
one GPU."""
from __future__ import annotations

import csv
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_decode_bytes_match_the_workloads_algorithmic_work(bench):
    """Whole-step bytes: weights 83,886,080 + B*P*4096 (cache read) + B*4096
    (cache write) + B*8192 (x) + B*16384 (out, fp32) + 512 (the RoPE row), the
    count of the page "Llama 3.1 8B . Grouped-query attention", In numbers,
    evaluated at the five workloads."""
    assert bench.decode_bytes(1, 128)["step"] == 84_439_552
    assert bench.decode_bytes(1, 1000)["step"] == 88_011_264
    assert bench.decode_bytes(64, 8192)["step"] == 2_233_205_248
    assert bench.decode_bytes(8, 131071)["step"] == 4_379_050_496
    # per kernel: attention reads rows 0..P of K and V (row P just written)
    # plus Q and writes O's two parts
    a = bench.decode_bytes(8, 131071)["attn"]
    assert a == 8 * 131072 * 8 * 128 * 2 * 2 + 8 * 4096 * 4 + 8 * 4096 * 2 * 2
    # multi-head: 32 key/value heads, 4x the cache bytes and 4096 + 8192 QKV rows
    m = bench.decode_bytes(1, 1000, 32)
    assert m["step"] == (4096 + 8192 + 4096) * 4096 * 2 + 1000 * 32 * 128 * 4 + 32 * 128 * 4 \
        + 8192 + 16384 + 512


def test_prefill_flops_match_the_workloads_algorithmic_work(bench):
    """B = 4, T = 2048 from position 0: QKV 412.32, causal attention 137.51
    and wo 274.88 GFLOP (824.70 in all)."""
    f = bench.prefill_flops(4, 2048)
    assert round(f["qkv"] / 1e9, 2) == 412.32
    assert round(f["attn"] / 1e9, 2) == 137.51
    assert round(f["wo"] / 1e9, 2) == 274.88
    assert round(f["total"] / 1e9, 2) == 824.70
    # chunked: token i after 2048 cached rows sees 2048 + i + 1 keys
    c = bench.prefill_flops(4, 2048, 2048)
    assert c["attn"] == 4.0 * 4 * (2048 * 2048 + 2048 * 2049 / 2) * 32 * 128


def test_roofline_is_work_over_time_against_the_peak(bench):
    r = bench.roofline("k", "hbm", 88_011_264, 22.0)
    assert r["achieved"] == round(88_011_264 / 22e-6 / 1e9, 1)
    assert r["frac"] == round(r["achieved"] / 8000.0, 4)
    r = bench.roofline("g", "mfma", 412.32e9, 330.0)
    assert r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["achieved"] - 412.32e9 / 330e-6 / 1e12) < 0.1


def test_code_digest_ignores_comments_only(bench, tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() {\n  return 1;  // one\n}\n/* block\n comment */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.code_digest("k.hip")
    src.write_text("// header\nint f() {\n\n  return 1;  // the value one\n}\n")
    assert bench.code_digest("k.hip") == d0
    src.write_text("int f() {\n  return 2;\n}\n")
    assert bench.code_digest("k.hip") != d0
    # several sources: a change in any of them changes the digest
    hdr = tmp_path / "k.h"
    hdr.write_text("#define K 1\n")
    d1 = bench.code_digest(("k.hip", "k.h"))
    hdr.write_text("#define K 1  // one\n")
    assert bench.code_digest(("k.hip", "k.h")) == d1
    hdr.write_text("#define K 2\n")
    assert bench.code_digest(("k.hip", "k.h")) != d1
    assert set(bench.DECODE_SRC) >= {"grouped_query_attention_gemv_amd/csrc/decode.hip",
                                     "grouped_query_attention_gemv_amd/csrc/common.h"}


def test_committed_traffic_summaries_match_the_current_decode_code(bench):
    """roofline.traffic comes from profiles/*_hbm_traffic.md only while the
    kernels' code is the code the counters were taken on."""
    for summary, kernel in (("decode_p1000_hbm_traffic.md", "decode_step_kernel<1, 8>"),
                            ("decode_p128_hbm_traffic.md", "decode_step_kernel<1, 8>"),
                            ("decode_b64_p8192_hbm_traffic.md", "decode_attn_kernel<8>"),
                            ("stacked_b8_p131071_hbm_traffic.md", "decode_attn_kernel<8>")):
        t = bench.counter_traffic(summary, kernel)
        assert t is not None, f"{summary}: stale or missing for {kernel}"
        assert t > 0


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_pmc_summary_scales_by_the_copy_probe(bench, tmp_path):
    """FETCH_SIZE and WRITE_SIZE are each scaled by what they read for the
    256 MiB copy the counter runs start with."""
    fc, wc = tmp_path / "f.csv", tmp_path / "w.csv"
    copy = "__amd_rocclr_copyBuffer"          # the runtime copy kernel of the 256 MiB probe
    k = "void gqa::decode_attn_kernel<8>(gqa::DecodeParams)"
    _write_counters(fc, [(copy, "FETCH_SIZE", 131072.0), (k, "FETCH_SIZE", 1000.0), (k, "FETCH_SIZE", 1000.0)])
    _write_counters(wc, [(copy, "WRITE_SIZE", 262144.0), (k, "WRITE_SIZE", 10.0), (k, "WRITE_SIZE", 10.0)])
    out = tmp_path / "s.md"
    bench.pmc_summary(str(fc), str(wc), 256, "t", ["cmd"], str(out))
    text = out.read_text()
    want = int(round((1000.0 * 2.0 + 10.0 * 1.0) * 1024))
    assert f"traffic_bytes_per_launch[decode_attn_kernel<8>]: {want}" in text


def test_counter_summary_derives_matrix_core_busy(bench, tmp_path):
    """busy / (SQ_BUSY_CYCLES / 32 engines * 1024 SIMDs)."""
    c = tmp_path / "c.csv"
    k = "void gqa::gemm_kernel<0>(gqa::GemmArgs)"
    _write_counters(c, [(k, "SQ_BUSY_CYCLES", 32.0 * 1000), (k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 500),
                        (k, "SQ_VALU_MFMA_COEXEC_CYCLES", 1024.0 * 100),
                        (k, "SQ_INSTS_MFMA", 100.0), (k, "SQ_INSTS_VALU", 250.0)])
    out = tmp_path / "s.md"
    bench.counter_summary([str(c)], "t", ["cmd"], str(out))
    text = out.read_text()
    assert "gemm_kernel<0>: matrix cores busy 50.0% of 1,000 cycles" in text
    assert "VALU co-executing in 20.0% of them" in text
    assert "1.50 other VALU instructions per MFMA" in text
    # the LDS figure appears when its two counters are there
    assert "LDS bank conflicts" not in text
    c2 = tmp_path / "c2.csv"
    _write_counters(c2, [(k, "SQ_LDS_BANK_CONFLICT", 25.0), (k, "SQ_LDS_IDX_ACTIVE", 1000.0)])
    bench.counter_summary([str(c), str(c2)], "t", ["cmd"], str(out))
    assert "LDS bank conflicts in 2.5% of LDS-active cycles" in out.read_text()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
