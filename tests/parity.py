"""Helpers shared by the GPU parity tests: comparisons against the oracle and
runners that stage seeded inputs, call the library and return what it wrote.

Tolerances (written here, used by every parity test):
  * floating point (Delta_attn, and the post-RoPE Q, K, V probes):
    max|gpu - oracle| / rms(oracle) <= 1e-2 and mean|gpu - oracle| / rms <= 2e-3;
  * cache placement: bit-exact (every element outside the written rows keeps
    its bits; the written rows sit exactly where the layout says);
  * cache values: each written bf16 is bit-exactly the round-to-nearest-even
    of the GPU's own pre-rounding value (the fp32 probe, itself within the
    tolerance above), and at most 1e-3 of them differ from the oracle's
    rounding of the fp64 value (fp32 sums may cross a rounding boundary; near
    zero such a crossing can span several bf16 steps, so no step bound).
"""
from __future__ import annotations

import os

import numpy as np
import torch

import grouped_query_attention_gemv_amd as G
from grouped_query_attention_gemv_amd import synth
from oracle import gqa_oracle as O

MAX_TOL = 1e-2
MEAN_TOL = 2e-3
FLIP_TOL = 1e-3
FLIP_FLOOR = 8     # flips allowed in any sample, however small


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a bf16/fp32 tensor."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 patterns of a bf16 tensor."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def norm_err(gpu: np.ndarray, ref: np.ndarray):
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = np.abs(gpu - ref)
    return float(d.max() / rms), float(d.mean() / rms)


_LOG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
                    "parity_errors.log")


def log_errs(case: str, errs: dict):
    """Append the measured error figures of a case to gpurun_out/parity_errors.log."""
    os.makedirs(os.path.dirname(_LOG), exist_ok=True)
    with open(_LOG, "a") as f:
        f.write(f"{case}: " + ", ".join(
            f"{k}=" + ("/".join(f"{v:.3e}" for v in val) if isinstance(val, tuple) else f"{val:.3e}")
            for k, val in errs.items()) + "\n")


def assert_close(name: str, gpu, ref, max_tol=MAX_TOL, mean_tol=MEAN_TOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    mx, mn = norm_err(gpu, ref)
    assert mx <= max_tol and mn <= mean_tol, f"{name}: normalised max {mx:.3e}, mean {mn:.3e}"
    return mx, mn


def assert_bf16_rows(name: str, gpu_bits: np.ndarray, ref_bits: np.ndarray, probe=None,
                     flip_tol=FLIP_TOL):
    """Cache values: exact rounding of the GPU's fp32 value (when the probe is
    given) and rarely different from the oracle's rounding: at most a fraction
    flip_tol of them, or FLIP_FLOOR values in a sample too small for a rate
    (the flips are near-ties, ~3e-4 of all values, so a 2,048-value sample
    expects 0.6 of them)."""
    assert gpu_bits.shape == ref_bits.shape
    if probe is not None:
        want = O.bf16_bits_from_f64(np.asarray(probe, dtype=np.float64))
        bad = int(np.sum(want != gpu_bits))
        assert bad == 0, f"{name}: {bad} values are not the bf16 rounding of the GPU's fp32 value"
    n_flip = int(np.sum(gpu_bits != ref_bits))
    flips = n_flip / max(1, gpu_bits.size)
    assert n_flip <= max(flip_tol * gpu_bits.size, FLIP_FLOOR), \
        f"{name}: {flips:.2e} of the values ({n_flip}) differ from the oracle's rounding"
    return flips


# ----------------------------------------------------------------------------
# runners
# ----------------------------------------------------------------------------

class DecodeCase:
    """Seeded decode workload staged on the GPU (cache rows 0..P-1 from the
    generator, sentinel NaN everywhere else)."""

    def __init__(self, B: int, P: int, T_max: int, seed: int = 0, dev="cuda", theta=5e5,
                 scaled=True, cache_on_device=False, n_kv=8):
        self.B, self.P, self.T_max, self.dev = B, P, T_max, torch.device(dev)
        self.theta, self.scaled, self.n_kv = theta, scaled, n_kv
        self.kcache, self.vcache = G.empty_caches(B, T_max, self.dev, n_kv)
        if not cache_on_device:
            self.x, self.w, self.kc_rows, self.vc_rows = synth.decode_workload(seed, B, P,
                                                                                n_kv_heads=n_kv)
            self.kcache.copy_(synth.sentinel_like(self.kcache.shape, self.dev))
            self.vcache.copy_(synth.sentinel_like(self.vcache.shape, self.dev))
            G.kcache_by_position(self.kcache)[:, :P] = self.kc_rows.to(self.dev)
            G.vcache_write(self.vcache, 0, self.vc_rows.to(self.dev))
        else:
            # large caches: x and weights from the host generator, cache values
            # drawn on the device straight into the cache buffers
            gen = synth.generator(seed)
            self.x = synth.randn_bf16(gen, (B, synth.D_MODEL))
            self.w = synth.block_weights(gen, n_kv_heads=n_kv)
            dgen = synth.generator(seed + 1, self.dev)
            synth.fill_randn_bf16_(self.kcache, dgen)
            synth.fill_randn_bf16_(self.vcache, dgen)
            n = T_max - P
            G.kcache_by_position(self.kcache)[:, P:] = synth.sentinel_like((B, n, n_kv, 128),
                                                                            self.dev)
            G.vcache_write(self.vcache, P, synth.sentinel_like((B, n, n_kv, 128), self.dev))
            self.kc_rows = self.vc_rows = None
        self.k_before = self.kcache.clone()
        self.v_before = self.vcache.clone()
        self.rope = G.rope_table(T_max, theta, scaled, device=self.dev)
        self.wd = [t.to(self.dev) for t in self.w]
        self.xd = self.x.to(self.dev)

    def run(self, probe=True):
        nqkv = G.D_MODEL + 2 * self.n_kv * G.HEAD_DIM
        self.probe = torch.empty((self.B, nqkv), dtype=torch.float32, device=self.dev) \
            if probe else None
        self.ws = G.workspace(self.B, 1, self.T_max, self.dev)
        self.out = G.block_decode(self.xd, *self.wd, self.kcache, self.vcache, self.rope,
                                  self.P, ws=self.ws, probe=self.probe)
        torch.cuda.synchronize()
        assert G.workspace_errors(self.ws) == 0, "a bounded wait of the fused decode timed out"
        return self.out

    def oracle(self, seqs=None):
        seqs = list(range(self.B)) if seqs is None else list(seqs)
        x = f64(self.x[seqs])[:, None, :]
        w = [f64(t) for t in self.w]
        if self.kc_rows is not None:
            kc, vc = f64(self.kc_rows[seqs]), f64(self.vc_rows[seqs])
        else:   # the generator's values, as staged before the call
            kc = f64(G.kcache_by_position(self.k_before)[seqs, :self.P])
            vc = f64(G.vcache_read(self.v_before[seqs], 0, self.P))
        return O.gqa_block(x, *w, kc, vc, self.P, self.theta, self.scaled,
                           n_kv_heads=self.n_kv)

    def check(self, res, seqs=None):
        """Compare the GPU results of sequences ``seqs`` with oracle result res."""
        seqs = list(range(self.B)) if seqs is None else list(seqs)
        B = len(seqs)
        P = self.P
        nk = self.n_kv * 128
        errs = {}
        errs["delta"] = assert_close("delta", f64(self.out[seqs]), res.delta[:, 0])
        if self.probe is not None:
            pr = f64(self.probe[seqs])
            errs["q"] = assert_close("Q", pr[:, :4096], res.q.reshape(B, 4096))
            errs["k"] = assert_close("K", pr[:, 4096:4096 + nk], res.k.reshape(B, nk))
            errs["v"] = assert_close("V", pr[:, 4096 + nk:], res.v.reshape(B, nk))
        kpos = G.kcache_by_position(self.kcache)
        vrow = G.vcache_read(self.vcache[seqs], P, P + 1)[:, 0]
        kp = vp = None
        if self.probe is not None:
            kp = pr[:, 4096:4096 + nk].reshape(B, self.n_kv, 128)
            vp = pr[:, 4096 + nk:].reshape(B, self.n_kv, 128)
        errs["k_flips"] = assert_bf16_rows("kcache row", bits(kpos[seqs, P]), res.k_bits[:, 0], kp)
        errs["v_flips"] = assert_bf16_rows("vcache row", bits(vrow), res.v_bits[:, 0], vp)
        log_errs(f"decode B={self.B} P={P} seqs={seqs if len(seqs) < self.B else 'all'}", errs)
        return errs

    def check_untouched(self):
        """Every cache element except row P is bit-identical to before."""
        P = self.P
        a = self.kcache.clone()
        b = self.k_before.clone()
        G.kcache_by_position(a)[:, P] = 0
        G.kcache_by_position(b)[:, P] = 0
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "key cache changed off row P"
        a = self.vcache.clone()
        b = self.v_before.clone()
        G.vcache_blocks(a)[:, P // G.V_BLOCK, P % G.V_BLOCK] = 0
        G.vcache_blocks(b)[:, P // G.V_BLOCK, P % G.V_BLOCK] = 0
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "value cache changed off row P"


class PrefillCase:
    """Seeded prefill of T tokens per sequence at positions start_pos.. (cache
    rows 0..start_pos-1 from the generator, sentinel NaN everywhere else)."""

    def __init__(self, B: int, T: int, T_max: int, seed: int = 0, dev="cuda", theta=5e5,
                 scaled=True, start_pos: int = 0, n_kv=8):
        self.B, self.T, self.T_max, self.dev = B, T, T_max, torch.device(dev)
        self.theta, self.scaled, self.start_pos, self.n_kv = theta, scaled, start_pos, n_kv
        if start_pos:
            self.x, self.w, self.kc_rows, self.vc_rows = synth.chunked_prefill_workload(
                seed, B, start_pos, T, n_kv_heads=n_kv)
        else:
            self.x, self.w = synth.prefill_workload(seed, B, T, n_kv_heads=n_kv)
            self.kc_rows = self.vc_rows = None
        self.kcache, self.vcache = G.empty_caches(B, T_max, self.dev, n_kv)
        self.kcache.copy_(synth.sentinel_like(self.kcache.shape, self.dev))
        self.vcache.copy_(synth.sentinel_like(self.vcache.shape, self.dev))
        if start_pos:
            G.kcache_by_position(self.kcache)[:, :start_pos] = self.kc_rows.to(self.dev)
            G.vcache_write(self.vcache, 0, self.vc_rows.to(self.dev))
        self.k_before = self.kcache.clone()
        self.v_before = self.vcache.clone()
        self.rope = G.rope_table(T_max, theta, scaled, device=self.dev)
        self.wd = [t.to(self.dev) for t in self.w]
        self.xd = self.x.to(self.dev)

    def run(self, probe=True):
        nqkv = G.D_MODEL + 2 * self.n_kv * G.HEAD_DIM
        self.probe = torch.empty((self.B, self.T, nqkv), dtype=torch.float32,
                                 device=self.dev) if probe else None
        self.out = G.block_prefill(self.xd, *self.wd, self.kcache, self.vcache, self.rope,
                                   probe=self.probe, start_pos=self.start_pos)
        torch.cuda.synchronize()
        return self.out

    def oracle(self, seqs=None):
        seqs = list(range(self.B)) if seqs is None else list(seqs)
        w = [f64(t) for t in self.w]
        kc = f64(self.kc_rows[seqs]) if self.start_pos else None
        vc = f64(self.vc_rows[seqs]) if self.start_pos else None
        return O.gqa_block(f64(self.x[seqs]), *w, kc, vc, self.start_pos, self.theta,
                           self.scaled, n_kv_heads=self.n_kv)

    def check(self, res, seqs=None):
        seqs = list(range(self.B)) if seqs is None else list(seqs)
        B, T, sp = len(seqs), self.T, self.start_pos
        nk = self.n_kv * 128
        errs = {}
        errs["delta"] = assert_close("delta", f64(self.out[seqs]), res.delta)
        if self.probe is not None:
            pr = f64(self.probe[seqs])
            errs["q"] = assert_close("Q", pr[..., :4096], res.q.reshape(B, T, 4096))
            errs["k"] = assert_close("K", pr[..., 4096:4096 + nk], res.k.reshape(B, T, nk))
            errs["v"] = assert_close("V", pr[..., 4096 + nk:], res.v.reshape(B, T, nk))
        kpos = G.kcache_by_position(self.kcache)
        vrows = G.vcache_read(self.vcache[seqs], sp, sp + T)
        kp = vp = None
        if self.probe is not None:
            kp = pr[..., 4096:4096 + nk].reshape(B, T, self.n_kv, 128)
            vp = pr[..., 4096 + nk:].reshape(B, T, self.n_kv, 128)
        errs["k_flips"] = assert_bf16_rows("kcache rows", bits(kpos[seqs, sp:sp + T]), res.k_bits,
                                           kp)
        errs["v_flips"] = assert_bf16_rows("vcache rows", bits(vrows), res.v_bits, vp)
        log_errs(f"prefill B={self.B} start_pos={sp} T={T} n_kv={self.n_kv}", errs)
        return errs

    def check_untouched(self):
        """Rows 0..start_pos-1 keep the cached prefix and rows start_pos+T..
        the sentinel, bit for bit."""
        sp, end, T_max = self.start_pos, self.start_pos + self.T, self.T_max
        kb = lambda c: G.kcache_by_position(c).contiguous().view(torch.int16)
        a, b = kb(self.kcache), kb(self.k_before)
        assert torch.equal(a[:, :sp], b[:, :sp]), "cached key rows changed"
        assert torch.equal(a[:, end:], b[:, end:]), "key rows past the chunk changed"
        assert bool((b[:, end:] == synth.SENTINEL_BITS).all())
        if sp:
            assert torch.equal(G.vcache_read(self.vcache, 0, sp).view(torch.int16),
                               G.vcache_read(self.v_before, 0, sp).view(torch.int16)), \
                "cached value rows changed"
        if end < T_max:
            a = G.vcache_read(self.vcache, end, T_max).view(torch.int16)
            b = G.vcache_read(self.v_before, end, T_max).view(torch.int16)
            assert torch.equal(a, b) and bool((b == synth.SENTINEL_BITS).all()), \
                "value rows past the chunk changed"
