"""Helpers shared by the GPU parity tests: comparisons against the oracle and
runners that stage seeded inputs, call the library and return what it wrote.

Tolerances (written here, used by every parity test):
  * floating point (Delta_attn, and the post-RoPE Q, K, V probes):
    max|gpu - oracle| / rms(oracle) <= 1e-2 and mean|gpu - oracle| / rms <= 2e-3;
  * cache placement: bit-exact (every element outside the written rows keeps
    its bits; the written rows sit exactly where the layout says);
  * cache values: each written bf16 is bit-exactly the round-to-nearest-even
    of the GPU's own pre-rounding value (the fp32 probe, itself within the
    tolerance above).  Where it differs from the oracle's rounding of the
    exact value, that one element is checked against the rounding bound of
    the fp32 arithmetic that produced it (``round_bounds``): the GPU value
    must lie within that bound of the exact value, so the two sit on either
    side of a bf16 rounding midpoint only because the exact value is that
    close to it.  No count of differing values is allowed beyond that.

Rounding bound.  A projected feature y = sum_i x_i w_i over 4096 bf16 inputs
is formed in fp32: each bf16 product is exact in fp32, and the products are
summed along a chain of at most N_ACC roundings (GEMV: 64 per lane plus the
8 levels of the cross-lane tree; matrix cores: 128 steps of 32-term products,
each step rounded once into the accumulator, 4 split-K partials at most),
so |y_fp32 - y| <= N_ACC * 2^-24 * sum_i |x_i w_i|.  A rotated key pair adds
the two features' bounds plus 4 roundings of the rotation and the fp32
table entries.
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
N_ACC = 256                # longest rounding chain of a projected feature (see above)
U32 = 2.0 ** -24           # unit roundoff of fp32


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


_LOG = os.path.join(os.environ.get("GQA_TEST_LOG_DIR") or
                    os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                 "gpurun_out"), "parity_errors.log")


def log_errs(case: str, errs: dict):
    """Append the measured error figures of a case to the parity error log
    (parity_errors.log in the test log folder, see conftest.py)."""
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


def bf16_half_step(v: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values around each (bf16) value v: the widest
    distance from v at which a number still rounds to v."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def round_bounds(x: np.ndarray, w: np.ndarray, rotated: bool) -> np.ndarray:
    """Per-feature bound on |fp32 value - exact value| of y = x w^T (x
    [..., 4096], w [n, 4096], both holding bf16 values): N_ACC * 2^-24 *
    sum_i |x_i w_i|.  With ``rotated`` the features are RoPE pairs (2i, 2i+1),
    each rotated value mixing both features of its pair."""
    s = np.abs(x) @ np.abs(w).T
    if not rotated:
        return N_ACC * U32 * s
    pair = s.reshape(*s.shape[:-1], -1, 2).sum(-1, keepdims=True)
    return ((N_ACC + 4) * U32 * np.broadcast_to(pair, pair.shape[:-1] + (2,))).reshape(s.shape)


def tie_slack(xn_exact: np.ndarray, w: np.ndarray, rel: float = 2.0 ** -16) -> np.ndarray:
    """Extra bound for a projection of a bf16-rounded input computed on both
    sides (the layers' normalised input): an element whose exact value lies
    within ``rel`` of a bf16 rounding midpoint may round one step apart on
    the GPU (fp32) and in the oracle (fp64), which moves each feature by at
    most that step times |w|."""
    v = O.f64_from_bf16_bits(O.bf16_bits_from_f64(xn_exact))
    half = bf16_half_step(v)
    near = (half - np.abs(xn_exact - v)) <= rel * np.abs(xn_exact)
    return np.where(near, 2.0 * half, 0.0) @ np.abs(w).T


def assert_bf16_rows(name: str, gpu_bits: np.ndarray, exact: np.ndarray, bound: np.ndarray,
                     probe=None):
    """Cache values (or any bf16 output) against the oracle's exact value.

    gpu_bits  uint16 patterns the GPU wrote
    exact     the oracle's fp64 value before rounding, same shape
    bound     per-element rounding bound of the GPU's fp32 value (round_bounds)
    probe     the GPU's fp32 value before rounding, when it was captured

    Every written value must be the RNE rounding of the probe.  A value that
    differs from the oracle's rounding is accepted only if the GPU's fp32
    value is within ``bound`` of the exact one (with no probe: if the GPU's
    bf16 value is within bound + half a bf16 step of it).  Returns the
    fraction of values that differ."""
    exact = np.asarray(exact, dtype=np.float64)
    assert gpu_bits.shape == exact.shape, (name, gpu_bits.shape, exact.shape)
    bound = np.broadcast_to(np.asarray(bound, dtype=np.float64), exact.shape)
    if probe is not None:
        probe = np.asarray(probe, dtype=np.float64)
        want = O.bf16_bits_from_f64(probe)
        bad = int(np.sum(want != gpu_bits))
        assert bad == 0, f"{name}: {bad} values are not the bf16 rounding of the GPU's fp32 value"
    flip = gpu_bits != O.bf16_bits_from_f64(exact)
    if probe is not None:
        off = np.abs(probe - exact) > bound
    else:
        g = O.f64_from_bf16_bits(gpu_bits)
        off = np.abs(g - exact) > bound + bf16_half_step(g)
    bad = flip & off
    n_bad = int(np.sum(bad))
    if n_bad:
        i = tuple(int(a[0]) for a in np.nonzero(bad))
        raise AssertionError(
            f"{name}: {n_bad} of {int(np.sum(flip))} values that round differently from the "
            f"oracle lie outside the fp32 rounding bound (first at {i}: exact {exact[i]:.9g}, "
            f"gpu {O.f64_from_bf16_bits(gpu_bits[i]):.9g}, bound {bound[i]:.3g})")
    return float(np.mean(flip))


def kv_bounds(x: np.ndarray, w, n_kv: int):
    """Rounding bounds [..., n_kv, 128] of the post-RoPE keys and the values
    projected from x [..., 4096] (w = (wq, wk, wv, wo) as fp64)."""
    bk = round_bounds(x, w[1], rotated=True)
    bv = round_bounds(x, w[2], rotated=False)
    shape = x.shape[:-1] + (n_kv, 128)
    return bk.reshape(shape), bv.reshape(shape)


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

    def run(self, probe=True, schedule=G.DECODE_AUTO):
        nqkv = G.D_MODEL + 2 * self.n_kv * G.HEAD_DIM
        self.probe = torch.empty((self.B, nqkv), dtype=torch.float32, device=self.dev) \
            if probe else None
        self.ws = G.workspace(G.OP_DECODE, self.B, self.T_max, self.dev, n_kv_heads=self.n_kv)
        self.out = G.block_decode(self.xd, *self.wd, self.kcache, self.vcache, self.rope,
                                  self.P, ws=self.ws, probe=self.probe, schedule=schedule)
        torch.cuda.synchronize()
        assert G.workspace_errors(self.ws) == 0, "the decode reported an error in its workspace"
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
        bk, bv = kv_bounds(f64(self.x[seqs]), [f64(t) for t in self.w], self.n_kv)
        errs["k_flips"] = assert_bf16_rows("kcache row", bits(kpos[seqs, P]), res.k[:, 0], bk, kp)
        errs["v_flips"] = assert_bf16_rows("vcache row", bits(vrow), res.v[:, 0], bv, vp)
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
        bk, bv = kv_bounds(f64(self.x[seqs]), [f64(t) for t in self.w], self.n_kv)
        errs["k_flips"] = assert_bf16_rows("kcache rows", bits(kpos[seqs, sp:sp + T]), res.k, bk,
                                           kp)
        errs["v_flips"] = assert_bf16_rows("vcache rows", bits(vrows), res.v, bv, vp)
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
