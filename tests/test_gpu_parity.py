"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Every case compares the library's output with the oracle on the same seeded
inputs, to the tolerances stated in tests/parity.py: normalised max 1e-2 and
mean 2e-3 for Delta_attn and the post-RoPE Q/K/V probes, bit-exact cache
placement, and cache values equal to the oracle's bf16 rounding or its
neighbour.
"""
import numpy as np
import pytest
import torch

import grouped_query_attention_gemv_amd as G
from grouped_query_attention_gemv_amd import synth
from oracle import gqa_oracle as O
from tests.parity import (MEAN_TOL, DecodeCase, PrefillCase, assert_bf16_rows, assert_close, bits,
                          f64, kv_bounds, norm_err, round_bounds, tie_slack)

pytestmark = pytest.mark.gpu

DEV = "cuda"


# ----------------------------------------------------------------------------
# RoPE table
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("scaled", [True, False])
def test_rope_table_matches_oracle(scaled):
    T_max = 131072
    tab = G.rope_table(T_max, 500000.0, scaled, device=DEV)
    torch.cuda.synchronize()
    got = tab.cpu().numpy().astype(np.float64)
    pos = np.arange(T_max)
    cos, sin = O.rope_cos_sin(pos, 128, 500000.0, scaled)
    # one rounding of an fp64 value to fp32: at most half an fp32 ulp of 1
    assert np.max(np.abs(got[..., 0] - cos)) <= 2 ** -24 * 1.01
    assert np.max(np.abs(got[..., 1] - sin)) <= 2 ** -24 * 1.01


# ----------------------------------------------------------------------------
# Decode
# ----------------------------------------------------------------------------

@pytest.fixture(params=["split", "fused"])
def schedule(request):
    """The decode schedule a test asks for in each call: the three-launch and
    the one-launch one (every shape these tests use is admitted by both)."""
    return {"split": G.DECODE_SPLIT, "fused": G.DECODE_FUSED}[request.param]


def _decode_full(B, P, T_max, schedule=G.DECODE_AUTO, **kw):
    c = DecodeCase(B, P, T_max, dev=DEV, **kw)
    c.run(schedule=schedule)
    errs = c.check(c.oracle())
    c.check_untouched()
    return c, errs


def test_decode_start_pos_128(schedule):
    """B=1, start_pos=128: rows 0-127 cached, row 128 written, rows 0-128 read."""
    _decode_full(1, 128, 256, schedule)


def test_decode_p1000(schedule):
    """B=1 at the pages' decode point: P = 1,000 cached, row 1,000 written."""
    _, errs = _decode_full(1, 1000, 1024, schedule)
    # fp32 Q/P/O with hi/lo bf16 matrix-core operands: far inside the bound
    assert errs["delta"][0] < 1e-3


@pytest.mark.parametrize("P", [0, 1, 31, 32, 33, 127, 128, 129, 255, 1023])
def test_decode_positions(P, schedule):
    """Single key, tile and split edges."""
    _decode_full(2, P, 1024, schedule)


@pytest.mark.parametrize("B", [3, 5, 6, 7, 8, 9, 17])
def test_decode_batches(B):
    """Batch sizes across the projection paths: the GEMVs (wo below 5 tokens,
    QKV up to 8), wo on the matrix cores for 5 to 8 tokens, the split-K
    matrix-core projections above 8 (ragged last chunk)."""
    _decode_full(B, 300, 512)


def test_decode_unscaled_rope():
    """Llama 3 setting (use_scaled_rope False) at a position where scaling matters."""
    _decode_full(1, 5000, 5024, scaled=False)


@pytest.mark.parametrize("n_kv,B,P", [(16, 1, 1000), (32, 1, 1000), (32, 1, 1023), (32, 2, 300),
                                      (16, 2, 1000), (8, 1, 3000), (8, 2, 1500), (32, 1, 0)])
def test_decode_fused_head_counts_and_long_splits(n_kv, B, P):
    """The one-launch schedule at 16 and 32 kv heads, and with splits capped
    at 128 attention workgroups (two 32-position tiles per wave, the appended
    row in the second tile for the last split), within the oracle's bounds.
    AUTO picks it at 8 kv heads and at B = 1."""
    c, errs = _decode_full(B, P, ((P + 1 + 31) // 32) * 32 + 32, G.DECODE_FUSED, n_kv=n_kv)
    auto = G.DECODE_FUSED if (n_kv == 8 or B == 1) else G.DECODE_SPLIT
    assert G.decode_schedule(B, P, c.T_max, n_kv, G.DECODE_AUTO) == auto
    assert errs["delta"][0] < 1e-3


@pytest.mark.parametrize("n_kv,B,P", [(32, 1, 1000), (32, 3, 777), (16, 1, 1000), (16, 2, 100),
                                      (32, 8, 129), (16, 5, 0), (16, 9, 300), (32, 17, 65),
                                      (16, 64, 31), (32, 70, 200)])
def test_decode_other_kv_head_counts(n_kv, B, P):
    """n_rep = 32 / n_kv query heads per key/value head: 1 is multi-head
    attention, 2 a wider GQA; the same kernels templated on the head count.
    B > 8 takes the matrix-core projections (B = 70: two 64-token launches,
    the second ragged)."""
    _, errs = _decode_full(B, P, 1024, n_kv=n_kv)
    assert errs["delta"][0] < 1e-3


def test_decode_accumulate_and_bf16_out(schedule):
    """out += Delta with the bf16 copy of the updated residual."""
    c = DecodeCase(2, 100, 128, dev=DEV)
    res = c.oracle()
    h0 = torch.randn(2, 4096, generator=torch.Generator().manual_seed(5)).to(DEV)
    out = h0.clone()
    ob = torch.empty(2, 4096, dtype=torch.bfloat16, device=DEV)
    G.block_decode(c.xd, *c.wd, c.kcache, c.vcache, c.rope, c.P, out=out, out_bf16=ob,
                   accumulate=True, schedule=schedule)
    torch.cuda.synchronize()
    want = f64(h0) + res.delta[:, 0]
    assert_close("h + delta", f64(out) - f64(h0), res.delta[:, 0])
    assert torch.equal(ob.cpu(), out.cpu().to(torch.bfloat16))
    assert np.max(np.abs(f64(out) - want)) < 1e-2


def test_decode_batched_b64_p8192_sampled():
    """B=64 sequences with 8,192 cached positions each (caches ~2 GiB), one new
    token each; sampled sequences against the oracle, every cache bit outside
    row 8,192 unchanged."""
    c = DecodeCase(64, 8192, 8224, dev=DEV, cache_on_device=True)
    c.run()
    seqs = [0, 13, 63]
    c.check(c.oracle(seqs), seqs)
    c.check_untouched()


def test_decode_batched_mha_b64_p8192_sampled():
    """The multi-head variant (32 key/value heads) at the batched bench size:
    B=64, 8,192 cached positions (caches ~8.6 GiB); sampled sequences against
    the oracle, every cache bit outside row 8,192 unchanged."""
    c = DecodeCase(64, 8192, 8224, dev=DEV, cache_on_device=True, n_kv=32)
    c.run()
    seqs = [0, 31, 63]
    c.check(c.oracle(seqs), seqs)
    c.check_untouched()


def test_decode_long_context_p131071_sampled():
    """One block at the long-context point: B=8 sequences with 131,071 cached
    positions each (2 GiB per cache tensor), row 131,071 written; sampled
    sequences against the oracle, every other cache bit unchanged."""
    c = DecodeCase(8, 131071, 131072, dev=DEV, cache_on_device=True)
    c.run()
    seqs = [0, 5]
    c.check(c.oracle(seqs), seqs)
    c.check_untouched()


def test_decode_stacked_blocks_residual():
    """32 stacked blocks, each with its own weights and cache, h <- h + Delta
    (no norms, no FFN), the next block's input being bf16(h): B=8, P=4095,
    against the oracle's block-by-block chain for sampled sequences."""
    from grouped_query_attention_gemv_amd import synth
    from oracle import gqa_oracle as O
    B, P, T_max, L = 8, 4095, 4096, 32
    gen = synth.generator(7)
    x0 = synth.randn_bf16(gen, (B, 4096))
    blocks = []
    dgen = synth.generator(8, DEV)
    for _ in range(L):
        w = [t.to(DEV) for t in synth.block_weights(gen)]
        kc, vc = G.empty_caches(B, T_max, DEV)
        synth.fill_randn_bf16_(kc, dgen)
        synth.fill_randn_bf16_(vc, dgen)
        blocks.append((w, kc, vc, kc.clone(), vc.clone()))
    rope = G.rope_table(T_max, device=DEV)
    ws = G.workspace(G.OP_DECODE, B, T_max, DEV)
    h = x0.to(DEV).float()
    xa = x0.to(DEV)
    xb = torch.empty_like(xa)
    for w, kc, vc, _, _ in blocks:
        G.block_decode(xa, *w, kc, vc, rope, P, out=h, out_bf16=xb, accumulate=True, ws=ws)
        xa, xb = xb, xa
    torch.cuda.synchronize()
    seqs = [1, 6]
    # generators: one block's fp64 copies exist on the host at a time
    ws_ = ([f64(t) for t in w] for w, *_ in blocks)
    kcs = (f64(G.kcache_by_position(k0[seqs])[:, :P]) for *_, k0, _ in blocks)
    vcs = (f64(G.vcache_read(v0[seqs], 0, P)) for *_, v0 in blocks)
    h_ref, _ = O.stacked_decode(f64(x0[seqs]), ws_, kcs, vcs, P)
    # compare the accumulated residual update h - x0 (the 32 summed deltas)
    assert_close("stacked residual", f64(h[seqs]) - f64(x0[seqs]), h_ref - f64(x0[seqs]))
    assert torch.equal(xa.cpu(), h.cpu().to(torch.bfloat16))


@pytest.mark.timeout(600)
def test_decode_stacked_blocks_at_full_context():
    """Three stacked blocks at the long-context point (B = 8, P = 131,071 in
    every block, 4 GiB of cache per block), h <- h + Delta with bf16(h) as the
    next block's input; one sampled sequence against the oracle's block by
    block chain, and every other cache bit of every block unchanged."""
    B, P, T_max, L = 8, 131071, 131072, 3
    gen = synth.generator(17)
    x0 = synth.randn_bf16(gen, (B, 4096))
    dgen = synth.generator(18, DEV)
    blocks = []
    for _ in range(L):
        w = [t.to(DEV) for t in synth.block_weights(gen)]
        kc, vc = G.empty_caches(B, T_max, DEV)
        synth.fill_randn_bf16_(kc, dgen)
        synth.fill_randn_bf16_(vc, dgen)
        blocks.append((w, kc, vc, kc.clone(), vc.clone()))
    rope = G.rope_table(T_max, device=DEV)
    ws = G.workspace(G.OP_DECODE, B, T_max, DEV)
    h = x0.to(DEV).float()
    xa, xb = x0.to(DEV), torch.empty((B, 4096), dtype=torch.bfloat16, device=DEV)
    for w, kc, vc, _, _ in blocks:
        G.block_decode(xa, *w, kc, vc, rope, P, out=h, out_bf16=xb, accumulate=True, ws=ws)
        xa, xb = xb, xa
    torch.cuda.synchronize()
    assert G.workspace_errors(ws) == 0
    seq = [5]
    ws_ = ([f64(t) for t in w] for w, *_ in blocks)
    kcs = (f64(G.kcache_by_position(k0[seq])[:, :P]) for *_, k0, _ in blocks)
    vcs = (f64(G.vcache_read(v0[seq], 0, P)) for *_, v0 in blocks)
    h_ref, _ = O.stacked_decode(f64(x0[seq]), ws_, kcs, vcs, P)
    assert_close("stacked residual at P=131071", f64(h[seq]) - f64(x0[seq]), h_ref - f64(x0[seq]))
    for _, kc, vc, k0, v0 in blocks:           # only row P of each cache changed
        a, b = kc.clone(), k0.clone()
        G.kcache_by_position(a)[:, P] = 0
        G.kcache_by_position(b)[:, P] = 0
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        a, b = vc.clone(), v0.clone()
        G.vcache_blocks(a)[:, P // 32, P % 32] = 0
        G.vcache_blocks(b)[:, P // 32, P % 32] = 0
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_resumes_from_copied_caches():
    """Checkpoint and resume: prefill 300 tokens, copy the caches out (to the
    host and back into fresh buffers), and decode token 300 from the copy.
    Delta and the appended rows equal the decode on the original caches bit
    for bit, and match the oracle of the 301-token prefill's last row."""
    T = 300
    full = PrefillCase(2, T + 1, 320, dev=DEV)
    ref = full.oracle()
    kc, vc = G.empty_caches(2, 320, DEV)
    G.block_prefill(full.xd[:, :T].contiguous(), *full.wd, kc, vc, full.rope)
    torch.cuda.synchronize()
    k_host, v_host = kc.cpu(), vc.cpu()                 # the checkpoint
    kc2, vc2 = G.empty_caches(2, 320, DEV)
    kc2.copy_(k_host)
    vc2.copy_(v_host)
    x = full.xd[:, T].contiguous()
    a = G.block_decode(x, *full.wd, kc, vc, full.rope, T)
    b = G.block_decode(x, *full.wd, kc2, vc2, full.rope, T)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))
    assert_close("resumed decode vs oracle", f64(b), ref.delta[:, T])


def test_decode_fused_largest_admitted_context(schedule):
    """B=1 at start_pos 2,047: 16 splits x 8 kv heads, the most attention
    workgroups the one-launch schedule admits."""
    _decode_full(1, 2047, 2048, schedule)


def test_decode_schedules_agree_bitwise():
    """Both schedules run the same arithmetic in the same order: identical
    outputs and caches.  Every call of either schedule leaves the workspace's
    synchronisation region as gqa_workspace_init wrote it: zero words but the
    magic word, and "not yet" markers in every hand-off buffer."""
    outs, caches = [], []
    ws = G.workspace(G.OP_DECODE, 2, 1024, DEV)
    torch.cuda.synchronize()
    region = ws[:G.SYNC_BYTES].view(torch.int32).clone()
    assert int(region[1].item()) == G.WS_MAGIC
    assert int(region[2:16384].abs().sum().item()) == 0
    for mode in (G.DECODE_FUSED, G.DECODE_SPLIT, G.DECODE_FUSED):
        c = DecodeCase(2, 777, 1024, dev=DEV)
        out = G.block_decode(c.xd, *c.wd, c.kcache, c.vcache, c.rope, c.P, ws=ws, schedule=mode)
        torch.cuda.synchronize()
        outs.append(out.clone())
        caches.append((c.kcache.clone(), c.vcache.clone()))
        assert torch.equal(ws[:G.SYNC_BYTES].view(torch.int32), region)
    for o, (k, v) in zip(outs[1:], caches[1:]):
        assert torch.equal(o, outs[0])
        assert torch.equal(k.view(torch.int16), caches[0][0].view(torch.int16))
        assert torch.equal(v.view(torch.int16), caches[0][1].view(torch.int16))


def test_decode_is_deterministic():
    for B in (1, 4):     # one-launch and three-launch schedules
        c = DecodeCase(B, 1000, 1024, dev=DEV)
        a = c.run().clone()
        b = c.run().clone()
        assert torch.equal(a, b)


def test_decode_in_hip_graph_matches_eager(schedule):
    """A captured decode call, replayed several times with eager work and
    synchronisations between replays, reproduces the eager result bit for bit
    (the library issues no memset, so nothing in the graph depends on one)."""
    c = DecodeCase(2, 300, 320, dev=DEV)
    eager = c.run(probe=False, schedule=schedule).clone()
    out = torch.zeros_like(eager)
    ws = G.workspace(G.OP_DECODE, 2, 320, DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        G.block_decode(c.xd, *c.wd, c.kcache, c.vcache, c.rope, c.P, out=out, ws=ws,
                       schedule=schedule)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.block_decode(c.xd, *c.wd, c.kcache, c.vcache, c.rope, c.P, out=out, ws=ws,
                       schedule=schedule)
    for _ in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    c.check_untouched()


def test_fused_decode_reads_this_calls_data():
    """The one-launch schedule hands Q, the new K/V row, the split partials
    and O from workgroup to workgroup through memory that earlier calls wrote
    at the same addresses (the wo workgroups read O through their L2, after
    every producer's device-scope stores completed).  Calls on one workspace
    and one set of buffers, each with a new x, replayed from a graph with the
    input changed between replays: every replay must equal a fresh
    three-launch result on that x."""
    B, P, T_max = 1, 777, 1024
    c = DecodeCase(B, P, T_max, dev=DEV)
    ws = G.workspace(G.OP_DECODE, B, T_max, DEV)
    x = c.xd.clone()
    out = torch.zeros((B, 4096), dtype=torch.float32, device=DEV)
    k0, v0 = c.kcache.clone(), c.vcache.clone()
    xs = [synth.randn_bf16(synth.generator(100 + i), (B, 4096)).to(DEV) for i in range(5)]
    F = G.DECODE_FUSED

    def reference(xi):
        kc, vc = k0.clone(), v0.clone()
        r = G.block_decode(xi, *c.wd, kc, vc, c.rope, P, schedule=G.DECODE_SPLIT)
        torch.cuda.synchronize()
        return r

    for xi in xs[:2]:                       # eager calls, one workspace
        x.copy_(xi)
        r = G.block_decode(x, *c.wd, c.kcache, c.vcache, c.rope, P, out=out, ws=ws, schedule=F)
        torch.cuda.synchronize()
        assert torch.equal(r, reference(xi))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        G.block_decode(x, *c.wd, c.kcache, c.vcache, c.rope, P, out=out, ws=ws, schedule=F)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.block_decode(x, *c.wd, c.kcache, c.vcache, c.rope, P, out=out, ws=ws, schedule=F)
    for xi in xs[2:] + xs[:2]:              # graph replays, new x each time
        x.copy_(xi)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, reference(xi))
    assert G.workspace_errors(ws) == 0
    # how often the first attention workgroup ran away from the XCD that its
    # index modulo 8 would give (nothing relies on it; this only records it)
    print("fused launches placed away from their XCDs:", G.workspace_off_home(ws), "of 7")


@pytest.mark.parametrize("B", [6, 16])
def test_three_launch_decode_graph_replays_match_eager(B):
    """The three-launch schedule captured in a graph: B = 6 runs wo on the
    matrix cores (131 KiB of dynamic LDS), B = 16 the split-K projections.
    Replayed with a new x each time, with eager work and synchronisations
    between the replays; every replay equals an eager call on that x bit for
    bit (caches restored before each)."""
    P, T_max = 200, 224
    c = DecodeCase(B, P, T_max, dev=DEV)
    ws = G.workspace(G.OP_DECODE, B, T_max, DEV)
    x = c.xd.clone()
    out = torch.zeros((B, 4096), dtype=torch.float32, device=DEV)
    k0, v0 = c.kcache.clone(), c.vcache.clone()
    xs = [synth.randn_bf16(synth.generator(200 + i), (B, 4096)).to(DEV) for i in range(4)]
    S = G.DECODE_SPLIT

    def eager(xi):
        kc, vc = k0.clone(), v0.clone()
        r = G.block_decode(xi, *c.wd, kc, vc, c.rope, P, schedule=S)
        torch.cuda.synchronize()
        return r, kc, vc

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        G.block_decode(x, *c.wd, c.kcache, c.vcache, c.rope, P, out=out, ws=ws, schedule=S)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.block_decode(x, *c.wd, c.kcache, c.vcache, c.rope, P, out=out, ws=ws, schedule=S)
    for xi in xs:
        c.kcache.copy_(k0)
        c.vcache.copy_(v0)
        x.copy_(xi)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref, kc, vc = eager(xi)
        assert torch.equal(out, ref)
        assert torch.equal(c.kcache.view(torch.int16), kc.view(torch.int16))
        assert torch.equal(c.vcache.view(torch.int16), vc.view(torch.int16))
    assert G.workspace_errors(ws) == 0


def test_decode_rejects_small_workspace_without_side_effects():
    c = DecodeCase(1, 64, 128, dev=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    out = torch.full((1, 4096), 7.0, device=DEV)
    with pytest.raises(G.GQAError):
        G.block_decode(c.xd, *c.wd, c.kcache, c.vcache, c.rope, c.P, out=out, ws=ws)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    assert torch.equal(c.kcache.view(torch.int16), c.k_before.view(torch.int16))
    assert torch.equal(c.vcache.view(torch.int16), c.v_before.view(torch.int16))


def test_workspace_init_writes_words_and_markers():
    """gqa_workspace_init on a workspace full of garbage: zero synchronisation
    words (64 KiB) but the magic word, then the one-launch decode's hand-off
    buffers holding their "not yet" markers -- an fp32 signalling NaN in Q
    (2 x 4096 floats) and in the partials, a pair of bf16 signalling NaNs in
    the appended rows (2 x 2 x 32 x 128 bf16) -- then the wo slots (512 x 64
    words) zero, and nothing written past the region."""
    n = G.SYNC_BYTES + 4096
    ws = torch.full((n,), 0x5a, dtype=torch.uint8, device=DEV)
    G.workspace_init(ws)
    torch.cuda.synchronize()
    w = ws.view(torch.int32).cpu().numpy().view(np.uint32)
    assert w[0] == 0 and w[1] == G.WS_MAGIC and not w[2:16384].any()
    q_end = 16384 + 2 * 4096
    kv_end = q_end + 2 * 2 * 32 * 64
    part_end = kv_end + 128 * 4 * 132 + 2 * 32 * 32
    assert (w[16384:q_end] == 0x7f800001).all()
    assert (w[q_end:kv_end] == 0x7f817f81).all()
    assert (w[kv_end:part_end] == 0x7f800001).all()
    assert not w[part_end:part_end + 512 * 64].any()
    assert not w[part_end + 512 * 64:G.SYNC_BYTES // 4].any()
    assert (w[G.SYNC_BYTES // 4:] == 0x5a5a5a5a).all()


@pytest.mark.parametrize("B,P,schedule", [(1, 300, G.DECODE_FUSED), (16, 300, G.DECODE_SPLIT)])
def test_decode_on_uninitialised_workspace_reports_it(B, P, schedule):
    """A workspace that never saw gqa_workspace_init (zero-filled here, as
    fresh memory often is) has no magic word: the kernels that rely on its
    synchronisation words (the one-launch step, the batched projections) wait
    for nothing, write NaN into Delta and set the INIT bit.  Initialising the
    same workspace makes the next call correct."""
    c = DecodeCase(B, P, 320, dev=DEV)
    ws = torch.zeros(G.workspace_bytes(G.OP_DECODE, B, 320), dtype=torch.uint8, device=DEV)
    out = torch.zeros((B, 4096), dtype=torch.float32, device=DEV)
    G.block_decode(c.xd, *c.wd, c.kcache, c.vcache, c.rope, P, out=out, ws=ws, schedule=schedule)
    torch.cuda.synchronize()
    assert G.workspace_errors(ws) & G.WS_ERR_INIT
    assert bool(torch.isnan(out).all())
    G.workspace_init(ws)
    c.kcache.copy_(c.k_before)
    c.vcache.copy_(c.v_before)
    G.block_decode(c.xd, *c.wd, c.kcache, c.vcache, c.rope, P, out=out, ws=ws, schedule=schedule)
    torch.cuda.synchronize()
    assert G.workspace_errors(ws) == 0
    assert_close("delta after init", f64(out), c.oracle().delta[:, 0])


# ----------------------------------------------------------------------------
# Prefill
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("B,T", [(1, 1), (2, 63), (1, 64), (2, 65), (3, 130), (1, 257),
                                 (2, 300)])
def test_prefill_small(B, T):
    c = PrefillCase(B, T, ((T + 31) // 32) * 32 + 32, dev=DEV)
    c.run()
    c.check(c.oracle())
    c.check_untouched()


def test_prefill_b4_t2048():
    """Causal prefill B=4, T=2048 from position 0: Delta [4, 2048, 4096] and
    cache rows 0-2047 of each sequence."""
    c = PrefillCase(4, 2048, 2048, dev=DEV)
    c.run()
    errs = c.check(c.oracle())
    print("prefill B=4 T=2048 errors", errs)


def test_prefill_unscaled_rope():
    """Llama 3 setting (use_scaled_rope False): prefill and a chunk after it."""
    c = PrefillCase(1, 300, 640, dev=DEV, scaled=False)
    c.run()
    c.check(c.oracle())
    c = PrefillCase(1, 200, 640, dev=DEV, scaled=False, start_pos=300)
    c.run()
    c.check(c.oracle())
    c.check_untouched()


def test_prefill_with_caller_fp16_wo_matches():
    """A caller-held fp16 copy of Wo (gqa_wo_to_fp16, converted once) gives
    the same Delta bit for bit as the per-call conversion, with wo not read."""
    c = PrefillCase(2, 130, 192, dev=DEV)
    a = c.run(probe=False).clone()
    wo16 = G.wo_to_fp16(c.wd[3])
    torch.cuda.synchronize()
    assert torch.equal(wo16.cpu(), c.wd[3].cpu().to(torch.float16))
    c.kcache.copy_(c.k_before)
    c.vcache.copy_(c.v_before)
    b = G.block_prefill(c.xd, *c.wd[:3], None, c.kcache, c.vcache, c.rope, wo16=wo16)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _prefill_with_prefix_values(scale_k, scale_v, rows):
    """Chunked prefill whose cached prefix holds a few rows scaled up."""
    B, sp, T, T_max = 1, 96, 40, 160
    c = PrefillCase(B, T, T_max, dev=DEV, start_pos=sp)
    kr = c.kc_rows.float()
    vr = c.vc_rows.float()
    kr[:, rows] *= scale_k
    vr[:, rows] *= scale_v
    c.kc_rows = kr.to(torch.bfloat16)
    c.vc_rows = vr.to(torch.bfloat16)
    G.kcache_by_position(c.kcache)[:, :sp] = c.kc_rows.to(DEV)
    G.vcache_write(c.vcache, 0, c.vc_rows.to(DEV))
    c.k_before = c.kcache.clone()
    c.v_before = c.vcache.clone()
    ws = G.workspace(G.OP_PREFILL, B, T_max, DEV, T, sp)
    out = G.block_prefill(c.xd, *c.wd, c.kcache, c.vcache, c.rope, ws=ws, start_pos=sp)
    torch.cuda.synchronize()
    c.out = out
    return c, ws


def test_prefill_large_cached_values_within_fp16_range():
    """Cached values up to ~5e4 (bf16 holds them, and so does fp16): the fp16
    attention operands stay exact, parity holds and no range bit is set."""
    c, ws = _prefill_with_prefix_values(1.0, 1e4, [3, 50, 77])
    assert float(c.vc_rows.float().abs().max()) < 65504
    assert G.workspace_errors(ws) == 0
    assert_close("delta", f64(c.out), c.oracle().delta)


def test_prefill_values_beyond_fp16_range_saturate_and_flag():
    """Cached keys and values beyond 65504 (bf16 holds them, fp16 does not)
    are saturated to +-65504 instead of turning Delta into inf/NaN, and the
    call sets WS_ERR_FP16_RANGE in its workspace's error word."""
    c, ws = _prefill_with_prefix_values(3e4, 3e4, [5, 60])
    assert float(c.vc_rows.float().abs().max()) > 65504
    assert G.workspace_errors(ws) & G.WS_ERR_FP16_RANGE
    assert bool(torch.isfinite(c.out).all())


def test_prefill_is_deterministic():
    c = PrefillCase(2, 200, 256, dev=DEV)
    a = c.run().clone()
    b = c.run().clone()
    assert torch.equal(a, b)


@pytest.mark.parametrize("n_kv,B,start_pos,T", [
    (32, 1, 0, 300), (32, 2, 0, 257), (32, 3, 0, 64), (32, 1, 130, 129), (32, 2, 1000, 48),
    (16, 2, 0, 130), (16, 1, 37, 200), (16, 1, 0, 1), (16, 3, 64, 256)])
def test_prefill_other_kv_head_counts(n_kv, B, start_pos, T):
    """n_rep = 32 / n_kv query heads per key/value head (1: multi-head
    attention, 256-query tiles; 2: 128-query tiles), from position 0 and after
    cached rows, with ragged query tiles."""
    T_max = ((start_pos + T + 31) // 32) * 32 + 32
    c = PrefillCase(B, T, T_max, dev=DEV, start_pos=start_pos, n_kv=n_kv)
    c.run()
    c.check(c.oracle())
    c.check_untouched()


@pytest.mark.parametrize("n_kv", [16, 32])
def test_kv_variant_decode_after_prefill(n_kv):
    """Multi-head / n_rep = 2 models: prefill 700 tokens, decode token 700 on
    the cache it wrote, against a 701-token prefill and its oracle."""
    T = 700
    full = PrefillCase(1, T + 1, 704, dev=DEV, n_kv=n_kv)
    full.run(probe=False)
    ref = full.oracle()
    assert_close("prefill 701", f64(full.out), ref.delta)
    kc, vc = G.empty_caches(1, 704, DEV, n_kv)
    G.block_prefill(full.xd[:, :T].contiguous(), *full.wd, kc, vc, full.rope)
    out = G.block_decode(full.xd[:, T].contiguous(), *full.wd, kc, vc, full.rope, T)
    torch.cuda.synchronize()
    assert_close("decode vs oracle", f64(out), ref.delta[:, T])
    assert np.array_equal(bits(G.kcache_by_position(kc)[:, :T]),
                          bits(G.kcache_by_position(full.kcache)[:, :T]))
    assert np.array_equal(bits(G.vcache_read(vc, 0, T)), bits(G.vcache_read(full.vcache, 0, T)))


def test_prefill_mha_b2_t1024():
    """Multi-head attention (n_kv = 32) prefill at B=2, T=1024: four full
    256-query tiles per sequence and head."""
    c = PrefillCase(2, 1024, 1024, dev=DEV, n_kv=32)
    c.run()
    c.check(c.oracle())


# ----------------------------------------------------------------------------
# Chunked prefill: T new tokens after start_pos cached rows
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("B,start_pos,T", [(1, 1, 1), (1, 64, 64), (2, 37, 70), (1, 130, 5),
                                           (3, 200, 129), (2, 1000, 48), (1, 960, 300)])
def test_prefill_chunked_small(B, start_pos, T):
    T_max = ((start_pos + T + 31) // 32) * 32 + 32
    c = PrefillCase(B, T, T_max, dev=DEV, start_pos=start_pos)
    c.run()
    c.check(c.oracle())
    c.check_untouched()


def test_prefill_chunked_b2_p1024_t1024():
    """1,024 new tokens after 1,024 cached rows; the oracle checks sequence 1."""
    c = PrefillCase(2, 1024, 2048, dev=DEV, start_pos=1024)
    c.run()
    print("chunked prefill B=2 P=1024 T=1024 errors", c.check(c.oracle([1]), [1]))
    c.check_untouched()


def test_chunked_prefill_continues_a_prefill():
    """Prefill 300 tokens, then the next 200 from start_pos 300 on the same
    cache.  The cache rows equal those of one 500-token prefill bit for bit
    (same GEMM rows, same positions); the chunk's Delta matches the oracle of
    the 500-token prefill."""
    P, T = 300, 200
    full = PrefillCase(1, P + T, 512, dev=DEV)
    full.run(probe=False)
    ref = full.oracle()
    kc, vc = G.empty_caches(1, 512, DEV)
    G.block_prefill(full.xd[:, :P].contiguous(), *full.wd, kc, vc, full.rope)
    out = G.block_prefill(full.xd[:, P:].contiguous(), *full.wd, kc, vc, full.rope, start_pos=P)
    torch.cuda.synchronize()
    assert_close("chunk vs oracle", f64(out), ref.delta[:, P:])
    assert_close("chunk vs one prefill", f64(out), f64(full.out[:, P:]))
    assert np.array_equal(bits(G.kcache_by_position(kc)[:, :P + T]),
                          bits(G.kcache_by_position(full.kcache)[:, :P + T]))
    assert np.array_equal(bits(G.vcache_read(vc, 0, P + T)), bits(G.vcache_read(full.vcache, 0, P + T)))


# ----------------------------------------------------------------------------
# Layers: h = x + Delta(RMSNorm(x) * g)
# ----------------------------------------------------------------------------
#
# The normalised input is rounded to bf16 on both sides, from fp32 on the GPU
# and from fp64 in the oracle, so an element whose exact value sits at a
# rounding midpoint (to within the fp32 error of the norm) may land one bf16
# step apart.  Such a step moves every projected feature by the step times
# its weight; tests.parity.tie_slack bounds that per feature, and the cache
# rows' rounding check adds it to the fp32 accumulation bound.


def _layer_kv_bounds(xn_exact, w, n_kv):
    """Rounding bounds [..., n_kv, 128] of keys and values projected from the
    bf16 rounding of xn_exact, including the near-tie slack of that rounding."""
    xn = O.f64_from_bf16_bits(O.bf16_bits_from_f64(xn_exact))
    bk, bv = kv_bounds(xn, w, n_kv)
    sk = tie_slack(xn_exact, w[1])
    sk = sk.reshape(*sk.shape[:-1], -1, 2).sum(-1, keepdims=True)
    sk = np.broadcast_to(sk, sk.shape[:-1] + (2,)).reshape(bk.shape)
    sv = tie_slack(xn_exact, w[2]).reshape(bv.shape)
    return bk + sk, bv + sv


@pytest.mark.parametrize("B,P,mode", [(1, 1000, "fused"), (1, 1000, "split"), (4, 300, "auto"),
                                      (6, 300, "auto"), (16, 200, "auto")])
def test_layer_decode(B, P, mode):
    c = DecodeCase(B, P, ((P + 1 + 31) // 32) * 32 + 32, dev=DEV)
    g = synth.norm_gain(5)
    gd = g.to(DEV)
    h_bf16 = torch.empty((B, G.D_MODEL), dtype=torch.bfloat16, device=DEV)
    sched = {"fused": G.DECODE_FUSED, "split": G.DECODE_SPLIT, "auto": G.DECODE_AUTO}[mode]
    ws = G.workspace(G.OP_LAYER_DECODE, B, c.T_max, DEV)
    h = G.layer_decode(c.xd, gd, *c.wd, c.kcache, c.vcache, c.rope, P, h_bf16=h_bf16, ws=ws,
                       schedule=sched)
    torch.cuda.synchronize()
    assert G.workspace_errors(ws) == 0
    w = [f64(t) for t in c.w]
    ref_h, res = O.gqa_layer(f64(c.x)[:, None, :], f64(g), G.NORM_EPS, *w, f64(c.kc_rows),
                             f64(c.vc_rows), P)
    x = f64(c.x)
    errs = {"h": assert_close("h", f64(h), ref_h[:, 0]),
            "delta": assert_close("h - x", f64(h) - x, res.delta[:, 0])}
    want = O.bf16_bits_from_f64(f64(h))
    assert np.array_equal(bits(h_bf16), want), "h_bf16 is not the bf16 rounding of h"
    bk, bv = _layer_kv_bounds(O.rms_norm(x, f64(g), G.NORM_EPS), w, 8)
    errs["k_flips"] = assert_bf16_rows("kcache row", bits(G.kcache_by_position(c.kcache)[:, P]),
                                       res.k[:, 0], bk)
    errs["v_flips"] = assert_bf16_rows("vcache row", bits(G.vcache_read(c.vcache, P, P + 1)[:, 0]),
                                       res.v[:, 0], bv)
    c.check_untouched()
    print(f"layer decode B={B} P={P} {mode}", errs)


@pytest.mark.parametrize("n_kv,B,P", [(16, 2, 300), (32, 1, 1000), (16, 7, 100), (16, 12, 100),
                                      (32, 9, 65)])
def test_layer_decode_other_kv_head_counts(n_kv, B, P):
    """The layer (RMSNorm, block, residual) with 16 and 32 key/value heads, on
    the projection paths: B <= 8 with the norm in the QKV GEMV and the
    residual in the wo epilogue (GEMV up to 4 tokens, matrix cores above),
    and B > 8 with the norm pass and the accumulating block."""
    c = DecodeCase(B, P, ((P + 1 + 31) // 32) * 32 + 32, dev=DEV, n_kv=n_kv)
    g = synth.norm_gain(7)
    ws = G.workspace(G.OP_LAYER_DECODE, B, c.T_max, DEV, n_kv_heads=n_kv)
    h = G.layer_decode(c.xd, g.to(DEV), *c.wd, c.kcache, c.vcache, c.rope, P, ws=ws)
    torch.cuda.synchronize()
    assert G.workspace_errors(ws) == 0
    w = [f64(t) for t in c.w]
    ref_h, res = O.gqa_layer(f64(c.x)[:, None, :], f64(g), G.NORM_EPS, *w, f64(c.kc_rows),
                             f64(c.vc_rows), P, n_kv_heads=n_kv)
    errs = {"h": assert_close("h", f64(h), ref_h[:, 0]),
            "delta": assert_close("h - x", f64(h) - f64(c.x), res.delta[:, 0])}
    bk, _ = _layer_kv_bounds(O.rms_norm(f64(c.x), f64(g), G.NORM_EPS), w, n_kv)
    errs["k_flips"] = assert_bf16_rows("kcache row", bits(G.kcache_by_position(c.kcache)[:, P]),
                                       res.k[:, 0], bk)
    c.check_untouched()
    print(f"layer decode n_kv={n_kv} B={B} P={P}", errs)


@pytest.mark.parametrize("n_kv,B,start_pos,T", [(16, 2, 0, 70), (32, 1, 64, 100)])
def test_layer_prefill_other_kv_head_counts(n_kv, B, start_pos, T):
    """The prefill layer with 16 and 32 key/value heads (also after cached rows)."""
    T_max = ((start_pos + T + 31) // 32) * 32 + 32
    c = PrefillCase(B, T, T_max, dev=DEV, start_pos=start_pos, n_kv=n_kv)
    g = synth.norm_gain(8)
    ws = G.workspace(G.OP_LAYER_PREFILL, B, T_max, DEV, T, start_pos, n_kv_heads=n_kv)
    h = G.layer_prefill(c.xd, g.to(DEV), *c.wd, c.kcache, c.vcache, c.rope, start_pos=start_pos,
                        ws=ws)
    torch.cuda.synchronize()
    w = [f64(t) for t in c.w]
    kc = f64(c.kc_rows) if start_pos else None
    vc = f64(c.vc_rows) if start_pos else None
    ref_h, res = O.gqa_layer(f64(c.x), f64(g), G.NORM_EPS, *w, kc, vc, start_pos,
                             n_kv_heads=n_kv)
    errs = {"h": assert_close("h", f64(h), ref_h),
            "delta": assert_close("h - x", f64(h) - f64(c.x), res.delta)}
    c.check_untouched()
    print(f"layer prefill n_kv={n_kv} B={B} start_pos={start_pos} T={T}", errs)


def _check_xn(ws, B, start_pos, T, T_max, ref_xn):
    base = G.workspace_bytes(G.OP_PREFILL, B, T_max, T, start_pos)
    base = (base + 255) // 256 * 256
    xn = ws[base:base + B * T * G.D_MODEL * 2].view(torch.bfloat16).reshape(ref_xn.shape)
    got = bits(xn).astype(np.int32)
    want = O.bf16_bits_from_f64(ref_xn).astype(np.int32)
    off = got != want
    assert np.mean(off) <= 1e-4, f"normalised input: {np.mean(off):.2e} off"
    assert np.all(np.abs(got - want) <= 1), "normalised input more than one bf16 step off"
    return float(np.mean(off))


@pytest.mark.parametrize("B,start_pos,T", [(2, 0, 70), (1, 64, 100), (2, 200, 8)])
def test_layer_prefill(B, start_pos, T):
    T_max = ((start_pos + T + 31) // 32) * 32 + 32
    c = PrefillCase(B, T, T_max, dev=DEV, start_pos=start_pos)
    g = synth.norm_gain(6)
    ws = G.workspace(G.OP_LAYER_PREFILL, B, T_max, DEV, T, start_pos)
    probe = torch.empty((B, T, G.QKV_DIM), dtype=torch.float32, device=DEV)
    h = G.layer_prefill(c.xd, g.to(DEV), *c.wd, c.kcache, c.vcache, c.rope, start_pos=start_pos,
                        ws=ws, probe=probe)
    torch.cuda.synchronize()
    w = [f64(t) for t in c.w]
    kc = f64(c.kc_rows) if start_pos else None
    vc = f64(c.vc_rows) if start_pos else None
    ref_h, res = O.gqa_layer(f64(c.x), f64(g), G.NORM_EPS, *w, kc, vc, start_pos)
    errs = {"h": assert_close("h", f64(h), ref_h),
            "delta": assert_close("h - x", f64(h) - f64(c.x), res.delta)}
    xn_exact = O.rms_norm(f64(c.x), f64(g), G.NORM_EPS)
    errs["xn_off"] = _check_xn(ws, B, start_pos, T, T_max, xn_exact)
    pr = f64(probe)
    kpos = G.kcache_by_position(c.kcache)
    bk, bv = _layer_kv_bounds(xn_exact, w, 8)
    errs["k_flips"] = assert_bf16_rows("kcache rows", bits(kpos[:, start_pos:start_pos + T]),
                                       res.k, bk, pr[..., 4096:5120].reshape(B, T, 8, 128))
    errs["v_flips"] = assert_bf16_rows("vcache rows",
                                       bits(G.vcache_read(c.vcache, start_pos, start_pos + T)),
                                       res.v, bv, pr[..., 5120:].reshape(B, T, 8, 128))
    c.check_untouched()
    print(f"layer prefill B={B} start_pos={start_pos} T={T}", errs)


# ----------------------------------------------------------------------------
# Vocabulary projection
# ----------------------------------------------------------------------------

def _check_logits(got, exact, bound, name):
    """Logits are bf16 values, each the rounding of an fp32 dot product whose
    summation order the page leaves open: every logit equals the oracle's
    (its rounding of the exact product) unless the exact product lies within
    the fp32 accumulation bound of a rounding midpoint, where another order
    may round the other way (assert_bf16_rows); the mean difference from the
    oracle's logits stays at the usual tolerance."""
    g = f64(got)
    assert np.array_equal(O.f64_from_bf16_bits(O.bf16_bits_from_f64(g)), g), f"{name}: not bf16 values"
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    errs = {"logits": norm_err(g, O.f64_from_bf16_bits(O.bf16_bits_from_f64(exact)))}
    assert errs["logits"][1] <= MEAN_TOL, f"{name}: normalised mean {errs['logits'][1]:.3e}"
    errs["flips"] = assert_bf16_rows(name, O.bf16_bits_from_f64(g), exact, bound)
    return errs


def _vocab_exact(h, w, g):
    """The oracle's logits before their final bf16 rounding, and the fp32
    rounding bound of each (with the near-tie slack of the normalised input)."""
    if g is None:
        return h @ w.T, round_bounds(h, w, rotated=False)
    zx = O.rms_norm(h, g, G.NORM_EPS)
    z = O.f64_from_bf16_bits(O.bf16_bits_from_f64(zx))
    return z @ w.T, round_bounds(z, w, rotated=False) + tie_slack(zx, w)


@pytest.mark.parametrize("B,V,norm", [(3, 1001, True), (5, 130, False),
                                      # from 6 sequences: the matrix-core path, 1 to 4 column
                                      # tiles of 16 (a partial last block of 128 rows; 70: two
                                      # launches, the second ragged)
                                      (6, 130, True), (8, 130, True), (11, 4096, False),
                                      (9, 4096, True), (20, 1001, True), (40, 300, False),
                                      (70, 130, True), (64, 257, False)])
def test_vocab_logits_small(B, V, norm):
    from grouped_query_attention_gemv_amd import synth
    gen = synth.generator(40 + B)
    h = synth.randn_bf16(gen, (B, G.D_MODEL))
    w = synth.randn_bf16(gen, (V, G.D_MODEL), 0.02)
    g = synth.norm_gain(41) if norm else None
    L = G.vocab_logits(h.to(DEV), w.to(DEV), g.to(DEV) if norm else None)
    torch.cuda.synchronize()
    ref = O.vocab_logits(f64(h), f64(w), f64(g) if norm else None, G.NORM_EPS)
    exact, bound = _vocab_exact(f64(h), f64(w), f64(g) if norm else None)
    assert np.array_equal(O.f64_from_bf16_bits(O.bf16_bits_from_f64(exact)), ref)
    print(f"vocab B={B} V={V} norm={norm}", _check_logits(L, exact, bound, "logits"))


@pytest.mark.parametrize("B", [2, 6, 24])
def test_vocab_logits_llama31_size(B):
    """V = 128,256 (the Llama 3 vocabulary), final norm on: weights drawn on
    the device, 4,096 sampled rows checked against the oracle.  B = 2 runs
    the GEMV, B = 6 and 24 the matrix-core path (one and two column tiles)."""
    from grouped_query_attention_gemv_amd import synth
    V = G.VOCAB
    gen = synth.generator(50)
    h = synth.randn_bf16(gen, (B, G.D_MODEL))
    g = synth.norm_gain(51)
    w = torch.empty((V, G.D_MODEL), dtype=torch.bfloat16, device=DEV)
    synth.fill_randn_bf16_(w, synth.generator(52, DEV), 0.02)
    L = G.vocab_logits(h.to(DEV), w, g.to(DEV))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(53).choice(V, 4096, replace=False))
    rows[-1] = V - 1
    wr = f64(w[torch.from_numpy(rows).to(DEV)])
    ref = O.vocab_logits(f64(h), wr, f64(g), G.NORM_EPS)
    exact, bound = _vocab_exact(f64(h), wr, f64(g))
    assert np.array_equal(O.f64_from_bf16_bits(O.bf16_bits_from_f64(exact)), ref)
    print(f"vocab B={B} V=128256", _check_logits(L[:, torch.from_numpy(rows).to(DEV)], exact, bound,
                                                 "logits"))
    assert bool(torch.isfinite(L).all())


# ----------------------------------------------------------------------------
# Decode after prefill
# ----------------------------------------------------------------------------

def test_decode_after_prefill_equals_prefill_1001():
    """Prefill 1,000 tokens, then decode token 1,000 on the cache the prefill
    wrote; the result must match the last row of a 1,001-token prefill (and
    the oracle of that prefill)."""
    T = 1000
    full = PrefillCase(1, T + 1, 1024, dev=DEV)
    full.run(probe=False)
    ref = full.oracle()
    assert_close("prefill 1001", f64(full.out), ref.delta)

    kc, vc = G.empty_caches(1, 1024, DEV)
    G.block_prefill(full.xd[:, :T].contiguous(), *full.wd, kc, vc, full.rope)
    out = G.block_decode(full.xd[:, T].contiguous(), *full.wd, kc, vc, full.rope, T)
    torch.cuda.synchronize()
    assert_close("decode vs oracle", f64(out), ref.delta[:, T])
    assert_close("decode vs gpu prefill", f64(out), f64(full.out[:, T]))
    # rows 0..999 come from the same GEMM tiles on both routes: bit-identical;
    # row 1000 (GEMV vs GEMM summation order) may sit one bf16 step away
    assert np.array_equal(bits(G.kcache_by_position(kc)[:, :T]),
                          bits(G.kcache_by_position(full.kcache)[:, :T]))
    assert np.array_equal(bits(G.vcache_read(vc, 0, T)), bits(G.vcache_read(full.vcache, 0, T)))
    bk, _ = kv_bounds(f64(full.x[:, T]), [f64(t) for t in full.w], 8)
    assert_bf16_rows("row 1000", bits(G.kcache_by_position(kc)[:, T]), ref.k[:, T], bk)


# ---------------------------------------------------------------------------
# Seeded shape sweep: combinations the cases above do not spell out
# ---------------------------------------------------------------------------

def _sweep_cases():
    rng = np.random.default_rng(20261203)
    dec, pre = [], []
    for i in range(16):
        n_kv = int(rng.choice([8, 16, 32]))
        B = int(rng.integers(1, 5 if n_kv == 32 else 13))
        P = int(rng.integers(0, 2000))
        T_max = (P + 1 + int(rng.integers(0, 64)) + 31) // 32 * 32
        schedule = [G.DECODE_AUTO, G.DECODE_SPLIT, G.DECODE_FUSED][int(rng.integers(0, 3))]
        dec.append((i, n_kv, B, P, T_max, schedule))
    for i in range(8):
        n_kv = int(rng.choice([8, 16, 32]))
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, 300))
        sp = 0 if rng.random() < 0.5 else int(rng.integers(1, 600))
        T_max = (sp + T + int(rng.integers(0, 64)) + 31) // 32 * 32
        pre.append((i, n_kv, B, T, sp, T_max))
    return dec, pre


_SWEEP_DECODE, _SWEEP_PREFILL = _sweep_cases()


@pytest.mark.parametrize("i,n_kv,B,P,T_max,schedule", _SWEEP_DECODE)
def test_decode_shape_sweep(i, n_kv, B, P, T_max, schedule):
    """Seeded random (kv heads, batch, position, cache length, schedule):
    Delta, Q, K, V and the appended rows against the oracle, every other
    cache bit unchanged.  A one-launch request the shape does not admit runs
    the library's choice instead."""
    if schedule == G.DECODE_FUSED:
        try:
            G.decode_schedule(B, P, T_max, n_kv, schedule)
        except G.GQAError:
            schedule = G.DECODE_AUTO
    c = DecodeCase(B, P, T_max, seed=300 + i, dev=DEV, n_kv=n_kv)
    c.run(schedule=schedule)
    c.check(c.oracle())
    c.check_untouched()


@pytest.mark.parametrize("i,n_kv,B,T,start_pos,T_max", _SWEEP_PREFILL)
def test_prefill_shape_sweep(i, n_kv, B, T, start_pos, T_max):
    """Seeded random (kv heads, batch, new tokens, cached prefix, cache
    length) prefill against the oracle, every other cache bit unchanged."""
    c = PrefillCase(B, T, T_max, seed=400 + i, dev=DEV, start_pos=start_pos, n_kv=n_kv)
    c.run()
    c.check(c.oracle())
    c.check_untouched()
