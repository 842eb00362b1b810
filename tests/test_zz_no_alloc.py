"""The decode entry point that allocates nothing (gqa_block_decode_noalloc)
against gqa_block_decode on the same inputs (needs an MI355X).

Both run the same kernels in the same order, so Delta, the probe and the
cache rows must agree bit for bit; Delta is also held to the oracle's
tolerance.  Each case makes two calls in a row on the library's one scratch
array, the second with a smaller input, so the second call must not depend
on what the first left there.
"""
import pytest
import torch

import grouped_query_attention_gemv_amd as G
from tests.parity import DecodeCase, assert_close, f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _pair(B, P, T_max, schedule):
    """Run one case through both entry points on identical caches; return
    the no-allocation result after checking it against the other."""
    c = DecodeCase(B, P, T_max, dev=DEV)
    nqkv = G.QKV_DIM
    # reference: the workspace entry point on copies of the caches
    kc, vc = c.kcache.clone(), c.vcache.clone()
    ref_probe = torch.empty((B, nqkv), dtype=torch.float32, device=DEV)
    ref = G.block_decode(c.xd, *c.wd, kc, vc, c.rope, P, probe=ref_probe, schedule=schedule)
    out = torch.full((B, G.D_MODEL), 7.0, dtype=torch.float32, device=DEV)
    probe = torch.empty((B, nqkv), dtype=torch.float32, device=DEV)
    G.block_decode_noalloc(c.xd, *c.wd, c.kcache, c.vcache, c.rope, P, out=out, probe=probe,
                           schedule=schedule)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), f"B={B} P={P}: Delta differs from gqa_block_decode"
    assert torch.equal(probe, ref_probe)
    assert torch.equal(c.kcache.view(torch.int16), kc.view(torch.int16))
    assert torch.equal(c.vcache.view(torch.int16), vc.view(torch.int16))
    assert_close("delta vs oracle", f64(out), c.oracle().delta[:, 0])
    c.check_untouched()
    return out


@pytest.mark.parametrize("first,second", [
    ((2, 777, 1024, G.DECODE_FUSED), (1, 100, 128, G.DECODE_FUSED)),    # one launch
    ((5, 300, 320, G.DECODE_SPLIT), (2, 64, 96, G.DECODE_SPLIT)),       # three launches
    ((16, 200, 224, G.DECODE_AUTO), (9, 31, 64, G.DECODE_AUTO)),        # matrix-core projections
])
def test_noalloc_decode_matches_the_workspace_entry_point(first, second):
    _pair(*first)
    _pair(*second)


def test_noalloc_decode_in_a_graph_matches_eager():
    """Captured once and replayed with eager work and synchronisations between
    the replays: every replay equals the eager call bit for bit."""
    B, P, T_max = 1, 500, 512
    c = DecodeCase(B, P, T_max, dev=DEV)
    k0, v0 = c.kcache.clone(), c.vcache.clone()
    eager = G.block_decode_noalloc(c.xd, *c.wd, c.kcache, c.vcache, c.rope, P).clone()
    out = torch.zeros_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        G.block_decode_noalloc(c.xd, *c.wd, c.kcache, c.vcache, c.rope, P, out=out)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        G.block_decode_noalloc(c.xd, *c.wd, c.kcache, c.vcache, c.rope, P, out=out)
    # an eager call of another shape between replays reuses the scratch
    x3 = c.xd.repeat(3, 1).contiguous()
    kc3, vc3 = G.empty_caches(3, 64, DEV)
    kc3.zero_()
    vc3.zero_()
    rope3 = G.rope_table(64, device=DEV)
    for _ in range(4):
        out.zero_()
        G.block_decode_noalloc(x3, *c.wd, kc3, vc3, rope3, 10)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    assert torch.equal(c.kcache.view(torch.int16)[:, :, :P], k0.view(torch.int16)[:, :, :P])
