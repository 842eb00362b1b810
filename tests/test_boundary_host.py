"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/gqa.h declares, and
reject bad arguments with the documented status before making any HIP call
(so the fake device addresses used here are never dereferenced).
"""
import ctypes
import os
import re
import subprocess

import pytest

import grouped_query_attention_gemv_amd as G
from grouped_query_attention_gemv_amd import gqa as GB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

OK, ENULL, ESHAPE, ERANGE, EALIGN, EWS, EHIP, EALIAS, EARG = 0, -1, -2, -3, -4, -5, -6, -7, -8


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_documented_entry_points():
    names = _declared_functions()
    for n in ("gqa_rope_table", "gqa_workspace_bytes", "gqa_block_prefill", "gqa_block_decode",
              "gqa_status_string", "gqa_block_prefill_profiled", "gqa_block_decode_profiled",
              "gqa_block_prefill_from", "gqa_workspace_bytes_from"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = G.lib()
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", GB.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in _declared_functions():
        assert n in exported, n
    assert set(GB._SIGS) == set(_declared_functions())


def test_status_strings():
    for code in (OK, ENULL, ESHAPE, ERANGE, EALIGN, EWS, EHIP, EALIAS, EARG):
        assert G.status_string(code).startswith(GB.STATUS[code])
    assert "unknown" in G.status_string(12345)


def test_workspace_bytes():
    assert G.workspace_bytes(0, 1, 64) == 0
    assert G.workspace_bytes(1, 0, 64) == 0
    assert G.workspace_bytes(1, 1, 0) == 0
    # prefill needs fp16 Q and O, fp16 K/V copies and an fp16 Wo: at B=4, T=2048
    n = G.workspace_bytes(4, 2048, 2048)
    assert n >= 4 * 2048 * 4096 * 2 * 2 + 2 * 4 * 8 * 2048 * 128 * 2 + 4096 * 4096 * 2
    assert G.workspace_bytes(8, 1, 131072) > 0


# fake, 16-byte aligned device addresses: validation rejects every call below
# before any of them could be used
BASE = 0x7F0000000000


def _fake(i, size=1 << 32):
    return ctypes.c_void_p(BASE + i * size)


def _decode_args(**kw):
    a = dict(x=_fake(0), wq=_fake(1), wk=_fake(2), wv=_fake(3), wo=_fake(4), kc=_fake(5),
             vc=_fake(6), T_max=1024, rope=_fake(7), start_pos=10, B=1, out=_fake(8),
             out_bf16=None, accumulate=0, ws=_fake(9), ws_bytes=1 << 40, probe=None,
             stream=None)
    a.update(kw)
    return [a[k] for k in ("x", "wq", "wk", "wv", "wo", "kc", "vc", "T_max", "rope", "start_pos",
                           "B", "out", "out_bf16", "accumulate", "ws", "ws_bytes", "probe",
                           "stream")]


def _decode_kv_args(n_kv, **kw):
    a = _decode_args(**kw)
    return a[:7] + [n_kv] + a[7:] + [None]


@pytest.mark.parametrize("n_kv,kw,code", [
    (4, {}, EARG), (24, {}, EARG), (0, {}, EARG), (-8, {}, EARG),
    (16, dict(B=0), ESHAPE), (32, dict(B=64, ws_bytes=1024), EWS),
    (32, dict(x=None), ENULL), (16, dict(start_pos=1024), ERANGE), (32, dict(ws_bytes=1024), EWS),
    (32, dict(out=_fake(0)), EALIAS), (16, dict(probe=_fake(8)), EALIAS),
])
def test_decode_kv_rejects_bad_arguments(n_kv, kw, code):
    assert G.lib().gqa_block_decode_kv(*_decode_kv_args(n_kv, **kw)) == code


def test_decode_kv_fused_schedule_is_rejected_off_eight_heads():
    """The one-launch schedule is built for 8 key/value heads; forcing it
    makes the other head counts fail before any launch."""
    prev = G.set_decode_schedule(G.DECODE_FUSED)
    try:
        assert G.lib().gqa_block_decode_kv(*_decode_kv_args(16)) == EARG
        assert G.lib().gqa_block_decode_kv(*_decode_kv_args(32)) == EARG
    finally:
        G.set_decode_schedule(prev)


def _prefill_args(**kw):
    a = dict(x=_fake(0), wq=_fake(1), wk=_fake(2), wv=_fake(3), wo=_fake(4), kc=_fake(5),
             vc=_fake(6), T_max=1024, rope=_fake(7), B=1, T=16, out=_fake(8), ws=_fake(9),
             ws_bytes=1 << 40, probe=None, stream=None)
    a.update(kw)
    return [a[k] for k in ("x", "wq", "wk", "wv", "wo", "kc", "vc", "T_max", "rope", "B", "T",
                           "out", "ws", "ws_bytes", "probe", "stream")]


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), ENULL), (dict(wo=None), ENULL), (dict(kc=None), ENULL), (dict(ws=None), ENULL),
    (dict(rope=None), ENULL), (dict(out=None), ENULL),
    (dict(B=0), ESHAPE), (dict(B=100000), ESHAPE), (dict(T_max=0), ESHAPE),
    (dict(T_max=1004), EALIGN), (dict(T_max=1000), EALIGN), (dict(x=ctypes.c_void_p(BASE + 2)), EALIGN),
    (dict(probe=ctypes.c_void_p(BASE + (20 << 32) + 4)), EALIGN),
    (dict(start_pos=-1), ERANGE), (dict(start_pos=1024), ERANGE),
    (dict(ws_bytes=1024), EWS), (dict(accumulate=2), EARG),
    (dict(out=_fake(0)), EALIAS), (dict(probe=_fake(8)), EALIAS),
    (dict(out_bf16=_fake(5)), EALIAS), (dict(ws=_fake(6)), EALIAS),
])
def test_decode_rejects_bad_arguments(kw, code):
    assert G.lib().gqa_block_decode(*_decode_args(**kw)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), ENULL), (dict(vc=None), ENULL),
    (dict(B=0), ESHAPE), (dict(T=0), ESHAPE), (dict(T_max=-8), ESHAPE),
    (dict(T_max=1020), EALIGN), (dict(wq=ctypes.c_void_p(BASE + (1 << 32) + 8)), EALIGN),
    (dict(T=1025), ERANGE),
    (dict(ws_bytes=4096), EWS),
    (dict(out=_fake(3)), EALIAS), (dict(kc=_fake(6)), EALIAS),
])
def test_prefill_rejects_bad_arguments(kw, code):
    assert G.lib().gqa_block_prefill(*_prefill_args(**kw)) == code


def _prefill_from_args(**kw):
    a = dict(x=_fake(0), wq=_fake(1), wk=_fake(2), wv=_fake(3), wo=_fake(4), kc=_fake(5),
             vc=_fake(6), T_max=1024, rope=_fake(7), start_pos=100, B=1, T=16, out=_fake(8),
             ws=_fake(9), ws_bytes=1 << 40, probe=None, stream=None)
    a.update(kw)
    return [a[k] for k in ("x", "wq", "wk", "wv", "wo", "kc", "vc", "T_max", "rope", "start_pos",
                           "B", "T", "out", "ws", "ws_bytes", "probe", "stream")]


def _prefill_kv_args(n_kv, **kw):
    a = _prefill_from_args(**kw)
    return a[:7] + [n_kv] + a[7:] + [None]


@pytest.mark.parametrize("n_kv,kw,code", [
    (4, {}, EARG), (12, {}, EARG), (64, {}, EARG), (0, {}, EARG),
    (32, dict(x=None), ENULL), (16, dict(T=0), ESHAPE), (32, dict(start_pos=1009), ERANGE),
    (32, dict(ws_bytes=4096), EWS), (16, dict(out=_fake(3)), EALIAS),
    (32, dict(probe=_fake(8)), EALIAS),
])
def test_prefill_kv_rejects_bad_arguments(n_kv, kw, code):
    assert G.lib().gqa_block_prefill_kv(*_prefill_kv_args(n_kv, **kw)) == code


def test_workspace_bytes_kv():
    L = G.lib()
    for B, sp, T, T_max in [(1, 0, 1, 32), (4, 0, 2048, 2048), (2, 100, 300, 512)]:
        assert L.gqa_workspace_bytes_kv(B, sp, T, T_max, 8) == \
            L.gqa_workspace_bytes_from(B, sp, T, T_max)
        n8, n16, n32 = (L.gqa_workspace_bytes_kv(B, sp, T, T_max, k) for k in (8, 16, 32))
        assert 0 < n8 <= n16 <= n32
    # the fp16 K/V copies: B * n_kv * Tp * 128 * 2 bytes each, Tp = 2048
    assert L.gqa_workspace_bytes_kv(4, 0, 2048, 2048, 32) - \
        L.gqa_workspace_bytes_kv(4, 0, 2048, 2048, 8) == 2 * 4 * 24 * 2048 * 128 * 2
    for k in (0, 4, 24, 33):
        assert L.gqa_workspace_bytes_kv(1, 0, 16, 64, k) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), ENULL), (dict(rope=None), ENULL),
    (dict(B=0), ESHAPE), (dict(T=0), ESHAPE),
    (dict(start_pos=-1), ERANGE), (dict(start_pos=1009), ERANGE), (dict(T=925), ERANGE),
    (dict(ws_bytes=4096), EWS),
    (dict(out=_fake(3)), EALIAS), (dict(vc=_fake(5)), EALIAS),
])
def test_prefill_from_rejects_bad_arguments(kw, code):
    assert G.lib().gqa_block_prefill_from(*_prefill_from_args(**kw)) == code


def test_workspace_bytes_from():
    lib = G.lib()
    assert lib.gqa_workspace_bytes_from(1, -1, 16, 1024) == 0
    assert lib.gqa_workspace_bytes_from(1, 1009, 16, 1024) == 0
    assert lib.gqa_workspace_bytes_from(1, 1008, 16, 1024) > 0
    assert lib.gqa_workspace_bytes_from(4, 0, 2048, 4096) == lib.gqa_workspace_bytes(4, 2048, 4096)
    # the fp16 K and V^T copies hold all start_pos + T keys: 2048 more rows of
    # 8 heads x 128 fp16 per sequence, twice
    grow = lib.gqa_workspace_bytes_from(4, 2048, 2048, 4096) - lib.gqa_workspace_bytes(4, 2048, 4096)
    assert grow == 2 * 4 * 8 * 2048 * 128 * 2
    assert G.workspace_bytes(4, 2048, 4096, start_pos=2048) == grow + lib.gqa_workspace_bytes(4, 2048, 4096)


def test_layer_workspace_bytes():
    lib = G.lib()
    for (B, sp, T, Tm) in [(1, 0, 1, 1024), (4, 2048, 2048, 4096), (2, 0, 70, 128)]:
        base = lib.gqa_workspace_bytes_from(B, sp, T, Tm)
        assert lib.gqa_layer_workspace_bytes(B, sp, T, Tm) == ((base + 255) // 256) * 256 + B * T * 4096 * 2
    assert lib.gqa_layer_workspace_bytes(1, 1020, 8, 1024) == 0


def _layer_decode_args(**kw):
    a = dict(x=_fake(0), g=_fake(10), eps=ctypes.c_float(1e-5), wq=_fake(1), wk=_fake(2),
             wv=_fake(3), wo=_fake(4), kc=_fake(5), vc=_fake(6), T_max=1024, rope=_fake(7),
             start_pos=10, B=1, h=_fake(8), h_bf16=None, ws=_fake(9), ws_bytes=1 << 40,
             probe=None, stream=None)
    a.update(kw)
    return [a[k] for k in ("x", "g", "eps", "wq", "wk", "wv", "wo", "kc", "vc", "T_max", "rope",
                           "start_pos", "B", "h", "h_bf16", "ws", "ws_bytes", "probe", "stream")]


@pytest.mark.parametrize("kw,code", [
    (dict(g=None), ENULL), (dict(h=None), ENULL), (dict(wq=None), ENULL),
    (dict(B=0), ESHAPE), (dict(start_pos=1024), ERANGE), (dict(start_pos=-3), ERANGE),
    (dict(eps=ctypes.c_float(0.0)), EARG), (dict(eps=ctypes.c_float(float("nan"))), EARG),
    (dict(g=ctypes.c_void_p(BASE + (10 << 32) + 2)), EALIGN),
    (dict(ws_bytes=4096), EWS),
    (dict(h=_fake(0)), EALIAS), (dict(h=_fake(10)), EALIAS), (dict(h=_fake(9)), EALIAS),
    (dict(h_bf16=_fake(5)), EALIAS),
])
def test_layer_decode_rejects_bad_arguments(kw, code):
    assert G.lib().gqa_layer_decode(*_layer_decode_args(**kw)) == code


def test_layer_workspace_bytes_kv():
    lib = G.lib()
    for (B, sp, T, Tm) in [(1, 0, 1, 1024), (4, 2048, 2048, 4096), (2, 0, 70, 128)]:
        assert lib.gqa_layer_workspace_bytes_kv(B, sp, T, Tm, 8) == \
            lib.gqa_layer_workspace_bytes(B, sp, T, Tm)
        for kv in (16, 32):
            base = lib.gqa_workspace_bytes_kv(B, sp, T, Tm, kv)
            assert lib.gqa_layer_workspace_bytes_kv(B, sp, T, Tm, kv) == \
                ((base + 255) // 256) * 256 + B * T * 4096 * 2
    assert lib.gqa_layer_workspace_bytes_kv(1, 0, 1, 1024, 24) == 0
    assert lib.gqa_layer_workspace_bytes_kv(1, 1020, 8, 1024, 16) == 0


def _layer_kv_args(n_kv, **kw):
    a = _layer_decode_args(**kw)
    return a[:9] + [n_kv] + a[9:]


@pytest.mark.parametrize("n_kv,kw,code", [
    (4, {}, EARG), (24, {}, EARG), (0, {}, EARG),
    (16, dict(g=None), ENULL), (32, dict(B=0), ESHAPE), (16, dict(start_pos=1024), ERANGE),
    (32, dict(ws_bytes=4096), EWS), (16, dict(h=_fake(10)), EALIAS),
])
def test_layer_decode_kv_rejects_bad_arguments(n_kv, kw, code):
    assert G.lib().gqa_layer_decode_kv(*_layer_kv_args(n_kv, **kw)) == code


@pytest.mark.parametrize("n_kv,kw,code", [
    (4, {}, EARG), (24, {}, EARG),
    (16, dict(x=None), ENULL), (32, dict(T=0), ESHAPE), (16, dict(start_pos=1020), ERANGE),
    (32, dict(ws_bytes=4096), EWS), (16, dict(h=_fake(9)), EALIAS),
])
def test_layer_prefill_kv_rejects_bad_arguments(n_kv, kw, code):
    a = dict(x=_fake(0), g=_fake(10), eps=ctypes.c_float(1e-5), wq=_fake(1), wk=_fake(2),
             wv=_fake(3), wo=_fake(4), kc=_fake(5), vc=_fake(6), T_max=1024, rope=_fake(7),
             start_pos=0, B=1, T=8, h=_fake(8), ws=_fake(9), ws_bytes=1 << 40, probe=None,
             stream=None)
    a.update(kw)
    args = [a[k] for k in ("x", "g", "eps", "wq", "wk", "wv", "wo", "kc", "vc")] + [n_kv] + \
        [a[k] for k in ("T_max", "rope", "start_pos", "B", "T", "h", "ws", "ws_bytes", "probe",
                        "stream")]
    assert G.lib().gqa_layer_prefill_kv(*args) == code


def _vocab_args(**kw):
    a = dict(h=_fake(0), g=None, eps=ctypes.c_float(1e-5), w=_fake(1), V=128256, B=1,
             logits=_fake(2), stream=None)
    a.update(kw)
    return [a[k] for k in ("h", "g", "eps", "w", "V", "B", "logits", "stream")]


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), ENULL), (dict(w=None), ENULL), (dict(logits=None), ENULL),
    (dict(B=0), ESHAPE), (dict(V=0), ESHAPE), (dict(V=(1 << 20) + 1), ESHAPE),
    (dict(logits=ctypes.c_void_p(BASE + (2 << 32) + 4)), EALIGN),
    (dict(g=_fake(3), eps=ctypes.c_float(-1.0)), EARG),
    (dict(logits=_fake(1)), EALIAS), (dict(logits=_fake(0)), EALIAS),
])
def test_vocab_logits_rejects_bad_arguments(kw, code):
    assert G.lib().gqa_vocab_logits(*_vocab_args(**kw)) == code


def test_profiled_variants_need_events():
    l = G.lib()
    assert l.gqa_block_decode_profiled(*_decode_args(), None) == ENULL
    assert l.gqa_block_prefill_profiled(*_prefill_args(), None) == ENULL


def test_rope_table_rejects_bad_arguments():
    l = G.lib()
    assert l.gqa_rope_table(0, 5e5, 1, _fake(0), None) == ESHAPE
    assert l.gqa_rope_table(16, 0.0, 1, _fake(0), None) == EARG
    assert l.gqa_rope_table(16, 5e5, 2, _fake(0), None) == EARG
    assert l.gqa_rope_table(16, 5e5, 1, None, None) == ENULL
    assert l.gqa_rope_table(16, 5e5, 1, ctypes.c_void_p(BASE + 4), None) == EALIGN


def test_binding_raises_without_gpu_tensors():
    import torch
    x = torch.zeros(1, 4096, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        G.block_decode(x, x, x, x, x, x, x, x, 0)


def test_workspace_starts_with_the_sync_region():
    assert G.SYNC_BYTES == 65536
    for args in ((1, 1, 64), (4, 2048, 2048), (64, 1, 8224)):
        assert G.workspace_bytes(*args) > G.SYNC_BYTES
    src = open(HEADER).read()
    assert "#define GQA_SYNC_BYTES  65536" in src


def test_workspace_init_rejections():
    lib = G.lib()
    assert lib.gqa_workspace_init(None, 1 << 20, None) == ENULL
    assert lib.gqa_workspace_init(ctypes.c_void_p(BASE + 8), 1 << 20, None) == EALIGN
    assert lib.gqa_workspace_init(_fake(1), G.SYNC_BYTES - 1, None) == EWS


def test_decode_schedule_selection():
    prev = G.set_decode_schedule(G.DECODE_AUTO)
    try:
        F, S = G.DECODE_FUSED, G.DECODE_SPLIT
        # fused while the attention grid (splits of 128 positions x 8 kv heads x B)
        # stays within 128 workgroups, and B <= 2
        assert G.decode_schedule(1, 0, 64) == F
        assert G.decode_schedule(1, 1000, 1024) == F
        assert G.decode_schedule(1, 2047, 4096) == F
        assert G.decode_schedule(1, 2048, 4096) == S
        assert G.decode_schedule(2, 1023, 2048) == F
        assert G.decode_schedule(2, 1024, 2048) == S
        assert G.decode_schedule(3, 10, 64) == S
        assert G.decode_schedule(64, 8192, 8224) == S
        G.set_decode_schedule(G.DECODE_SPLIT)
        assert G.decode_schedule(1, 1000, 1024) == S
        G.set_decode_schedule(G.DECODE_FUSED)
        assert G.decode_schedule(1, 1000, 1024) == F
        with pytest.raises(G.GQAError):
            G.decode_schedule(3, 10, 64)
        assert G.lib().gqa_decode_schedule(1, 64, 64) == ERANGE
        assert G.lib().gqa_decode_schedule(0, 1, 64) == ESHAPE
        assert G.lib().gqa_set_decode_schedule(7) == EARG
    finally:
        G.set_decode_schedule(prev)


def test_fused_schedule_rejects_shapes_it_does_not_admit():
    # B = 3 under a forced fused schedule: rejected before any device call
    prev = G.set_decode_schedule(G.DECODE_FUSED)
    try:
        assert G.lib().gqa_block_decode(*_decode_args(B=3)) == EARG
        assert G.lib().gqa_block_decode(*_decode_args(B=1, start_pos=4000, T_max=4096)) == EARG
    finally:
        G.set_decode_schedule(prev)


def test_library_has_no_unresolved_symbols_of_its_own():
    # a kernel whose host-side launch stub failed to instantiate shows up as
    # an undefined gqa:: symbol; loading the library lazily would not notice
    out = subprocess.run(["nm", "-D", "--undefined-only", "-C", GB.LIB_PATH], capture_output=True,
                         text=True).stdout
    mine = [l for l in out.splitlines() if "gqa::" in l or "gqa_" in l]
    assert mine == [], mine
