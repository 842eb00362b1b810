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
AUTO, SPLIT, FUSED = G.DECODE_AUTO, G.DECODE_SPLIT, G.DECODE_FUSED


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_documented_entry_points():
    names = _declared_functions()
    for n in ("gqa_rope_table", "gqa_workspace_bytes", "gqa_workspace_init", "gqa_block_prefill",
              "gqa_block_decode", "gqa_decode_schedule", "gqa_status_string", "gqa_wo_to_fp16",
              "gqa_layer_prefill", "gqa_layer_decode", "gqa_vocab_logits",
              "gqa_block_decode_noalloc"):
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
    # the binding declares exactly the header's functions, and the library
    # exports no other gqa_ entry point
    assert set(GB._SIGS) == set(_declared_functions())
    assert set(n for n in exported if n.startswith("gqa_")) == set(_declared_functions())


def test_library_has_no_mutable_global_state_symbols():
    """No writable data of the library's own but the no-allocation decode's
    scratch array and its per-device address cache: every choice is an
    argument (the old process-wide decode-schedule setting is gone)."""
    # the product library itself (not a sanitizer build named by GQA_LIB)
    product = os.path.join(os.path.dirname(GB.__file__), "libgqa.so")
    out = subprocess.run(["nm", "-C", "--defined-only", product], capture_output=True,
                         text=True).stdout
    # (kernel launch handles are data symbols too, but carry a signature)
    mine = [l.split(None, 2)[2] for l in out.splitlines()
            if len(l.split()) >= 3 and l.split()[1] in "bBdD" and
            ("gqa" in l or "anonymous namespace" in l) and "(" not in l.split(None, 2)[2]
            .replace("(anonymous namespace)", "")]
    assert sorted(mine) == ["(anonymous namespace)::g_scratch_ptr",
                            "(anonymous namespace)::scratch"], mine


def test_status_strings():
    for code in (OK, ENULL, ESHAPE, ERANGE, EALIGN, EWS, EHIP, EALIAS, EARG):
        assert G.status_string(code).startswith(GB.STATUS[code])
    assert "unknown" in G.status_string(12345)


# ----------------------------------------------------------------------------
# workspace sizes
# ----------------------------------------------------------------------------

def _wsb(op, B, T_max, T=1, start_pos=0, n_kv=8):
    return G.lib().gqa_workspace_bytes(op, n_kv, B, start_pos, T, T_max)


def test_workspace_bytes_rejects_out_of_range():
    for op in (G.OP_PREFILL, G.OP_DECODE, G.OP_LAYER_PREFILL, G.OP_LAYER_DECODE):
        assert _wsb(op, 0, 64) == 0
        assert _wsb(op, 1, 0) == 0
        assert _wsb(op, 1, 64, T=0) == 0
        assert _wsb(op, 1, 64, start_pos=-1) == 0
        for k in (0, 4, 24, 33):
            assert _wsb(op, 1, 64, n_kv=k) == 0
    assert _wsb(7, 1, 64) == 0
    assert _wsb(G.OP_DECODE, 1, 64, T=2) == 0              # decode is one token
    assert _wsb(G.OP_DECODE, 1, 64, start_pos=64) == 0     # row start_pos must exist
    assert _wsb(G.OP_PREFILL, 1, 1024, T=16, start_pos=1009) == 0
    assert _wsb(G.OP_PREFILL, 1, 1024, T=16, start_pos=1008) > 0


def test_decode_workspace_excludes_prefill_copies():
    """Decode needs the sync region, Q, O and the partials: about 1.5 MiB at
    B = 1, not the 32 MiB fp16 Wo of prefill, and no dependence on T_max."""
    n = _wsb(G.OP_DECODE, 1, 1024)
    assert G.SYNC_BYTES < n < 2 << 20
    assert n == _wsb(G.OP_DECODE, 1, 131072, start_pos=131071)
    assert _wsb(G.OP_PREFILL, 1, 1024) > 32 << 20
    # the split-K partials of the batched projections grow with n_kv
    assert _wsb(G.OP_DECODE, 64, 8224, n_kv=8) < _wsb(G.OP_DECODE, 64, 8224, n_kv=32)


def test_prefill_workspace_sizes():
    # fp16 Q and O, fp16 K/V copies and an fp16 Wo: at B=4, T=2048
    n = _wsb(G.OP_PREFILL, 4, 2048, T=2048)
    assert n >= 4 * 2048 * 4096 * 2 * 2 + 2 * 4 * 8 * 2048 * 128 * 2 + 4096 * 4096 * 2
    # the fp16 K and V^T copies hold all start_pos + T keys: 2048 more rows of
    # 8 heads x 128 fp16 per sequence, twice
    grow = _wsb(G.OP_PREFILL, 4, 4096, T=2048, start_pos=2048) - _wsb(G.OP_PREFILL, 4, 4096, T=2048)
    assert grow == 2 * 4 * 8 * 2048 * 128 * 2
    # and with the head count: B * n_kv * Tp * 128 * 2 bytes each
    assert _wsb(G.OP_PREFILL, 4, 2048, T=2048, n_kv=32) - _wsb(G.OP_PREFILL, 4, 2048, T=2048) == \
        2 * 4 * 24 * 2048 * 128 * 2


def test_layer_workspace_sizes():
    for (B, sp, T, Tm) in [(4, 2048, 2048, 4096), (2, 0, 70, 128)]:
        for kv in (8, 16, 32):
            base = _wsb(G.OP_PREFILL, B, Tm, T, sp, kv)
            assert _wsb(G.OP_LAYER_PREFILL, B, Tm, T, sp, kv) == \
                ((base + 255) // 256) * 256 + B * T * 4096 * 2
    for B in (1, 16):
        base = _wsb(G.OP_DECODE, B, 1024)
        assert _wsb(G.OP_LAYER_DECODE, B, 1024) == ((base + 255) // 256) * 256 + B * 4096 * 2


def test_workspace_starts_with_the_sync_region():
    # 64 KiB of synchronisation words, then the one-launch decode's hand-off
    # buffers: Q and the appended rows of 2 sequences at up to 32 kv heads,
    # the partials of 128 attention workgroups (up to 4 heads x 132 floats,
    # 128-byte aligned per (sequence, kv head)), then 512 wo workgroups' slots
    # of 64 words, rounded up to whole 4 KiB fill blocks
    handoff = 2 * 4096 * 4 + 2 * 2 * 32 * 128 * 2 + (128 * 4 * 132 + 2 * 32 * 32) * 4 + 512 * 64 * 4
    assert G.SYNC_BYTES == (65536 + handoff + 4095) // 4096 * 4096 == 540672
    for op, B, T, Tm in ((G.OP_DECODE, 1, 1, 64), (G.OP_PREFILL, 4, 2048, 2048),
                         (G.OP_DECODE, 64, 1, 8224)):
        assert _wsb(op, B, Tm, T) > G.SYNC_BYTES
    src = open(HEADER).read()
    assert "#define GQA_SYNC_BYTES  540672" in src
    assert f"#define GQA_VOCAB_MFMA_MIN_B  {G.VOCAB_MFMA_MIN_B}" in src


def test_workspace_init_rejections():
    lib = G.lib()
    assert lib.gqa_workspace_init(None, 1 << 20, None) == ENULL
    assert lib.gqa_workspace_init(ctypes.c_void_p(BASE + 8), 1 << 20, None) == EALIGN
    assert lib.gqa_workspace_init(_fake(1), G.SYNC_BYTES - 1, None) == EWS


# ----------------------------------------------------------------------------
# argument checks of the block calls (fake, 16-byte aligned device addresses:
# validation rejects every call below before any of them could be used)
# ----------------------------------------------------------------------------

BASE = 0x7F0000000000


def _fake(i, size=1 << 32):
    return ctypes.c_void_p(BASE + i * size)


_DECODE_KEYS = ("x", "wq", "wk", "wv", "wo", "kc", "vc", "n_kv", "T_max", "rope", "start_pos",
                "B", "out", "out_bf16", "accumulate", "schedule", "ws", "ws_bytes", "probe",
                "events", "stream")


def _decode_args(**kw):
    a = dict(x=_fake(0), wq=_fake(1), wk=_fake(2), wv=_fake(3), wo=_fake(4), kc=_fake(5),
             vc=_fake(6), n_kv=8, T_max=1024, rope=_fake(7), start_pos=10, B=1, out=_fake(8),
             out_bf16=None, accumulate=0, schedule=AUTO, ws=_fake(9), ws_bytes=1 << 40,
             probe=None, events=None, stream=None)
    a.update(kw)
    return [a[k] for k in _DECODE_KEYS]


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), ENULL), (dict(wo=None), ENULL), (dict(kc=None), ENULL), (dict(ws=None), ENULL),
    (dict(rope=None), ENULL), (dict(out=None), ENULL),
    (dict(B=0), ESHAPE), (dict(B=100000), ESHAPE), (dict(T_max=0), ESHAPE),
    (dict(T_max=1004), EALIGN), (dict(T_max=1000), EALIGN),
    (dict(x=ctypes.c_void_p(BASE + 2)), EALIGN),
    (dict(probe=ctypes.c_void_p(BASE + (20 << 32) + 4)), EALIGN),
    (dict(start_pos=-1), ERANGE), (dict(start_pos=1024), ERANGE),
    (dict(ws_bytes=1024), EWS), (dict(accumulate=2), EARG),
    (dict(schedule=3), EARG), (dict(schedule=-1), EARG),
    (dict(out=_fake(0)), EALIAS), (dict(probe=_fake(8)), EALIAS),
    (dict(out_bf16=_fake(5)), EALIAS), (dict(ws=_fake(6)), EALIAS),
    # other head counts
    (dict(n_kv=4), EARG), (dict(n_kv=24), EARG), (dict(n_kv=0), EARG), (dict(n_kv=-8), EARG),
    (dict(n_kv=16, B=0), ESHAPE), (dict(n_kv=32, B=64, ws_bytes=1024), EWS),
    (dict(n_kv=32, x=None), ENULL), (dict(n_kv=16, start_pos=1024), ERANGE),
    (dict(n_kv=32, out=_fake(0)), EALIAS), (dict(n_kv=16, probe=_fake(8)), EALIAS),
])
def test_decode_rejects_bad_arguments(kw, code):
    assert G.lib().gqa_block_decode(*_decode_args(**kw)) == code


_NOALLOC_KEYS = ("x", "wq", "wk", "wv", "wo", "kc", "vc", "n_kv", "T_max", "rope", "start_pos",
                 "B", "out", "out_bf16", "accumulate", "schedule", "probe", "stream")


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), ENULL), (dict(out=None), ENULL), (dict(B=0), ESHAPE), (dict(n_kv=12), EARG),
    (dict(start_pos=1024), ERANGE), (dict(accumulate=3), EARG), (dict(schedule=7), EARG),
    (dict(B=3, schedule=FUSED), EARG), (dict(out=_fake(0)), EALIAS),
    # beyond the 16 MiB scratch array: rejected before anything runs
    (dict(B=512), EWS), (dict(B=128, n_kv=32), EWS),
])
def test_decode_noalloc_rejects_bad_arguments(kw, code):
    a = dict(zip(_DECODE_KEYS, _decode_args()))
    a.update(kw)
    assert G.lib().gqa_block_decode_noalloc(*[a[k] for k in _NOALLOC_KEYS]) == code


def test_decode_noalloc_scratch_limit_matches_the_workspace_sizes():
    """The shapes the scratch array admits are those whose decode workspace
    fits in GQA_NOALLOC_SCRATCH_BYTES."""
    assert "#define GQA_NOALLOC_SCRATCH_BYTES  (16u << 20)" in open(HEADER).read()
    lim = G.NOALLOC_SCRATCH_BYTES
    assert _wsb(G.OP_DECODE, 200, 1024) <= lim < _wsb(G.OP_DECODE, 512, 1024)
    assert _wsb(G.OP_DECODE, 64, 1024, n_kv=32) <= lim < _wsb(G.OP_DECODE, 128, 1024, n_kv=32)


def test_decode_workspace_check_uses_the_decode_size():
    """A workspace of exactly the decode size is accepted by validation (the
    call then fails only at launch on fake addresses, which dry shapes never
    reach: here the alias check on a wrong-sized buffer is what answers)."""
    n = _wsb(G.OP_DECODE, 1, 1024)
    assert G.lib().gqa_block_decode(*_decode_args(ws_bytes=n - 1)) == EWS
    # with the size met, the next check to fail is the planted alias
    assert G.lib().gqa_block_decode(*_decode_args(ws_bytes=n, out=_fake(0))) == EALIAS


def test_fused_schedule_is_rejected_where_it_does_not_apply():
    """The one-launch schedule takes B <= 2 and at most 128 attention
    workgroups of at most 256 positions each; asking for it elsewhere fails
    before any launch.  The request is per call: the next call is
    unaffected."""
    L = G.lib()
    assert L.gqa_block_decode(*_decode_args(B=3, schedule=FUSED)) == EARG
    assert L.gqa_block_decode(*_decode_args(start_pos=5000, T_max=8192, schedule=FUSED)) == EARG
    assert L.gqa_block_decode(*_decode_args(n_kv=32, start_pos=1024, T_max=2048, schedule=FUSED)) == EARG
    # the same arguments with AUTO pass validation up to the planted alias
    assert L.gqa_block_decode(*_decode_args(B=3, schedule=AUTO, out=_fake(0))) == EALIAS
    # 16 and 32 kv heads take the one-launch schedule too
    assert L.gqa_block_decode(*_decode_args(n_kv=16, schedule=FUSED, out=_fake(0))) == EALIAS
    assert L.gqa_block_decode(*_decode_args(n_kv=32, schedule=FUSED, out=_fake(0))) == EALIAS


def test_decode_schedule_selection():
    sch = G.lib().gqa_decode_schedule
    F, S = FUSED, SPLIT
    # fused for B <= 2 while the attention grid (splits x kv heads x B) fits
    # in 128 workgroups of at most 256 positions: the splits of 128 positions,
    # fewer and longer where needed
    assert sch(8, 1, 0, 64, AUTO) == F
    assert sch(8, 1, 1000, 1024, AUTO) == F
    assert sch(8, 1, 2047, 4096, AUTO) == F
    assert sch(8, 1, 4095, 4096, AUTO) == F          # 16 splits of 256
    assert sch(8, 1, 4096, 8192, AUTO) == S          # 16 would need 257 each
    assert sch(8, 2, 1023, 2048, AUTO) == F
    assert sch(8, 2, 2047, 2048, AUTO) == F          # 8 splits of 256 per sequence
    assert sch(8, 2, 2048, 4096, AUTO) == S
    assert sch(8, 3, 10, 64, AUTO) == S
    assert sch(8, 64, 8192, 8224, AUTO) == S
    # 16 kv heads: 8 splits per sequence at B = 1; 32: 4
    assert sch(16, 1, 1000, 1024, AUTO) == F
    assert sch(16, 1, 2047, 4096, AUTO) == F
    assert sch(16, 1, 2048, 4096, AUTO) == S
    assert sch(32, 1, 0, 64, AUTO) == F
    assert sch(32, 1, 1023, 1024, AUTO) == F
    assert sch(32, 1, 1024, 2048, AUTO) == S
    # at B = 2 with 16 or 32 kv heads the one-launch schedule is admitted but
    # AUTO keeps the three launches (measured faster there)
    assert sch(32, 2, 511, 1024, FUSED) == F
    assert sch(32, 2, 511, 1024, AUTO) == S
    assert sch(16, 2, 1000, 1024, FUSED) == F
    assert sch(16, 2, 1000, 1024, AUTO) == S
    assert sch(32, 2, 512, 1024, FUSED) == EARG
    assert sch(32, 1, 1024, 2048, FUSED) == EARG
    # the documented limit, start_pos + 1 <= 32768 / (n_kv * B), at every admitted pair
    for n_kv in (8, 16, 32):
        for B in (1, 2):
            lim = 32768 // (n_kv * B)
            assert sch(n_kv, B, lim - 1, lim, FUSED) == F
            assert sch(n_kv, B, lim, 2 * lim, FUSED) == EARG
    # explicit requests
    assert sch(8, 1, 1000, 1024, SPLIT) == S
    assert sch(8, 1, 1000, 1024, FUSED) == F
    assert sch(8, 3, 10, 64, FUSED) == EARG
    assert sch(8, 1, 1000, 1024, 9) == EARG
    # invalid shapes
    assert sch(8, 1, 64, 64, AUTO) == ERANGE
    assert sch(8, 0, 1, 64, AUTO) == ESHAPE
    assert sch(12, 1, 1, 64, AUTO) == EARG
    with pytest.raises(G.GQAError):
        G.decode_schedule(3, 10, 64, schedule=FUSED)
    assert G.decode_schedule(1, 1000, 1024) == F


_PREFILL_KEYS = ("x", "wq", "wk", "wv", "wo", "wo16", "kc", "vc", "n_kv", "T_max", "rope",
                 "start_pos", "B", "T", "out", "ws", "ws_bytes", "probe", "events", "stream")


def _prefill_args(**kw):
    a = dict(x=_fake(0), wq=_fake(1), wk=_fake(2), wv=_fake(3), wo=_fake(4), wo16=None,
             kc=_fake(5), vc=_fake(6), n_kv=8, T_max=1024, rope=_fake(7), start_pos=0, B=1,
             T=16, out=_fake(8), ws=_fake(9), ws_bytes=1 << 40, probe=None, events=None,
             stream=None)
    a.update(kw)
    return [a[k] for k in _PREFILL_KEYS]


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), ENULL), (dict(vc=None), ENULL), (dict(rope=None), ENULL),
    (dict(wo=None), ENULL),                                  # neither wo nor wo16
    (dict(B=0), ESHAPE), (dict(T=0), ESHAPE), (dict(T_max=-8), ESHAPE),
    (dict(T_max=1020), EALIGN), (dict(wq=ctypes.c_void_p(BASE + (1 << 32) + 8)), EALIGN),
    (dict(wo16=ctypes.c_void_p(BASE + (11 << 32) + 8)), EALIGN),
    (dict(T=1025), ERANGE), (dict(start_pos=-1), ERANGE), (dict(start_pos=1009), ERANGE),
    (dict(start_pos=100, T=925), ERANGE),
    (dict(ws_bytes=4096), EWS),
    (dict(out=_fake(3)), EALIAS), (dict(kc=_fake(6)), EALIAS), (dict(start_pos=100, vc=_fake(5)), EALIAS),
    (dict(wo16=_fake(8)), EALIAS),                           # the fp16 Wo is an input
    (dict(n_kv=4), EARG), (dict(n_kv=12), EARG), (dict(n_kv=64), EARG), (dict(n_kv=0), EARG),
    (dict(n_kv=32, x=None), ENULL), (dict(n_kv=16, T=0), ESHAPE),
    (dict(n_kv=32, start_pos=1009), ERANGE), (dict(n_kv=32, ws_bytes=4096), EWS),
    (dict(n_kv=16, out=_fake(3)), EALIAS), (dict(n_kv=32, probe=_fake(8)), EALIAS),
])
def test_prefill_rejects_bad_arguments(kw, code):
    assert G.lib().gqa_block_prefill(*_prefill_args(**kw)) == code


def test_prefill_accepts_wo16_in_place_of_wo():
    # with wo NULL and a caller fp16 copy, validation runs to the planted alias
    assert G.lib().gqa_block_prefill(*_prefill_args(wo=None, wo16=_fake(11),
                                                     out=_fake(3))) == EALIAS


def test_wo_to_fp16_rejections():
    L = G.lib()
    assert L.gqa_wo_to_fp16(None, _fake(1), None) == ENULL
    assert L.gqa_wo_to_fp16(_fake(0), None, None) == ENULL
    assert L.gqa_wo_to_fp16(ctypes.c_void_p(BASE + 4), _fake(1), None) == EALIGN
    assert L.gqa_wo_to_fp16(_fake(0), ctypes.c_void_p(BASE + 4096), None) == EALIAS


_LAYER_DECODE_KEYS = ("x", "g", "eps", "wq", "wk", "wv", "wo", "kc", "vc", "n_kv", "T_max",
                      "rope", "start_pos", "B", "h", "h_bf16", "schedule", "ws", "ws_bytes",
                      "probe", "stream")


def _layer_decode_args(**kw):
    a = dict(x=_fake(0), g=_fake(10), eps=ctypes.c_float(1e-5), wq=_fake(1), wk=_fake(2),
             wv=_fake(3), wo=_fake(4), kc=_fake(5), vc=_fake(6), n_kv=8, T_max=1024,
             rope=_fake(7), start_pos=10, B=1, h=_fake(8), h_bf16=None, schedule=AUTO,
             ws=_fake(9), ws_bytes=1 << 40, probe=None, stream=None)
    a.update(kw)
    return [a[k] for k in _LAYER_DECODE_KEYS]


@pytest.mark.parametrize("kw,code", [
    (dict(g=None), ENULL), (dict(h=None), ENULL), (dict(wq=None), ENULL),
    (dict(B=0), ESHAPE), (dict(start_pos=1024), ERANGE), (dict(start_pos=-3), ERANGE),
    (dict(eps=ctypes.c_float(0.0)), EARG), (dict(eps=ctypes.c_float(float("nan"))), EARG),
    (dict(g=ctypes.c_void_p(BASE + (10 << 32) + 2)), EALIGN),
    (dict(ws_bytes=4096), EWS), (dict(schedule=5), EARG),
    (dict(h=_fake(0)), EALIAS), (dict(h=_fake(10)), EALIAS), (dict(h=_fake(9)), EALIAS),
    (dict(h_bf16=_fake(5)), EALIAS),
    (dict(n_kv=4), EARG), (dict(n_kv=24), EARG), (dict(n_kv=16, g=None), ENULL),
    (dict(n_kv=32, B=0), ESHAPE), (dict(n_kv=16, start_pos=1024), ERANGE),
    (dict(n_kv=32, ws_bytes=4096), EWS), (dict(n_kv=16, h=_fake(10)), EALIAS),
    (dict(n_kv=32, B=2, start_pos=600, schedule=FUSED), EARG),
])
def test_layer_decode_rejects_bad_arguments(kw, code):
    assert G.lib().gqa_layer_decode(*_layer_decode_args(**kw)) == code


_LAYER_PREFILL_KEYS = ("x", "g", "eps", "wq", "wk", "wv", "wo", "wo16", "kc", "vc", "n_kv",
                       "T_max", "rope", "start_pos", "B", "T", "h", "ws", "ws_bytes", "probe",
                       "stream")


@pytest.mark.parametrize("kw,code", [
    (dict(n_kv=4), EARG), (dict(n_kv=24), EARG),
    (dict(x=None), ENULL), (dict(n_kv=32, T=0), ESHAPE), (dict(n_kv=16, start_pos=1020), ERANGE),
    (dict(ws_bytes=4096), EWS), (dict(h=_fake(9)), EALIAS), (dict(h=_fake(0)), EALIAS),
    (dict(eps=ctypes.c_float(2.0)), EARG),
])
def test_layer_prefill_rejects_bad_arguments(kw, code):
    a = dict(x=_fake(0), g=_fake(10), eps=ctypes.c_float(1e-5), wq=_fake(1), wk=_fake(2),
             wv=_fake(3), wo=_fake(4), wo16=None, kc=_fake(5), vc=_fake(6), n_kv=8, T_max=1024,
             rope=_fake(7), start_pos=0, B=1, T=8, h=_fake(8), ws=_fake(9), ws_bytes=1 << 40,
             probe=None, stream=None)
    a.update(kw)
    assert G.lib().gqa_layer_prefill(*[a[k] for k in _LAYER_PREFILL_KEYS]) == code


def _vocab_args(**kw):
    a = dict(h=_fake(0), g=None, eps=ctypes.c_float(1e-5), w=_fake(1), V=128256, B=1,
             logits=_fake(2), ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return [a[k] for k in ("h", "g", "eps", "w", "V", "B", "logits", "ws", "ws_bytes", "stream")]


def _vocab_ws(B):
    return G.workspace_bytes(G.OP_VOCAB, B, 1)


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), ENULL), (dict(w=None), ENULL), (dict(logits=None), ENULL),
    (dict(B=0), ESHAPE), (dict(V=0), ESHAPE), (dict(V=(1 << 20) + 1), ESHAPE),
    (dict(logits=ctypes.c_void_p(BASE + (2 << 32) + 4)), EALIGN),
    (dict(g=_fake(3), eps=ctypes.c_float(-1.0)), EARG),
    (dict(logits=_fake(1)), EALIAS), (dict(logits=_fake(0)), EALIAS),
    # from GQA_VOCAB_MFMA_MIN_B sequences on, with a norm, the normalised
    # tokens need the workspace
    (dict(B=6, g=_fake(3)), EWS), (dict(B=9, g=_fake(3)), EWS),
    (dict(B=9, g=_fake(3), ws=_fake(4), ws_bytes=_vocab_ws(9) - 1), EWS),
    (dict(B=9, g=_fake(3), ws=ctypes.c_void_p(BASE + (4 << 32) + 8), ws_bytes=_vocab_ws(9)), EALIGN),
    (dict(B=9, g=_fake(3), ws=ctypes.c_void_p(BASE - G.SYNC_BYTES), ws_bytes=_vocab_ws(9)), EALIAS),
    (dict(B=9, g=_fake(3), ws=ctypes.c_void_p(BASE + (2 << 32) - (G.SYNC_BYTES + 4096)),
          ws_bytes=_vocab_ws(9)), EALIAS),
])
def test_vocab_logits_rejects_bad_arguments(kw, code):
    assert G.lib().gqa_vocab_logits(*_vocab_args(**kw)) == code


def test_vocab_workspace_size():
    """The synchronisation region, then the normalised tokens (B x 4096 bf16,
    256-byte aligned); the size depends on B alone."""
    for B in (1, 9, 64, 1024):
        assert _vocab_ws(B) == G.SYNC_BYTES + (B * 4096 * 2 + 255) // 256 * 256
    assert G.workspace_bytes(G.OP_VOCAB, 9, 1) == G.workspace_bytes(G.OP_VOCAB, 9, 4096, T=7, n_kv_heads=32)


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


def test_library_has_no_unresolved_symbols_of_its_own():
    # a kernel whose host-side launch stub failed to instantiate shows up as
    # an undefined gqa:: symbol; loading the library lazily would not notice
    out = subprocess.run(["nm", "-D", "--undefined-only", "-C", GB.LIB_PATH], capture_output=True,
                         text=True).stdout
    mine = [l for l in out.splitlines() if "gqa::" in l or "gqa_" in l]
    assert mine == [], mine
