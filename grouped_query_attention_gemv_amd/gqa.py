"""Python binding of libgqa.so: argument marshalling only.

Every function checks dtypes, devices, shapes and contiguity of the torch
tensors it is given, then passes raw device pointers and the current HIP
stream to the C ABI declared in ``include/gqa.h``.  All computation happens
in the library's kernels; if the library is missing or fails to load, calls
raise instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import torch

D_MODEL = 4096
N_HEADS = 32
N_KV_HEADS = 8
KV_HEAD_COUNTS = (8, 16, 32)   # key/value head counts the block entry points take
HEAD_DIM = 128
QKV_DIM = 6144
ROPE_PAIRS = 64
V_BLOCK = 32
DECODE_STAGES = 3
PREFILL_STAGES = 4
SYNC_BYTES = 540672
VOCAB_MFMA_MIN_B = 6   # gqa_vocab_logits: matrix cores (and, with a norm, a workspace) from here
NOALLOC_SCRATCH_BYTES = 16 << 20   # the no-allocation decode's scratch array per GPU
DECODE_AUTO, DECODE_SPLIT, DECODE_FUSED = 0, 1, 2
OP_PREFILL, OP_DECODE, OP_LAYER_PREFILL, OP_LAYER_DECODE, OP_VOCAB = 0, 1, 2, 3, 4
# bits of the workspace error word
WS_ERR_WAIT, WS_ERR_WO_WAIT, WS_ERR_INIT, WS_ERR_FP16_RANGE = 0x1, 0x2, 0x4, 0x100
WS_MAGIC = 0x31415147

# With GQA_DEBUG=1 in the environment every block and layer call synchronises
# and raises if its workspace's error word is nonzero.
DEBUG = os.environ.get("GQA_DEBUG", "") == "1"

_HERE = os.path.dirname(os.path.abspath(__file__))
# GQA_LIB names another build of the same library (the host-sanitizer build
# of the tests); by default the in-tree libgqa.so is loaded
LIB_PATH = os.environ.get("GQA_LIB") or os.path.join(_HERE, "libgqa.so")

STATUS = {
    0: "GQA_OK", -1: "GQA_ERR_NULL", -2: "GQA_ERR_SHAPE", -3: "GQA_ERR_RANGE",
    -4: "GQA_ERR_ALIGN", -5: "GQA_ERR_WORKSPACE", -6: "GQA_ERR_HIP", -7: "GQA_ERR_ALIAS",
    -8: "GQA_ERR_ARG",
}

# exported entry points and their C signatures
_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_F = ctypes.c_float
_SIGS = {
    "gqa_status_string": (ctypes.c_char_p, [_I]),
    "gqa_rope_table": (_I, [_I, ctypes.c_double, _I, _P, _P]),
    "gqa_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I]),
    "gqa_workspace_init": (_I, [_P, _Z, _P]),
    "gqa_decode_schedule": (_I, [_I, _I, _I, _I, _I]),
    "gqa_wo_to_fp16": (_I, [_P, _P, _P]),
    # x wq wk wv wo wo16 kc vc n_kv T_max rope start_pos B T out ws ws_bytes probe events stream
    "gqa_block_prefill": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _P, _P, _Z,
                               _P, _P, _P]),
    # x wq wk wv wo kc vc n_kv T_max rope start_pos B out out_bf16 accumulate schedule ws
    # ws_bytes probe events stream
    "gqa_block_decode": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _P, _P, _I, _I, _P,
                              _Z, _P, _P, _P]),
    # x wq wk wv wo kc vc n_kv T_max rope start_pos B out out_bf16 accumulate schedule probe
    # stream
    "gqa_block_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _P, _P,
                                      _I, _I, _P, _P]),
    # x norm_w eps wq wk wv wo wo16 kc vc n_kv T_max rope start_pos B T h ws ws_bytes probe stream
    "gqa_layer_prefill": (_I, [_P, _P, _F, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _P,
                               _P, _Z, _P, _P]),
    # x norm_w eps wq wk wv wo kc vc n_kv T_max rope start_pos B h h_bf16 schedule ws ws_bytes
    # probe stream
    "gqa_layer_decode": (_I, [_P, _P, _F, _P, _P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _P, _P, _I,
                              _P, _Z, _P, _P]),
    "gqa_vocab_logits": (_I, [_P, _P, _F, _P, _I, _I, _P, _P, _Z, _P]),
}

_lib = None


class GQAError(RuntimeError):
    """A libgqa call returned an error status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def lib() -> ctypes.CDLL:
    """Load libgqa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m grouped_query_attention_gemv_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().gqa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise GQAError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must live on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ----------------------------------------------------------------------------
# Allocation helpers (layouts of include/gqa.h)
# ----------------------------------------------------------------------------

def workspace_bytes(op: int, B: int, T_max: int, T: int = 1, start_pos: int = 0,
                    n_kv_heads: int = N_KV_HEADS) -> int:
    """Scratch bytes of one call of operation ``op`` (OP_PREFILL, OP_DECODE,
    OP_LAYER_PREFILL, OP_LAYER_DECODE, OP_VOCAB); 0 for arguments out of range."""
    return int(lib().gqa_workspace_bytes(int(op), int(n_kv_heads), int(B), int(start_pos),
                                         int(T), int(T_max)))


def workspace(op: int, B: int, T_max: int, device, T: int = 1, start_pos: int = 0,
              n_kv_heads: int = N_KV_HEADS) -> torch.Tensor:
    """A workspace for one call of operation ``op`` with these arguments,
    initialised (gqa_workspace_init) on the current stream."""
    n = workspace_bytes(op, B, T_max, T, start_pos, n_kv_heads)
    if n == 0:
        raise ValueError(f"no workspace size for op={op}, B={B}, start_pos={start_pos}, T={T}, "
                         f"T_max={T_max}, n_kv_heads={n_kv_heads}")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


def workspace_init(ws: torch.Tensor) -> None:
    """Zero the synchronisation words, write the magic word and mark the
    one-launch decode's hand-off buffers empty (again, e.g. after the error
    word turned nonzero)."""
    _check(lib().gqa_workspace_init(_ptr(ws), ws.numel(), _stream(ws.device)),
           "gqa_workspace_init")


def workspace_errors(ws: torch.Tensor) -> int:
    """The workspace's sticky error word (WS_ERR_* bits).  Synchronises with
    the device."""
    return int(ws[:4].view(torch.int32).item())


def workspace_off_home(ws: torch.Tensor) -> int:
    """One-launch decodes since the workspace was initialised whose
    workgroups the dispatcher did not place on their kv head's XCD (their
    hand-off reads then miss the shared L2 line; results are unaffected: a
    performance diagnostic, not an error).  Synchronises."""
    return int(ws[8:12].view(torch.int32).item())


def _debug_check(ws: torch.Tensor, where: str):
    if DEBUG:
        err = workspace_errors(ws)
        if err:
            raise RuntimeError(f"{where}: workspace error word {err:#x}")


def decode_schedule(B: int, start_pos: int, T_max: int, n_kv_heads: int = N_KV_HEADS,
                    schedule: int = DECODE_AUTO) -> int:
    """The schedule (DECODE_SPLIT or DECODE_FUSED) a decode call of this shape
    runs when it asks for ``schedule``."""
    r = int(lib().gqa_decode_schedule(int(n_kv_heads), int(B), int(start_pos), int(T_max),
                                      int(schedule)))
    if r < 0:
        raise GQAError(r, "gqa_decode_schedule")
    return r


def empty_caches(B: int, T_max: int, device, n_kv_heads: int = N_KV_HEADS):
    """(kcache [B, n_kv, T_max, 128], vcache [B, n_kv, T_max/32, 128, 32])
    bf16, uninitialised; T_max must be a multiple of 32; n_kv defaults to
    Llama 3.1 8B's 8 key/value heads."""
    if T_max % V_BLOCK:
        raise ValueError(f"T_max must be a multiple of {V_BLOCK}")
    k = torch.empty((B, n_kv_heads, T_max, HEAD_DIM), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, n_kv_heads, T_max // V_BLOCK, HEAD_DIM, V_BLOCK), dtype=torch.bfloat16,
                    device=device)
    return k, v


def kcache_by_position(kcache: torch.Tensor) -> torch.Tensor:
    """View [B, T_max, n_kv, 128] of the head-major key cache."""
    return kcache.permute(0, 2, 1, 3)


def vcache_blocks(vcache: torch.Tensor) -> torch.Tensor:
    """View [B, T_max/32, 32, n_kv, 128] of the blocked value cache: block,
    position within the block, kv head, dim."""
    return vcache.permute(0, 2, 4, 1, 3)


def _block_pieces(lo: int, hi: int):
    """Split positions [lo, hi) into (block, first, last) pieces of 32-blocks."""
    pos = lo
    while pos < hi:
        blk, r0 = divmod(pos, V_BLOCK)
        r1 = min(V_BLOCK, r0 + hi - pos)
        yield blk, r0, r1
        pos += r1 - r0


def vcache_read(vcache: torch.Tensor, lo: int, hi: int) -> torch.Tensor:
    """Copy of value rows [lo, hi) as [B, hi - lo, n_kv, 128]."""
    v5 = vcache_blocks(vcache)
    return torch.cat([v5[:, b, r0:r1] for b, r0, r1 in _block_pieces(lo, hi)], dim=1)


def vcache_write(vcache: torch.Tensor, lo: int, rows: torch.Tensor) -> None:
    """Store rows [B, n, n_kv, 128] at positions lo .. lo + n - 1."""
    v5 = vcache_blocks(vcache)
    off = 0
    n = rows.shape[1]
    first_full = -(-lo // V_BLOCK)
    last_full = (lo + n) // V_BLOCK
    for b, r0, r1 in _block_pieces(lo, lo + n):
        if first_full <= b < last_full and r0 == 0 and r1 == V_BLOCK:
            if b == first_full:   # all full blocks in one strided copy
                nb = last_full - first_full
                v5[:, b:b + nb] = rows[:, off:off + nb * V_BLOCK].reshape(
                    rows.shape[0], nb, V_BLOCK, rows.shape[2], HEAD_DIM)
                off += nb * V_BLOCK
            continue
        v5[:, b, r0:r1] = rows[:, off:off + r1 - r0]
        off += r1 - r0


class HipEvents:
    """A set of HIP events created through the HIP runtime, for the
    *_profiled entry points."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                  ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events[i] = h
        self.n = n

    def elapsed_ms(self, i: int, j: int) -> float:
        """Milliseconds between events i and j (synchronises on j)."""
        if self._hip.hipEventSynchronize(self.events[j]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.events[i], self.events[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for i in range(self.n):
            if self.events[i]:
                self._hip.hipEventDestroy(self.events[i])
                self.events[i] = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------------------
# Entry points
# ----------------------------------------------------------------------------

def rope_table(T_max: int, theta: float = 500000.0, scaled: bool = True, device="cuda",
               out: torch.Tensor | None = None) -> torch.Tensor:
    """[T_max, 64, 2] fp32 (cos, sin) table on ``device``."""
    device = torch.device(device)
    if out is None:
        out = torch.empty((T_max, ROPE_PAIRS, 2), dtype=torch.float32, device=device)
    _need(out, "rope", torch.float32, (T_max, ROPE_PAIRS, 2), out.device)
    _check(lib().gqa_rope_table(int(T_max), float(theta), int(bool(scaled)), _ptr(out),
                                _stream(out.device)), "gqa_rope_table")
    return out


def _check_block(x, wq, wk, wv, wo, kcache, vcache, rope, kv_heads=KV_HEAD_COUNTS):
    """Validate the weights, caches and rope table; the number of key/value
    heads comes from wk's rows and must be one of kv_heads.  wo may be None
    when a prefill gets its fp16 copy instead."""
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    if wk.dim() != 2 or wk.shape[0] % HEAD_DIM or wk.shape[0] // HEAD_DIM not in kv_heads:
        raise ValueError(f"wk must be [n_kv*128, 4096] with n_kv in {tuple(kv_heads)}")
    n_kv = wk.shape[0] // HEAD_DIM
    _need(wq, "wq", torch.bfloat16, (D_MODEL, D_MODEL), dev)
    _need(wk, "wk", torch.bfloat16, (n_kv * HEAD_DIM, D_MODEL), dev)
    _need(wv, "wv", torch.bfloat16, (n_kv * HEAD_DIM, D_MODEL), dev)
    if wo is not None:
        _need(wo, "wo", torch.bfloat16, (D_MODEL, D_MODEL), dev)
    if kcache.dim() != 4:
        raise ValueError(f"kcache must be [B, {n_kv}, T_max, 128]")
    B, T_max = kcache.shape[0], kcache.shape[2]
    _need(kcache, "kcache", torch.bfloat16, (B, n_kv, T_max, HEAD_DIM), dev)
    _need(vcache, "vcache", torch.bfloat16,
          (B, n_kv, T_max // V_BLOCK, HEAD_DIM, V_BLOCK), dev)
    if rope.dim() != 3 or rope.shape[0] < T_max:
        raise ValueError("rope must be [>= T_max, 64, 2]")
    _need(rope, "rope", torch.float32, (rope.shape[0], ROPE_PAIRS, 2), dev)
    return dev, B, T_max, n_kv


def _events(events):
    return None if events is None else events.events


def wo_to_fp16(wo, out=None) -> torch.Tensor:
    """fp16 copy [4096, 4096] of wo for the prefill's output projection
    (gqa_wo_to_fp16; entries beyond +-65504 saturate)."""
    _need(wo, "wo", torch.bfloat16, (D_MODEL, D_MODEL), wo.device)
    if out is None:
        out = torch.empty((D_MODEL, D_MODEL), dtype=torch.float16, device=wo.device)
    _need(out, "wo16", torch.float16, (D_MODEL, D_MODEL), wo.device)
    _check(lib().gqa_wo_to_fp16(_ptr(wo), _ptr(out), _stream(wo.device)), "gqa_wo_to_fp16")
    return out


def block_prefill(x, wq, wk, wv, wo, kcache, vcache, rope, out=None, ws=None, probe=None,
                  events: HipEvents | None = None, start_pos: int = 0,
                  wo16=None) -> torch.Tensor:
    """Delta_attn [B, T, 4096] fp32 for x [B, T, 4096] bf16 at positions
    start_pos..start_pos+T-1; reads cache rows 0..start_pos-1 and writes rows
    start_pos..start_pos+T-1.  The number of key/value heads is
    wk.shape[0] / 128: 8 (Llama 3.1 8B), 16 or 32.  wo16: optional fp16 copy
    of wo from wo_to_fp16 (then wo may be None)."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, 4096]")
    dev, B, T_max, n_kv = _check_block(x, wq, wk, wv, wo, kcache, vcache, rope)
    if wo is None and wo16 is None:
        raise ValueError("wo or wo16 is needed")
    if wo16 is not None:
        _need(wo16, "wo16", torch.float16, (D_MODEL, D_MODEL), dev)
    T = x.shape[1]
    _need(x, "x", torch.bfloat16, (B, T, D_MODEL), dev)
    if out is None:
        out = torch.empty((B, T, D_MODEL), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, T, D_MODEL), dev)
    if probe is not None:
        _need(probe, "probe", torch.float32, (B, T, D_MODEL + 2 * n_kv * HEAD_DIM), dev)
    if ws is None:
        ws = workspace(OP_PREFILL, B, T_max, dev, T, start_pos, n_kv)
    _check(lib().gqa_block_prefill(
        _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(wo16), _ptr(kcache), _ptr(vcache),
        n_kv, int(T_max), _ptr(rope), int(start_pos), int(B), int(T), _ptr(out), _ptr(ws),
        ws.numel(), _ptr(probe), _events(events), _stream(dev)), "gqa_block_prefill")
    _debug_check(ws, "gqa_block_prefill")
    return out


def block_decode(x, wq, wk, wv, wo, kcache, vcache, rope, start_pos: int, out=None,
                 out_bf16=None, accumulate: bool = False, ws=None, probe=None,
                 events: HipEvents | None = None, schedule: int = DECODE_AUTO) -> torch.Tensor:
    """One token per sequence at position start_pos: x [B, 4096] bf16 ->
    out [B, 4096] fp32 (= Delta, or += Delta with accumulate).  The number of
    key/value heads is wk.shape[0] / 128: 8 (Llama 3.1 8B), 16 or 32.
    schedule: DECODE_AUTO, DECODE_SPLIT or DECODE_FUSED."""
    if x.dim() != 2:
        raise ValueError("x must be [B, 4096]")
    if wo is None:
        raise ValueError("decode needs wo")
    dev, B, T_max, n_kv = _check_block(x, wq, wk, wv, wo, kcache, vcache, rope)
    _need(x, "x", torch.bfloat16, (B, D_MODEL), dev)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty((B, D_MODEL), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, D_MODEL), dev)
    if out_bf16 is not None:
        _need(out_bf16, "out_bf16", torch.bfloat16, (B, D_MODEL), dev)
    if probe is not None:
        _need(probe, "probe", torch.float32, (B, D_MODEL + 2 * n_kv * HEAD_DIM), dev)
    if ws is None:
        ws = workspace(OP_DECODE, B, T_max, dev, n_kv_heads=n_kv)
    _check(lib().gqa_block_decode(
        _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(kcache), _ptr(vcache), n_kv,
        int(T_max), _ptr(rope), int(start_pos), int(B), _ptr(out), _ptr(out_bf16),
        int(bool(accumulate)), int(schedule), _ptr(ws), ws.numel(), _ptr(probe), _events(events),
        _stream(dev)), "gqa_block_decode")
    _debug_check(ws, "gqa_block_decode")
    return out


def block_decode_noalloc(x, wq, wk, wv, wo, kcache, vcache, rope, start_pos: int, out=None,
                         out_bf16=None, accumulate: bool = False, probe=None,
                         schedule: int = DECODE_AUTO) -> torch.Tensor:
    """block_decode with the library's own per-GPU scratch array as the
    workspace (gqa_block_decode_noalloc): no workspace argument and no device
    allocation inside the call when out is given.  Calls that overlap on one
    GPU race on the shared array."""
    if x.dim() != 2:
        raise ValueError("x must be [B, 4096]")
    if wo is None:
        raise ValueError("decode needs wo")
    dev, B, T_max, n_kv = _check_block(x, wq, wk, wv, wo, kcache, vcache, rope)
    _need(x, "x", torch.bfloat16, (B, D_MODEL), dev)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty((B, D_MODEL), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, D_MODEL), dev)
    if out_bf16 is not None:
        _need(out_bf16, "out_bf16", torch.bfloat16, (B, D_MODEL), dev)
    if probe is not None:
        _need(probe, "probe", torch.float32, (B, D_MODEL + 2 * n_kv * HEAD_DIM), dev)
    _check(lib().gqa_block_decode_noalloc(
        _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(kcache), _ptr(vcache), n_kv,
        int(T_max), _ptr(rope), int(start_pos), int(B), _ptr(out), _ptr(out_bf16),
        int(bool(accumulate)), int(schedule), _ptr(probe), _stream(dev)),
        "gqa_block_decode_noalloc")
    return out


NORM_EPS = 1e-5   # norm_eps of the Llama 3.1 8B catalogue entry
VOCAB = 128256    # vocabulary size of Llama 3


def vocab_logits(h, w_out, norm_w=None, eps: float = NORM_EPS, logits=None,
                 ws=None) -> torch.Tensor:
    """Logits [B, V] fp32 (bf16-rounded values) = z W_out^T for h [B, 4096]
    bf16, z = RMSNorm(h) * norm_w when norm_w is given, else h.  From
    VOCAB_MFMA_MIN_B sequences on, with a norm, the call needs a workspace
    (allocated here unless ``ws`` is given)."""
    if h.dim() != 2 or w_out.dim() != 2:
        raise ValueError("h must be [B, 4096] and w_out [V, 4096]")
    dev = h.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    B, V = h.shape[0], w_out.shape[0]
    _need(h, "h", torch.bfloat16, (B, D_MODEL), dev)
    _need(w_out, "w_out", torch.bfloat16, (V, D_MODEL), dev)
    if norm_w is not None:
        _need(norm_w, "norm_w", torch.bfloat16, (D_MODEL,), dev)
    if logits is None:
        logits = torch.empty((B, V), dtype=torch.float32, device=dev)
    _need(logits, "logits", torch.float32, (B, V), dev)
    if ws is None and B >= VOCAB_MFMA_MIN_B and norm_w is not None:
        ws = workspace(OP_VOCAB, B, 1, dev)
    _check(lib().gqa_vocab_logits(_ptr(h), _ptr(norm_w), float(eps), _ptr(w_out), int(V), int(B),
                                  _ptr(logits), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(dev)), "gqa_vocab_logits")
    return logits


def layer_prefill(x, norm_w, wq, wk, wv, wo, kcache, vcache, rope, start_pos: int = 0,
                  eps: float = NORM_EPS, h=None, ws=None, probe=None, wo16=None) -> torch.Tensor:
    """h = x + Delta_attn(RMSNorm(x) * norm_w) [B, T, 4096] fp32 for x
    [B, T, 4096] bf16 at positions start_pos..; the block's cache rows as in
    block_prefill.  The number of key/value heads is wk.shape[0] / 128."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, 4096]")
    dev, B, T_max, n_kv = _check_block(x, wq, wk, wv, wo, kcache, vcache, rope)
    if wo is None and wo16 is None:
        raise ValueError("wo or wo16 is needed")
    if wo16 is not None:
        _need(wo16, "wo16", torch.float16, (D_MODEL, D_MODEL), dev)
    T = x.shape[1]
    _need(x, "x", torch.bfloat16, (B, T, D_MODEL), dev)
    _need(norm_w, "norm_w", torch.bfloat16, (D_MODEL,), dev)
    if h is None:
        h = torch.empty((B, T, D_MODEL), dtype=torch.float32, device=dev)
    _need(h, "h", torch.float32, (B, T, D_MODEL), dev)
    if probe is not None:
        _need(probe, "probe", torch.float32, (B, T, D_MODEL + 2 * n_kv * HEAD_DIM), dev)
    if ws is None:
        ws = workspace(OP_LAYER_PREFILL, B, T_max, dev, T, start_pos, n_kv)
    _check(lib().gqa_layer_prefill(
        _ptr(x), _ptr(norm_w), float(eps), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(wo16),
        _ptr(kcache), _ptr(vcache), n_kv, int(T_max), _ptr(rope), int(start_pos), int(B), int(T),
        _ptr(h), _ptr(ws), ws.numel(), _ptr(probe), _stream(dev)), "gqa_layer_prefill")
    _debug_check(ws, "gqa_layer_prefill")
    return h


def layer_decode(x, norm_w, wq, wk, wv, wo, kcache, vcache, rope, start_pos: int,
                 eps: float = NORM_EPS, h=None, h_bf16=None, ws=None, probe=None,
                 schedule: int = DECODE_AUTO) -> torch.Tensor:
    """h = x + Delta_attn(RMSNorm(x) * norm_w) [B, 4096] fp32 for one token per
    sequence at start_pos; h_bf16 (optional) receives its bf16 rounding.  The
    number of key/value heads is wk.shape[0] / 128 (8, 16 or 32)."""
    if x.dim() != 2:
        raise ValueError("x must be [B, 4096]")
    if wo is None:
        raise ValueError("decode needs wo")
    dev, B, T_max, n_kv = _check_block(x, wq, wk, wv, wo, kcache, vcache, rope)
    _need(x, "x", torch.bfloat16, (B, D_MODEL), dev)
    _need(norm_w, "norm_w", torch.bfloat16, (D_MODEL,), dev)
    if h is None:
        h = torch.empty((B, D_MODEL), dtype=torch.float32, device=dev)
    _need(h, "h", torch.float32, (B, D_MODEL), dev)
    if h_bf16 is not None:
        _need(h_bf16, "h_bf16", torch.bfloat16, (B, D_MODEL), dev)
    if probe is not None:
        _need(probe, "probe", torch.float32, (B, D_MODEL + 2 * n_kv * HEAD_DIM), dev)
    if ws is None:
        ws = workspace(OP_LAYER_DECODE, B, T_max, dev, n_kv_heads=n_kv)
    _check(lib().gqa_layer_decode(
        _ptr(x), _ptr(norm_w), float(eps), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(kcache),
        _ptr(vcache), n_kv, int(T_max), _ptr(rope), int(start_pos), int(B), _ptr(h),
        _ptr(h_bf16), int(schedule), _ptr(ws), ws.numel(), _ptr(probe), _stream(dev)),
        "gqa_layer_decode")
    _debug_check(ws, "gqa_layer_decode")
    return h
