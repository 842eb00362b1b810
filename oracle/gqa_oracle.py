"""Plain fp64 CPU oracle for one Llama-3.1-8B grouped-query attention block.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this module imports nothing from the product path.

What it computes is the plain definition of the block as the model-atlas pages
state it (no blocking, no online softmax, no split merge):

  * page "Llama 3.1 8B . Query projection": Q = x W_Q with the weight stored
    [out, in] (F.linear computes x A^T), no bias;
  * page "Llama 3.1 8B . Grouped-query attention" (decode, P = 1,000):
      - evidence "qkv": separate bias-free Q/K/V projections, viewed as
        heads with feature f -> (head f // 128, dim f % 128);
      - evidence "rope": adjacent element pairs (2i, 2i+1) of Q and K form a
        complex number that is multiplied by the position's rotation;
      - header "state": the KV cache gets row start_pos written and rows
        0..start_pos read;
      - evidence "gqa": KV head g serves query heads 4g..4g+3
        (repeat_interleave over the head axis);
      - evidence "scores": Q K^T / sqrt(head_dim), causal mask where key j is
        hidden from query row i iff j > start_pos + i, softmax over keys;
      - evidence "retrieval": P V, heads merged back to feature h*128 + d, then
        the bias-free output projection wo gives Delta_attn.

Readings taken where the pages are silent (each also listed in the design
notes of the repository):

  * Rounding: everything is fp64 except the KV cache, which the pages size
    as 16-bit ("In numbers": 2 bytes per element).  New K/V rows are rounded
    to bf16 (round to nearest even) when appended, and attention reads the
    appended rows back from the cache, i.e. in their rounded form.
  * RoPE frequencies: f_i = theta ** (-2i / head_dim).  With ``scaled`` the
    Llama 3.1 long-context wavelength rule is applied (scale 8, low-frequency
    factor 1, high-frequency factor 4, original context 8192).  The pages cite
    but do not print that rule, so its constants are "parity unpinned";
    only its shape (continuity, limits) is pinned by the tests.
  * Pre-norm (``rms_norm``, ``gqa_layer``): the page constructs
    attention_norm = RMSNorm(dim, eps=norm_eps) (norm_eps 1e-5 in the
    catalogue entry) and adds the attention's update to x, but does not print
    the norm's body.  It is read as the standard root-mean-square norm with a
    per-feature gain, x / sqrt(mean(x^2) + eps) * g, and its output is
    rounded once to bf16 because the block consumes bf16 input.
  * Cache layout: the oracle's logical cache is [B][position][kv_head][dim]
    (the keys comment in evidence "gqa" indexes keys by batch, position,
    head, dim).  How the GPU lays it out in memory is not the oracle's concern.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Llama 3.1 8B attention shapes (page "Query projection", catalogue entry
# arch_args: dim 4096, n_heads 32, n_kv_heads 8, rope_theta 500000.0).
D_MODEL = 4096
N_HEADS = 32
N_KV_HEADS = 8
HEAD_DIM = D_MODEL // N_HEADS
ROPE_THETA = 500000.0

# Llama 3.1 scaled-RoPE rule constants (Meta's public release; not printed on
# the pages, hence unpinned).
SCALE_FACTOR = 8.0
LOW_FREQ_FACTOR = 1.0
HIGH_FREQ_FACTOR = 4.0
OLD_CONTEXT_LEN = 8192.0


# --------------------------------------------------------------------------
# Sizes printed on the pages
# --------------------------------------------------------------------------

def weight_shapes(d_model: int = D_MODEL, n_heads: int = N_HEADS,
                  n_kv_heads: int = N_KV_HEADS) -> dict:
    """[out, in] weight shapes of the block (page "Query projection": the
    module holds the weight output by input; page "Grouped-query attention",
    Parameters table: wk/wv are 4,096 x (8 x 128))."""
    hd = d_model // n_heads
    return {
        "wq": (n_heads * hd, d_model),
        "wk": (n_kv_heads * hd, d_model),
        "wv": (n_kv_heads * hd, d_model),
        "wo": (d_model, n_heads * hd),
    }


def parameter_counts(d_model: int = D_MODEL, n_heads: int = N_HEADS,
                     n_kv_heads: int = N_KV_HEADS) -> dict:
    """Element counts of the block's weights and their total (Parameters
    table of page "Grouped-query attention")."""
    shapes = weight_shapes(d_model, n_heads, n_kv_heads)
    counts = {k: int(np.prod(v)) for k, v in shapes.items()}
    counts["total"] = sum(counts.values())
    return counts


def kv_cache_bytes_per_token(n_layers: int = 32, n_kv_heads: int = N_KV_HEADS,
                             head_dim: int = HEAD_DIM, elem_bytes: int = 2) -> int:
    """K and V rows of every layer for one position ("In numbers" on page
    "Grouped-query attention": 2 (K, V) x layers x kv heads x dim x bytes)."""
    return 2 * n_layers * n_kv_heads * head_dim * elem_bytes


# --------------------------------------------------------------------------
# bf16 rounding (the cache is 16-bit)
# --------------------------------------------------------------------------

def bf16_bits_from_f64(a) -> np.ndarray:
    """Round fp64 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns.

    bf16 keeps 8 significant bits, so for normal numbers the rounding point in
    an fp64 significand is bit 45.  The value rounded there is exactly
    representable in fp32, whose upper 16 bits are then the bf16 pattern.
    Values below the fp32 normal range (never produced by the block at its
    magnitudes) are rounded through fp32 instead.
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    bits = a.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    r64 = rounded.view(np.float64)
    r32 = r64.astype(np.float32)
    out = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    tiny = np.abs(a) < 2.0 ** -126
    if np.any(tiny):
        t32 = a[tiny].astype(np.float32).view(np.uint32)
        t_lsb = (t32 >> np.uint32(16)) & np.uint32(1)
        out[tiny] = ((t32 + np.uint32(0x7FFF) + t_lsb) >> np.uint32(16)).astype(np.uint16)
    return out


def f64_from_bf16_bits(bits) -> np.ndarray:
    """Exact value of bf16 patterns, in fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def rope_inv_freq(head_dim: int = HEAD_DIM, theta: float = ROPE_THETA,
                  scaled: bool = True) -> np.ndarray:
    """Per-pair angular frequency f_i, i < head_dim/2, in fp64.

    Unscaled (Llama 3, page "Attention update", use_scaled_rope False):
    f_i = theta^(-2i/head_dim).  Scaled (Llama 3.1, use_scaled_rope True):
    wavelengths 2*pi/f shorter than OLD_CONTEXT_LEN/HIGH_FREQ_FACTOR keep f,
    longer than OLD_CONTEXT_LEN/LOW_FREQ_FACTOR use f/SCALE_FACTOR, and in
    between f is blended linearly in OLD_CONTEXT_LEN/wavelength.
    """
    i = np.arange(head_dim // 2, dtype=np.float64)
    f = np.power(float(theta), -2.0 * i / head_dim)
    if not scaled:
        return f
    wavelen = 2.0 * math.pi / f
    short_edge = OLD_CONTEXT_LEN / HIGH_FREQ_FACTOR
    long_edge = OLD_CONTEXT_LEN / LOW_FREQ_FACTOR
    blend = (OLD_CONTEXT_LEN / wavelen - LOW_FREQ_FACTOR) / (HIGH_FREQ_FACTOR - LOW_FREQ_FACTOR)
    mid = (1.0 - blend) * f / SCALE_FACTOR + blend * f
    return np.where(wavelen < short_edge, f,
                    np.where(wavelen > long_edge, f / SCALE_FACTOR, mid))


def rope_cos_sin(positions, head_dim: int = HEAD_DIM, theta: float = ROPE_THETA,
                 scaled: bool = True):
    """cos and sin of the angle position * f_i, shape [len(positions), head_dim/2],
    all in fp64 (the table R [positions, 64 pairs] of page "Grouped-query
    attention")."""
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    ang = pos * rope_inv_freq(head_dim, theta, scaled).reshape(1, -1)
    return np.cos(ang), np.sin(ang)


def apply_rope(z: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (z[2i], z[2i+1]) by the angle whose cos/sin are
    given (evidence "rope": the pair is a complex number multiplied by the
    rotation).  z: [..., T, heads, head_dim]; cos/sin: [T, head_dim/2]."""
    a = z[..., 0::2]
    b = z[..., 1::2]
    c = cos[:, None, :]
    s = sin[:, None, :]
    out = np.empty_like(z)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# --------------------------------------------------------------------------
# Attention pieces
# --------------------------------------------------------------------------

def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """exp(s - max) / sum exp(s - max) along ``axis``; -inf entries get 0."""
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def causal_visible(T: int, start_pos: int) -> np.ndarray:
    """Boolean [T, start_pos + T]: query row i sees key j iff j <= start_pos + i
    (the mask comment in evidence "scores")."""
    i = np.arange(T).reshape(-1, 1)
    j = np.arange(start_pos + T).reshape(1, -1)
    return j <= start_pos + i


def kv_head_of(h: int, n_heads: int, n_kv_heads: int) -> int:
    """KV head serving query head h: repeat_interleave over the head axis
    (evidence "gqa": keys are expanded with a new axis after the kv-head
    axis, so copies of one kv head sit next to each other)."""
    return h // (n_heads // n_kv_heads)


@dataclass
class BlockResult:
    delta: np.ndarray      # [B, T, d_model] fp64, Delta_attn
    q: np.ndarray          # [B, T, n_heads, hd] fp64, after RoPE
    k: np.ndarray          # [B, T, n_kv_heads, hd] fp64, after RoPE, before rounding
    v: np.ndarray          # [B, T, n_kv_heads, hd] fp64, before rounding
    k_bits: np.ndarray     # [B, T, n_kv_heads, hd] uint16, the appended cache rows
    v_bits: np.ndarray     # [B, T, n_kv_heads, hd] uint16
    attn_out: np.ndarray   # [B, T, n_heads * hd] fp64, merged heads before wo
    probs: list | None = None  # per b: [n_heads, T, start_pos + T] when asked


def gqa_block(x, wq, wk, wv, wo, k_cached, v_cached, start_pos: int,
              theta: float = ROPE_THETA, scaled: bool = True,
              n_heads: int = N_HEADS, n_kv_heads: int = N_KV_HEADS,
              keep_probs: bool = False) -> BlockResult:
    """One attention block over T new tokens per sequence.

    x:        [B, T, d] bf16 values (any float dtype; promoted to fp64)
    wq, wk, wv, wo: [out, in] weights (bf16 values)
    k_cached, v_cached: [B, start_pos, n_kv_heads, hd], the cache rows
              0..start_pos-1 before the call (ignored when start_pos == 0)
    Returns Delta_attn and the intermediate tensors (see BlockResult).
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, d = x.shape
    hd = d // n_heads
    wq = np.asarray(wq, dtype=np.float64)
    wk = np.asarray(wk, dtype=np.float64)
    wv = np.asarray(wv, dtype=np.float64)
    wo = np.asarray(wo, dtype=np.float64)

    # Projections: F.linear(x, W) = x W^T, weights [out, in].
    q = (x @ wq.T).reshape(B, T, n_heads, hd)
    k = (x @ wk.T).reshape(B, T, n_kv_heads, hd)
    v = (x @ wv.T).reshape(B, T, n_kv_heads, hd)

    # RoPE on Q and K at positions start_pos .. start_pos + T - 1.
    cos, sin = rope_cos_sin(np.arange(start_pos, start_pos + T), hd, theta, scaled)
    q = apply_rope(q, cos, sin)
    k = apply_rope(k, cos, sin)

    # Append to the 16-bit cache, then read keys/values back from it.
    k_bits = bf16_bits_from_f64(k)
    v_bits = bf16_bits_from_f64(v)
    k_new = f64_from_bf16_bits(k_bits)
    v_new = f64_from_bf16_bits(v_bits)

    L = start_pos + T
    visible = causal_visible(T, start_pos)
    scale = 1.0 / math.sqrt(hd)
    attn = np.empty((B, T, n_heads, hd), dtype=np.float64)
    probs_all = [] if keep_probs else None
    for b in range(B):
        if start_pos > 0:
            keys_b = np.concatenate(
                [np.asarray(k_cached[b, :start_pos], dtype=np.float64), k_new[b]], axis=0)
            vals_b = np.concatenate(
                [np.asarray(v_cached[b, :start_pos], dtype=np.float64), v_new[b]], axis=0)
        else:
            keys_b, vals_b = k_new[b], v_new[b]
        probs_b = np.empty((n_heads, T, L)) if keep_probs else None
        for h in range(n_heads):
            g = kv_head_of(h, n_heads, n_kv_heads)
            s = (q[b, :, h, :] @ keys_b[:, g, :].T) * scale      # [T, L]
            s = np.where(visible, s, -np.inf)
            p = softmax(s, axis=-1)
            attn[b, :, h, :] = p @ vals_b[:, g, :]
            if keep_probs:
                probs_b[h] = p
        if keep_probs:
            probs_all.append(probs_b)

    merged = attn.reshape(B, T, n_heads * hd)     # feature = h * hd + dim
    delta = merged @ wo.T
    return BlockResult(delta=delta, q=q, k=k, v=v, k_bits=k_bits, v_bits=v_bits,
                       attn_out=merged, probs=probs_all)


def stacked_decode(x_bits_first, weights, k_cached_list, v_cached_list, start_pos: int,
                   theta: float = ROPE_THETA, scaled: bool = True,
                   n_heads: int = N_HEADS, n_kv_heads: int = N_KV_HEADS):
    """Decode one token through a stack of attention blocks with the residual
    stream h_{l+1} = h_l + Delta_l(bf16(h_l)) and no norms or FFN (the layer
    loop of page "Vocabulary projection" and the block residual of evidence
    "handoff", read without RMSNorm and without the feed-forward half).

    x_bits_first: [B, d] fp64 values of the first block's input (bf16 values)
    weights: list of (wq, wk, wv, wo) per block
    k_cached_list/v_cached_list: per block [B, start_pos, kv, hd]
    Returns the final fp64 residual h [B, d] and the per-block Delta list.
    """
    h = np.asarray(x_bits_first, dtype=np.float64)
    deltas = []
    for (wq, wk, wv, wo), kc, vc in zip(weights, k_cached_list, v_cached_list):
        x_in = f64_from_bf16_bits(bf16_bits_from_f64(h))
        res = gqa_block(x_in[:, None, :], wq, wk, wv, wo, kc, vc, start_pos, theta, scaled,
                        n_heads, n_kv_heads)
        d = res.delta[:, 0, :]
        deltas.append(d)
        h = h + d
    return h, deltas


def rms_norm(x, g, eps: float) -> np.ndarray:
    """Root-mean-square norm over the last axis with gain g:
    x / sqrt(mean(x^2) + eps) * g (the reading of attention_norm above)."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def gqa_layer(x, norm_w, eps: float, wq, wk, wv, wo, k_cached, v_cached, start_pos: int,
              theta: float = ROPE_THETA, scaled: bool = True,
              n_heads: int = N_HEADS, n_kv_heads: int = N_KV_HEADS):
    """The block inside its residual branch (page "Llama 3.1 8B . Grouped-query
    attention", code section: h = x + attention(attention_norm(x), ...)).

    x: [B, T, d] bf16 values; norm_w: [d] bf16 values.  The normalised input
    is rounded to bf16 (the block's input dtype) before the block.
    Returns (h [B, T, d] fp64, the block's BlockResult).
    """
    x = np.asarray(x, dtype=np.float64)
    xn = f64_from_bf16_bits(bf16_bits_from_f64(rms_norm(x, norm_w, eps)))
    res = gqa_block(xn, wq, wk, wv, wo, k_cached, v_cached, start_pos, theta, scaled,
                    n_heads, n_kv_heads)
    return x + res.delta, res


def vocab_logits(h, w_out, norm_w=None, eps: float = 1e-5) -> np.ndarray:
    """Page "Llama 3.1 8B . Vocabulary projection": L = z W_out with the
    weight stored [out, in] (F.linear, no bias), z the final norm of h (the
    page's code applies self.norm first; read as ``rms_norm`` with its output
    rounded to bf16) or h itself when no gain is given.  The projection's
    output is in the model's bf16 and is cast to float32 on return, so each
    logit is the bf16 rounding of the exact dot product.

    h: [B, d] bf16 values; w_out: [V, d] bf16 values.  Returns [B, V] fp64
    holding bf16 values.
    """
    h = np.asarray(h, dtype=np.float64)
    z = h if norm_w is None else f64_from_bf16_bits(bf16_bits_from_f64(rms_norm(h, norm_w, eps)))
    return f64_from_bf16_bits(bf16_bits_from_f64(z @ np.asarray(w_out, dtype=np.float64).T))
