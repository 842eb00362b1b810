"""Seeded synthetic inputs for the attention block.

Holds no arithmetic of the method: only random draws, rounding of the draws
to bf16 (the inputs' storage type) and a NaN sentinel for cache rows that a
call must neither read nor write.  Both the tests (for the oracle and the
GPU path) and the benchmark take their inputs from here.

Recipe: ``torch.randn`` in fp32 times a scale, rounded to bf16; one
``torch.Generator`` seeded per workload; draws in the order x, Wq, Wk, Wv,
Wo, K cache, V cache.  Scales: x 1, weights 0.02, cache rows 1.
"""
from __future__ import annotations

import torch

D_MODEL = 4096
N_HEADS = 32
N_KV_HEADS = 8
HEAD_DIM = 128
WEIGHT_STD = 0.02
# a quiet-NaN bf16 pattern that no draw produces; marks cache rows that must
# stay untouched
SENTINEL_BITS = 0x7FA1


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn_bf16(gen: torch.Generator, shape, scale: float = 1.0, device="cpu") -> torch.Tensor:
    """N(0, scale^2) drawn in fp32 and stored as bf16."""
    t = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(torch.bfloat16)


def fill_randn_bf16_(dst: torch.Tensor, gen: torch.Generator, scale: float = 1.0,
                     chunk_elems: int = 1 << 28) -> torch.Tensor:
    """Fill a large contiguous bf16 tensor with N(0, scale^2) draws in chunks
    (for caches too large to draw in fp32 at once)."""
    flat = dst.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        tmp = torch.randn(e - s, generator=gen, dtype=torch.float32, device=dst.device)
        if scale != 1.0:
            tmp.mul_(scale)
        flat[s:e].copy_(tmp)
        del tmp
    return dst


def block_weights(gen: torch.Generator, device="cpu", n_kv_heads: int = N_KV_HEADS):
    """(Wq, Wk, Wv, Wo), [out, in] bf16, N(0, 0.02^2), drawn on ``device``
    (which must be the generator's device)."""
    wq = randn_bf16(gen, (N_HEADS * HEAD_DIM, D_MODEL), WEIGHT_STD, device)
    wk = randn_bf16(gen, (n_kv_heads * HEAD_DIM, D_MODEL), WEIGHT_STD, device)
    wv = randn_bf16(gen, (n_kv_heads * HEAD_DIM, D_MODEL), WEIGHT_STD, device)
    wo = randn_bf16(gen, (D_MODEL, N_HEADS * HEAD_DIM), WEIGHT_STD, device)
    return wq, wk, wv, wo


def sentinel_like(shape, device="cpu") -> torch.Tensor:
    """bf16 tensor whose every element holds the sentinel NaN pattern."""
    return torch.full(shape, SENTINEL_BITS, dtype=torch.int16, device=device).view(torch.bfloat16)


def cache_rows(gen: torch.Generator, B: int, P: int, device="cpu", n_kv_heads: int = N_KV_HEADS):
    """Logical cache rows [B, P, n_kv, 128] for K then V, bf16 N(0, 1)."""
    k = randn_bf16(gen, (B, P, n_kv_heads, HEAD_DIM), 1.0, device)
    v = randn_bf16(gen, (B, P, n_kv_heads, HEAD_DIM), 1.0, device)
    return k, v


def decode_workload(seed: int, B: int, P: int, device="cpu", n_kv_heads: int = N_KV_HEADS):
    """x [B, 4096], weights, and cached rows [B, P, n_kv, 128] for K and V
    (n_kv key/value heads, 8 for Llama 3.1 8B)."""
    gen = generator(seed, device)
    x = randn_bf16(gen, (B, D_MODEL), 1.0, device)
    w = block_weights(gen, device, n_kv_heads)
    k, v = cache_rows(gen, B, P, device, n_kv_heads)
    return x, w, k, v


def prefill_workload(seed: int, B: int, T: int, device="cpu", n_kv_heads: int = N_KV_HEADS):
    """x [B, T, 4096] and weights."""
    gen = generator(seed, device)
    x = randn_bf16(gen, (B, T, D_MODEL), 1.0, device)
    w = block_weights(gen, device, n_kv_heads)
    return x, w


def chunked_prefill_workload(seed: int, B: int, start_pos: int, T: int, device="cpu",
                             n_kv_heads: int = N_KV_HEADS):
    """x [B, T, 4096], weights, and cached rows [B, start_pos, n_kv, 128] for
    K and V (the keys and values of the earlier chunk)."""
    gen = generator(seed, device)
    x = randn_bf16(gen, (B, T, D_MODEL), 1.0, device)
    w = block_weights(gen, device, n_kv_heads)
    k, v = cache_rows(gen, B, start_pos, device, n_kv_heads)
    return x, w, k, v


def norm_gain(seed: int, device="cpu") -> torch.Tensor:
    """bf16 [4096] gain of a pre-norm: 1 + N(0, 0.1^2)."""
    gen = generator(seed, device)
    g = 1.0 + 0.1 * torch.randn((D_MODEL,), generator=gen, dtype=torch.float32, device=device)
    return g.to(torch.bfloat16)
