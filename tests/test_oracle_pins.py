"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a printed value of the pages, a library
routine, a closed form, an invariant or the scalar brute force, chosen so a
plausible slip in the oracle (dropped term, wrong sign or index, transposed
operand, tiled instead of interleaved heads) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import gqa_oracle as O
from tests import brute_force as BF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _bf16_vals(rng, shape, scale):
    """fp64 arrays holding bf16 values (N(0, scale^2) rounded to bf16)."""
    a = rng.standard_normal(shape) * scale
    return O.f64_from_bf16_bits(O.bf16_bits_from_f64(a))


# ----------------------------------------------------------------------------
# Printed sizes
# ----------------------------------------------------------------------------

def test_parameter_counts_match_pages():
    g = _golden()
    c = O.parameter_counts()
    assert c["wq"] == g["wq_params"]["value"]
    assert c["wk"] == g["wk_params"]["value"]
    assert c["wv"] == g["wv_params"]["value"]
    assert c["wo"] == g["wo_params"]["value"]
    assert c["total"] == g["block_params"]["value"]
    assert 32 * c["total"] == g["block_params_32_blocks"]["value"]
    assert 32 * c["wq"] == g["wq_params_32_blocks"]["value"]
    # the [out, in] orientation of each weight
    s = O.weight_shapes()
    assert s["wk"] == (8 * 128, 4096) and s["wo"] == (4096, 4096)


def test_kv_cache_sizes_match_pages():
    g = _golden()
    per_tok = O.kv_cache_bytes_per_token()
    assert per_tok == g["kv_bytes_per_token_gqa"]["value"]
    assert O.kv_cache_bytes_per_token(n_kv_heads=32) == g["kv_bytes_per_token_mha"]["value"]
    mib = per_tok * g["decode_keys_read_p1000"]["value"] / 2 ** 20
    assert round(mib, 1) == g["kv_mib_at_1001_positions"]["value"]
    assert per_tok * 131072 == g["kv_gib_at_131072_tokens"]["value"] * 2 ** 30
    assert O.kv_cache_bytes_per_token(n_kv_heads=32) * 131072 == \
        g["kv_gib_at_131072_tokens_mha"]["value"] * 2 ** 30
    assert O.HEAD_DIM // 2 == g["rope_pairs"]["value"]


# ----------------------------------------------------------------------------
# bf16 rounding
# ----------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    a32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    mine = O.bf16_bits_from_f64(a32.astype(np.float64))
    ref = torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_rounding_ties_and_direct_rounding():
    # exact ties go to even: 1 + 2^-8 lies between 1 and 1 + 2^-7
    assert O.bf16_bits_from_f64(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert O.bf16_bits_from_f64(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # slightly below a tie: must round down even though fp32 rounding would
    # first land exactly on the tie (a double-rounding trap)
    v = 1.0 + 2.0 ** -8 - 2.0 ** -40
    assert O.bf16_bits_from_f64(np.array([v]))[0] == 0x3F80
    v = 1.0 + 3 * 2.0 ** -8 - 2.0 ** -40
    assert O.bf16_bits_from_f64(np.array([v]))[0] == 0x3F81
    assert O.bf16_bits_from_f64(np.array([-2.0]))[0] == 0xC000


def test_bf16_rounding_matches_scalar_brute_force():
    rng = np.random.default_rng(2)
    a = rng.standard_normal(20000) * np.exp(rng.uniform(-10, 10, 20000))
    mine = O.f64_from_bf16_bits(O.bf16_bits_from_f64(a))
    ref = np.array([BF.bf16_round_scalar(float(v)) for v in a])
    assert np.array_equal(mine, ref)


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def test_rope_frequencies_match_transformers_llama3_rule():
    """Default and Llama-3-scaled inverse frequencies against the independent
    implementation in transformers (it works in fp32, hence 1e-6)."""
    from transformers import LlamaConfig
    from transformers import modeling_rope_utils as mru
    base = LlamaConfig(hidden_size=4096, num_attention_heads=32, num_key_value_heads=8,
                       rope_theta=500000.0, max_position_embeddings=131072)
    inv, _ = mru._compute_default_rope_parameters(base) if hasattr(
        mru, "_compute_default_rope_parameters") else (None, None)
    if inv is not None:
        r = O.rope_inv_freq(128, 500000.0, scaled=False)
        assert np.max(np.abs(r - inv.double().numpy()) / r) < 1e-6
    cfg = LlamaConfig(hidden_size=4096, num_attention_heads=32, num_key_value_heads=8,
                      rope_theta=500000.0, max_position_embeddings=131072,
                      rope_scaling={"rope_type": "llama3", "factor": 8.0,
                                    "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                                    "original_max_position_embeddings": 8192})
    inv, _ = mru._compute_llama3_parameters(cfg)
    r = O.rope_inv_freq(128, 500000.0, scaled=True)
    assert np.max(np.abs(r - inv.double().numpy()) / r) < 1e-6


def test_rope_unscaled_closed_forms():
    f = O.rope_inv_freq(128, 500000.0, scaled=False)
    assert f[0] == 1.0                                  # pair 0 turns 1 rad per position
    ratios = f[1:] / f[:-1]
    assert np.allclose(ratios, 500000.0 ** (-2.0 / 128), rtol=1e-13, atol=0)
    assert math.isclose(f[63], 500000.0 ** (-126.0 / 128), rel_tol=1e-13)


def test_scaled_rope_shape():
    """Structure of the long-context rule: the highest frequencies are kept,
    the lowest are divided by 8, the blend is continuous and monotone."""
    fs = O.rope_inv_freq(128, 500000.0, scaled=True)
    fu = O.rope_inv_freq(128, 500000.0, scaled=False)
    lam = 2 * np.pi / fu
    keep = lam < 2048.0
    div = lam > 8192.0
    assert np.array_equal(fs[keep], fu[keep])
    assert np.allclose(fs[div], fu[div] / 8.0, rtol=0, atol=0)
    assert np.all(np.diff(fs) < 0)                       # still strictly decreasing
    assert keep.sum() == 29 and div.sum() == 29          # pairs 0-28 kept, 35-63 divided
    # continuity of the blend at both edges
    for edge, expect in ((2048.0, 1.0), (8192.0, 1.0 / 8.0)):
        f_edge = 2 * np.pi / edge
        t = (8192.0 / edge - 1.0) / 3.0
        blended = (1 - t) * f_edge / 8.0 + t * f_edge
        assert math.isclose(blended, f_edge * expect, rel_tol=1e-14)


def test_rope_is_complex_multiplication_of_adjacent_pairs():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((5, 3, 128))             # [T, heads, hd]
    pos = np.array([0, 1, 7, 1000, 131071])
    cos, sin = O.rope_cos_sin(pos)
    got = O.apply_rope(z, cos, sin)
    zc = z[..., 0::2] + 1j * z[..., 1::2]            # view_as_complex over adjacent pairs
    ang = pos[:, None] * O.rope_inv_freq()[None, :]
    rc = zc * np.exp(1j * ang)[:, None, :]
    ref = np.empty_like(z)
    ref[..., 0::2] = rc.real
    ref[..., 1::2] = rc.imag
    assert np.max(np.abs(got - ref)) < 1e-12


def test_rope_invariants():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((4, 2, 128))
    cos0, sin0 = O.rope_cos_sin([0, 0, 0, 0])
    assert np.array_equal(O.apply_rope(z, cos0, sin0), z)           # R(0) = identity, exactly
    pos = np.array([3, 500, 9000, 131071])
    cos, sin = O.rope_cos_sin(pos)
    r = O.apply_rope(z, cos, sin)
    n0 = z[..., 0::2] ** 2 + z[..., 1::2] ** 2
    n1 = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    assert np.max(np.abs(n0 - n1)) < 1e-12                          # pair norms kept
    # <R(m) q, R(n) k> depends only on m - n
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    for scaled in (False, True):
        for m, n in ((10, 3), (4000, 4000), (70000, 12345)):
            cm, sm = O.rope_cos_sin([m], scaled=scaled)
            cn, sn = O.rope_cos_sin([n], scaled=scaled)
            cd, sd = O.rope_cos_sin([m - n], scaled=scaled)
            lhs = np.sum(O.apply_rope(q, cm, sm) * O.apply_rope(k, cn, sn))
            rhs = np.sum(O.apply_rope(q, cd, sd) * k)
            assert abs(lhs - rhs) < 1e-9


# ----------------------------------------------------------------------------
# Small-shape block checks
# ----------------------------------------------------------------------------

def _tiny_inputs(rng, B, T, start_pos, d, H, KV):
    hd = d // H
    x = _bf16_vals(rng, (B, T, d), 1.0)
    wq = _bf16_vals(rng, (H * hd, d), 0.3)
    wk = _bf16_vals(rng, (KV * hd, d), 0.3)
    wv = _bf16_vals(rng, (KV * hd, d), 0.3)
    wo = _bf16_vals(rng, (d, H * hd), 0.3)
    kc = _bf16_vals(rng, (B, start_pos, KV, hd), 1.0)
    vc = _bf16_vals(rng, (B, start_pos, KV, hd), 1.0)
    return x, wq, wk, wv, wo, kc, vc


@pytest.mark.parametrize("B,T,start_pos,scaled", [
    (1, 1, 0, True), (2, 3, 0, True), (1, 4, 2, False), (2, 2, 3, True), (1, 1, 5, False)])
def test_oracle_matches_scalar_brute_force(B, T, start_pos, scaled):
    d, H, KV = 32, 4, 2          # head_dim 8: pairs 0-3 hit all three branches of the scaled rule
    rng = np.random.default_rng(10 + B * 7 + T * 3 + start_pos)
    x, wq, wk, wv, wo, kc, vc = _tiny_inputs(rng, B, T, start_pos, d, H, KV)
    theta = 5.0e5
    res = O.gqa_block(x, wq, wk, wv, wo, kc, vc, start_pos, theta, scaled, H, KV)
    delta, q, k_r = BF.block(x.tolist(), wq.tolist(), wk.tolist(), wv.tolist(), wo.tolist(),
                             kc.tolist(), vc.tolist(), start_pos, H, KV, theta, scaled)
    assert np.max(np.abs(res.delta - np.array(delta))) < 1e-12
    assert np.max(np.abs(res.q - np.array(q))) < 1e-12
    assert np.array_equal(O.f64_from_bf16_bits(res.k_bits), np.array(k_r))


def test_attention_matches_torch_sdpa_gqa_and_linear():
    """Projections vs F.linear and the attention core vs torch's own
    scaled_dot_product_attention with enable_gqa (repeat_interleave heads) and
    an explicit offset causal mask, all in fp64 on the CPU."""
    rng = np.random.default_rng(5)
    B, T, sp, d, H, KV = 2, 6, 5, 64, 8, 2
    hd = d // H
    x, wq, wk, wv, wo, kc, vc = _tiny_inputs(rng, B, T, sp, d, H, KV)
    res = O.gqa_block(x, wq, wk, wv, wo, kc, vc, sp, 5.0e5, True, H, KV)
    tx = torch.from_numpy(x)
    # projections (before RoPE) of V are untouched by RoPE
    v_lin = F.linear(tx, torch.from_numpy(wv)).numpy().reshape(B, T, KV, hd)
    assert np.max(np.abs(v_lin - res.v)) < 1e-12
    q = torch.from_numpy(res.q).transpose(1, 2)                      # [B, H, T, hd]
    keys = np.concatenate([kc, O.f64_from_bf16_bits(res.k_bits)], axis=1)
    vals = np.concatenate([vc, O.f64_from_bf16_bits(res.v_bits)], axis=1)
    k_t = torch.from_numpy(keys).transpose(1, 2).contiguous()         # [B, KV, L, hd]
    v_t = torch.from_numpy(vals).transpose(1, 2).contiguous()
    vis = torch.from_numpy(O.causal_visible(T, sp))
    o = F.scaled_dot_product_attention(q, k_t, v_t, attn_mask=vis, enable_gqa=True)
    merged = o.transpose(1, 2).reshape(B, T, H * hd).numpy()
    assert np.max(np.abs(merged - res.attn_out)) < 1e-12
    delta = F.linear(torch.from_numpy(merged), torch.from_numpy(wo)).numpy()
    assert np.max(np.abs(delta - res.delta)) < 1e-12


def test_mha_special_case_equals_textbook_per_head_attention():
    """n_kv_heads == n_heads (the MHA comparison on the GQA page) reduces to
    independent causal attention per head: torch SDPA with is_causal."""
    rng = np.random.default_rng(6)
    B, T, d, H = 2, 7, 64, 4
    hd = d // H
    x, wq, wk, wv, wo, kc, vc = _tiny_inputs(rng, B, T, 0, d, H, H)
    res = O.gqa_block(x, wq, wk, wv, wo, kc, vc, 0, 5.0e5, False, H, H)
    q = torch.from_numpy(res.q).transpose(1, 2)
    k = torch.from_numpy(O.f64_from_bf16_bits(res.k_bits)).transpose(1, 2).contiguous()
    v = torch.from_numpy(O.f64_from_bf16_bits(res.v_bits)).transpose(1, 2).contiguous()
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    assert np.max(np.abs(o.transpose(1, 2).reshape(B, T, d).numpy() - res.attn_out)) < 1e-12


def test_softmax_rows_sum_to_one_and_mask():
    rng = np.random.default_rng(7)
    B, T, sp, d, H, KV = 1, 5, 3, 32, 4, 2
    x, wq, wk, wv, wo, kc, vc = _tiny_inputs(rng, B, T, sp, d, H, KV)
    res = O.gqa_block(x, wq, wk, wv, wo, kc, vc, sp, 5.0e5, True, H, KV, keep_probs=True)
    p = res.probs[0]                                   # [H, T, L]
    assert np.max(np.abs(p.sum(-1) - 1.0)) < 1e-14
    for t in range(T):
        assert np.all(p[:, t, sp + t + 1:] == 0.0)      # keys after the query's position
        assert np.all(p[:, t, :sp + t + 1] > 0.0)


def test_gqa_head_map_is_interleaved():
    """Constant V = g on kv head g, wo = identity: head h must output h // 4,
    which tells repeat_interleave apart from tiling (h % 8)."""
    d, H, KV = 4096, 32, 8
    hd = 128
    B, T, sp = 1, 2, 3
    x = np.zeros((B, T, d)); x[..., 0] = 1.0
    rng = np.random.default_rng(8)
    wq = _bf16_vals(rng, (d, d), 0.02)
    wk = _bf16_vals(rng, (KV * hd, d), 0.02)
    wv = np.zeros((KV * hd, d))
    for g in range(KV):
        wv[g * hd:(g + 1) * hd, 0] = float(g)
    wo = np.eye(d)
    kc = _bf16_vals(rng, (B, sp, KV, hd), 1.0)
    vc = np.zeros((B, sp, KV, hd))
    for g in range(KV):
        vc[:, :, g, :] = float(g)
    res = O.gqa_block(x, wq, wk, wv, wo, kc, vc, sp)
    want = np.repeat(np.arange(H) // 4, hd).astype(np.float64)
    assert np.max(np.abs(res.delta[0, :, :] - want[None, :])) < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(9)
    d, H, KV = 64, 8, 2
    hd = d // H
    # T = 1 at position 0: one key, P = [1], O = V0 (as rounded into the cache)
    x, wq, wk, wv, wo, kc, vc = _tiny_inputs(rng, 2, 1, 0, d, H, KV)
    res = O.gqa_block(x, wq, wk, wv, wo, kc, vc, 0, n_heads=H, n_kv_heads=KV)
    v0 = O.f64_from_bf16_bits(res.v_bits)[:, 0]                       # [B, KV, hd]
    want = np.repeat(v0, H // KV, axis=1).reshape(2, 1, d)
    assert np.max(np.abs(res.attn_out - want)) < 1e-15
    assert np.max(np.abs(res.delta - want @ wo.T)) < 1e-12
    # all cached keys equal and the new key too: uniform P, O = mean of V
    sp = 6
    x, wq, wk, wv, wo, kc, vc = _tiny_inputs(rng, 1, 1, sp, d, H, KV)
    wk = np.zeros_like(wk)                                            # new key = 0
    kc = np.zeros_like(kc)
    res = O.gqa_block(x, wq, wk, wv, wo, kc, vc, sp, n_heads=H, n_kv_heads=KV)
    vals = np.concatenate([vc, O.f64_from_bf16_bits(res.v_bits)], axis=1)[0]  # [L, KV, hd]
    mean = vals.mean(axis=0)
    want = np.repeat(mean, H // KV, axis=0).reshape(d)
    assert np.max(np.abs(res.attn_out[0, 0] - want)) < 1e-14


def test_one_hot_layout_is_exact():
    """x = e_f picks column f of each [out, in] weight; with small-integer
    weights every projection is exact and position 0 leaves Q/K unrotated."""
    d, H, KV = 4096, 32, 8
    hd = 128
    rng = np.random.default_rng(11)
    f = 1234
    x = np.zeros((1, 1, d)); x[0, 0, f] = 1.0
    wq = rng.integers(-8, 9, (d, d)).astype(np.float64)
    wk = rng.integers(-8, 9, (KV * hd, d)).astype(np.float64)
    wv = rng.integers(-8, 9, (KV * hd, d)).astype(np.float64)
    wo = rng.integers(-2, 3, (d, d)).astype(np.float64)
    res = O.gqa_block(x, wq, wk, wv, wo, None, None, 0)
    assert np.array_equal(res.q.reshape(-1), wq[:, f])
    assert np.array_equal(O.f64_from_bf16_bits(res.k_bits).reshape(-1), wk[:, f])
    assert np.array_equal(O.f64_from_bf16_bits(res.v_bits).reshape(-1), wv[:, f])
    # one key: O = V0 per group, Delta = O wo^T exactly (integers)
    o = np.repeat(wv[:, f].reshape(KV, hd), 4, axis=0).reshape(d)
    assert np.array_equal(res.delta.reshape(-1), wo @ o)


def test_decode_after_prefill_equals_longer_prefill():
    """Prefill of T+1 tokens, last row == prefill of T tokens followed by a
    decode at start_pos = T on the cache that prefill wrote."""
    rng = np.random.default_rng(12)
    d, H, KV = 128, 8, 2
    B, T = 2, 9
    x, wq, wk, wv, wo, _, _ = _tiny_inputs(rng, B, T + 1, 0, d, H, KV)
    full = O.gqa_block(x, wq, wk, wv, wo, None, None, 0, n_heads=H, n_kv_heads=KV)
    pre = O.gqa_block(x[:, :T], wq, wk, wv, wo, None, None, 0, n_heads=H, n_kv_heads=KV)
    kc = O.f64_from_bf16_bits(pre.k_bits)
    vc = O.f64_from_bf16_bits(pre.v_bits)
    dec = O.gqa_block(x[:, T:], wq, wk, wv, wo, kc, vc, T, n_heads=H, n_kv_heads=KV)
    assert np.max(np.abs(dec.delta[:, 0] - full.delta[:, T])) < 1e-12
    assert np.array_equal(dec.k_bits[:, 0], full.k_bits[:, T])
    assert np.max(np.abs(pre.delta - full.delta[:, :T])) < 1e-12       # causal: later tokens unseen


def test_stacked_decode_hand_computed_chain():
    """Three stacked blocks at position 0 (one key, so every softmax is [1]
    and O is the appended V row of the head's kv head), with one-hot input and
    small-integer weights: every value is exact and the residual stream was
    worked out by hand.  d = 8, 2 query heads sharing 1 kv head of width 4.

      x0 = e_0
      block 0: v = (1, 5, -2, 256) from column 0 of wv;  O = (v, v);
               wo reverses the features: D0 = (256, -2, 5, 1, 256, -2, 5, 1)
               h1 = (257, -2, 5, 1, 256, -2, 5, 1)
      block 1 reads bf16(h1) = (256, -2, 5, 1, 256, -2, 5, 1) (257 is a tie
               of 256 and 258 and goes to even):
               v = (3*256, 3*5, -1*1, 2*(-2)) = (768, 15, -1, -4)
               (768, not the 772 that the unrounded 257 would give)
               D1 = (O[6], -O[0], 0, 0, 0, 2*O[1], 0, O[3])
                  = (-1, -768, 0, 0, 0, 30, 0, -4)
               h2 = (256, -770, 5, 1, 256, 28, 5, -3)   (the stream keeps -770)
      block 2 reads bf16(h2); v = (0, 0, h2[5], 0) = (0, 0, 28, 0); O[6] is
               head 1's copy of v[2]; D2 = (0, 0, O[6], 0, ...) = 28 at [2]
               h3 = (256, -770, 33, 1, 256, 28, 5, -3)

    A dropped residual, an unrounded block input, a transposed wv or wo, or a
    head expanded from the wrong kv head changes h3."""
    d, H, KV, hd = 8, 2, 1, 4
    rng = np.random.default_rng(14)
    x0 = np.zeros((1, d))
    x0[0, 0] = 1.0

    def block(wv_entries, wo_entries):
        wq = _bf16_vals(rng, (H * hd, d), 0.5)       # irrelevant with one key
        wk = _bf16_vals(rng, (KV * hd, d), 0.5)
        wv = np.zeros((KV * hd, d))
        for (r, c), val in wv_entries.items():
            wv[r, c] = val
        wo = np.zeros((d, H * hd))
        for (r, c), val in wo_entries.items():
            wo[r, c] = val
        return wq, wk, wv, wo

    blocks = [
        block({(0, 0): 1, (1, 0): 5, (2, 0): -2, (3, 0): 256},
              {(i, 7 - i): 1 for i in range(8)}),
        block({(0, 0): 3, (1, 2): 3, (2, 7): -1, (3, 5): 2},
              {(0, 6): 1, (1, 0): -1, (5, 1): 2, (7, 3): 1}),
        block({(2, 5): 1}, {(2, 6): 1}),
    ]
    empty = [np.zeros((1, 0, KV, hd))] * 3
    h, deltas = O.stacked_decode(x0, blocks, empty, empty, 0, n_heads=H, n_kv_heads=KV)
    assert np.array_equal(deltas[0][0], [256, -2, 5, 1, 256, -2, 5, 1])
    assert np.array_equal(deltas[1][0], [-1, -768, 0, 0, 0, 30, 0, -4])
    assert np.array_equal(deltas[2][0], [0, 0, 28, 0, 0, 0, 0, 0])
    assert np.array_equal(h[0], [256, -770, 33, 1, 256, 28, 5, -3])


def test_stacked_decode_with_zero_output_projections_keeps_the_input():
    """Real shapes, cached rows and RoPE at position 3: with every wo = 0 each
    block's update is exactly zero, so the residual stream leaves the stack
    bit for bit equal to its input (and every Delta is zero)."""
    rng = np.random.default_rng(13)
    d, KV, hd = 4096, 8, 128
    B, sp = 2, 3
    x = _bf16_vals(rng, (B, d), 1.0)
    ws, kcs, vcs = [], [], []
    for _ in range(3):
        ws.append((_bf16_vals(rng, (d, d), 0.02), _bf16_vals(rng, (KV * hd, d), 0.02),
                   _bf16_vals(rng, (KV * hd, d), 0.02), np.zeros((d, d))))
        kcs.append(_bf16_vals(rng, (B, sp, KV, hd), 1.0))
        vcs.append(_bf16_vals(rng, (B, sp, KV, hd), 1.0))
    h, deltas = O.stacked_decode(x, ws, kcs, vcs, sp)
    assert np.array_equal(h, x)
    assert all(not np.any(dl) for dl in deltas)


def test_rms_norm_matches_torch_rms_norm():
    """The pre-norm reading against the library routine, in fp64."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 5, 4096)) * 3.0
    g = rng.standard_normal(4096)
    for eps in (1e-5, 0.3):
        want = F.rms_norm(torch.from_numpy(x), (4096,), weight=torch.from_numpy(g), eps=eps).numpy()
        assert np.max(np.abs(O.rms_norm(x, g, eps) - want)) < 1e-12


def test_rms_norm_closed_forms():
    d, eps = 4096, 1e-5
    g = np.linspace(-2.0, 2.0, d)
    c = 0.75
    y = O.rms_norm(np.full((1, d), c), np.ones(d), eps)
    assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=0, atol=1e-15)
    x = np.zeros((1, d))
    x[0, 17] = 5.0                                    # one nonzero feature: mean = 25 / d
    y = O.rms_norm(x, g, eps)
    assert abs(y[0, 17] - 5.0 / math.sqrt(25.0 / d + eps) * g[17]) < 1e-12
    assert np.count_nonzero(y) == 1
    # scale equivariance: norm(s x, s^2 eps) == norm(x, eps)
    rng = np.random.default_rng(22)
    x = rng.standard_normal((2, d))
    assert np.max(np.abs(O.rms_norm(7.0 * x, g, 49.0 * eps) - O.rms_norm(x, g, eps))) < 1e-12


def test_layer_with_zero_gain_is_the_identity():
    """norm_w = 0 makes the block's input zero: every q, k, v is zero, the
    attention averages zero values, Delta = 0 and h == x bit for bit."""
    rng = np.random.default_rng(23)
    d, KV, hd = 4096, 8, 128
    x = _bf16_vals(rng, (2, 3, d), 1.0)
    w = (_bf16_vals(rng, (d, d), 0.02), _bf16_vals(rng, (KV * hd, d), 0.02),
         _bf16_vals(rng, (KV * hd, d), 0.02), _bf16_vals(rng, (d, d), 0.02))
    h, res = O.gqa_layer(x, np.zeros(d), 1e-5, *w, None, None, 0)
    assert np.array_equal(h, x)
    assert not np.any(res.delta)


def test_vocab_logits_one_hot_and_library():
    """A one-hot h picks a weight column exactly (W holds bf16 values); a
    general h matches F.linear in fp64 rounded to bf16."""
    rng = np.random.default_rng(31)
    V, d = 257, 4096
    w = _bf16_vals(rng, (V, d), 0.02)
    h = np.zeros((2, d))
    h[0, 5] = 1.0
    h[1, 4095] = -1.0
    L = O.vocab_logits(h, w)
    assert np.array_equal(L[0], w[:, 5]) and np.array_equal(L[1], -w[:, 4095])
    h = _bf16_vals(rng, (3, d), 1.0)
    want = F.linear(torch.from_numpy(h), torch.from_numpy(w)).numpy()
    assert np.array_equal(O.vocab_logits(h, w), O.f64_from_bf16_bits(O.bf16_bits_from_f64(want)))
    g = _bf16_vals(rng, (d,), 1.0)
    z = O.f64_from_bf16_bits(O.bf16_bits_from_f64(O.rms_norm(h, g, 1e-5)))
    assert np.array_equal(O.vocab_logits(h, w, g, 1e-5), O.vocab_logits(z, w))
