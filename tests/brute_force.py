"""Scalar pure-Python attention block for tiny shapes.

Written independently of the NumPy oracle (no shared helpers): every sum is
an explicit loop over scalars, RoPE frequencies come from ``math.pow``, and
bf16 rounding uses ``math.frexp`` with Python's round-half-to-even.  It exists
only to pin the oracle on tiny inputs.
"""
from __future__ import annotations

import math


def bf16_round_scalar(a: float) -> float:
    """Nearest bfloat16 value (8 significant bits, ties to even)."""
    if a == 0.0 or not math.isfinite(a):
        return a
    m, e = math.frexp(a)               # a = m * 2**e with 0.5 <= |m| < 1
    r = round(m * 256.0)               # 8 significant bits, half to even
    return math.ldexp(r / 256.0, e)


def inv_freq_scalar(head_dim, theta, scaled):
    out = []
    for i in range(head_dim // 2):
        f = 1.0 / math.pow(theta, (2.0 * i) / head_dim)
        if scaled:
            lam = 2.0 * math.pi / f
            if lam < 8192.0 / 4.0:
                pass
            elif lam > 8192.0 / 1.0:
                f = f / 8.0
            else:
                t = (8192.0 / lam - 1.0) / (4.0 - 1.0)
                f = (1.0 - t) * (f / 8.0) + t * f
        out.append(f)
    return out


def block(x, wq, wk, wv, wo, kc, vc, start_pos, n_heads, n_kv, theta, scaled):
    """x: nested lists [B][T][d]; weights nested [out][in]; kc/vc [B][start_pos][n_kv][hd].

    Returns (delta [B][T][d], q [B][T][H][hd], k_rounded [B][T][KV][hd]).
    """
    B = len(x)
    T = len(x[0])
    d = len(x[0][0])
    hd = d // n_heads
    rep = n_heads // n_kv
    freqs = inv_freq_scalar(hd, theta, scaled)

    def matvec(W, vec):
        res = []
        for row in W:
            acc = 0.0
            for a, b in zip(row, vec):
                acc += a * b
            res.append(acc)
        return res

    def rot(vec, pos):
        out = list(vec)
        for i in range(hd // 2):
            ang = pos * freqs[i]
            c, s = math.cos(ang), math.sin(ang)
            a, b = vec[2 * i], vec[2 * i + 1]
            out[2 * i] = a * c - b * s
            out[2 * i + 1] = a * s + b * c
        return out

    delta, q_all, k_all = [], [], []
    for b in range(B):
        # cache rows for this sequence: list over positions of [n_kv][hd]
        keys = [[list(kc[b][p][g]) for g in range(n_kv)] for p in range(start_pos)]
        vals = [[list(vc[b][p][g]) for g in range(n_kv)] for p in range(start_pos)]
        qs = []
        for t in range(T):
            pos = start_pos + t
            qf = matvec(wq, x[b][t])
            kf = matvec(wk, x[b][t])
            vf = matvec(wv, x[b][t])
            qh = [rot(qf[h * hd:(h + 1) * hd], pos) for h in range(n_heads)]
            kh = [rot(kf[g * hd:(g + 1) * hd], pos) for g in range(n_kv)]
            vh = [vf[g * hd:(g + 1) * hd] for g in range(n_kv)]
            keys.append([[bf16_round_scalar(e) for e in kh[g]] for g in range(n_kv)])
            vals.append([[bf16_round_scalar(e) for e in vh[g]] for g in range(n_kv)])
            qs.append(qh)
        q_all.append(qs)
        k_all.append([keys[start_pos + t] for t in range(T)])
        d_b = []
        for t in range(T):
            pos = start_pos + t
            merged = []
            for h in range(n_heads):
                g = h // rep
                scores = []
                for j in range(pos + 1):
                    acc = 0.0
                    for e in range(hd):
                        acc += qs[t][h][e] * keys[j][g][e]
                    scores.append(acc / math.sqrt(hd))
                mx = max(scores)
                ex = [math.exp(s - mx) for s in scores]
                tot = sum(ex)
                o = [0.0] * hd
                for j in range(pos + 1):
                    w = ex[j] / tot
                    for e in range(hd):
                        o[e] += w * vals[j][g][e]
                merged.extend(o)
            d_b.append(matvec(wo, merged))
        delta.append(d_b)
    return delta, q_all, k_all
