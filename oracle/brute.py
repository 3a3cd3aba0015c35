"""Brute-force attention in pure Python.  TEST INFRASTRUCTURE ONLY.

An independent second writing of the definition (Cleave §2.2 "FlashAttention",
Fig. 2: QK-Matmul, softmax, V-Matmul) with explicit loops, ``math.exp`` and
``math.fsum`` (exactly rounded sums), for tiny shapes only.  It pins the numpy
oracle in ``oracle.attention``; the two share no code.

Conventions are the oracle's: GQA head h reads KV head h // (Hq // Hkv);
causal masking is bottom-right aligned (row i sees key j iff
j <= i + L_b - Lq); a row with no visible key gives O = 0, LSE = -inf.
"""
from __future__ import annotations

import math


def brute_attention(q, k, v, causal, scale, dv):
    """q: nested lists [B][Lq][Hq][D]; k[b]: [L_b][Hkv][D]; v[b]: [L_b][Hkv][Dv].

    Returns (O [B][Lq][Hq][Dv], LSE [B][Lq][Hq]) as nested lists of floats.
    """
    out_o, out_l = [], []
    for b in range(len(q)):
        lq = len(q[b])
        n = len(k[b])
        o_b, l_b = [], []
        for i in range(lq):
            o_i, l_i = [], []
            hq = len(q[b][i])
            hkv = len(k[b][0]) if n else 1
            g = hq // hkv
            for h in range(hq):
                kvh = h // g
                keys = [j for j in range(n) if (not causal) or j <= i + n - lq]
                if not keys:
                    o_i.append([0.0] * dv)
                    l_i.append(-math.inf)
                    continue
                scores = {}
                for j in keys:
                    dot = math.fsum(float(q[b][i][h][d]) * float(k[b][j][kvh][d])
                                    for d in range(len(q[b][i][h])))
                    scores[j] = scale * dot
                mx = max(scores.values())
                ex = {j: math.exp(scores[j] - mx) for j in keys}
                total = math.fsum(ex.values())
                row = [math.fsum(ex[j] * float(v[b][j][kvh][c]) for j in keys) / total
                       for c in range(dv)]
                o_i.append(row)
                l_i.append(mx + math.log(total))
            o_b.append(o_i)
            l_b.append(l_i)
        out_o.append(o_b)
        out_l.append(l_b)
    return out_o, out_l


def brute_rmsnorm_matmul(x, g, w, eps):
    """RMSNorm then Matmul with explicit loops (Cleave §1, Fig. 1), for tiny
    shapes: x [M][K], g [K], w [N][K] as nested lists.  Returns Y [M][N]."""
    out = []
    for row in x:
        k = len(row)
        mean_sq = math.fsum(v * v for v in row) / k
        inv = 1.0 / math.sqrt(mean_sq + eps)
        normed = [row[c] * inv * g[c] for c in range(k)]
        out.append([math.fsum(normed[c] * wrow[c] for c in range(k)) for wrow in w])
    return out


def brute_swiglu(x, w_gate, w_up):
    """silu(x . w_gate_n) * (x . w_up_n) with explicit loops, for tiny shapes:
    x [M][K], w_gate and w_up [N][K] as nested lists.  Returns H [M][N]."""
    out = []
    for row in x:
        hrow = []
        for wg, wu in zip(w_gate, w_up):
            gsum = math.fsum(a * b for a, b in zip(row, wg))
            usum = math.fsum(a * b for a, b in zip(row, wu))
            hrow.append(gsum / (1.0 + math.exp(-gsum)) * usum)
        out.append(hrow)
    return out


def brute_matmul_matmul(q, k, v, causal, scale, dv):
    """MatMul+MatMul (Cleave §7.3 subgraph list) with explicit loops and exact sums.

    q: [B][Lq][Hq][D]; k[b]: [L_b][Hkv][D]; v[b]: [L_b][Hkv][Dv].  For each
    output (b, i, h, c): sum over visible keys j of t_j * V[b][j][h // G][c],
    where t_j = scale * sum_d Q[b][i][h][d] K[b][j][h // G][d].  A row with no
    visible key gives 0.  Returns O [B][Lq][Hq][Dv] as nested lists.
    """
    out = []
    for b in range(len(q)):
        lq = len(q[b])
        n = len(k[b])
        o_b = []
        for i in range(lq):
            hq = len(q[b][i])
            hkv = len(k[b][0]) if n else 1
            g = hq // hkv
            o_i = []
            for h in range(hq):
                kvh = h // g
                keys = [j for j in range(n) if (not causal) or j <= i + n - lq]
                t = {j: scale * math.fsum(q[b][i][h][d] * k[b][j][kvh][d]
                                          for d in range(len(q[b][i][h]))) for j in keys}
                o_i.append([math.fsum(t[j] * v[b][j][kvh][c] for j in keys) for c in range(dv)])
            o_b.append(o_i)
        out.append(o_b)
    return out
