"""Scalar-loop, pure-Python Sol-Attn and Sol-Attn2 for tiny inputs (test infrastructure only).

An independent, deliberately naive restatement of the same definitions as
``oracle.sol_attn`` and ``oracle.sol_attn2`` (plain lists, ``math.exp``, one
token at a time, the threshold statistics computed as a literal mean and
variance of the proxy row where the paper's appendix "Threshold variance
derivation" allows it).  Used only to cross-check the vectorized oracle on
N <= ~200, d <= 16.
"""
from __future__ import annotations

import math


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def _blocks(n, block):
    out = []
    s = 0
    while s < n:
        out.append(list(range(s, min(s + block, n))))
        s += block
    return out


def _mean_rows(rows):
    d = len(rows[0])
    return [sum(r[c] for r in rows) / len(rows) for c in range(d)]


def routing(q, k, beta, block=64, thresh="diag", sink_blocks=()):
    """Returns (sel[i][j] bool, s_hat[i][j], tau[i]) for one head given as lists of rows."""
    n, d = len(q), len(q[0])
    scale = 1.0 / math.sqrt(d)
    blocks = _blocks(n, block)
    qbar = [_mean_rows([q[t] for t in b]) for b in blocks]
    kbar = [_mean_rows([k[t] for t in b]) for b in blocks]
    nb = len(blocks)
    s_hat = [[_dot(qbar[i], kbar[j]) * scale for j in range(nb)] for i in range(nb)]
    tau = []
    for i in range(nb):
        if thresh == "exact":
            # literal row mean and population variance of the proxy row
            mu = sum(s_hat[i]) / nb
            var = sum((x - mu) ** 2 for x in s_hat[i]) / nb
        else:
            mu_k = [sum(kbar[j][c] for j in range(nb)) / nb for c in range(d)]
            v_k = [sum(kbar[j][c] ** 2 for j in range(nb)) / nb - mu_k[c] ** 2 for c in range(d)]
            mu = _dot(qbar[i], mu_k) * scale
            var = sum(qbar[i][c] ** 2 * v_k[c] for c in range(d)) * scale * scale
        tau.append(mu + beta * math.sqrt(max(var, 0.0)))
    sel = [[(s_hat[i][j] > tau[i]) or (j in sink_blocks) for j in range(nb)] for i in range(nb)]
    return sel, s_hat, tau


def sol_attn(q, k, v, beta, block=64, thresh="diag", sink_blocks=()):
    """Sol-Attn output rows for one head (lists of rows)."""
    n, d = len(q), len(q[0])
    scale = 1.0 / math.sqrt(d)
    blocks = _blocks(n, block)
    sel, _, _ = routing(q, k, beta, block, thresh, sink_blocks)
    out = []
    for t in range(n):
        i = t // block
        num = [0.0] * d
        den = 0.0
        terms = []  # (logit, weight multiplier, value vector)
        for j, b in enumerate(blocks):
            if sel[i][j]:
                for u in b:
                    terms.append((_dot(q[t], k[u]) * scale, 1.0, v[u]))
            else:
                kb = _mean_rows([k[u] for u in b])
                vs = [sum(v[u][c] for u in b) for c in range(d)]
                terms.append((_dot(q[t], kb) * scale, float(len(b)), vs, True))
        m = max(x[0] for x in terms)
        for term in terms:
            e = math.exp(term[0] - m)
            if len(term) == 4:          # pooled block: numerator e*V-sum, denominator n*e
                den += term[1] * e
                for c in range(d):
                    num[c] += e * term[2][c]
            else:
                den += e
                for c in range(d):
                    num[c] += e * term[2][c]
        out.append([x / den for x in num])
    return out


def sol_attn2(q, k, v, beta, block=64, anchor=32, thresh="diag", sink_blocks=(), grouping="split2"):
    """Sol-Attn2 output rows for one head, no quantization (q, k already dequantized)."""
    n, d = len(q), len(q[0])
    scale = 1.0 / math.sqrt(d)
    blocks = _blocks(n, block)
    sel, _, _ = routing(q, k, beta, block, thresh, sink_blocks)
    qhat = _mean_rows(q)
    groups = []
    for b in blocks:
        if grouping == "whole":
            members = [b]
        elif grouping == "singleton":
            members = [[u] for u in b]
        else:
            proj = {u: _dot(k[u], qhat) for u in b}
            thr = sum(proj.values()) / len(b)
            members = [[u for u in b if proj[u] >= thr], [u for u in b if proj[u] < thr]]
        gl = []
        for mem in members:
            if mem:
                gl.append((len(mem), _mean_rows([k[u] for u in mem]), _mean_rows([v[u] for u in mem])))
        groups.append(gl)
    out = [None] * n
    for i, b in enumerate(blocks):
        tail = [g for j in range(len(blocks)) if not sel[i][j] for g in groups[j]]
        exact = [u for j, bb in enumerate(blocks) if sel[i][j] for u in bb]
        for a0 in range(b[0], b[-1] + 1, anchor):
            a = list(range(a0, min(a0 + anchor, b[-1] + 1)))
            qbar_a = _mean_rows([q[t] for t in a])
            if tail:
                w = [ng * math.exp(_dot(qbar_a, kg) * scale) for ng, kg, _ in tail]
                z_a = sum(w)
                mu = [sum(w[g] * tail[g][1][c] for g in range(len(tail))) / z_a for c in range(d)]
                nu = [sum(w[g] * tail[g][2][c] for g in range(len(tail))) / z_a for c in range(d)]
            else:
                z_a, mu, nu = 0.0, [0.0] * d, [0.0] * d
            for t in a:
                delta = _dot([q[t][c] - qbar_a[c] for c in range(d)], mu) * scale
                zhat = z_a * math.exp(delta)
                num = [zhat * nu[c] for c in range(d)]
                den = zhat
                for u in exact:
                    e = math.exp(_dot(q[t], k[u]) * scale)
                    den += e
                    for c in range(d):
                        num[c] += e * v[u][c]
                out[t] = [x / den for x in num]
    return out
