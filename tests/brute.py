"""Brute-force attention at 50 significant digits, for tiny inputs only.

An independent second implementation used to pin the fp64 oracle: it builds
the whole masked score matrix from its own position lists (written straight
from the pages' descriptions of the splits), then takes the softmax by direct
exponentiation in mpmath — no max shift, no two-pass structure, no code shared
with ``oracle/`` or the GPU library.
"""
import mpmath

from synth import bf16_bits_to_f32

mpmath.mp.dps = 50


def rank_tokens(S, cp, r, layout):
    """Global positions held by rank r (one sequence of length S)."""
    if layout == "contiguous":        # equal contiguous slices (PCP page, §3.5)
        n = S // cp
        return list(range(r * n, (r + 1) * n))
    if layout == "striped":           # the literal example: t mod cp == r (zig-zag page, §4.2)
        return [t for t in range(S) if t % cp == r]
    if layout == "zigzag":            # 2*cp chunks; rank r takes the r-th from each end
        c = S // (2 * cp)
        chunks = [list(range(i * c, (i + 1) * c)) for i in range(2 * cp)]
        return chunks[r] + chunks[2 * cp - 1 - r]
    raise ValueError(layout)


def rank_tokens_docs(doc_lens, cp, r, layout):
    """Per-document split; returns (positions, document start of each)."""
    pos, starts, base = [], [], 0
    for L in doc_lens:
        p = [base + t for t in rank_tokens(int(L), cp, r, layout)]
        pos += p
        starts += [base] * len(p)
        base += int(L)
    return pos, starts


def _vals(a):
    """Exact values of a uint16-bf16 or float32 array as nested Python floats."""
    import numpy as np
    if a.dtype == np.uint16:
        a = bf16_bits_to_f32(a)
    return a.astype(np.float64).tolist()


def attention(q, k, v, q_pos, k_pos, q_start=None, causal=True, scale=None):
    """Dense attention; returns (o[i][h][t], lse[i][h]) as mpmath numbers."""
    return attention_values(_vals(q), _vals(k), _vals(v), q_pos, k_pos, q_start, causal, scale)


def attention_values(Q, K, V, q_pos, k_pos, q_start=None, causal=True, scale=None, only_rows=None):
    """Dense attention of nested lists Q[i][h][t], K[j][g][t], V[j][g][t]
    (numbers or mpf); `only_rows` limits the computed query rows (others None)."""
    lq, hq, d = len(Q), len(Q[0]), len(Q[0][0])
    lk, hkv = len(K), len(K[0])
    scale = mpmath.mpf(1) / mpmath.sqrt(d) if scale is None else mpmath.mpf(scale)
    group = hq // hkv
    o = [[None] * hq for _ in range(lq)]
    lse = [[None] * hq for _ in range(lq)]
    for i in (range(lq) if only_rows is None else only_rows):
        for h in range(hq):
            g = h // group
            weights, rows = [], []
            for j in range(lk):
                if causal:
                    if k_pos[j] > q_pos[i]:
                        continue
                    if q_start is not None and k_pos[j] < q_start[i]:
                        continue
                s = scale * mpmath.fsum(mpmath.mpf(Q[i][h][t]) * mpmath.mpf(K[j][g][t]) for t in range(d))
                weights.append(mpmath.exp(s))
                rows.append(j)
            if not rows:
                o[i][h] = [mpmath.mpf(0)] * d
                lse[i][h] = mpmath.mpf("-inf")
                continue
            Z = mpmath.fsum(weights)
            o[i][h] = [mpmath.fsum(w * mpmath.mpf(V[j][g][t]) for w, j in zip(weights, rows)) / Z
                       for t in range(d)]
            lse[i][h] = mpmath.log(Z)
    return o, lse


def grad_fd(q, k, v, dout, q_pos, k_pos, q_start=None, causal=True, scale=None, step="1e-15"):
    """Gradients of loss = sum dout * O with respect to q, k, v by central
    differences of ``attention_values`` at 50 digits (truncation error of
    order step^2, far below fp64 rounding). Returns nested lists of mpf:
    dq[i][h][t], dk[j][g][t], dv[j][g][t]."""
    Q, K, V = _vals(q), _vals(k), _vals(v)
    dO = dout.tolist()
    hstep = mpmath.mpf(step)
    lq, hq, d = len(Q), len(Q[0]), len(Q[0][0])
    lk, hkv = len(K), len(K[0])

    def loss(Qx, Kx, Vx, rows=None):
        o, _ = attention_values(Qx, Kx, Vx, q_pos, k_pos, q_start, causal, scale, rows)
        return mpmath.fsum(mpmath.mpf(dO[i][h][t]) * o[i][h][t]
                           for i in (range(lq) if rows is None else rows) for h in range(hq) for t in range(d))

    def perturbed(X, idx, delta):
        Y = [[list(r) for r in m] for m in X]
        a, b, c = idx
        Y[a][b][c] = mpmath.mpf(Y[a][b][c]) + delta
        return Y

    dq = [[[None] * d for _ in range(hq)] for _ in range(lq)]
    for i in range(lq):             # q_i only moves row i's output
        for h in range(hq):
            for t in range(d):
                up = loss(perturbed(Q, (i, h, t), hstep), K, V, [i])
                dn = loss(perturbed(Q, (i, h, t), -hstep), K, V, [i])
                dq[i][h][t] = (up - dn) / (2 * hstep)
    dk = [[[None] * d for _ in range(hkv)] for _ in range(lk)]
    dv = [[[None] * d for _ in range(hkv)] for _ in range(lk)]
    for j in range(lk):
        for g in range(hkv):
            for t in range(d):
                dk[j][g][t] = (loss(Q, perturbed(K, (j, g, t), hstep), V)
                               - loss(Q, perturbed(K, (j, g, t), -hstep), V)) / (2 * hstep)
                dv[j][g][t] = (loss(Q, K, perturbed(V, (j, g, t), hstep))
                               - loss(Q, K, perturbed(V, (j, g, t), -hstep))) / (2 * hstep)
    return dq, dk, dv
