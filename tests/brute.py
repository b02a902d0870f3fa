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
    Q, K, V = _vals(q), _vals(k), _vals(v)
    lq, hq, d = len(Q), len(Q[0]), len(Q[0][0])
    lk, hkv = len(K), len(K[0])
    scale = mpmath.mpf(1) / mpmath.sqrt(d) if scale is None else mpmath.mpf(scale)
    group = hq // hkv
    o = [[None] * hq for _ in range(lq)]
    lse = [[None] * hq for _ in range(lq)]
    for i in range(lq):
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
