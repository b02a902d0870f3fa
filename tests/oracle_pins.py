"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError if
the oracle disagrees with:
  * a 50-digit brute force built from its own position lists (tests/brute.py),
  * closed forms (Q = 0, constant V, a single visible key, huge score gaps),
  * invariants (softmax rows sum to 1, merge-order independence, the
    global-max/global-sum normaliser of the PCP page §4.2, GQA = repeated KV
    heads and the Ulysses head split of the Halo page),
  * the pages' literal index facts (the striped example and the split
    arithmetic) and closed-form pair counts.
  * for the gradients: central differences at 50 digits of the brute-force
    forward, the zero-sum and sum-to-dO invariants of dK and dV, invariance
    under a common key shift, GQA = repeated heads, and closed forms (one
    visible key per row, Q = 0).

``tests/test_oracle.py`` runs them on the real oracle; ``tests/test_oracle_mutants.py``
runs them on copies of the oracle with planted mistakes and requires each
mistake to fail at least one pin.
"""
import itertools
import math
import os

import numpy as np

import brute
from synth import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed, dtype, sigma=1.0):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _widen(a):
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def mpinf():
    import mpmath
    return mpmath.mpf("-inf")


# ---------------------------------------------------------------------------
# 1. brute force on tiny inputs

BRUTE_CASES = [
    # (S, cp, rank, layout, hq, hkv, d, dtype, doc_lens, key_ranks)
    (32, 2, 1, "zigzag", 4, 2, 8, "bf16", None, "all"),
    (24, 4, 2, "striped", 2, 1, 4, "f32", None, "all"),
    (16, 2, 1, "contiguous", 2, 2, 4, "bf16", None, "all"),
    (32, 2, 1, "zigzag", 2, 2, 4, "bf16", (8, 16, 8), "all"),
    (32, 4, 1, "zigzag", 2, 1, 4, "f32", None, (2, 3)),      # one block subset: some rows see nothing
    (16, 2, 0, "zigzag", 4, 4, 4, "f32", None, (0,)),
]


def pin_brute_force(orc, tol=1e-13):
    for case_i, (S, cp, r, layout, hq, hkv, d, dtype, docs, key_ranks) in enumerate(BRUTE_CASES):
        seed = 77 + case_i
        if docs is None:
            qp, qs = orc.local_positions(S, cp, r, layout)
            bq = brute.rank_tokens(S, cp, r, layout)
            bqs = None
            qs = None
        else:
            qp, qs = orc.local_positions(S, cp, r, layout, doc_lens=list(docs))
            bq, bqs = brute.rank_tokens_docs(docs, cp, r, layout)
        ranks = range(cp) if key_ranks == "all" else key_ranks
        kp_parts, bk = [], []
        for kr in ranks:
            if docs is None:
                kp_parts.append(orc.local_positions(S, cp, kr, layout)[0])
                bk += brute.rank_tokens(S, cp, kr, layout)
            else:
                kp_parts.append(orc.local_positions(S, cp, kr, layout, doc_lens=list(docs))[0])
                bk += brute.rank_tokens_docs(docs, cp, kr, layout)[0]
        kp = np.concatenate(kp_parts)
        q = _rand((len(qp), hq, d), seed, dtype)
        k = _rand((len(kp), hkv, d), seed + 100, dtype)
        v = _rand((len(kp), hkv, d), seed + 200, dtype)
        # the oracle's result, computed from its own positions, against brute force on brute's positions
        o, lse, _ = orc.attention(q, k, v, qp, kp, qs, True)
        bo, bl = brute.attention(q, k, v, bq, bk, bqs, True)
        for i in range(len(bq)):
            for h in range(hq):
                n = i * hq + h
                if bl[i][h] == mpinf():
                    assert lse[n] == -math.inf and np.all(o[n] == 0.0), \
                        "case %d: empty row (%d,%d) must be (0, -inf)" % (case_i, i, h)
                    continue
                assert abs(float(bl[i][h]) - lse[n]) <= tol, "case %d: lse row (%d,%d)" % (case_i, i, h)
                for t in range(d):
                    assert abs(float(bo[i][h][t]) - o[n, t]) <= tol, "case %d: o (%d,%d,%d)" % (case_i, i, h, t)
    # non-causal on arbitrary positions
    q = _rand((5, 2, 4), 5, "f32")
    k = _rand((7, 1, 4), 6, "f32")
    v = _rand((7, 1, 4), 7, "f32")
    o, lse, _ = orc.attention(q, k, v, None, None, None, False)
    bo, bl = brute.attention(q, k, v, None, None, None, False)
    for i in range(5):
        for h in range(2):
            assert abs(float(bl[i][h]) - lse[i * 2 + h]) <= tol
            assert max(abs(float(bo[i][h][t]) - o[i * 2 + h, t]) for t in range(4)) <= tol


# ---------------------------------------------------------------------------
# 2. softmax rows sum to 1 over exactly the visible keys


def pin_rows_sum_to_one(orc):
    S, cp, r, hq, hkv, d = 256, 4, 1, 2, 1, 16
    qp, _ = orc.local_positions(S, cp, r, "zigzag")
    kp = np.arange(S, dtype=np.int32)
    bq = brute.rank_tokens(S, cp, r, "zigzag")
    q = _rand((len(qp), hq, d), 11, "bf16")
    k = _rand((S, hkv, d), 12, "bf16")
    for i in (0, 1, 31, 32, 63):
        for h in range(hq):
            p = orc.softmax_row(q, k, i, h, qp, kp)
            n_vis = sum(1 for j in range(S) if j <= bq[i])
            assert np.all(p >= 0.0)
            assert abs(p.sum() - 1.0) <= 1e-14 * n_vis, "softmax row must sum to 1"
            assert np.count_nonzero(p[bq[i] + 1:]) == 0, "future keys must get zero weight"
            assert np.count_nonzero(p[:bq[i] + 1]) == n_vis, "every earlier key gets weight"


# ---------------------------------------------------------------------------
# 3. merge-order independence and the global max / global sum normaliser


def _block_partials(orc, q, k, v, qp, kps, bounds):
    parts = []
    for (a, b), kp in zip(bounds, kps):
        o, lse, _ = orc.attention(q, k[a:b], v[a:b], qp, kp)
        parts.append((o, lse))
    return parts


def pin_merge_order(orc, tol=1e-12):
    S, cp, r, hq, hkv, d = 1024, 4, 1, 1, 1, 64     # the shape of the smallest workload
    qp, _ = orc.local_positions(S, cp, r, "zigzag")
    kps = [orc.local_positions(S, cp, b, "zigzag")[0] for b in range(cp)]
    kp = np.concatenate(kps)
    q = _rand((len(qp), hq, d), 21, "f32")
    k = _rand((S, hkv, d), 22, "f32")
    v = _rand((S, hkv, d), 23, "f32")
    o_full, lse_full, _ = orc.attention(q, k, v, qp, kp)
    n = S // cp
    parts = _block_partials(orc, q, k, v, qp, kps, [(b * n, (b + 1) * n) for b in range(cp)])
    assert any(np.isneginf(p[1]).any() for p in parts), "some block must leave rows empty here"
    for order in itertools.permutations(range(cp)):
        o, lse = parts[order[0]]
        for b in order[1:]:
            o, lse = orc.merge(o, lse, *parts[b])
        assert np.max(np.abs(lse - lse_full)) <= tol, "merge order %s changes lse" % (order,)
        assert np.max(np.abs(o - o_full)) <= tol, "merge order %s changes o" % (order,)
    # a tree order
    a = orc.merge(*parts[3], *parts[0])
    b = orc.merge(*parts[1], *parts[2])
    o, lse = orc.merge(*a, *b)
    assert np.max(np.abs(lse - lse_full)) <= tol and np.max(np.abs(o - o_full)) <= tol


def pin_global_softmax(orc, tol=1e-13):
    """The PCP page's normaliser (§4.2): shard maxima -> global max -> local
    exponentials -> global sum -> divide. Weights applied to V must equal the
    merged partials of the same shards."""
    S, cp, hq, d = 128, 4, 1, 8
    qp, _ = orc.local_positions(S, cp, 2, "zigzag")
    kps = [orc.local_positions(S, cp, b, "zigzag")[0] for b in range(cp)]
    q = _rand((len(qp), hq, d), 31, "f32")
    ks = [_rand((len(kp), 1, d), 40 + b, "f32") for b, kp in enumerate(kps)]
    vs = [_rand((len(kp), 1, d), 50 + b, "f32") for b, kp in enumerate(kps)]
    parts = [orc.attention(q, kb, vb, qp, kp)[:2] for kb, vb, kp in zip(ks, vs, kps)]
    o, lse = parts[0]
    for p in parts[1:]:
        o, lse = orc.merge(o, lse, *p)
    qw = _widen(q)[:, 0, :]
    scale = 1.0 / math.sqrt(d)
    for i in range(len(qp)):
        scores = []
        for kb, kp in zip(ks, kps):
            s = (_widen(kb)[:, 0, :] @ qw[i]) * scale
            s[kp > qp[i]] = -np.inf
            scores.append(s)
        gmax = max(np.max(s) for s in scores)                    # all-reduce MAX
        local = [np.exp(s - gmax) for s in scores]               # local exp
        gsum = sum(float(np.sum(e)) for e in local)              # all-reduce SUM
        out = sum(e @ _widen(vb)[:, 0, :] for e, vb in zip(local, vs)) / gsum
        assert np.max(np.abs(out - o[i])) <= tol, "merged partials differ from the global normaliser"
        assert abs(gmax + math.log(gsum) - lse[i]) <= tol


def pin_merge_special(orc):
    d = 3
    oa = np.array([[1.0, 2.0, 3.0], [0.0, 0.0, 0.0], [0.0, 0.0, 0.0], [1.0, -1.0, 0.5]])
    la = np.array([0.5, -np.inf, -np.inf, 2.0])
    ob = np.array([[0.0, 0.0, 0.0], [4.0, 5.0, 6.0], [0.0, 0.0, 0.0], [-2.0, 3.0, 0.25]])
    lb = np.array([-np.inf, 1.5, -np.inf, 2.0])
    o, L = orc.merge(oa, la, ob, lb)
    assert np.array_equal(o[0], oa[0]) and L[0] == 0.5, "x merged with empty must be x exactly"
    assert np.array_equal(o[1], ob[1]) and L[1] == 1.5
    assert np.array_equal(o[2], np.zeros(d)) and L[2] == -np.inf, "empty with empty stays empty"
    assert np.allclose(o[3], 0.5 * (oa[3] + ob[3]), atol=1e-15, rtol=0) and abs(L[3] - (2.0 + math.log(2))) < 1e-15
    o2, L2 = orc.merge(ob, lb, oa, la)
    assert np.array_equal(o, o2) and np.array_equal(L, L2), "merge must be commutative"
    # unequal weights: e^1 : e^0
    o3, L3 = orc.merge(np.array([[1.0]]), np.array([1.0]), np.array([[0.0]]), np.array([0.0]))
    w = math.e / (math.e + 1.0)
    assert abs(o3[0, 0] - w) < 1e-15 and abs(L3[0] - math.log(math.e + 1.0)) < 1e-15


# ---------------------------------------------------------------------------
# 4. closed forms


def pin_closed_forms(orc):
    S, cp, r, hq, hkv, d = 512, 2, 1, 4, 2, 16
    qp, _ = orc.local_positions(S, cp, r, "zigzag")
    bq = np.array(brute.rank_tokens(S, cp, r, "zigzag"))
    kp = np.arange(S, dtype=np.int32)
    k = _rand((S, hkv, d), 61, "bf16")
    v = _rand((S, hkv, d), 62, "bf16")
    # Q = 0: uniform weights over the visible keys
    q0 = np.zeros((len(qp), hq, d), np.uint16)
    o, lse, cnt = orc.attention(q0, k, v, qp, kp)
    vw = _widen(v)
    csum = np.cumsum(vw, axis=0)
    for i in range(len(qp)):
        nvis = bq[i] + 1
        for h in range(hq):
            n = i * hq + h
            assert cnt[n] == nvis
            assert abs(lse[n] - math.log(nvis)) <= 1e-13, "Q=0 gives lse = ln(#visible)"
            mean = csum[bq[i], h // (hq // hkv)] / nvis
            assert np.max(np.abs(o[n] - mean)) <= 1e-12, "Q=0 gives the mean of the visible values"
    # constant V
    q = _rand((len(qp), hq, d), 63, "bf16")
    vc = np.full((S, hkv, d), f32_to_bf16_bits(np.float32(0.375)), np.uint16)
    o, _, _ = orc.attention(q, k, vc, qp, kp)
    assert np.max(np.abs(o - 0.375)) <= 1e-15, "constant V gives O = V"
    # exactly one visible key: row i sees only key 0 when keys sit at positions 0, and > q_pos
    qp1 = np.array([10, 20], np.int32)
    kp1 = np.array([5, 30, 40], np.int32)
    q1 = _rand((2, 1, d), 64, "f32")
    k1 = _rand((3, 1, d), 65, "f32")
    v1 = _rand((3, 1, d), 66, "f32")
    o, lse, cnt = orc.attention(q1, k1, v1, qp1, kp1)
    for i in range(2):
        s = float(_widen(q1)[i, 0] @ _widen(k1)[0, 0]) / math.sqrt(d)
        assert cnt[i] == 1 and abs(lse[i] - s) <= 1e-14 and np.max(np.abs(o[i] - _widen(v1)[0, 0])) <= 1e-15
    # huge score gap: the largest score dominates completely, without overflow
    q2 = np.ones((1, 1, 4), np.float32)
    k2 = np.array([[[1.0] * 4], [[300.0] * 4], [[2.0] * 4]], np.float32)
    v2 = np.array([[[1.0] * 4], [[7.0] * 4], [[3.0] * 4]], np.float32)
    o, lse, _ = orc.attention(q2, k2, v2, np.array([5], np.int32), np.array([0, 1, 2], np.int32))
    assert np.all(np.isfinite(o)) and np.max(np.abs(o - 7.0)) <= 1e-12
    assert abs(lse[0] - 600.0) <= 1e-9, "scores 2, 600, 4 give lse 600 + ln(1 + e^-598 + e^-596)"


# ---------------------------------------------------------------------------
# 5. GQA = repeated KV heads, and the Ulysses head split


def pin_gqa_and_head_split(orc):
    S, hq, hkv, d = 64, 8, 2, 8
    pos = np.arange(S, dtype=np.int32)
    q = _rand((S, hq, d), 71, "bf16")
    k = _rand((S, hkv, d), 72, "bf16")
    v = _rand((S, hkv, d), 73, "bf16")
    o, lse, _ = orc.attention(q, k, v, pos, pos)
    G = hq // hkv
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    o2, lse2, _ = orc.attention(q, kr, vr, pos, pos)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "GQA must equal repeat_kv exactly"
    # head split: cp ranks each take hq/cp query heads and hkv/cp KV heads over the whole sequence
    cp = 2
    for r in range(cp):
        qs = np.ascontiguousarray(q[:, r * hq // cp:(r + 1) * hq // cp])
        ks = np.ascontiguousarray(k[:, r * hkv // cp:(r + 1) * hkv // cp])
        vs = np.ascontiguousarray(v[:, r * hkv // cp:(r + 1) * hkv // cp])
        os_, ls_, _ = orc.attention(qs, ks, vs, pos, pos)
        ref_o = o.reshape(S, hq, d)[:, r * hq // cp:(r + 1) * hq // cp].reshape(-1, d)
        ref_l = lse.reshape(S, hq)[:, r * hq // cp:(r + 1) * hq // cp].reshape(-1)
        assert np.array_equal(os_, ref_o) and np.array_equal(ls_, ref_l), "head split must be exact"


# ---------------------------------------------------------------------------
# 6. index maps


def read_golden_positions(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":")
            rows[int(key)] = [int(x) for x in vals.split()]
    return rows


def pair_count(q_pos, k_pos, q_start=None):
    """Visible (query, key) pairs by counting, from sorted key positions."""
    kp = np.sort(np.asarray(k_pos, np.int64))
    hi = np.searchsorted(kp, np.asarray(q_pos, np.int64), side="right")
    lo = 0 if q_start is None else np.searchsorted(kp, np.asarray(q_start, np.int64), side="left")
    return int(np.sum(hi - lo))


def pin_index_maps(orc):
    # the striped example printed on the zig-zag page
    gold = read_golden_positions("striped_cp4_S16.txt")
    for r, expect in gold.items():
        got, _ = orc.local_positions(16, 4, r, "striped")
        assert got.tolist() == expect, "striped rank %d" % r
    # the PCP page's split arithmetic: 32768 tokens over 4 ranks -> 8192 each, contiguous
    for r in range(4):
        got, _ = orc.local_positions(32768, 4, r, "contiguous")
        assert len(got) == 8192 and got[0] == 8192 * r and got[-1] == 8192 * r + 8191
        assert np.all(np.diff(got) == 1)
    # every layout partitions [0, S) and agrees with the brute-force lists
    for S, cp in ((16, 4), (64, 2), (96, 3), (1024, 4), (4096, 8)):
        for layout in ("contiguous", "zigzag", "striped"):
            allp = []
            for r in range(cp):
                got, st = orc.local_positions(S, cp, r, layout)
                assert got.tolist() == brute.rank_tokens(S, cp, r, layout), (S, cp, r, layout)
                assert np.all(np.diff(got) > 0) and np.all(st == 0)
                allp.append(got)
            assert np.array_equal(np.sort(np.concatenate(allp)), np.arange(S)), "layouts partition the sequence"
    # zig-zag balance: every rank has 2*cp*c^2 + c visible pairs against the whole sequence
    for S, cp, expect in ((1024, 4, 131200), (65536, 8, 268439552)):
        c = S // (2 * cp)
        assert 2 * cp * c * c + c == expect
        for r in range(cp):
            got, _ = orc.local_positions(S, cp, r, "zigzag")
            assert pair_count(got, np.arange(S)) == expect, "zig-zag rank %d unbalanced" % r
    # per-document zig-zag: rank share is exactly 1/cp of each document's causal pairs
    docs = [16, 48, 8, 24]
    cp = 4
    for r in range(cp):
        got, st = orc.local_positions(sum(docs), cp, r, "zigzag", doc_lens=docs)
        bq, bst = brute.rank_tokens_docs(docs, cp, r, "zigzag")
        assert got.tolist() == bq and st.tolist() == bst
        expect = sum(L * (L + 1) // (2 * cp) for L in docs)
        assert pair_count(got, np.arange(sum(docs)), st) == expect
    # divisibility is enforced
    for bad in ((30, 4, "zigzag"), (10, 4, "contiguous"), (10, 4, "striped")):
        try:
            orc.local_positions(bad[0], bad[1], 0, bad[2])
        except ValueError:
            continue
        raise AssertionError("non-divisible split must be rejected: %s" % (bad,))


# ---------------------------------------------------------------------------
# 7. gradients: 50-digit finite differences of the brute-force forward

GRAD_CASES = [
    # (S, cp, rank, layout, hq, hkv, d, dtype, doc_lens, key_ranks, causal)
    (8, 2, 1, "zigzag", 2, 1, 3, "bf16", None, "all", True),      # GQA, diagonal and off-diagonal keys
    (16, 2, 0, "zigzag", 1, 1, 2, "f32", (4, 8, 4), "all", True),  # documents
    (16, 4, 0, "zigzag", 2, 2, 2, "bf16", None, (1, 2), True),     # some rows see none of these keys
    (8, 2, 0, "contiguous", 2, 1, 3, "f32", None, (1,), False),    # no mask
]


def _grad_case(orc, case_i, case):
    S, cp, r, layout, hq, hkv, d, dtype, docs, key_ranks, causal = case
    seed = 500 + case_i
    if docs is None:
        qp, _ = orc.local_positions(S, cp, r, layout)
        bq, bqs, qs = brute.rank_tokens(S, cp, r, layout), None, None
    else:
        qp, qs = orc.local_positions(S, cp, r, layout, doc_lens=list(docs))
        bq, bqs = brute.rank_tokens_docs(docs, cp, r, layout)
    ranks = range(cp) if key_ranks == "all" else key_ranks
    kp, bk = [], []
    for kr in ranks:
        if docs is None:
            kp.append(orc.local_positions(S, cp, kr, layout)[0])
            bk += brute.rank_tokens(S, cp, kr, layout)
        else:
            kp.append(orc.local_positions(S, cp, kr, layout, doc_lens=list(docs))[0])
            bk += brute.rank_tokens_docs(docs, cp, kr, layout)[0]
    kp = np.concatenate(kp)
    q = _rand((len(qp), hq, d), seed, dtype)
    k = _rand((len(kp), hkv, d), seed + 1, dtype)
    v = _rand((len(kp), hkv, d), seed + 2, dtype)
    dout = np.random.default_rng(seed + 3).standard_normal((len(qp), hq, d))
    return q, k, v, dout, (qp, kp, qs), (bq, bk, bqs), causal


def pin_grad_brute_force(orc, tol=1e-12):
    for case_i, case in enumerate(GRAD_CASES):
        q, k, v, dout, (qp, kp, qs), (bq, bk, bqs), causal = _grad_case(orc, case_i, case)
        dq, dk, dv, _ = orc.attention_grad(q, k, v, dout, qp, kp, qs, causal)
        bdq, bdk, bdv = brute.grad_fd(q, k, v, dout, bq, bk, bqs, causal)
        for name, got, ref in (("dq", dq, bdq), ("dk", dk, bdk), ("dv", dv, bdv)):
            a, b, c = got.shape
            for x, y, z in itertools.product(range(a), range(b), range(c)):
                assert abs(float(ref[x][y][z]) - got[x, y, z]) <= tol, \
                    "case %d: %s[%d,%d,%d] %r vs brute %s" % (case_i, name, x, y, z, got[x, y, z], ref[x][y][z])


# ---------------------------------------------------------------------------
# 8. gradient invariants and closed forms


def pin_grad_invariants(orc):
    rng = np.random.default_rng(91)
    lq, lk, hq, hkv, d = 24, 40, 4, 2, 8
    qp = np.sort(rng.choice(np.arange(10, 60), lq, replace=False)).astype(np.int32)
    kp = np.sort(rng.choice(np.arange(0, 60), lk, replace=False)).astype(np.int32)
    # values on a 1/64 grid, so that shifting every key by a grid vector is exact in float32
    q = (rng.integers(-64, 65, (lq, hq, d)) / 64.0).astype(np.float32)
    k = (rng.integers(-64, 65, (lk, hkv, d)) / 64.0).astype(np.float32)
    v = (rng.integers(-64, 65, (lk, hkv, d)) / 64.0).astype(np.float32)
    dout = rng.standard_normal((lq, hq, d))
    dq, dk, dv, delta = orc.attention_grad(q, k, v, dout, qp, kp, None, True)
    o, _, cnt = orc.attention(q, k, v, qp, kp, None, True)
    group = hq // hkv
    seen = (cnt.reshape(lq, hq) > 0)
    for g in range(hkv):
        # each row's dS sums to zero over its keys, so the key gradients of a KV head sum to zero
        assert np.abs(dk[:, g].sum(0)).max() <= 1e-12 * max(1.0, np.abs(dk).max()), "sum_j dK_j != 0"
        # each row's weights sum to one, so the value gradients sum to the rows' output gradients
        rows_dout = (dout[:, g * group:(g + 1) * group] * seen[:, g * group:(g + 1) * group, None]).sum((0, 1))
        assert np.abs(dv[:, g].sum(0) - rows_dout).max() <= 1e-12 * max(1.0, np.abs(rows_dout).max()), \
            "sum_j dV_j != sum_i dO_i"
    # D = <dO, O>
    assert np.abs(delta - (dout * o.reshape(lq, hq, d)).sum(-1)).max() <= 1e-12
    # shifting every key by one vector shifts each row's scores by a constant: no gradient changes
    c = (rng.integers(-32, 33, d) / 64.0).astype(np.float32)
    dq2, dk2, dv2, _ = orc.attention_grad(q, k + c, v, dout, qp, kp, None, True)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert np.abs(a - b).max() <= 1e-11 * max(1.0, np.abs(a).max()), "key shift changed a gradient"
    # GQA = the KV heads repeated for every query head, key gradients summed over the group
    kr, vr = np.repeat(k, group, axis=1), np.repeat(v, group, axis=1)
    dq3, dk3, dv3, _ = orc.attention_grad(q, kr, vr, dout, qp, kp, None, True)
    assert np.abs(dq3 - dq).max() <= 1e-12
    assert np.abs(dk3.reshape(lk, hkv, group, d).sum(2) - dk).max() <= 1e-12
    assert np.abs(dv3.reshape(lk, hkv, group, d).sum(2) - dv).max() <= 1e-12
    # (row, head) list = the same rows of the full result
    rows = np.array([0, 5, 23, 11], np.int64)
    heads = np.array([3, 0, 1, 2], np.int32)
    dqs, _, _, ds = orc.attention_grad(q, k, v, dout, qp, kp, None, True, rows=rows, heads=heads)
    assert np.array_equal(dqs, dq[rows, heads]) and np.array_equal(ds, delta[rows, heads])


def pin_grad_closed_forms(orc):
    rng = np.random.default_rng(92)
    # every row sees exactly one key (documents of length one): O_i = v_i, so dV_i = dO_i and
    # the softmax has no freedom: dQ = dK = 0
    n, hq, hkv, d = 6, 2, 1, 4
    pos = np.arange(n, dtype=np.int32)
    q = rng.standard_normal((n, hq, d)).astype(np.float32)
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    dout = rng.standard_normal((n, hq, d))
    dq, dk, dv, delta = orc.attention_grad(q, k, v, dout, pos, pos, pos, True)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    assert np.abs(dv[:, 0] - dout.sum(1)).max() <= 1e-14
    assert np.abs(delta - (dout * v.astype(np.float64)).sum(-1)).max() <= 1e-13
    # Q = 0: uniform weights 1/n_i over the n_i visible keys, so
    # dV_j = sum over rows i seeing j of dO_i / n_i, dK = 0, and
    # dQ_i = scale / n_i * sum_j <dO_i, v_j - mean_i(v)> k_j
    lq, lk, d = 5, 7, 3
    qp = np.array([1, 2, 4, 5, 6], np.int32)
    kp = np.arange(lk, dtype=np.int32)
    q = np.zeros((lq, 1, d), np.float32)
    k = rng.standard_normal((lk, 1, d)).astype(np.float32)
    v = rng.standard_normal((lk, 1, d)).astype(np.float32)
    dout = rng.standard_normal((lq, 1, d))
    scale = 0.7
    dq, dk, dv, _ = orc.attention_grad(q, k, v, dout, qp, kp, None, True, scale=scale)
    kk, vv = k[:, 0].astype(np.float64), v[:, 0].astype(np.float64)
    dv_ref = np.zeros((lk, d))
    for i in range(lq):
        vis = kp <= qp[i]
        ni = vis.sum()
        dv_ref[vis] += dout[i, 0] / ni
        vbar = vv[vis].mean(0)
        dq_ref = scale / ni * ((vv[vis] - vbar) @ dout[i, 0]) @ kk[vis]
        assert np.abs(dq[i, 0] - dq_ref).max() <= 1e-13, "uniform-weight dQ row %d" % i
    assert np.all(dk == 0.0)
    assert np.abs(dv[:, 0] - dv_ref).max() <= 1e-13


ALL_PINS = [pin_brute_force, pin_rows_sum_to_one, pin_merge_order, pin_global_softmax, pin_merge_special,
            pin_closed_forms, pin_gqa_and_head_split, pin_index_maps, pin_grad_invariants, pin_grad_closed_forms,
            pin_grad_brute_force]
