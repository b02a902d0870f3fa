"""The plan of a document call (cpattn_varlen_plan).

Host logic (CPU): the records' tiles are a permutation of the call's
workgroups; each XCD (workgroup id b runs on XCD b % 8) keeps the set of
logical tiles the kernel's default order gives it; within an XCD the tiles go
in decreasing order of the key tiles their workgroup loads, ties by logical
id. Every field of every record (key range, per-wave fully visible keys,
document starts, per-lane search flag) is recomputed here from the positions
with numpy, and the work of a tile on a small case by brute force over keys.
GPU: the planned call gives results bit-identical to the unplanned one, in
the planned record order and in a random one.
"""
import numpy as np
import pytest

import context_long_sequence_amd as cp
from context_long_sequence_amd.share import block_positions


def _geometry(lq, hq, hkv):
    G = hq // hkv
    g_wg = 8 if G % 8 == 0 else 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    r_wg = 8 // g_wg
    n_qtiles = (lq + 32 * r_wg - 1) // (32 * r_wg)
    return n_qtiles, hq // g_wg, r_wg


def _default_logical(n, units):
    """Logical tile of each workgroup id in the kernel's default order."""
    bid = np.arange(n, dtype=np.int64)
    if units % 8 != 0:
        return bid
    x, slot = bid & 7, bid >> 3
    q, rem = n >> 3, n & 7
    return x * q + np.minimum(x, rem) + slot


def _tile_keys(in_bf16, d):
    return (128 if d == 64 else 64) if in_bf16 else 32


def _work(q_pos, k_pos, cu, lq, hq, hkv, d, in_bf16):
    """Key tiles each logical tile's workgroup loads: keys from the first row's
    document start to the last row's position."""
    n_qtiles, units, r_wg = _geometry(lq, hq, hkv)
    BK = _tile_keys(in_bf16, d)
    L = np.arange(n_qtiles * units, dtype=np.int64)
    qt = n_qtiles - 1 - L % n_qtiles
    r0 = qt * 32 * r_wg
    r1 = np.minimum(r0 + 32 * r_wg, lq)
    first, last = q_pos[r0], q_pos[r1 - 1]
    start = cu[np.searchsorted(cu, first, side="right") - 1]
    kb = np.searchsorted(k_pos, start, side="left")
    ke = np.searchsorted(k_pos, last, side="right")
    nt = np.where(ke > kb, (ke + BK - 1) // BK - kb // BK, 0)
    if len(k_pos) == 0:
        return np.zeros_like(nt)
    return np.where(k_pos[0] > last, 0, nt)


REC = cp.VARLEN_PLAN_RECORD
TILE, KB, KE, SLAST, SFIRST, FLO, FHI, FLAGS = 0, 1, 2, 4, 12, 20, 28, 36


def _fields(q_pos, k_pos, cu, lq, hq, hkv):
    """Every record field by logical tile, recomputed with numpy searches."""
    n_qtiles, units, r_wg = _geometry(lq, hq, hkv)
    n = n_qtiles * units
    g_wg = 8 // r_wg
    L = np.arange(n, dtype=np.int64)
    qt = n_qtiles - 1 - L % n_qtiles
    wg_r0 = qt * 32 * r_wg
    wg_r1 = np.minimum(wg_r0 + 32 * r_wg, lq)
    lk = len(k_pos)
    k_first = k_pos[0] if lk else 0
    k_last = k_pos[-1] if lk else 0
    start_of = lambda x: cu[np.maximum(np.searchsorted(cu, x, side="right") - 1, 0)]
    didx = lambda x: np.searchsorted(cu, x, side="right")
    rec = np.zeros((n, REC), np.int64)
    rec[:, TILE] = L
    wq_hi = q_pos[wg_r1 - 1]
    sees = (lk > 0) & ~(k_first > wq_hi)
    s_wg = start_of(q_pos[wg_r0])
    kb = np.where(k_first >= s_wg, 0, np.searchsorted(k_pos, s_wg, side="left"))
    ke = np.where(k_last <= wq_hi, lk, np.searchsorted(k_pos, wq_hi, side="right"))
    rec[:, KB] = np.where(sees, kb, 0)
    rec[:, KE] = np.where(sees, ke, 0)
    for w in range(8):
        r0 = wg_r0 + 32 * (w // g_wg)
        r1 = np.minimum(r0 + 32, lq)
        act = r0 < lq
        qf = np.where(act, q_pos[np.minimum(r0, lq - 1)], wq_hi)
        ql = np.where(act, q_pos[np.maximum(r1 - 1, 0)], wq_hi)
        sf, sl = start_of(qf), start_of(ql)
        rec[:, SFIRST + w] = sf
        rec[:, SLAST + w] = sl
        rec[:, FLAGS + w] = (didx(ql) > didx(qf) + 1).astype(np.int64)
        rec[:, FLO + w] = np.where(k_first >= sl, 0, np.searchsorted(k_pos, sl, side="left"))
        rec[:, FHI + w] = np.where(k_last <= qf, lk, np.searchsorted(k_pos, qf, side="right"))
    return rec


def _check_plan(plan, q_pos, k_pos, cu, lq, hq, hkv, d, in_bf16):
    n_qtiles, units, _ = _geometry(lq, hq, hkv)
    n = n_qtiles * units
    assert len(plan) == n * REC and n == cp.cpattn_partial_workgroups(lq, hq, hkv)
    recs = plan.reshape(n, REC).astype(np.int64)
    order = recs[:, TILE]
    assert np.array_equal(np.sort(order), np.arange(n)), "not a permutation"
    want = _fields(q_pos, k_pos, cu, lq, hq, hkv)
    assert np.array_equal(recs, want[order]), "a record differs from its recomputation"
    work = _work(q_pos, k_pos, cu, lq, hq, hkv, d, in_bf16)
    default = _default_logical(n, units)
    for x in range(8):
        ids = order[x::8]
        assert np.array_equal(np.sort(ids), np.sort(default[x::8])), "XCD %d's set changed" % x
        w = work[ids]
        assert np.all(np.diff(w) <= 0), "XCD %d: work not non-increasing" % x
        ties = np.diff(w) == 0
        assert np.all(np.diff(ids)[ties] > 0), "XCD %d: ties not by logical id" % x
    return work


def _documents_share(S, cp_size, docs_seed, min_doc, max_doc):
    """cu_seqlens of seeded document lengths (multiples of 2 cp_size, as the
    per-document zig-zag split needs) that fill S."""
    rng = np.random.default_rng(docs_seed)
    u = 2 * cp_size
    lens = []
    while sum(lens) < S:
        lens.append(u * int(rng.integers(max(1, min_doc // u), max_doc // u + 1)))
    lens[-1] -= sum(lens) - S
    if lens[-1] <= 0:
        extra = lens.pop()
        lens[-1] += extra
    assert sum(lens) == S and all(x > 0 and x % u == 0 for x in lens)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


@pytest.mark.parametrize("S,cp_size,rank,hq,hkv,d,in_bf16", [
    (131072, 4, 1, 32, 32, 128, True),     # the documents share: 32 heads (units split over the 8 XCDs)
    (16384, 4, 2, 16, 2, 64, True),        # grouped KV heads, d 64 (2 units: the hardware's order)
    (8192, 4, 0, 4, 4, 128, False),        # float32 tiles
])
def test_plan_keeps_xcd_sets_and_orders_by_work(S, cp_size, rank, hq, hkv, d, in_bf16):
    cu = _documents_share(S, cp_size, 11, 256, 8192)
    q_pos, _ = cp.cpattn_zigzag_index(S, cp_size, rank, "zigzag", cu)
    kps = block_positions(S, cp_size, cp_size, "rank_shares", "zigzag", cu)
    lq = len(q_pos)
    for b, kp in enumerate(kps):
        plan = cp.cpattn_varlen_plan(q_pos, kp, cu, hq, hkv, d, "bf16" if in_bf16 else "f32")
        work = _check_plan(plan, q_pos, kp, cu, lq, hq, hkv, d, in_bf16)
        assert work.max() > 0
        again = cp.cpattn_varlen_plan(q_pos, kp, cu, hq, hkv, d, "bf16" if in_bf16 else "f32")
        assert np.array_equal(plan, again), "the plan must be deterministic"


def test_work_estimate_brute_force():
    """On a small share, the work of each tile equals the key tiles spanned
    from the first key at or after the first row's document start to the last
    key at or before the last row, found by scanning every key."""
    S, cps = 4096, 4
    cu = _documents_share(S, cps, 5, 64, 700)
    q_pos, _ = cp.cpattn_zigzag_index(S, cps, 3, "zigzag", cu)
    kps = block_positions(S, cps, cps, "rank_shares", "zigzag", cu)
    hq = hkv = 8
    d = 128
    n_qtiles, units, r_wg = _geometry(len(q_pos), hq, hkv)
    BK = _tile_keys(True, d)
    for kp in kps:
        plan = cp.cpattn_varlen_plan(q_pos, kp, cu, hq, hkv, d)
        work = _check_plan(plan, q_pos, kp, cu, len(q_pos), hq, hkv, d, True)
        for L in range(n_qtiles * units):
            qt = n_qtiles - 1 - L % n_qtiles
            r0 = qt * 32 * r_wg
            r1 = min(r0 + 32 * r_wg, len(q_pos))
            start = max(c for c in cu[:-1] if c <= q_pos[r0])
            if kp[0] > q_pos[r1 - 1]:
                want = 0
            else:
                kb = next((j for j in range(len(kp)) if kp[j] >= start), len(kp))
                ke = max((j + 1 for j in range(len(kp)) if kp[j] <= q_pos[r1 - 1]), default=0)
                want = -(-ke // BK) - kb // BK if ke > kb else 0
            assert work[L] == want, (L, work[L], want)


def test_plan_errors():
    q_pos = np.arange(256, dtype=np.int32)
    k_pos = np.arange(256, dtype=np.int32)
    cu = np.array([0, 100, 256], np.int32)
    lib = cp.load_library()
    n = cp.cpattn_partial_workgroups(256, 4, 4) * REC
    out = np.zeros(n + 1, np.int32)
    st = lib.cpattn_varlen_plan(q_pos.ctypes.data, 256, k_pos.ctypes.data, 256, cu.ctypes.data, 2, 4, 4, 128, 0,
                                out.ctypes.data, n + 1)
    assert st == 2  # CPATTN_ERR_SHAPE: plan_len is not workgroups x the record size
    bad = q_pos[::-1].copy()
    with pytest.raises(cp.CpattnError) as e:
        cp.cpattn_varlen_plan(bad, k_pos, cu, 4, 4, 128)
    assert e.value.status == 4  # CPATTN_ERR_UNSORTED
    with pytest.raises(cp.CpattnError) as e:
        cp.cpattn_varlen_plan(q_pos, k_pos, cu, 4, 4, 96)
    assert e.value.status == 2
    assert cp.cpattn_partial_workgroups(-1, 4, 4) == -1
    assert cp.cpattn_partial_workgroups(256, 6, 4) == -1
    assert cp.cpattn_partial_workgroups(0, 4, 4) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["docs8k_zigzag_cp4_h4_d128", "docs8k_zigzag_cp4_h4kv2_d64",
                                  "docs4k_zigzag_cp4_h2kv1_d64_tiny"])
def test_planned_calls_bit_identical(name):
    """The share's plans, the same records in a random order and the unplanned
    calls give bit-identical O and LSE (accumulate mode, every block)."""
    import torch
    from test_gpu_parity import _reduced, say
    from context_long_sequence_amd.share import share_from_workload
    wl = _reduced()[name]
    say("%s: planned / shuffled records / unplanned" % name)
    planned = share_from_workload(wl)
    assert planned.plans is not None
    o1, l1 = [t.clone() for t in planned.step(wl.arrival())]
    rng = np.random.default_rng(3)
    shuffled = []
    for pl in planned.plans:
        recs = pl.view(-1, REC)
        shuffled.append(recs[torch.from_numpy(rng.permutation(recs.shape[0])).cuda()].contiguous().view(-1))
    planned.plans = shuffled
    o2, l2 = [t.clone() for t in planned.step(wl.arrival())]
    plain = share_from_workload(wl, plan=False)
    assert plain.plans is None
    o3, l3 = plain.step(wl.arrival())
    torch.cuda.synchronize()
    for o, l in ((o2, l2), (o3, l3)):
        assert torch.equal(o1.view(torch.int16), o.view(torch.int16))
        assert torch.equal(l1, l)


# ---------------------------------------------------------------------------
# The plan of a document gradient call (cpattn_varlen_bwd_plan): the query
# kernel's dispatch order.

def _bwd_query_work(q_pos, k_pos, cu, lq, hq):
    """Key tiles (32 keys) each logical tile of the query kernel loads: keys from
    its first row's document start to its last row (128 rows of one head)."""
    n_tiles = (lq + 127) // 128
    L = np.arange(n_tiles * hq, dtype=np.int64)
    qt = n_tiles - 1 - L % n_tiles
    r0 = qt * 128
    r1 = np.minimum(r0 + 128, lq)
    start = cu[np.searchsorted(cu, q_pos[r0], side="right") - 1]
    kb = np.searchsorted(k_pos, start, side="left")
    ke = np.searchsorted(k_pos, q_pos[r1 - 1], side="right")
    return np.where(ke > kb, (ke - kb + 31) // 32, 0)


@pytest.mark.parametrize("S,cp_size,rank,hq,hkv", [
    (131072, 4, 1, 32, 32),     # the documents share (heads split over the 8 XCDs)
    (16384, 4, 2, 12, 4),       # 12 heads: the hardware's order
])
def test_bwd_plan_keeps_xcd_sets_and_orders_by_work(S, cp_size, rank, hq, hkv):
    cu = _documents_share(S, cp_size, 13, 256, 8192)
    q_pos, _ = cp.cpattn_zigzag_index(S, cp_size, rank, "zigzag", cu)
    kps = block_positions(S, cp_size, cp_size, "rank_shares", "zigzag", cu)
    lq = len(q_pos)
    n = cp.cpattn_bwd_query_workgroups(lq, hq)
    assert n == (lq + 127) // 128 * hq
    default = _default_logical(n, hq)
    for kp in kps:
        plan = cp.cpattn_varlen_bwd_plan(q_pos, kp, cu, hq, hkv)
        assert plan.shape == (n,)
        assert np.array_equal(np.sort(plan), np.arange(n)), "the plan must be a permutation of the tiles"
        work = _bwd_query_work(q_pos.astype(np.int64), kp.astype(np.int64), cu.astype(np.int64), lq, hq)
        assert work.max() > 0
        for x in range(8):
            mine = plan[x::8]
            assert np.array_equal(np.sort(mine), np.sort(default[x::8])), "each XCD keeps its set of tiles"
            w = work[mine]
            assert np.all((w[:-1] > w[1:]) | ((w[:-1] == w[1:]) & (mine[:-1] < mine[1:]))), \
                "longest first, ties by tile id"
        assert np.array_equal(plan, cp.cpattn_varlen_bwd_plan(q_pos, kp, cu, hq, hkv))


def test_bwd_plan_errors():
    q_pos = np.arange(300, dtype=np.int32)
    k_pos = np.arange(300, dtype=np.int32)
    cu = np.array([0, 100, 300], np.int32)
    lib = cp.load_library()
    n = cp.cpattn_bwd_query_workgroups(300, 4)
    assert n == 12
    out = np.zeros(n + 1, np.int32)
    st = lib.cpattn_varlen_bwd_plan(q_pos.ctypes.data, 300, k_pos.ctypes.data, 300, cu.ctypes.data, 2, 4, 4,
                                    out.ctypes.data, n + 1)
    assert st == 2  # CPATTN_ERR_SHAPE: plan_len is not the query kernel's workgroups
    with pytest.raises(cp.CpattnError) as e:
        cp.cpattn_varlen_bwd_plan(q_pos, k_pos[::-1].copy(), cu, 4, 4)
    assert e.value.status == 4  # CPATTN_ERR_UNSORTED
    with pytest.raises(cp.CpattnError) as e:
        cp.cpattn_varlen_bwd_plan(q_pos, k_pos, cu, 6, 4)
    assert e.value.status == 2
    assert cp.cpattn_bwd_query_workgroups(-1, 4) == -1
    assert cp.cpattn_bwd_query_workgroups(0, 4) == 0


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["docs8k_zigzag_cp4_h2_d128", "docs8k_zigzag_cp4_h4kv2_d64"])
def test_planned_gradients_bit_identical(name):
    """The share's backward plans, a random order and the unplanned calls give
    bit-identical dq, dk and dv."""
    import torch
    from test_backward import _reduced
    from test_gpu_parity import say
    from context_long_sequence_amd.share import bits_to_device, share_from_workload
    wl = _reduced()[name]
    say("%s: planned / random order / unplanned gradients" % name)
    share = share_from_workload(wl)
    assert share.bwd_plans is not None
    order = list(wl.arrival())
    share.step(order)
    dout = bits_to_device(wl.dout())
    res = []
    dq, dk, dv = share.backward(dout, order)
    res.append((dq.clone(), [x.clone() for x in dk], [x.clone() for x in dv]))
    rng = np.random.default_rng(5)
    share.bwd_plans = [pl[torch.from_numpy(rng.permutation(pl.numel())).cuda()].contiguous() for pl in share.bwd_plans]
    dq, dk, dv = share.backward(dout, order)
    res.append((dq.clone(), [x.clone() for x in dk], [x.clone() for x in dv]))
    share.bwd_plans = None
    dq, dk, dv = share.backward(dout, order)
    res.append((dq.clone(), [x.clone() for x in dk], [x.clone() for x in dv]))
    torch.cuda.synchronize()
    for other in res[1:]:
        assert torch.equal(res[0][0], other[0])
        assert all(torch.equal(a, b) for a, b in zip(res[0][1], other[1]))
        assert all(torch.equal(a, b) for a, b in zip(res[0][2], other[2]))
