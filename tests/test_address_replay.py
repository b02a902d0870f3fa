"""CPU replay of the kernels' address arithmetic (tests/address_replay.py) at
the launches of two GPU test cases that are kept off the GPU, and at the
other ragged backward cases:

* the full-size documents share (packed 131072 tokens of documents,
  per-document zig-zag cp 4, rank 1: 32768 queries x 32 heads, d 128,
  against four 32768-key blocks): the forward step as the backward test runs
  it (four single-block calls with documents, the first writing, the others
  accumulating), the same blocks without documents (the path that requests
  the first tiles before the searches), the multi-block call, and the
  backward (D = <dO, O>, then one gradient call per block);
* lq 257, lk 300, three query and three KV heads, causal, d 64 (forward,
  D and gradients), with the same random positions as the GPU test.

Every workgroup of every launch is replayed; each descriptor, offset and
index is checked against the extent of the tensor it addresses. A planted
out-of-range tile shows that the checks catch that class of mistake.
"""
import numpy as np
import pytest

import address_replay as ar


def say(msg):
    print("[address-replay] " + msg, flush=True)


def _documents_share():
    from synth import WORKLOADS
    from context_long_sequence_amd import cpattn_zigzag_index
    from context_long_sequence_amd.share import block_positions
    wl = WORKLOADS["docs128k_zigzag_cp4_h32_d128"]
    docs = wl.doc_lens()
    cu = np.concatenate([[0], np.cumsum(docs)]).astype(np.int32)
    q_pos, _ = cpattn_zigzag_index(wl.S, wl.cp, wl.rank, wl.layout, cu)
    kps = block_positions(wl.S, wl.cp, wl.n_blocks, wl.block_kind, wl.layout, cu)
    return wl, cu, q_pos, kps


def _fwd_mem(lq, hq, hkv, d, kps, cu=None, in_esz=2, out_esz=2, plan_len=0):
    sizes = dict(q=lq * hq * d * in_esz, o=lq * hq * d * out_esz, lse=hq * lq * 4, q_pos=lq * 4, null=0,
                 cu=0 if cu is None else len(cu) * 4, wg_plan=plan_len * 4)
    for b, kp in enumerate(kps):
        lk = len(kp)
        sizes.update({"k%d" % b: lk * hkv * d * in_esz, "v%d" % b: lk * hkv * d * in_esz, "kp%d" % b: lk * 4})
    return ar.Mem(**sizes)


def _arrays(q_pos, kps, cu=None):
    a = {"q_pos": np.asarray(q_pos, np.int32)}
    for b, kp in enumerate(kps):
        a["kp%d" % b] = np.asarray(kp, np.int32)
    if cu is not None:
        a["cu"] = np.asarray(cu, np.int32)
    return a


def _report(what, mem, extra=""):
    say("%s: replayed%s" % (what, extra))
    for line in mem.summary():
        say("  " + line)


@pytest.fixture(scope="module")
def documents():
    return _documents_share()


@pytest.mark.parametrize("with_documents", [True, False], ids=["documents", "no-documents"])
def test_documents_share_forward_block_calls(documents, with_documents):
    """The forward step of the documents share: one call per block in arrival
    order, the first writing O and LSE, the others accumulating into them.
    With documents the kernel searches before loading its first tiles; the
    same blocks without documents take the path that requests Q and the
    first three tiles before the searches. The document calls also run
    planned, as the share runs them (the plan from the library's planner)."""
    from context_long_sequence_amd import cpattn_varlen_plan
    wl, cu, q_pos, kps = documents
    plan_len = ar.fwd_workgroups(wl.lq, wl.hq, wl.hkv) * ar.PLAN_REC
    mem = _fwd_mem(wl.lq, wl.hq, wl.hkv, wl.d, kps, cu, plan_len=plan_len)
    sr = ar.Searches(mem, _arrays(q_pos, kps, cu))
    tiles = 0
    for planned in ((False, True) if with_documents else (False,)):
        for i, b in enumerate(wl.arrival()):
            plan = cpattn_varlen_plan(q_pos, kps[b], cu, wl.hq, wl.hkv, wl.d) if planned else None
            tiles += ar.replay_forward(mem, sr, lq=wl.lq, hq=wl.hq, hkv=wl.hkv, D=wl.d, in_bf16=True,
                                       out_bf16=True, causal=True, accumulate=i > 0,
                                       blocks=[("k%d" % b, "v%d" % b, "kp%d" % b, len(kps[b]))],
                                       varlen=with_documents, n_seqs=len(cu) - 1, plan=plan)
    _report("documents share forward (%s)" % ("documents" if with_documents else "no documents"), mem,
            ", %d K/V tiles over %d calls" % (tiles, 8 if with_documents else 4))
    assert tiles > 0


def test_documents_share_forward_with_a_wrong_plan(documents):
    """A plan made for other positions (seeded random records: tile ids, key
    ranges and flags far outside their ranges) stays inside every tensor: the
    kernel clamps each addressing value it takes from a record."""
    wl, cu, q_pos, kps = documents
    n_wg = ar.fwd_workgroups(wl.lq, wl.hq, wl.hkv)
    mem = _fwd_mem(wl.lq, wl.hq, wl.hkv, wl.d, kps, cu, plan_len=n_wg * ar.PLAN_REC)
    sr = ar.Searches(mem, _arrays(q_pos, kps, cu))
    rng = np.random.default_rng(7)
    b = wl.arrival()[0]
    plan = rng.integers(-2 ** 31, 2 ** 31 - 1, size=n_wg * ar.PLAN_REC, dtype=np.int64).astype(np.int32)
    tiles = ar.replay_forward(mem, sr, lq=wl.lq, hq=wl.hq, hkv=wl.hkv, D=wl.d, in_bf16=True, out_bf16=True,
                              causal=True, accumulate=True, blocks=[("k%d" % b, "v%d" % b, "kp%d" % b, len(kps[b]))],
                              varlen=True, n_seqs=len(cu) - 1, plan=plan)
    _report("documents share forward, random plan", mem, ", %d K/V tiles" % tiles)
    assert tiles > 0


def test_documents_share_forward_multi_block(documents):
    wl, cu, q_pos, kps = documents
    mem = _fwd_mem(wl.lq, wl.hq, wl.hkv, wl.d, kps, cu)
    sr = ar.Searches(mem, _arrays(q_pos, kps, cu))
    order = list(wl.arrival())
    tiles = ar.replay_forward(mem, sr, lq=wl.lq, hq=wl.hq, hkv=wl.hkv, D=wl.d, in_bf16=True, out_bf16=True,
                              causal=True, accumulate=False,
                              blocks=[("k%d" % b, "v%d" % b, "kp%d" % b, len(kps[b])) for b in order],
                              varlen=True, n_seqs=len(cu) - 1, multi=True)
    _report("documents share multi-block forward", mem, ", %d K/V tiles" % tiles)
    assert tiles > 0


def _bwd_mem(lq, lk, hq, hkv, d, cu=None):
    return ar.Mem(q=lq * hq * d * 2, dout=lq * hq * d * 2, o=lq * hq * d * 2, k=lk * hkv * d * 2,
                  v=lk * hkv * d * 2, lse=hq * lq * 4, delta=hq * lq * 4, q_pos=lq * 4, k_pos=lk * 4, null=0,
                  cu=0 if cu is None else len(cu) * 4, dq=lq * hq * d * 4, dk=lk * hkv * d * 4,
                  dv=lk * hkv * d * 4, dq_plan=(lq + 127) // 128 * hq * 4)


def test_documents_share_backward(documents):
    """D = <dO, O>, then one gradient call per block (the first writing dQ,
    the others adding to it), as the backward test runs them."""
    wl, cu, q_pos, kps = documents
    for i, b in enumerate(wl.arrival()):
        mem = _bwd_mem(wl.lq, len(kps[b]), wl.hq, wl.hkv, wl.d, cu)
        if i == 0:
            ar.replay_delta(mem, lq=wl.lq, hq=wl.hq, D=wl.d, o_esz=2, do_esz=2)
        sr = ar.Searches(mem, {"q_pos": q_pos, "k_pos": kps[b], "cu": cu})
        ar.replay_backward(mem, sr, lq=wl.lq, lk=len(kps[b]), hq=wl.hq, hkv=wl.hkv, D=wl.d, causal=True,
                           varlen=True, n_seqs=len(cu) - 1, acc_dq=i > 0)
        _report("documents share backward, block %d" % b, mem)


def _bwd_multi_mem(lq, lks, hq, hkv, d, cu=None):
    sizes = dict(q=lq * hq * d * 2, dout=lq * hq * d * 2, lse=hq * lq * 4, delta=hq * lq * 4, q_pos=lq * 4, null=0,
                 cu=0 if cu is None else len(cu) * 4, dq=lq * hq * d * 4)
    for b, lk in enumerate(lks):
        sizes.update({"k%d" % b: lk * hkv * d * 2, "v%d" % b: lk * hkv * d * 2, "kp%d" % b: lk * 4,
                      "dk%d" % b: lk * hkv * d * 4, "dv%d" % b: lk * hkv * d * 4})
    return ar.Mem(**sizes)


def test_documents_share_backward_multi(documents):
    """The gradients of the documents share's four blocks in one
    cpattn_partial_bwd_multi call (key kernel over all blocks, query kernel
    walking them), accumulating dQ and not."""
    wl, cu, q_pos, kps = documents
    order = list(wl.arrival())
    lks = [len(kps[b]) for b in order]
    for acc in (False, True):
        mem = _bwd_multi_mem(wl.lq, lks, wl.hq, wl.hkv, wl.d, cu)
        sr = ar.Searches(mem, _arrays(q_pos, [kps[b] for b in order], cu))
        ar.replay_backward_multi(mem, sr, lq=wl.lq, lks=lks, hq=wl.hq, hkv=wl.hkv, D=wl.d, causal=True,
                                 varlen=True, n_seqs=len(cu) - 1, acc_dq=acc)
        _report("documents share multi-block backward (accumulate_dq %d)" % acc, mem)


def test_multi_backward_blocks_of_every_size():
    """A multi-block gradient call with an empty block, a one-key block, a
    ragged block, a block no row sees and the 64K share's block shape, GQA,
    causal with and without grouped heads, both head dims."""
    rng = np.random.default_rng(5)
    for d, hq, hkv in ((64, 6, 3), (128, 4, 1)):
        lq = 301
        qp = np.sort(rng.choice(5000, lq, replace=False)).astype(np.int32) + 1000
        lks = [0, 1, 333, 64, 128]
        kps = [np.sort(rng.choice(6000, n, replace=False)).astype(np.int32) + 500 for n in lks]
        kps[3] = np.arange(9000, 9064, dtype=np.int32)   # after every row
        for causal in (True, False):
            mem = _bwd_multi_mem(lq, lks, hq, hkv, d)
            sr = ar.Searches(mem, _arrays(qp, kps))
            ar.replay_backward_multi(mem, sr, lq=lq, lks=lks, hq=hq, hkv=hkv, D=d, causal=causal, acc_dq=causal)
    # a block length past its tensors is caught
    with pytest.raises(ar.AccessError):
        mem = _bwd_multi_mem(10, [40], 1, 1, 64)
        sr = ar.Searches(mem, _arrays(np.arange(10, dtype=np.int32), [np.arange(40, dtype=np.int32)]))
        ar.replay_backward_multi(mem, sr, lq=10, lks=[40 * 200], hq=1, hkv=1, D=64, causal=True)


def test_documents_share_backward_planned(documents):
    """The planned gradient calls of the documents share (the library's plans
    of the query kernel's order), and one with a seeded random plan of values
    outside the tiles, which the kernel clamps."""
    from context_long_sequence_amd import cpattn_varlen_bwd_plan
    wl, cu, q_pos, kps = documents
    rng = np.random.default_rng(9)
    for i, b in enumerate(wl.arrival()):
        plan = cpattn_varlen_bwd_plan(q_pos, kps[b], cu, wl.hq, wl.hkv)
        if i == 0:
            plan = rng.integers(-5, len(plan) + 5, len(plan))
        mem = _bwd_mem(wl.lq, len(kps[b]), wl.hq, wl.hkv, wl.d, cu)
        sr = ar.Searches(mem, {"q_pos": q_pos, "k_pos": kps[b], "cu": cu})
        ar.replay_backward(mem, sr, lq=wl.lq, lk=len(kps[b]), hq=wl.hq, hkv=wl.hkv, D=wl.d, causal=True,
                           varlen=True, n_seqs=len(cu) - 1, acc_dq=i > 0, dq_order=plan)
        _report("documents share planned backward, block %d%s" % (b, " (random plan)" if i == 0 else ""), mem)


RAGGED = [(100, 77, 2, 1), (257, 300, 3, 3), (33, 1, 4, 2), (70, 130, 16, 1), (50, 40, 3, 1)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lq,lk,hq,hkv", RAGGED)
def test_ragged_forward_and_backward(lq, lk, hq, hkv, causal, d):
    """The ragged backward test's launches (its positions: the same seeded
    draw), forward with bf16 O, D, and both gradient kernels. (257, 300, 3,
    3, causal, d 64) is the case kept off the GPU."""
    rng = np.random.default_rng(lq * 7 + lk + d + causal)
    qp = np.sort(rng.choice(4 * (lq + lk), lq, replace=False)).astype(np.int32)
    kp = np.sort(rng.choice(4 * (lq + lk), lk, replace=False)).astype(np.int32)
    mem = _fwd_mem(lq, hq, hkv, d, [kp])
    sr = ar.Searches(mem, _arrays(qp, [kp]))
    ar.replay_forward(mem, sr, lq=lq, hq=hq, hkv=hkv, D=d, in_bf16=True, out_bf16=True, causal=causal,
                      accumulate=False, blocks=[("k0", "v0", "kp0", lk)])
    bmem = _bwd_mem(lq, lk, hq, hkv, d)
    ar.replay_delta(bmem, lq=lq, hq=hq, D=d, o_esz=2, do_esz=2)
    bsr = ar.Searches(bmem, {"q_pos": qp, "k_pos": kp})
    ar.replay_backward(bmem, bsr, lq=lq, lk=lk, hq=hq, hkv=hkv, D=d, causal=causal)
    if (lq, lk, hq, hkv, causal, d) == (257, 300, 3, 3, True, 64):
        _report("ragged 257 x 300, 3 heads, causal, d 64: forward", mem)
        _report("ragged 257 x 300, 3 heads, causal, d 64: backward", bmem)


def test_checks_catch_a_tile_past_the_block():
    """Planted mistakes the checks must catch: a direct-to-LDS tile load or a
    positions load asked for at or past the block's last key (a negative
    record count, a negative offset), and a register fetch whose descriptor
    covers one row too many."""
    c = ar.FwdCfg(True, 128)
    lk, hkv = 300, 3
    row_stride = hkv * 128 * 2
    mem = ar.Mem(k=lk * row_stride, kp=lk * 4)
    ar.load_tile(mem, c, "k", 0, row_stride, 256, lk, 0, False)  # the real tail tile passes
    with pytest.raises(ar.AccessError):
        ar.load_tile(mem, c, "k", 0, row_stride, 320, lk, 0, False)
    with pytest.raises(ar.AccessError):
        ar.load_positions(mem, "kp", 320, lk, 0, c.BK)
    with pytest.raises(ar.AccessError):
        mem.buffer("k", np.array([256 * row_stride]), np.array([45 * row_stride]),
                        ar.LANES * 16 + 44 * row_stride, 16)


def test_search_model_is_an_upper_bound():
    """The replay's model of the wave-cooperative search returns the first
    index whose value exceeds x (numpy's right-sided searchsorted), on
    ascending arrays with repeats, at every size up to a few rounds."""
    rng = np.random.default_rng(7)
    for n in [0, 1, 2, 63, 64, 65, 4095, 4096, 4097, 300000]:
        a = np.sort(rng.integers(0, max(1, n // 3), n)).astype(np.int32)
        mem = ar.Mem(a=n * 4)
        sr = ar.Searches(mem, {"a": a})
        xs = np.concatenate([[-1, 0, n, n // 3], rng.integers(-2, max(2, n // 3) + 2, 50)])
        got = sr.wave_upper_bound("a", n, xs)
        assert np.array_equal(got, np.searchsorted(a, xs, side="right")), n
        cu = np.concatenate([[0], np.sort(rng.choice(np.arange(1, 10 * n + 2), min(n, 40), replace=False))])
        sr2 = ar.Searches(ar.Mem(cu=len(cu) * 4), {"cu": cu.astype(np.int32)})
        x = rng.integers(0, 10 * n + 2, 20)
        ub = np.searchsorted(cu, x, side="right")
        assert np.array_equal(sr2.doc_start("cu", len(cu) - 1, x), cu[np.maximum(ub - 1, 0)])
        assert np.array_equal(sr2.doc_end("cu", len(cu) - 1, x),
                              np.where(ub < len(cu), cu[np.minimum(ub, len(cu) - 1)], ar.INT32_MAX))


def _f32_bwd_mem(lq, lk, hq, hkv, d, cu=None):
    return ar.Mem(q=lq * hq * d * 4, dout=lq * hq * d * 4, k=lk * hkv * d * 4, v=lk * hkv * d * 4,
                  lse=hq * lq * 4, delta=hq * lq * 4, q_pos=lq * 4, k_pos=lk * 4, null=0,
                  cu=0 if cu is None else len(cu) * 4, dq=lq * hq * d * 4, dk=lk * hkv * d * 4,
                  dv=lk * hkv * d * 4)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lq,lk,hq,hkv", [(100, 77, 2, 1), (129, 200, 4, 4), (33, 1, 4, 2), (70, 130, 16, 1),
                                          (256, 256, 1, 1), (0, 5, 2, 1), (5, 0, 2, 1)])
def test_float32_backward_ragged(lq, lk, hq, hkv, causal, d):
    """The float32 gradient kernels at the float32 GPU tests' shapes (and empty sides)."""
    rng = np.random.default_rng(lq * 11 + lk + d + causal)
    qp = np.sort(rng.choice(4 * (lq + lk) + 1, lq, replace=False)).astype(np.int32)
    kp = np.sort(rng.choice(4 * (lq + lk) + 1, lk, replace=False)).astype(np.int32)
    mem = _f32_bwd_mem(lq, lk, hq, hkv, d)
    ar.replay_backward_f32(mem, ar.Searches(mem, {"q_pos": qp, "k_pos": kp}), lq=lq, lk=lk, hq=hq, hkv=hkv, D=d,
                           causal=causal)


def test_float32_backward_documents():
    """The float32 gradient kernels on the reduced documents workloads of the float32 GPU tests."""
    from synth import WORKLOADS
    from context_long_sequence_amd import cpattn_zigzag_index
    from context_long_sequence_amd.share import block_positions
    base = WORKLOADS["docs128k_zigzag_cp4_h32_d128"]
    for wl in [base.scaled(S=8192, hq=2, hkv=2, docs=(256, 2048), dtype="f32"),
               base.scaled(S=4096, hq=4, hkv=1, d=64, docs=(128, 1024), dtype="f32")]:
        cu = np.concatenate([[0], np.cumsum(wl.doc_lens())]).astype(np.int32)
        q_pos, _ = cpattn_zigzag_index(wl.S, wl.cp, wl.rank, wl.layout, cu)
        kps = block_positions(wl.S, wl.cp, wl.n_blocks, wl.block_kind, wl.layout, cu)
        for kp in kps:
            mem = _f32_bwd_mem(wl.lq, len(kp), wl.hq, wl.hkv, wl.d, cu)
            ar.replay_backward_f32(mem, ar.Searches(mem, {"q_pos": q_pos, "k_pos": kp, "cu": cu}), lq=wl.lq,
                                   lk=len(kp), hq=wl.hq, hkv=wl.hkv, D=wl.d, causal=True, varlen=True,
                                   n_seqs=len(cu) - 1)
