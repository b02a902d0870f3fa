"""Gradients through the C ABI (cpattn_bwd_delta + cpattn_partial_bwd) against
the fp64 oracle's gradients.

Tolerance: the kernels round P and dS to bf16 (unit roundoff 2^-9) before the
matrix products and accumulate in float32; O reaches D = <dO, O> rounded to
bf16 by the forward. Each gradient element is a sum of terms that each carry
a relative error of a few units of 2^-9, so the error is a small multiple of
2^-9 times the size of the terms. The bar is max|g - g_ref| <= 1e-2 *
max|g_ref| per tensor (five units of 2^-9 relative to the largest gradient),
and the root-mean-square error <= 4e-3 * the root-mean-square of g_ref. A
reference that is exactly zero by cancellation must come out below 1e-5.
"""
import numpy as np
import pytest

from test_gpu_parity import oracle_block_positions, record, say

pytestmark = pytest.mark.gpu

GRAD_TOL_MAX = 1e-2
GRAD_TOL_RMS = 4e-3
# float32 inputs: every step in float32 (unit roundoff 2^-24) with the exp2
# unit's few-ulp error; the forward's LSE and O (and so D) carry errors of the
# same relative order. Sums over at most a few thousand terms keep the error
# near 1e-6 of the terms' size: the bar is 1e-4 of max|g_ref| and 2e-5 of its
# root-mean-square.
GRAD_TOL_MAX_F32 = 1e-4
GRAD_TOL_RMS_F32 = 2e-5


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle.get()


def grad_compare(got, ref, what, tol_max=GRAD_TOL_MAX, tol_rms=GRAD_TOL_RMS):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite gradient"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    rms_ref = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    rms_err = float(np.sqrt(np.mean((got - ref) ** 2))) if ref.size else 0.0
    say("%s: max err %.3e of max %.3e (%.2e), rms err %.3e of rms %.3e (%.2e)" % (
        what, err, scale, err / scale if scale else 0.0, rms_err, rms_ref, rms_err / rms_ref if rms_ref else 0.0))
    record(what, elements=int(ref.size), max_abs_err=err, max_abs_ref=scale, rms_err=rms_err, rms_ref=rms_ref,
           max_tol_rel=tol_max, rms_tol_rel=tol_rms)
    if scale == 0.0:
        # a reference that is zero by cancellation (one visible key: dP = D, so
        # dS = 0) comes out at float32 rounding level: D and dP are summed in
        # different orders; inputs here are of unit size
        assert err <= 1e-5, what + ": gradient must vanish"
        return
    assert err <= tol_max * scale, "%s: max error %.3e > %.1e * %.3e" % (what, err, tol_max, scale)
    assert rms_err <= tol_rms * rms_ref, "%s: rms error %.3e > %.1e * %.3e" % (what, rms_err, tol_rms, rms_ref)


def oracle_grads(orc, wl, rows=None, heads=None):
    """The oracle's gradients for a workload (positions from its own closed forms,
    keys of every block in block-id order); dk, dv split per block."""
    docs = wl.doc_lens()
    qp, qs = orc.local_positions(wl.S, wl.cp, wl.rank, wl.layout, doc_lens=docs)
    kps = oracle_block_positions(orc, wl, None, docs)
    k = wl.kv_all("k")
    v = wl.kv_all("v")
    from synth import bf16_bits_to_f32
    dout = wl.dout()
    dout = (dout if dout.dtype == np.float32 else bf16_bits_to_f32(dout)).astype(np.float64)
    dq, dk, dv, _ = orc.attention_grad(wl.q(), k, v, dout, qp, np.concatenate(kps), qs if docs is not None else None,
                                       True, rows=rows, heads=heads)
    if rows is not None:
        return dq, None, None
    bounds = np.cumsum([0] + [len(p) for p in kps])
    return dq, [dk[bounds[b]:bounds[b + 1]] for b in range(wl.n_blocks)], \
        [dv[bounds[b]:bounds[b + 1]] for b in range(wl.n_blocks)]


def _reduced():
    from synth import WORKLOADS as W
    zz64k, contig, docs, zz1m = (W["zigzag64k_cp8_h32_d128"], W["contig128k_h16kv2_d64"],
                                 W["docs128k_zigzag_cp4_h32_d128"], W["zigzag1m_cp8_h32kv8_d128"])
    wls = [
        W["zigzag1k_cp4_h1_d64_f32"].scaled(name="zigzag1k_cp4_h1_d64_bf16", dtype="bf16"),
        zz64k.scaled(name="zigzag4k_cp8_h4_d128", S=4096, hq=4, hkv=4),
        contig.scaled(name="contig1k_h16kv2_d64", S=1024),
        docs.scaled(name="docs8k_zigzag_cp4_h2_d128", S=8192, hq=2, hkv=2, docs=(256, 2048)),
        zz1m.scaled(name="zigzag4k_cp8_h8kv2_d128", S=4096, hq=8, hkv=2),
        # documents at d 64 with grouped KV heads
        docs.scaled(name="docs8k_zigzag_cp4_h4kv2_d64", S=8192, hq=4, hkv=2, d=64, sigma=1.0, docs=(256, 2048)),
    ]
    return {w.name: w for w in wls}


def _run(torch, wl):
    from context_long_sequence_amd.share import bits_to_device, share_from_workload
    share = share_from_workload(wl)
    order = list(wl.arrival())
    share.step(order, "accumulate")
    dout = bits_to_device(wl.dout())
    dq, dk, dv = share.backward(dout, order)
    torch.cuda.synchronize()
    return share, dout, dq, dk, dv


@pytest.mark.parametrize("name", ["zigzag1k_cp4_h1_d64_bf16", "zigzag4k_cp8_h4_d128", "contig1k_h16kv2_d64",
                                  "docs8k_zigzag_cp4_h2_d128", "zigzag4k_cp8_h8kv2_d128",
                                  "docs8k_zigzag_cp4_h4kv2_d64"])
def test_backward_reduced_all(torch_cuda, orc, name):
    wl = _reduced()[name]
    say("backward %s: S=%d cp=%d hq=%d hkv=%d d=%d blocks=%d" % (name, wl.S, wl.cp, wl.hq, wl.hkv, wl.d, wl.n_blocks))
    _, _, dq, dk, dv = _run(torch_cuda, wl)
    rdq, rdk, rdv = oracle_grads(orc, wl)
    grad_compare(dq.cpu().numpy(), rdq, name + " dq")
    grad_compare(np.concatenate([x.cpu().numpy() for x in dk]), np.concatenate(rdk), name + " dk")
    grad_compare(np.concatenate([x.cpu().numpy() for x in dv]), np.concatenate(rdv), name + " dv")


def _large(name):
    """A full-size workload, or the documents workload at half its length
    (65536 packed tokens of log-uniform [1K, 32K] documents, per-document
    zig-zag cp 4, rank 1: 16384 queries x 32 heads, d 128, vs 4 blocks)."""
    from synth import WORKLOADS
    if name == "docs64k_zigzag_cp4_h32_d128":
        return WORKLOADS["docs128k_zigzag_cp4_h32_d128"].scaled(name="docs64k_zigzag_cp4_h32_d128", S=65536)
    return WORKLOADS[name]


# The full-size documents case faulted the GPU once, in its forward step, with
# a forward kernel that staged V transposed; that kernel was taken out, no
# cause was shown, and the case stays off the GPU until one is. (The CPU
# replay in test_address_replay.py finds every address of the committed
# kernels in range at this shape.) (The full-size
# documents forward is still compared with the oracle by the forward parity
# tests, and the documents backward at half length here and at reduced sizes.)
@pytest.mark.parametrize("name", ["zigzag64k_cp8_h32_d128",
                                  pytest.param("docs128k_zigzag_cp4_h32_d128", marks=pytest.mark.skip(
                                      reason="faulted the GPU with an earlier forward-kernel variant; "
                                             "cause not yet shown")),
                                  "docs64k_zigzag_cp4_h32_d128", "zigzag1m_cp8_h32kv8_d128",
                                  "contig128k_h16kv2_d64"])
def test_backward_full_size_sampled(torch_cuda, orc, name):
    """Full-size workloads (the 64K-token zig-zag share, the 128K-token
    documents share, the 1M-token GQA share, the 128K-token Ulysses head
    share at d 64) in the launch configuration the
    benchmark times: dq on sampled rows against the oracle; dk, dv of every
    key through invariants that hold at any size (each row's dS sums to zero
    over its keys, so dK sums to zero over all keys of a KV head; each row's
    P sums to one and every row sees at least its own key, so dV sums to the
    rows' dO over the query heads of the KV head)."""
    from synth import bf16_bits_to_f32
    wl = _large(name)
    say("backward %s full size: S=%d cp=%d hq=%d hkv=%d d=%d blocks=%d" % (name, wl.S, wl.cp, wl.hq, wl.hkv, wl.d,
                                                                          wl.n_blocks))
    share, dout, dq, dk, dv = _run(torch_cuda, wl)
    # dQ rows: as many as the forward checks (interior rows on top of every chunk's ends)
    from test_gpu_parity import FULL_SAMPLES
    rows, heads = wl.sample_pairs(n_pairs=FULL_SAMPLES.get(name, 8192))
    rdq, _, _ = oracle_grads(orc, wl, rows=rows, heads=heads)
    grad_compare(dq.cpu().numpy()[rows, heads], rdq, "%s dq (sampled)" % name)
    torch = torch_cuda
    group = wl.hq // wl.hkv
    ksum = torch.zeros((wl.hkv, wl.d), dtype=torch.float64, device="cuda")
    kabs = torch.zeros_like(ksum)
    vsum = torch.zeros_like(ksum)
    for b in range(wl.n_blocks):
        x = dk[b].double()
        ksum += x.sum(0)
        kabs += x.abs().sum(0)
        vsum += dv[b].double().sum(0)
    rel = float((ksum.abs() / kabs).max())
    say("%s: max |sum_j dK_j| / sum_j |dK_j| = %.3e" % (name, rel))
    assert rel <= 1e-3
    do64 = torch.from_numpy(bf16_bits_to_f32(wl.dout()).astype(np.float64)).cuda()
    want = do64.sum(0).reshape(wl.hkv, group, wl.d).sum(1)
    err = float((vsum - want).abs().max() / want.abs().max())
    say("%s: max |sum_j dV_j - sum_i dO_i| / max = %.3e" % (name, err))
    assert err <= 1e-3
    del share, dq, dk, dv
    torch.cuda.empty_cache()


def test_backward_deterministic_and_accumulate(torch_cuda):
    wl = _reduced()["zigzag4k_cp8_h8kv2_d128"]
    torch = torch_cuda
    from context_long_sequence_amd import cpattn_partial_bwd
    share, dout, dq, dk, dv = _run(torch, wl)
    dq1, dk1, dv1 = dq.clone(), [x.clone() for x in dk], [x.clone() for x in dv]
    share.backward(dout, list(wl.arrival()))
    torch.cuda.synchronize()
    assert torch.equal(dq, dq1) and all(torch.equal(a, b) for a, b in zip(dk, dk1))
    assert all(torch.equal(a, b) for a, b in zip(dv, dv1))
    # accumulate_dkv adds: a second call on the same block doubles its dk, dv (exactly: x + x)
    b = 3
    dqx = torch.zeros_like(dq)
    cpattn_partial_bwd(share.q, share.k_blocks[b], share.v_blocks[b], dout, share.q_pos, share.k_pos_blocks[b],
                       share.lse, share.delta, dqx, dk[b], dv[b], accumulate_dq=True, accumulate_dkv=True)
    torch.cuda.synchronize()
    assert torch.equal(dk[b], 2 * dk1[b]) and torch.equal(dv[b], 2 * dv1[b])


def _rand_bf16(torch, shape, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * 0.7).to(torch.bfloat16).cuda()


def _ragged_cases():
    out = []
    for lq, lk, hq, hkv in [(100, 77, 2, 1), (257, 300, 3, 3), (33, 1, 4, 2), (70, 130, 16, 1), (50, 40, 3, 1)]:
        for causal in (True, False):
            for d in (64, 128):
                marks = ()
                if (lq, lk, hq, hkv, causal, d) == (257, 300, 3, 3, True, 64):
                    # This case faulted the GPU once, with a query-gradient kernel that
                    # fetched two tiles ahead; that kernel was taken out, no cause was
                    # shown, and the case stays off the GPU until one is (the CPU replay
                    # in test_address_replay.py finds the committed kernels in range here).
                    marks = (pytest.mark.skip(reason="faulted the GPU with an earlier query-kernel variant; "
                                                     "cause not yet shown"),)
                out.append(pytest.param(d, causal, lq, lk, hq, hkv, marks=marks,
                                        id="%d-%d-%d-%d-%s-%d" % (lq, lk, hq, hkv, causal, d)))
    return out


@pytest.mark.parametrize("d,causal,lq,lk,hq,hkv", _ragged_cases())
def test_backward_ragged_random_positions(torch_cuda, orc, d, causal, lq, lk, hq, hkv):
    """Ragged sizes (not multiples of any tile), random ascending positions,
    GQA, one block: dq, dk, dv against the oracle."""
    torch = torch_cuda
    from context_long_sequence_amd import cpattn_bwd_delta, cpattn_partial, cpattn_partial_bwd
    say("ragged d=%d causal=%d lq=%d lk=%d hq=%d hkv=%d" % (d, causal, lq, lk, hq, hkv))
    rng = np.random.default_rng(lq * 7 + lk + d + causal)
    qp = np.sort(rng.choice(4 * (lq + lk), lq, replace=False)).astype(np.int32)
    kp = np.sort(rng.choice(4 * (lq + lk), lk, replace=False)).astype(np.int32)
    q = _rand_bf16(torch, (lq, hq, d), 1)
    k = _rand_bf16(torch, (lk, hkv, d), 2)
    v = _rand_bf16(torch, (lk, hkv, d), 3)
    dout = _rand_bf16(torch, (lq, hq, d), 4)
    qpd, kpd = torch.from_numpy(qp).cuda(), torch.from_numpy(kp).cuda()
    o = torch.empty((lq, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, lq), dtype=torch.float32, device="cuda")
    cpattn_partial(q, k, v, qpd, kpd, o, lse, causal=causal)
    delta = torch.empty((hq, lq), dtype=torch.float32, device="cuda")
    cpattn_bwd_delta(o, dout, delta)
    dq = torch.full((lq, hq, d), float("nan"), device="cuda")
    dk = torch.full((lk, hkv, d), float("nan"), device="cuda")
    dv = torch.full((lk, hkv, d), float("nan"), device="cuda")
    cpattn_partial_bwd(q, k, v, dout, qpd, kpd, lse, delta, dq, dk, dv, causal=causal)
    torch.cuda.synchronize()

    def bits(t):
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    from synth import bf16_bits_to_f32
    rdq, rdk, rdv, rdelta = orc.attention_grad(bits(q), bits(k), bits(v), bf16_bits_to_f32(bits(dout)), qp, kp,
                                               None, causal)
    grad_compare(dq.cpu().numpy(), rdq, "ragged dq")
    grad_compare(dk.cpu().numpy(), rdk, "ragged dk")
    grad_compare(dv.cpu().numpy(), rdv, "ragged dv")
    # D against the oracle's <dO, O> (O here is the kernel's bf16 output: within its rounding)
    err = float(np.max(np.abs(delta.cpu().numpy().T - rdelta)))
    say("ragged delta: max err %.3e" % err)
    assert err <= 2e-2 * max(1.0, float(np.max(np.abs(rdelta))))


def test_backward_empty_and_invisible_blocks(torch_cuda):
    """lk = 0 leaves dq as it is (accumulating) or zero; a block every key of
    which lies after every query gets dk = dv = 0 and adds nothing to dq;
    lq = 0 gives dk = dv = 0."""
    torch = torch_cuda
    from context_long_sequence_amd import cpattn_partial_bwd
    lq, lk, hq, hkv, d = 64, 96, 2, 2, 128
    q = _rand_bf16(torch, (lq, hq, d), 5)
    dout = _rand_bf16(torch, (lq, hq, d), 6)
    k = _rand_bf16(torch, (lk, hkv, d), 7)
    v = _rand_bf16(torch, (lk, hkv, d), 8)
    qp = torch.arange(lq, dtype=torch.int32, device="cuda")
    kp_late = torch.arange(1000, 1000 + lk, dtype=torch.int32, device="cuda")
    lse = torch.zeros((hq, lq), device="cuda")
    delta = torch.zeros((hq, lq), device="cuda")
    dq = torch.randn((lq, hq, d), device="cuda")
    dq0 = dq.clone()
    dk = torch.full((lk, hkv, d), float("nan"), device="cuda")
    dv = torch.full((lk, hkv, d), float("nan"), device="cuda")
    cpattn_partial_bwd(q, k, v, dout, qp, kp_late, lse, delta, dq, dk, dv, accumulate_dq=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0) and bool((dk == 0).all()) and bool((dv == 0).all())
    e = torch.empty((0, hkv, d), dtype=torch.bfloat16, device="cuda")
    ef = torch.empty((0, hkv, d), device="cuda")
    ep = torch.empty((0,), dtype=torch.int32, device="cuda")
    cpattn_partial_bwd(q, e, e, dout, qp, ep, lse, delta, dq, ef, ef, accumulate_dq=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0)
    cpattn_partial_bwd(q, e, e, dout, qp, ep, lse, delta, dq, ef, ef, accumulate_dq=False)
    torch.cuda.synchronize()
    assert bool((dq == 0).all())
    eq = torch.empty((0, hq, d), dtype=torch.bfloat16, device="cuda")
    cpattn_partial_bwd(eq, k, v, eq, torch.empty((0,), dtype=torch.int32, device="cuda"), kp_late,
                       torch.empty((hq, 0), device="cuda"), torch.empty((hq, 0), device="cuda"),
                       torch.empty((0, hq, d), device="cuda"), dk, dv)
    torch.cuda.synchronize()
    assert bool((dk == 0).all()) and bool((dv == 0).all())


# ---------------------------------------------------------------------------
# float32 inputs (the float32 kernels: every step in float32)

def _f32_workloads():
    from synth import WORKLOADS as W
    return {w.name: w for w in [
        W["zigzag1k_cp4_h1_d64_f32"],
        W["zigzag64k_cp8_h32_d128"].scaled(name="zigzag2k_cp8_h4kv2_d128_f32", S=2048, hq=4, hkv=2, dtype="f32"),
        W["docs128k_zigzag_cp4_h32_d128"].scaled(name="docs8k_zigzag_cp4_h2_d128_f32", S=8192, hq=2, hkv=2,
                                                 docs=(256, 2048), dtype="f32"),
        W["docs128k_zigzag_cp4_h32_d128"].scaled(name="docs4k_zigzag_cp4_h4kv1_d64_f32", S=4096, hq=4, hkv=1, d=64,
                                                 sigma=1.0, docs=(128, 1024), dtype="f32"),
    ]}


@pytest.mark.parametrize("name", ["zigzag1k_cp4_h1_d64_f32", "zigzag2k_cp8_h4kv2_d128_f32",
                                  "docs8k_zigzag_cp4_h2_d128_f32", "docs4k_zigzag_cp4_h4kv1_d64_f32"])
def test_backward_float32_inputs(torch_cuda, orc, name):
    """float32 q, k, v, dO (the 1K-token float32 workload, GQA and documents at
    reduced sizes): the forward step and one gradient call per block, against
    the oracle's gradients on every row and key."""
    wl = _f32_workloads()[name]
    say("backward float32 %s: S=%d cp=%d hq=%d hkv=%d d=%d blocks=%d" % (name, wl.S, wl.cp, wl.hq, wl.hkv, wl.d,
                                                                          wl.n_blocks))
    share, _, dq, dk, dv = _run(torch_cuda, wl)
    assert share.q.dtype == torch_cuda.float32 and share.o.dtype == torch_cuda.float32
    rdq, rdk, rdv = oracle_grads(orc, wl)
    tol = dict(tol_max=GRAD_TOL_MAX_F32, tol_rms=GRAD_TOL_RMS_F32)
    grad_compare(dq.cpu().numpy(), rdq, name + " dq", **tol)
    grad_compare(np.concatenate([x.cpu().numpy() for x in dk]), np.concatenate(rdk), name + " dk", **tol)
    grad_compare(np.concatenate([x.cpu().numpy() for x in dv]), np.concatenate(rdv), name + " dv", **tol)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lq,lk,hq,hkv", [(100, 77, 2, 1), (129, 200, 4, 4), (33, 1, 4, 2), (70, 130, 16, 1)])
def test_backward_float32_ragged(torch_cuda, orc, d, causal, lq, lk, hq, hkv):
    """float32 inputs at ragged sizes with random ascending positions, one
    block: the forward, D and the gradients against the oracle."""
    torch = torch_cuda
    from context_long_sequence_amd import cpattn_bwd_delta, cpattn_partial, cpattn_partial_bwd
    say("float32 ragged d=%d causal=%d lq=%d lk=%d hq=%d hkv=%d" % (d, causal, lq, lk, hq, hkv))
    rng = np.random.default_rng(lq * 11 + lk + d + causal)
    qp = np.sort(rng.choice(4 * (lq + lk), lq, replace=False)).astype(np.int32)
    kp = np.sort(rng.choice(4 * (lq + lk), lk, replace=False)).astype(np.int32)

    def rnd(shape, seed):
        return torch.randn(shape, generator=torch.Generator().manual_seed(seed)) * 0.7
    q, k, v, dout = rnd((lq, hq, d), 11), rnd((lk, hkv, d), 12), rnd((lk, hkv, d), 13), rnd((lq, hq, d), 14)
    qg, kg, vg, dg = (x.cuda() for x in (q, k, v, dout))
    qpd, kpd = torch.from_numpy(qp).cuda(), torch.from_numpy(kp).cuda()
    o = torch.empty((lq, hq, d), device="cuda")
    lse = torch.empty((hq, lq), device="cuda")
    cpattn_partial(qg, kg, vg, qpd, kpd, o, lse, causal=causal)
    delta = torch.empty((hq, lq), device="cuda")
    cpattn_bwd_delta(o, dg, delta)
    dq = torch.full((lq, hq, d), float("nan"), device="cuda")
    dk = torch.full((lk, hkv, d), float("nan"), device="cuda")
    dv = torch.full((lk, hkv, d), float("nan"), device="cuda")
    cpattn_partial_bwd(qg, kg, vg, dg, qpd, kpd, lse, delta, dq, dk, dv, causal=causal)
    torch.cuda.synchronize()
    rdq, rdk, rdv, _ = orc.attention_grad(q.numpy(), k.numpy(), v.numpy(), dout.numpy().astype(np.float64), qp, kp,
                                          None, causal)
    tol = dict(tol_max=GRAD_TOL_MAX_F32, tol_rms=GRAD_TOL_RMS_F32)
    grad_compare(dq.cpu().numpy(), rdq, "float32 ragged dq", **tol)
    grad_compare(dk.cpu().numpy(), rdk, "float32 ragged dk", **tol)
    grad_compare(dv.cpu().numpy(), rdv, "float32 ragged dv", **tol)
