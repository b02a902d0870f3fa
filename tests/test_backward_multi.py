"""The multi-block gradient call (cpattn_partial_bwd_multi) through the C ABI:
against the fp64 oracle's gradients, and against one cpattn_partial_bwd call
per block.

Every block's dk, dv come from the same key-kernel code as the per-block call
(only the grid spans the blocks), so they must be bit-identical to it. dq is
summed over the blocks in float32 registers and stored once, where the
per-block calls scale and add it to the stored float32 dq after every block:
the two differ by float32 rounding of a sum over at most a few dozen blocks,
bounded here by 1e-5 of max|dq| (about 80 float32 units of the largest
element); against the oracle dq holds the per-block call's bar (see
test_backward.py).
"""
import numpy as np
import pytest

from test_backward import _large, _reduced, grad_compare, oracle_grads
from test_gpu_parity import say

pytestmark = pytest.mark.gpu

MULTI_VS_BLOCKS_TOL = 1e-5


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


def _both(torch, wl):
    """One forward step, then the backward per block and fused; returns the
    share and both results (per-block dk, dv in block-id order)."""
    from context_long_sequence_amd.share import bits_to_device, share_from_workload
    share = share_from_workload(wl)
    order = list(wl.arrival())
    share.step(order, "accumulate")
    dout = bits_to_device(wl.dout())
    dq, dk, dv = share.backward(dout, order)
    torch.cuda.synchronize()
    blocks = (dq.clone(), [x.clone() for x in dk], [x.clone() for x in dv])
    for t in [share.dq] + share.dk + share.dv:
        t.fill_(float("nan"))
    dq, dk, dv = share.backward(dout, order, mode="fused")
    torch.cuda.synchronize()
    return share, dout, blocks, (dq, dk, dv)


def _same_keys_close_dq(torch, name, blocks, fused):
    for b, (x, y) in enumerate(zip(blocks[1], fused[1])):
        assert torch.equal(x, y), "%s: dk of block %d differs from the per-block call" % (name, b)
    for b, (x, y) in enumerate(zip(blocks[2], fused[2])):
        assert torch.equal(x, y), "%s: dv of block %d differs from the per-block call" % (name, b)
    assert bool(torch.isfinite(fused[0]).all()), name + ": non-finite dq"
    scale = float(blocks[0].abs().max())
    diff = float((fused[0] - blocks[0]).abs().max())
    say("%s: fused vs per-block: dk, dv bit-identical; max |ddq| %.3e of max %.3e" % (name, diff, scale))
    assert diff <= MULTI_VS_BLOCKS_TOL * scale


@pytest.mark.parametrize("name", ["zigzag1k_cp4_h1_d64_bf16", "zigzag4k_cp8_h4_d128", "contig1k_h16kv2_d64",
                                  "docs8k_zigzag_cp4_h2_d128", "zigzag4k_cp8_h8kv2_d128",
                                  "docs8k_zigzag_cp4_h4kv2_d64"])
def test_backward_multi_reduced_all(torch_cuda, orc, name):
    """Every reduced workload (all rows): the fused call against the oracle,
    and against the per-block calls."""
    wl = _reduced()[name]
    say("backward multi %s: S=%d cp=%d hq=%d hkv=%d d=%d blocks=%d" % (name, wl.S, wl.cp, wl.hq, wl.hkv, wl.d,
                                                                      wl.n_blocks))
    _, _, blocks, fused = _both(torch_cuda, wl)
    _same_keys_close_dq(torch_cuda, name, blocks, fused)
    rdq, rdk, rdv = oracle_grads(orc, wl)
    grad_compare(fused[0].cpu().numpy(), rdq, name + " multi dq")
    grad_compare(np.concatenate([x.cpu().numpy() for x in fused[1]]), np.concatenate(rdk), name + " multi dk")
    grad_compare(np.concatenate([x.cpu().numpy() for x in fused[2]]), np.concatenate(rdv), name + " multi dv")


@pytest.mark.parametrize("name", ["zigzag64k_cp8_h32_d128", "zigzag1m_cp8_h32kv8_d128"])
def test_backward_multi_full_size(torch_cuda, orc, name):
    """Full-size shares in the launch configuration the benchmark times: dq on
    sampled rows against the oracle, dk, dv bit for bit and dq to float32
    rounding against the per-block calls."""
    wl = _large(name)
    say("backward multi %s full size: S=%d cp=%d hq=%d hkv=%d d=%d blocks=%d" % (name, wl.S, wl.cp, wl.hq, wl.hkv,
                                                                                 wl.d, wl.n_blocks))
    share, _, blocks, fused = _both(torch_cuda, wl)
    _same_keys_close_dq(torch_cuda, name, blocks, fused)
    from test_gpu_parity import FULL_SAMPLES
    rows, heads = wl.sample_pairs(n_pairs=FULL_SAMPLES.get(name, 8192))
    rdq, _, _ = oracle_grads(orc, wl, rows=rows, heads=heads)
    grad_compare(fused[0].cpu().numpy()[rows, heads], rdq, "%s multi dq (sampled)" % name)
    del share, blocks, fused
    torch_cuda.cuda.empty_cache()


def test_backward_multi_empty_invisible_accumulate(torch_cuda):
    """Blocks without keys and blocks no row sees, among visible ones:
    accumulate_dq adds the visible blocks' share to dq and leaves it alone
    when no block is seen; the invisible block's dk, dv are zero (or, with
    accumulate_dkv, unchanged); two calls give identical results."""
    torch = torch_cuda
    from test_backward import _rand_bf16
    from context_long_sequence_amd import (cpattn_bwd_delta, cpattn_partial_bwd, cpattn_partial_bwd_multi,
                                           cpattn_partial_multi)
    lq, hq, hkv, d = 200, 4, 2, 128
    q = _rand_bf16(torch, (lq, hq, d), 11)
    dout = _rand_bf16(torch, (lq, hq, d), 12)
    qp = torch.arange(1000, 1000 + lq, dtype=torch.int32, device="cuda")
    lks = [150, 0, 90, 130]
    starts = [1050, 0, 5000, 900]   # block 2: every key after every row
    ks = [_rand_bf16(torch, (n, hkv, d), 20 + b) for b, n in enumerate(lks)]
    vs = [_rand_bf16(torch, (n, hkv, d), 30 + b) for b, n in enumerate(lks)]
    kps = [torch.arange(s, s + n, dtype=torch.int32, device="cuda") for s, n in zip(starts, lks)]
    o = torch.empty((lq, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, lq), dtype=torch.float32, device="cuda")
    cpattn_partial_multi(q, ks, vs, qp, kps, o, lse)
    delta = torch.empty((hq, lq), dtype=torch.float32, device="cuda")
    cpattn_bwd_delta(o, dout, delta)
    # per-block reference
    dq_ref = torch.zeros((lq, hq, d), device="cuda")
    dk_ref = [torch.empty((n, hkv, d), device="cuda") for n in lks]
    dv_ref = [torch.empty((n, hkv, d), device="cuda") for n in lks]
    for b in range(len(lks)):
        cpattn_partial_bwd(q, ks[b], vs[b], dout, qp, kps[b], lse, delta, dq_ref, dk_ref[b], dv_ref[b],
                           accumulate_dq=True)
    base = torch.randn((lq, hq, d), device="cuda")
    dq = base.clone()
    dk = [torch.full((n, hkv, d), float("nan"), device="cuda") for n in lks]
    dv = [torch.full((n, hkv, d), float("nan"), device="cuda") for n in lks]
    cpattn_partial_bwd_multi(q, ks, vs, dout, qp, kps, lse, delta, dq, dk, dv, accumulate_dq=True)
    torch.cuda.synchronize()
    for b in range(len(lks)):
        assert torch.equal(dk[b], dk_ref[b]) and torch.equal(dv[b], dv_ref[b]), b
    assert bool((dk[2] == 0).all()) and bool((dv[2] == 0).all())
    diff = float((dq - base - dq_ref).abs().max())
    assert diff <= 1e-5 * float(dq_ref.abs().max()) + 1e-6, diff
    # determinism: the same call again, written (not accumulated)
    dq1 = torch.empty_like(dq)
    dq2 = torch.empty_like(dq)
    cpattn_partial_bwd_multi(q, ks, vs, dout, qp, kps, lse, delta, dq1, dk, dv)
    cpattn_partial_bwd_multi(q, ks, vs, dout, qp, kps, lse, delta, dq2, dk, dv)
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2)
    # accumulate_dkv doubles every block's dk, dv exactly
    cpattn_partial_bwd_multi(q, ks, vs, dout, qp, kps, lse, delta, dq2, dk, dv, accumulate_dkv=True)
    torch.cuda.synchronize()
    for b in range(len(lks)):
        assert torch.equal(dk[b], 2 * dk_ref[b]) and torch.equal(dv[b], 2 * dv_ref[b]), b
    # only the invisible block and the empty one: dq left as it is when accumulating, zero otherwise
    dq3 = base.clone()
    cpattn_partial_bwd_multi(q, [ks[1], ks[2]], [vs[1], vs[2]], dout, qp, [kps[1], kps[2]], lse, delta, dq3,
                             [dk[1], dk[2]], [dv[1], dv[2]], accumulate_dq=True)
    torch.cuda.synchronize()
    assert torch.equal(dq3, base)
    cpattn_partial_bwd_multi(q, [ks[1], ks[2]], [vs[1], vs[2]], dout, qp, [kps[1], kps[2]], lse, delta, dq3,
                             [dk[1], dk[2]], [dv[1], dv[2]])
    torch.cuda.synchronize()
    assert bool((dq3 == 0).all())


def test_backward_multi_float32_inputs(torch_cuda):
    """float32 inputs run the single-block kernels block after block: the
    result equals the per-block calls bit for bit."""
    from synth import WORKLOADS
    wl = WORKLOADS["zigzag1k_cp4_h1_d64_f32"]
    _, _, blocks, fused = _both(torch_cuda, wl)
    assert torch_cuda.equal(blocks[0], fused[0])
    assert all(torch_cuda.equal(x, y) for x, y in zip(blocks[1], fused[1]))
    assert all(torch_cuda.equal(x, y) for x, y in zip(blocks[2], fused[2]))
