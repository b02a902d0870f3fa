"""The multi-block call (several arrived KV blocks in one launch) on the GPU:
against the oracle on every row of the reduced workloads and on sampled rows
at full size, against the single-block call, with an accumulated start, and
with empty and invisible blocks among the blocks."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("name", ["zigzag1k_cp4_h1_d64_f32", "zigzag4k_cp8_h4_d128", "contig2k_h16kv2_d64",
                                  "docs8k_zigzag_cp4_h4_d128", "zigzag16k_cp8_h8kv2_d128"])
def test_fused_all_rows(torch_cuda, orc, name):
    from context_long_sequence_amd.share import share_from_workload
    from test_gpu_parity import O_TOL_BF16, O_TOL_F32, _reduced, compare, oracle_share, say, to_np
    wl = _reduced()[name]
    say("%s fused: %d blocks" % (name, wl.n_blocks))
    share = share_from_workload(wl)
    o, lse = share.step(wl.arrival(), "fused")
    torch_cuda.cuda.synchronize()
    o, lse = to_np(o, lse)
    o_ref, lse_ref, _ = oracle_share(orc, wl)
    compare(o, lse, o_ref, lse_ref, None, None, O_TOL_F32 if wl.dtype == "f32" else O_TOL_BF16, name + " fused")


def test_fused_one_block_equals_single_block_call(torch_cuda):
    """One block through the multi-block kernel is the single-block call, bit for bit."""
    from context_long_sequence_amd.share import share_from_workload
    from test_gpu_parity import _reduced
    for name in ("zigzag4k_cp8_h4_d128", "docs8k_zigzag_cp4_h4_d128", "zigzag16k_cp8_h8kv2_d128"):
        wl = _reduced()[name]
        share = share_from_workload(wl)
        for b in range(wl.n_blocks):
            for acc in (False, True):
                share.call_block(0, share.o, share.lse, accumulate=False)
                o0, l0 = share.o.clone(), share.lse.clone()
                share.call_block(b, share.o, share.lse, accumulate=acc)
                o1, l1 = share.o.clone(), share.lse.clone()
                share.o.copy_(o0)
                share.lse.copy_(l0)
                share.call_multi([b], share.o, share.lse, accumulate=acc)
                torch_cuda.cuda.synchronize()
                assert torch_cuda.equal(share.o, o1) and torch_cuda.equal(share.lse, l1), (name, b, acc)


def test_fused_accumulate_and_split_order(torch_cuda, orc):
    """First half of the arrivals fused, the rest fused on top (accumulate), in
    another order: the union of all blocks."""
    from context_long_sequence_amd.share import share_from_workload
    from test_gpu_parity import O_TOL_BF16, _reduced, compare, oracle_share, to_np
    wl = _reduced()["zigzag4k_cp8_h4_d128"]
    share = share_from_workload(wl)
    order = list(wl.arrival())[::-1]
    share.call_multi(order[:3], share.o, share.lse, accumulate=False)
    share.call_multi(order[3:], share.o, share.lse, accumulate=True)
    torch_cuda.cuda.synchronize()
    o, lse = to_np(share.o, share.lse)
    o_ref, lse_ref, _ = oracle_share(orc, wl)
    compare(o, lse, o_ref, lse_ref, None, None, O_TOL_BF16, wl.name + " fused 3 + 5")


def test_fused_with_empty_and_invisible_blocks(torch_cuda):
    import torch
    from context_long_sequence_amd import cpattn_partial, cpattn_partial_multi
    from test_gpu_parity import _rand_dev
    lq, hq, d = 96, 2, 128
    q = _rand_dev((lq, hq, d), 1, "bf16")
    k = _rand_dev((64, hq, d), 2, "bf16")
    v = _rand_dev((64, hq, d), 3, "bf16")
    qp = torch.arange(100, 100 + lq, dtype=torch.int32, device="cuda")
    kp_past = torch.arange(0, 64, dtype=torch.int32, device="cuda")        # seen by every row
    kp_future = torch.arange(1000, 1064, dtype=torch.int32, device="cuda")  # seen by no row
    k0 = torch.empty((0, hq, d), dtype=torch.bfloat16, device="cuda")
    kp0 = torch.empty((0,), dtype=torch.int32, device="cuda")
    o = torch.empty((lq, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, lq), dtype=torch.float32, device="cuda")
    o1, l1 = torch.empty_like(o), torch.empty_like(lse)
    cpattn_partial(q, k, v, qp, kp_past, o1, l1, accumulate=False)
    cpattn_partial_multi(q, [k0, k, k, k], [k0, v, v, v], qp, [kp0, kp_future, kp_past, kp_future], o, lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, l1)
    cpattn_partial_multi(q, [k, k0], [v, k0], qp, [kp_future, kp0], o, lse)
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))
    o.copy_(q)
    lse.fill_(0.5)
    o0, l0 = o.clone(), lse.clone()
    cpattn_partial_multi(q, [k, k0], [v, k0], qp, [kp_future, kp0], o, lse, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)


@pytest.mark.parametrize("name", ["zigzag64k_cp8_h32_d128", "zigzag1m_cp8_h32kv8_d128"])
def test_fused_full_size_sampled(torch_cuda, orc, name):
    from context_long_sequence_amd.share import share_from_workload
    from synth import WORKLOADS
    from test_gpu_parity import FULL_SAMPLES, O_TOL_BF16, compare, oracle_share, say, to_np
    wl = WORKLOADS[name]
    share = share_from_workload(wl)
    say("%s fused, full size" % name)
    o, lse = share.step(wl.arrival(), "fused")
    torch_cuda.cuda.synchronize()
    o, lse = to_np(o, lse)
    assert np.all(np.isfinite(o)) and not np.any(np.isnan(lse)) and not np.any(np.isneginf(lse))
    rows, heads = wl.sample_pairs(FULL_SAMPLES[name])
    o_ref, lse_ref, _ = oracle_share(orc, wl, rows=rows, heads=heads)
    compare(o, lse, o_ref, lse_ref, rows, heads, O_TOL_BF16, name + " fused sampled")
