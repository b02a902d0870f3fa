"""The arrival pipeline: piece schedule and two-stream plan on the CPU; on the
GPU, the pipelined result against the same pieces folded without copies
(bit-identical) and against the oracle."""
import itertools

import numpy as np
import pytest

from context_long_sequence_amd.pipeline import plan, split_blocks


def test_split_blocks_covers_every_key_once_in_arrival_order():
    keys = [8192, 0, 300, 4096]
    order = [3, 0, 1, 2]
    for chunk in (1, 7, 1024, 4096, 8192, 10000):
        pieces = split_blocks(keys, order, chunk)
        assert [p[0] for p in pieces] == sorted([p[0] for p in pieces], key=order.index)
        for b in range(len(keys)):
            mine = [(lo, hi) for bb, lo, hi in pieces if bb == b]
            assert mine, "every block is folded in, even an empty one"
            assert all(0 < hi - lo <= chunk for lo, hi in mine) or keys[b] == 0
            assert mine[0][0] == 0 and mine[-1][1] == keys[b]
            assert all(a[1] == c[0] for a, c in zip(mine, mine[1:]))   # consecutive, no gap or overlap
    assert len(split_blocks([8192] * 8, range(8), 1024)) == 64
    with pytest.raises(ValueError):
        split_blocks([10], [0], 0)


@pytest.mark.parametrize("n_pieces,n_slots", [(1, 1), (5, 1), (8, 2), (64, 3), (3, 8)])
def test_plan_orders_copies_and_kernels_safely(n_pieces, n_slots):
    ops = plan(n_pieces, n_slots)
    assert len(ops) == 2 * n_pieces
    recorded = set()
    copies = [o for o in ops if o["kind"] == "copy"]
    kernels = [o for o in ops if o["kind"] == "kernel"]
    # each stream runs its ops in arrival order
    assert [o["piece"] for o in copies] == list(range(n_pieces))
    assert [o["piece"] for o in kernels] == list(range(n_pieces))
    for o in ops:
        # every wait names an event recorded earlier in issue order
        assert all(w in recorded for w in o["wait"])
        recorded.add(o["record"])
        assert o["slot"] == o["piece"] % n_slots
        if o["kind"] == "kernel":
            assert o["wait"] == ["arrived%d" % o["piece"]]
            assert o["accumulate"] == (o["piece"] > 0)
        else:
            i = o["piece"]
            # a slot is refilled only after the kernel that last read it has finished
            assert o["wait"] == (["free%d" % (i - n_slots)] if i >= n_slots else [])
    # no two pieces in flight share a slot: between the copy into a slot and the
    # kernel that frees it, no other copy targets that slot
    for i, j in itertools.combinations(range(n_pieces), 2):
        if i % n_slots == j % n_slots:
            assert j >= i + n_slots


@pytest.mark.gpu
@pytest.mark.parametrize("source", ["host", "device"])
@pytest.mark.parametrize("chunk,slots", [(128, 3), (1000, 2), (512, 1)])
def test_pipeline_matches_unpipelined_and_oracle(source, chunk, slots):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    from context_long_sequence_amd.pipeline import ArrivalPipeline
    from context_long_sequence_amd.share import share_from_workload
    from test_gpu_parity import O_TOL_BF16, _reduced, compare, oracle_share, say, to_np
    wl = _reduced()["zigzag4k_cp8_h4_d128"]
    share = share_from_workload(wl)
    order = list(wl.arrival())
    pipe = ArrivalPipeline(share, chunk, n_slots=slots, source=source)
    say("pipeline %s chunk=%d slots=%d: %d pieces" % (source, chunk, slots, len(pipe.pieces(order))))
    pipe.compute_only(order)
    torch.cuda.synchronize()
    o_ref, l_ref = share.o.clone(), share.lse.clone()
    share.o.zero_()
    share.lse.zero_()
    pipe.run(order)
    torch.cuda.synchronize()
    assert torch.equal(share.o, o_ref) and torch.equal(share.lse, l_ref)
    o, lse = to_np(share.o, share.lse)
    oo, lo, _ = oracle_share(oracle.get(), wl)
    compare(o, lse, oo, lo, None, None, O_TOL_BF16, "pipeline %s chunk %d" % (source, chunk))
    m = pipe.measure(order, reps=2, warmup=1)
    say("comm %.3f ms, compute %.3f ms, overlapped %.3f ms, hidden %.2f" % (
        m["comm_ms"], m["compute_ms"], m["overlapped_ms"], m["hidden"]))
    assert m["overlapped_ms"] > 0 and m["comm_ms"] > 0 and m["compute_ms"] > 0
    # after measure() the state is the last overlapped run's, still the same result
    torch.cuda.synchronize()
    assert torch.equal(share.o, o_ref) and torch.equal(share.lse, l_ref)
