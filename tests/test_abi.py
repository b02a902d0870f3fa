"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes

import numpy as np
import pytest

import context_long_sequence_amd as cp


@pytest.fixture(scope="module")
def lib():
    return cp.load_library()


def test_exports_every_declared_symbol(lib):
    names = cp.header_functions()
    assert set(names) == {"cpattn_version", "cpattn_last_error", "cpattn_zigzag_index", "cpattn_partial",
                          "cpattn_varlen_partial", "cpattn_partial_multi", "cpattn_merge_lse", "cpattn_bwd_delta",
                          "cpattn_partial_bwd", "cpattn_partial_workgroups", "cpattn_varlen_plan",
                          "cpattn_varlen_partial_planned", "cpattn_partial_bwd_multi",
                          "cpattn_bwd_query_workgroups", "cpattn_varlen_bwd_plan",
                          "cpattn_varlen_partial_bwd_planned"}
    for n in names:
        assert hasattr(lib, n), n


def test_version(lib):
    assert lib.cpattn_version() == 100


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Fake but aligned addresses: every case below is invalid on purpose, so the
# library must return before touching them. Skipped where a GPU is visible,
# so that a validation bug could never turn into a launch with these pointers.
A = 0x10000
B = 0x20000
C = 0x30000
O = 0x40000
L = 0x50000
P = 0x60000
K = 0x70000

# (status name, args for cpattn_partial)
PARTIAL_CASES = [
    ("ERR_NULL", (0, B, C, 0, 8, 8, 1, 1, 64, P, K, 1, 0.0, O, 0, L, 0, 0)),
    ("ERR_NULL", (A, B, C, 0, 8, 8, 1, 1, 64, P, K, 1, 0.0, O, 0, 0, 0, 0)),
    ("ERR_NULL", (A, B, C, 0, 8, 8, 1, 1, 64, 0, K, 1, 0.0, O, 0, L, 0, 0)),        # causal needs positions
    ("ERR_SHAPE", (A, B, C, 0, 8, 8, 1, 1, 96, P, K, 1, 0.0, O, 0, L, 0, 0)),       # head_dim 96
    ("ERR_SHAPE", (A, B, C, 0, 8, 8, 6, 4, 64, P, K, 1, 0.0, O, 0, L, 0, 0)),       # hq % hkv
    ("ERR_SHAPE", (A, B, C, 0, -1, 8, 1, 1, 64, P, K, 1, 0.0, O, 0, L, 0, 0)),      # lq < 0
    ("ERR_SHAPE", (A, B, C, 0, 8, 1 << 31, 1, 1, 64, P, K, 1, 0.0, O, 0, L, 0, 0)),  # lk >= 2^31
    ("ERR_DTYPE", (A, B, C, 1, 8, 8, 1, 1, 64, P, K, 1, 0.0, O, 0, L, 0, 0)),       # f32 in, bf16 out
    ("ERR_DTYPE", (A, B, C, 5, 8, 8, 1, 1, 64, P, K, 1, 0.0, O, 0, L, 0, 0)),
    ("ERR_RANGE", (A, B, C, 0, 8, 8, 1, 1, 64, P, K, 2, 0.0, O, 0, L, 0, 0)),       # causal flag
    ("ERR_RANGE", (A, B, C, 0, 8, 8, 1, 1, 64, P, K, 1, 0.0, O, 0, L, 3, 0)),       # accumulate flag
    ("ERR_ALIGN", (A + 2, B, C, 0, 8, 8, 1, 1, 64, P, K, 1, 0.0, O, 0, L, 0, 0)),
    ("ERR_ALIGN", (A, B, C, 0, 8, 8, 1, 1, 64, P + 2, K, 1, 0.0, O, 0, L, 0, 0)),
    ("ERR_ALIAS", (A, B, C, 0, 8, 8, 1, 1, 64, P, K, 1, 0.0, A + 16, 0, L, 0, 0)),  # o overlaps q
    ("ERR_ALIAS", (A, B, C, 0, 8, 8, 1, 1, 64, P, K, 1, 0.0, O, 0, B, 0, 0)),       # lse overlaps k
]
STATUS = {v: k for k, v in cp.STATUS.items()}


@pytest.mark.skipif(_gpu_visible(), reason="argument-rejection checks use fake addresses; CPU only")
@pytest.mark.parametrize("expect,args", PARTIAL_CASES)
def test_partial_rejects(lib, expect, args):
    st = lib.cpattn_partial(*args)
    assert st == STATUS[expect], (st, lib.cpattn_last_error())
    assert lib.cpattn_last_error().decode()


@pytest.mark.skipif(_gpu_visible(), reason="argument-rejection checks use fake addresses; CPU only")
def test_varlen_and_merge_reject(lib):
    base = (A, B, C, 0, 8, 8, 1, 1, 64, P, K)
    assert lib.cpattn_varlen_partial(*base, 0, 1, 0.0, O, 0, L, 0, 0) == STATUS["ERR_NULL"]   # no cu_seqlens
    assert lib.cpattn_varlen_partial(*base, 0x80000, 0, 0.0, O, 0, L, 0, 0) == STATUS["ERR_SHAPE"]  # n_seqs 0
    assert lib.cpattn_varlen_partial(*base, 0x80002, 1, 0.0, O, 0, L, 0, 0) == STATUS["ERR_ALIGN"]
    assert lib.cpattn_merge_lse(0, L, C, P, 0, 8, 1, 64, 0) == STATUS["ERR_NULL"]
    assert lib.cpattn_merge_lse(O, L, C, P, 0, 8, 1, 80, 0) == STATUS["ERR_SHAPE"]
    assert lib.cpattn_merge_lse(O, L, C, P, 7, 8, 1, 64, 0) == STATUS["ERR_DTYPE"]
    assert lib.cpattn_merge_lse(O, L, O + 16, P, 0, 8, 1, 64, 0) == STATUS["ERR_ALIAS"]
    assert lib.cpattn_merge_lse(O + 8, L, C, P, 0, 8, 1, 64, 0) == STATUS["ERR_ALIGN"]


@pytest.mark.skipif(_gpu_visible(), reason="argument-rejection checks use fake addresses; CPU only")
def test_multi_rejects(lib):
    import ctypes

    def arr(t, vals):
        a = (t * len(vals))(*vals)
        return a, ctypes.cast(a, ctypes.c_void_p).value

    kb, kbp = arr(ctypes.c_void_p, [B, B + 0x1000])
    vb, vbp = arr(ctypes.c_void_p, [C, C + 0x1000])
    pb, pbp = arr(ctypes.c_void_p, [K, K + 0x1000])
    lk, lkp = arr(ctypes.c_int64, [8, 8])

    def call(n=2, k=kbp, lks=lkp, hd=64, cu=0, ns=0, causal=1, o=O, acc=0):
        return lib.cpattn_partial_multi(A, k, vbp, 0, 8, lks, n, 1, 1, hd, P, pbp, cu, ns, causal, 0.0, o, 0, L,
                                        acc, 0)
    assert call(k=0) == STATUS["ERR_NULL"]                    # no block array
    assert call(n=0) == STATUS["ERR_RANGE"]                   # no block
    assert call(n=33) == STATUS["ERR_RANGE"]                  # over the table size
    assert call(hd=80) == STATUS["ERR_SHAPE"]                 # checked per block as cpattn_partial would
    assert call(cu=0x80000, ns=1, causal=0) == STATUS["ERR_RANGE"]   # documents need causal
    assert call(cu=0x80002, ns=1) == STATUS["ERR_ALIGN"]
    assert call(cu=0x80000, ns=0) == STATUS["ERR_SHAPE"]
    bad_lk, bad_lkp = arr(ctypes.c_int64, [8, 1 << 31])
    assert call(lks=bad_lkp) == STATUS["ERR_SHAPE"]           # the second block's length
    assert call(o=B + 0x1000 + 16) == STATUS["ERR_ALIAS"]     # o overlaps the second block's k
    assert call(acc=2) == STATUS["ERR_RANGE"]


DO, DL, DK, DV = 0x90000, 0xA0000, 0xB0000, 0xC0000


@pytest.mark.skipif(_gpu_visible(), reason="argument-rejection checks use fake addresses; CPU only")
def test_backward_rejects(lib):
    def bwd(q=A, dt=0, lq=8, lk=8, hq=1, hkv=1, hd=64, qp=P, kp=K, causal=1, cu=0, ns=0, scale=0.0, dq=O, adq=0,
            dk=DK, dv=DV, adkv=0, delta=DL):
        return lib.cpattn_partial_bwd(q, B, C, DO, dt, lq, lk, hq, hkv, hd, qp, kp, causal, cu, ns, scale, L, delta,
                                      dq, adq, dk, dv, adkv, 0)
    assert bwd(dq=0) == STATUS["ERR_NULL"]
    assert bwd(dk=0) == STATUS["ERR_NULL"]
    assert bwd(delta=0) == STATUS["ERR_NULL"]
    assert bwd(qp=0) == STATUS["ERR_NULL"]                     # causal needs positions
    assert bwd(dt=7) == STATUS["ERR_DTYPE"]                    # neither bf16 nor float32
    assert bwd(hd=96) == STATUS["ERR_SHAPE"]
    assert bwd(hq=6, hkv=4) == STATUS["ERR_SHAPE"]
    assert bwd(lk=1 << 31) == STATUS["ERR_SHAPE"]
    assert bwd(causal=2) == STATUS["ERR_RANGE"]
    assert bwd(adq=2) == STATUS["ERR_RANGE"]
    assert bwd(adkv=3) == STATUS["ERR_RANGE"]
    assert bwd(cu=0x80000, ns=1, causal=0) == STATUS["ERR_RANGE"]   # documents need causal
    assert bwd(cu=0x80000, ns=0) == STATUS["ERR_SHAPE"]
    assert bwd(scale=float("nan")) == STATUS["ERR_RANGE"]
    assert bwd(dq=O + 4) == STATUS["ERR_ALIGN"]
    assert bwd(dv=DK + 16) == STATUS["ERR_ALIAS"]              # dk and dv overlap
    assert bwd(dq=A + 16) == STATUS["ERR_ALIAS"]               # dq overlaps q
    assert bwd(dk=DL) == STATUS["ERR_ALIAS"]                   # dk overlaps delta
    # delta
    assert lib.cpattn_bwd_delta(0, 0, DO, 0, 8, 1, 64, DL, 0) == STATUS["ERR_NULL"]
    assert lib.cpattn_bwd_delta(O, 7, DO, 0, 8, 1, 64, DL, 0) == STATUS["ERR_DTYPE"]
    assert lib.cpattn_bwd_delta(O, 0, DO, 0, 8, 1, 80, DL, 0) == STATUS["ERR_SHAPE"]
    assert lib.cpattn_bwd_delta(O, 0, DO, 0, 8, 1, 64, O + 16, 0) == STATUS["ERR_ALIAS"]
    assert lib.cpattn_bwd_delta(O, 0, DO + 8, 0, 8, 1, 64, DL, 0) == STATUS["ERR_ALIGN"]


def test_last_error_is_thread_local(lib):
    import threading
    out = []
    pos = np.zeros(4, np.int32)
    assert lib.cpattn_zigzag_index(16, 4, 9, 1, None, 0, pos.ctypes.data, None) == STATUS["ERR_RANGE"]
    msg_main = lib.cpattn_last_error().decode()

    def other():
        out.append(lib.cpattn_last_error().decode())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert msg_main and out == [""]


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(cp.CpattnError):
        cp.load_library(str(tmp_path / "missing.so"))


def test_binding_rejects_position_arrays_of_the_wrong_length():
    """The kernels read lq (lk) positions and cannot see an array's length, so
    the binding checks it before anything reaches the library."""
    import torch
    q = torch.zeros((8, 2, 64), dtype=torch.bfloat16)
    k = torch.zeros((5, 2, 64), dtype=torch.bfloat16)
    o = torch.zeros_like(q)
    lse = torch.zeros((2, 8), dtype=torch.float32)
    good_q, good_k = torch.arange(8, dtype=torch.int32), torch.arange(5, dtype=torch.int32)
    short = torch.arange(4, dtype=torch.int32)
    for qp, kp in ((short, good_k), (good_q, short), (good_q.reshape(2, 4), good_k)):
        with pytest.raises(cp.CpattnError) as e:
            cp.cpattn_partial(q, k, k, qp, kp, o, lse)
        assert e.value.status == 2 and "entries" in str(e.value)
    with pytest.raises(cp.CpattnError):
        cp.cpattn_varlen_partial(q, k, k, good_q, short, torch.tensor([0, 8], dtype=torch.int32), o, lse)
    with pytest.raises(cp.CpattnError):
        cp.cpattn_partial_multi(q, [k], [k], good_q, [short], o, lse)
    g = torch.zeros((8, 2, 64), dtype=torch.float32)
    gk = torch.zeros((5, 2, 64), dtype=torch.float32)
    with pytest.raises(cp.CpattnError):
        cp.cpattn_partial_bwd(q, k, k, q, short, good_k, lse, lse, g, gk, gk)


def test_binding_rejects_multi_blocks_with_different_kv_heads():
    """cpattn_partial_multi takes one KV head count for all blocks and sizes
    every block's rows with it; a block with fewer KV heads than the first
    would be read past its end, so the binding rejects the call first."""
    import torch
    q = torch.zeros((8, 2, 64), dtype=torch.bfloat16)
    o = torch.zeros_like(q)
    lse = torch.zeros((2, 8), dtype=torch.float32)
    k2 = torch.zeros((5, 2, 64), dtype=torch.bfloat16)
    k1 = torch.zeros((5, 1, 64), dtype=torch.bfloat16)
    qp, kp = torch.arange(8, dtype=torch.int32), torch.arange(5, dtype=torch.int32)
    for blocks in ([k2, k1], [k1, k2]):
        with pytest.raises(cp.CpattnError) as e:
            cp.cpattn_partial_multi(q, blocks, blocks, qp, [kp, kp], o, lse)
        assert e.value.status == 2 and "KV heads" in str(e.value)


def test_status_table_matches_the_header():
    """The binding's status names carry the values the header's enum gives them."""
    import re
    with open(cp.HEADER) as f:
        text = f.read()
    enum = text[text.index("typedef enum {"):text.index("} cpattn_status;")]
    pairs = {int(v): k for k, v in re.findall(r"CPATTN_(\w+)\s*=\s*(\d+)", enum)}
    assert pairs == cp.STATUS


@pytest.mark.skipif(_gpu_visible(), reason="argument-rejection checks use fake addresses; CPU only")
def test_backward_multi_rejects(lib):
    def arr(t, vals):
        a = (t * len(vals))(*vals)
        return a, ctypes.cast(a, ctypes.c_void_p).value

    kb, kbp = arr(ctypes.c_void_p, [B, B + 0x1000])
    vb, vbp = arr(ctypes.c_void_p, [C, C + 0x1000])
    pb, pbp = arr(ctypes.c_void_p, [K, K + 0x1000])
    dkb, dkbp = arr(ctypes.c_void_p, [DK, DK + 0x1000])
    dvb, dvbp = arr(ctypes.c_void_p, [DV, DV + 0x1000])
    lk, lkp = arr(ctypes.c_int64, [8, 8])

    def call(n=2, k=kbp, lks=lkp, dks=dkbp, hd=64, dt=0, causal=1, cu=0, ns=0, dq=O, adq=0, adkv=0):
        return lib.cpattn_partial_bwd_multi(A, k, vbp, DO, dt, 8, lks, n, 1, 1, hd, P, pbp, causal, cu, ns, 0.0, L,
                                            DL, dq, adq, dks, dvbp, adkv, 0)
    assert call(k=0) == STATUS["ERR_NULL"]                    # no block array
    assert call(dks=0) == STATUS["ERR_NULL"]
    assert call(n=0) == STATUS["ERR_RANGE"]                   # no block
    assert call(n=33) == STATUS["ERR_RANGE"]                  # over the table size
    assert call(hd=96) == STATUS["ERR_SHAPE"]                 # checked per block as cpattn_partial_bwd would
    assert call(dt=7) == STATUS["ERR_DTYPE"]
    assert call(causal=2) == STATUS["ERR_RANGE"]
    assert call(adq=2) == STATUS["ERR_RANGE"]
    assert call(cu=0x80000, ns=1, causal=0) == STATUS["ERR_RANGE"]   # documents need causal
    bad_lk, bad_lkp = arr(ctypes.c_int64, [8, 1 << 31])
    assert call(lks=bad_lkp) == STATUS["ERR_SHAPE"]           # the second block's length
    assert call(dq=B + 0x1000 + 16) == STATUS["ERR_ALIAS"]    # dq overlaps the second block's k
    # block 0's dk overlaps block 1's v (within one block's call this would be allowed to pass
    # the single-block checks; across blocks it is caught)
    dk2, dk2p = arr(ctypes.c_void_p, [C + 0x1000, DK + 0x1000])
    assert call(dks=dk2p) == STATUS["ERR_ALIAS"]
    dk3, dk3p = arr(ctypes.c_void_p, [DK, DK + 0x10])         # the blocks' dk overlap each other
    assert call(dks=dk3p) == STATUS["ERR_ALIAS"]


@pytest.mark.skipif(_gpu_visible(), reason="argument-rejection checks use fake addresses; CPU only")
def test_backward_planned_rejects(lib):
    PL = 0xD0000

    def call(cu=0x80000, ns=1, plan=PL, plan_len=2, lq=8, hd=64, adq=0):
        return lib.cpattn_varlen_partial_bwd_planned(A, B, C, DO, 0, lq, 8, 2, 1, hd, P, K, cu, ns, 0.0, L, DL, O, adq,
                                                     DK, DV, 0, plan, plan_len, 0)
    assert call(cu=0) == STATUS["ERR_NULL"]                    # documents are required
    assert call(plan_len=3) == STATUS["ERR_SHAPE"]             # 1 row tile x 2 heads = 2 workgroups
    assert call(plan=0) == STATUS["ERR_NULL"]
    assert call(plan=PL + 2) == STATUS["ERR_ALIGN"]
    assert call(hd=96) == STATUS["ERR_SHAPE"]                  # checked as cpattn_partial_bwd would
    assert call(ns=0) == STATUS["ERR_SHAPE"]
    assert call(adq=2) == STATUS["ERR_RANGE"]
