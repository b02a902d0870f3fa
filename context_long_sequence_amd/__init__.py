"""Python binding of libcpattn.so: one context-parallel rank's exact blockwise
attention on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/cpattn.h). PyTorch supplies device memory
and the current stream. There is no fallback: if the library is missing or a
call fails, a ``CpattnError`` is raised.

Functions (same names as the C ABI):
  cpattn_zigzag_index(total_len, cp_size, rank, layout, cu_seqlens=None)
  cpattn_partial(q, k, v, q_pos, k_pos, o, lse, causal=True, softmax_scale=0.0, accumulate=False)
  cpattn_varlen_partial(q, k, v, q_pos, k_pos, cu_seqlens, o, lse, softmax_scale=0.0, accumulate=False)
  cpattn_partial_multi(q, k_blocks, v_blocks, q_pos, k_pos_blocks, o, lse, causal=True, softmax_scale=0.0,
                       accumulate=False, cu_seqlens=None)
  cpattn_merge_lse(o_acc, lse_acc, o_part, lse_part)
  cpattn_bwd_delta(o, dout, delta)
  cpattn_partial_bwd(q, k, v, dout, q_pos, k_pos, lse, delta, dq, dk, dv, causal=True, softmax_scale=0.0,
                     accumulate_dq=False, accumulate_dkv=False, cu_seqlens=None, plan=None)
  cpattn_bwd_query_workgroups(lq, hq), cpattn_varlen_bwd_plan(q_pos, k_pos, cu_seqlens, hq, hkv)
  cpattn_partial_bwd_multi(q, k_blocks, v_blocks, dout, q_pos, k_pos_blocks, lse, delta, dq, dk_blocks,
                           dv_blocks, causal=True, softmax_scale=0.0, accumulate_dq=False, accumulate_dkv=False,
                           cu_seqlens=None)

Layouts: q, o [lq, hq, d]; k, v [lk, hkv, d]; lse [hq, lq] float32; positions
int32 ascending. See include/cpattn.h for the full contract.
"""
import ctypes
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcpattn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "cpattn.h")

CPATTN_BF16, CPATTN_F32 = 0, 1
LAYOUTS = {"contiguous": 0, "zigzag": 1, "striped": 2}
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_DTYPE", 4: "ERR_UNSORTED", 5: "ERR_RANGE",
          6: "ERR_HIP", 7: "ERR_ALIGN", 8: "ERR_ALIAS"}


class CpattnError(RuntimeError):
    """A non-OK status from the library (or the library is missing)."""

    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status
        self.message = message


_lib = None


def load_library(path=LIB_PATH):
    """Load libcpattn.so (built by context_long_sequence_amd/build.py); raise if absent."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise CpattnError(-1, "libcpattn.so not found at %s; run `python -m context_long_sequence_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.cpattn_version.restype = ctypes.c_int
    lib.cpattn_version.argtypes = []
    lib.cpattn_last_error.restype = ctypes.c_char_p
    lib.cpattn_last_error.argtypes = []
    lib.cpattn_zigzag_index.restype = ctypes.c_int
    lib.cpattn_zigzag_index.argtypes = [i64, i32, i32, ctypes.c_int, vp, i32, vp, vp]
    lib.cpattn_partial.restype = ctypes.c_int
    lib.cpattn_partial.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i32, i32, i32, vp, vp, i32, f32,
                                   vp, ctypes.c_int, vp, i32, vp]
    lib.cpattn_varlen_partial.restype = ctypes.c_int
    lib.cpattn_varlen_partial.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i32, i32, i32, vp, vp, vp, i32, f32,
                                          vp, ctypes.c_int, vp, i32, vp]
    lib.cpattn_partial_workgroups.restype = ctypes.c_int64
    lib.cpattn_partial_workgroups.argtypes = [i64, i32, i32]
    lib.cpattn_varlen_plan.restype = ctypes.c_int
    lib.cpattn_varlen_plan.argtypes = [vp, i64, vp, i64, vp, i32, i32, i32, i32, ctypes.c_int, vp, i64]
    lib.cpattn_bwd_query_workgroups.restype = ctypes.c_int64
    lib.cpattn_bwd_query_workgroups.argtypes = [i64, i32]
    lib.cpattn_varlen_bwd_plan.restype = ctypes.c_int
    lib.cpattn_varlen_bwd_plan.argtypes = [vp, i64, vp, i64, vp, i32, i32, i32, vp, i64]
    lib.cpattn_varlen_partial_bwd_planned.restype = ctypes.c_int
    lib.cpattn_varlen_partial_bwd_planned.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i32, i32, i32, vp, vp,
                                                      vp, i32, f32, vp, vp, vp, i32, vp, vp, i32, vp, i64, vp]
    lib.cpattn_varlen_partial_planned.restype = ctypes.c_int
    lib.cpattn_varlen_partial_planned.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i32, i32, i32, vp, vp, vp, i32,
                                                  f32, vp, ctypes.c_int, vp, i32, vp, i64, vp]
    lib.cpattn_partial_multi.restype = ctypes.c_int
    lib.cpattn_partial_multi.argtypes = [vp, vp, vp, ctypes.c_int, i64, vp, i32, i32, i32, i32, vp, vp, vp, i32,
                                         i32, f32, vp, ctypes.c_int, vp, i32, vp]
    lib.cpattn_bwd_delta.restype = ctypes.c_int
    lib.cpattn_bwd_delta.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i32, i32, vp, vp]
    lib.cpattn_partial_bwd.restype = ctypes.c_int
    lib.cpattn_partial_bwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i32, i32, i32, vp, vp, i32, vp, i32,
                                       f32, vp, vp, vp, i32, vp, vp, i32, vp]
    lib.cpattn_partial_bwd_multi.restype = ctypes.c_int
    lib.cpattn_partial_bwd_multi.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, vp, i32, i32, i32, i32, vp, vp, i32,
                                             vp, i32, f32, vp, vp, vp, i32, vp, vp, i32, vp]
    lib.cpattn_merge_lse.restype = ctypes.c_int
    lib.cpattn_merge_lse.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i32, i32, vp]
    if path == LIB_PATH:
        _lib = lib
    return lib


def header_functions(path=HEADER):
    """Names of the functions declared in include/cpattn.h."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(cpattn_[a-z_]+)\s*\(", text, re.M)))


def _check(lib, status):
    if status != 0:
        raise CpattnError(status, lib.cpattn_last_error().decode())


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return CPATTN_BF16
    if t.dtype == torch.float32:
        return CPATTN_F32
    raise CpattnError(3, "tensor dtype %s is not bfloat16 or float32" % t.dtype)


def _dev(t, name, dtype=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise CpattnError(1, "%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise CpattnError(2, "%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise CpattnError(3, "%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _pos_len(t, n, name):
    """A position array must be 1-D with one entry per token: the kernels read
    n of them and cannot see the array's length."""
    if t is not None and (t.dim() != 1 or t.numel() != n):
        raise CpattnError(2, "%s must be 1-D with %d entries, got shape %s" % (name, n, tuple(t.shape)))


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def cpattn_version():
    return load_library().cpattn_version()


def cpattn_zigzag_index(total_len, cp_size, rank, layout="zigzag", cu_seqlens=None):
    """Global positions of `rank`'s tokens (and each token's document start), as int32 numpy arrays."""
    lib = load_library()
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    n = total_len // cp_size if cp_size > 0 else 0
    pos = np.zeros(max(n, 1), np.int32)
    start = np.zeros(max(n, 1), np.int32)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, np.int32)
    st = lib.cpattn_zigzag_index(int(total_len), int(cp_size), int(rank), lay,
                                 None if cu is None else cu.ctypes.data,
                                 0 if cu is None else len(cu) - 1, pos.ctypes.data, start.ctypes.data)
    _check(lib, st)
    return pos[:n], start[:n]


def _shapes(q, k, o, lse):
    if q.dim() != 3 or k.dim() != 3 or o.dim() != 3 or lse.dim() != 2:
        raise CpattnError(2, "q, k, v, o must be 3-D [tokens, heads, head_dim] and lse 2-D [heads, tokens]")
    lq, hq, d = q.shape
    lk, hkv, d2 = k.shape
    if d2 != d or tuple(o.shape) != (lq, hq, d) or tuple(lse.shape) != (hq, lq):
        raise CpattnError(2, "shape mismatch: q %s k %s o %s lse %s" % (tuple(q.shape), tuple(k.shape),
                                                                        tuple(o.shape), tuple(lse.shape)))
    return lq, lk, hq, hkv, d


def cpattn_partial(q, k, v, q_pos, k_pos, o, lse, causal=True, softmax_scale=0.0, accumulate=False, stream=None):
    """Fold one KV block into (o, lse); see cpattn_partial in include/cpattn.h."""
    import torch
    lib = load_library()
    lq, lk, hq, hkv, d = _shapes(q, k, o, lse)
    if tuple(v.shape) != tuple(k.shape):
        raise CpattnError(2, "v must have k's shape")
    _pos_len(q_pos, lq, "q_pos")
    _pos_len(k_pos, lk, "k_pos")
    st = lib.cpattn_partial(_dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dtype_code(q), lq, lk, hq,
                            hkv, d, _dev(q_pos, "q_pos", torch.int32), _dev(k_pos, "k_pos", torch.int32),
                            int(bool(causal)), float(softmax_scale), _dev(o, "o"), _dtype_code(o),
                            _dev(lse, "lse", torch.float32), int(bool(accumulate)), _stream(stream))
    _check(lib, st)


def cpattn_varlen_partial(q, k, v, q_pos, k_pos, cu_seqlens, o, lse, softmax_scale=0.0, accumulate=False,
                          stream=None, plan=None):
    """As cpattn_partial, causal within documents given by device cu_seqlens.
    plan (optional int32 device tensor, from cpattn_varlen_plan for these
    positions): the call runs planned (cpattn_varlen_partial_planned)."""
    import torch
    lib = load_library()
    lq, lk, hq, hkv, d = _shapes(q, k, o, lse)
    if tuple(v.shape) != tuple(k.shape):
        raise CpattnError(2, "v must have k's shape")
    _pos_len(q_pos, lq, "q_pos")
    _pos_len(k_pos, lk, "k_pos")
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise CpattnError(2, "cu_seqlens must be 1-D with n_seqs + 1 >= 2 entries")
    args = [_dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dtype_code(q), lq, lk, hq, hkv, d,
            _dev(q_pos, "q_pos", torch.int32), _dev(k_pos, "k_pos", torch.int32),
            _dev(cu_seqlens, "cu_seqlens", torch.int32), cu_seqlens.numel() - 1, float(softmax_scale), _dev(o, "o"),
            _dtype_code(o), _dev(lse, "lse", torch.float32), int(bool(accumulate))]
    if plan is None:
        st = lib.cpattn_varlen_partial(*args, _stream(stream))
    else:
        if plan.dim() != 1:
            raise CpattnError(2, "plan must be 1-D")
        st = lib.cpattn_varlen_partial_planned(*args, _dev(plan, "plan", torch.int32), plan.numel(), _stream(stream))
    _check(lib, st)


def cpattn_partial_workgroups(lq, hq, hkv):
    """Workgroups of one cpattn_partial / cpattn_varlen_partial call (-1 for invalid sizes)."""
    return int(load_library().cpattn_partial_workgroups(int(lq), int(hq), int(hkv)))


VARLEN_PLAN_RECORD = 48  # CPATTN_VARLEN_PLAN_RECORD: int32 per workgroup in a plan


def cpattn_varlen_plan(q_pos, k_pos, cu_seqlens, hq, hkv, head_dim, in_dtype="bf16"):
    """Plan of one document call (cpattn_varlen_partial(..., plan=)) from HOST
    positions and document offsets (numpy int32): an int32 numpy array of
    VARLEN_PLAN_RECORD entries per workgroup."""
    lib = load_library()
    qp = np.ascontiguousarray(q_pos, np.int32)
    kp = np.ascontiguousarray(k_pos, np.int32)
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    n = cpattn_partial_workgroups(len(qp), hq, hkv)
    if n < 0:
        raise CpattnError(2, "invalid sizes lq=%d hq=%d hkv=%d" % (len(qp), hq, hkv))
    n *= VARLEN_PLAN_RECORD
    plan = np.zeros(max(n, 1), np.int32)
    code = in_dtype if isinstance(in_dtype, int) else (CPATTN_BF16 if in_dtype == "bf16" else CPATTN_F32)
    st = lib.cpattn_varlen_plan(qp.ctypes.data, len(qp), kp.ctypes.data if len(kp) else None, len(kp),
                                cu.ctypes.data, len(cu) - 1, int(hq), int(hkv), int(head_dim), code,
                                plan.ctypes.data, n)
    _check(lib, st)
    return plan[:n]


def cpattn_bwd_query_workgroups(lq, hq):
    """Workgroups of the query-gradient kernel: the length of a backward plan."""
    return int(load_library().cpattn_bwd_query_workgroups(int(lq), int(hq)))


def cpattn_varlen_bwd_plan(q_pos, k_pos, cu_seqlens, hq, hkv):
    """Plan of one document gradient call (cpattn_partial_bwd(..., plan=)) from
    HOST positions and document offsets (numpy int32): the query kernel's
    dispatch order, one int32 per workgroup."""
    lib = load_library()
    qp = np.ascontiguousarray(q_pos, np.int32)
    kp = np.ascontiguousarray(k_pos, np.int32)
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    n = cpattn_bwd_query_workgroups(len(qp), hq)
    if n < 0:
        raise CpattnError(2, "invalid sizes lq=%d hq=%d" % (len(qp), hq))
    plan = np.zeros(max(n, 1), np.int32)
    st = lib.cpattn_varlen_bwd_plan(qp.ctypes.data, len(qp), kp.ctypes.data if len(kp) else None, len(kp),
                                    cu.ctypes.data, len(cu) - 1, int(hq), int(hkv), plan.ctypes.data, n)
    _check(lib, st)
    return plan[:n]


def cpattn_partial_multi(q, k_blocks, v_blocks, q_pos, k_pos_blocks, o, lse, causal=True, softmax_scale=0.0,
                         accumulate=False, cu_seqlens=None, stream=None):
    """Fold several arrived KV blocks into (o, lse) in one launch, in list
    order; see cpattn_partial_multi in include/cpattn.h."""
    import torch
    lib = load_library()
    n = len(k_blocks)
    if n == 0 or len(v_blocks) != n or len(k_pos_blocks) != n:
        raise CpattnError(5, "k_blocks, v_blocks and k_pos_blocks must be non-empty lists of one length")
    for k, v, p in zip(k_blocks, v_blocks, k_pos_blocks):
        _shapes(q, k, o, lse)
        if tuple(v.shape) != tuple(k.shape):
            raise CpattnError(2, "each v must have its k's shape")
        # the C ABI takes one KV head count for every block (it sizes each
        # block's rows with it), so blocks that differ are rejected here
        if k.shape[1] != k_blocks[0].shape[1]:
            raise CpattnError(2, "every KV block must have the same number of KV heads (%d and %d)" % (
                k_blocks[0].shape[1], k.shape[1]))
        _pos_len(p, k.shape[0], "k_pos")
    _pos_len(q_pos, q.shape[0], "q_pos")
    ptrs = ctypes.c_void_p * n
    kp = ptrs(*[_dev(k, "k", q.dtype) for k in k_blocks])
    vp_ = ptrs(*[_dev(v, "v", q.dtype) for v in v_blocks])
    pp = ptrs(*[_dev(p, "k_pos", torch.int32) for p in k_pos_blocks])
    lks = (ctypes.c_int64 * n)(*[int(k.shape[0]) for k in k_blocks])
    lq, hq, d = q.shape
    hkv = k_blocks[0].shape[1]
    st = lib.cpattn_partial_multi(_dev(q, "q"), ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp_, ctypes.c_void_p),
                                  _dtype_code(q), lq, ctypes.cast(lks, ctypes.c_void_p), n, hq, hkv, d,
                                  _dev(q_pos, "q_pos", torch.int32), ctypes.cast(pp, ctypes.c_void_p),
                                  _dev(cu_seqlens, "cu_seqlens", torch.int32),
                                  0 if cu_seqlens is None else cu_seqlens.numel() - 1, int(bool(causal)),
                                  float(softmax_scale), _dev(o, "o"), _dtype_code(o), _dev(lse, "lse", torch.float32),
                                  int(bool(accumulate)), _stream(stream))
    _check(lib, st)


def cpattn_merge_lse(o_acc, lse_acc, o_part, lse_part, stream=None):
    """In place: (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_part, lse_part))."""
    import torch
    lib = load_library()
    if o_acc.dim() != 3 or tuple(o_part.shape) != tuple(o_acc.shape) or o_part.dtype != o_acc.dtype:
        raise CpattnError(2, "o_acc and o_part must be [lq, hq, d] of one dtype")
    lq, hq, d = o_acc.shape
    if tuple(lse_acc.shape) != (hq, lq) or tuple(lse_part.shape) != (hq, lq):
        raise CpattnError(2, "lse tensors must be [hq, lq]")
    st = lib.cpattn_merge_lse(_dev(o_acc, "o_acc"), _dev(lse_acc, "lse_acc", torch.float32), _dev(o_part, "o_part"),
                              _dev(lse_part, "lse_part", torch.float32), _dtype_code(o_acc), lq, hq, d,
                              _stream(stream))
    _check(lib, st)


def cpattn_bwd_delta(o, dout, delta, stream=None):
    """delta[h, i] = <dout[i, h], o[i, h]> (float32), for the backward calls."""
    import torch
    lib = load_library()
    if o.dim() != 3 or tuple(dout.shape) != tuple(o.shape):
        raise CpattnError(2, "o and dout must both be [lq, hq, d]")
    lq, hq, d = o.shape
    if tuple(delta.shape) != (hq, lq):
        raise CpattnError(2, "delta must be [hq, lq]")
    st = lib.cpattn_bwd_delta(_dev(o, "o"), _dtype_code(o), _dev(dout, "dout"), _dtype_code(dout), lq, hq, d,
                              _dev(delta, "delta", torch.float32), _stream(stream))
    _check(lib, st)


def cpattn_partial_bwd(q, k, v, dout, q_pos, k_pos, lse, delta, dq, dk, dv, causal=True, softmax_scale=0.0,
                       accumulate_dq=False, accumulate_dkv=False, cu_seqlens=None, stream=None, plan=None):
    """Gradients of one KV block: dq (+)= this block's share, dk, dv (+)= the block's key gradients.

    q, dout [lq, hq, d] bf16; k, v [lk, hkv, d] bf16; lse, delta [hq, lq] float32 (the merged LSE of
    the forward and cpattn_bwd_delta's output); dq [lq, hq, d], dk, dv [lk, hkv, d] float32. With
    documents, `plan` (a device int32 tensor from cpattn_varlen_bwd_plan) selects the planned call
    (cpattn_varlen_partial_bwd_planned); the results are the same bit for bit.
    """
    import torch
    lib = load_library()
    if q.dim() != 3 or k.dim() != 3 or tuple(v.shape) != tuple(k.shape) or tuple(dout.shape) != tuple(q.shape):
        raise CpattnError(2, "q, dout must be [lq, hq, d] and k, v [lk, hkv, d]")
    lq, hq, d = q.shape
    lk, hkv, d2 = k.shape
    if d2 != d:
        raise CpattnError(2, "q and k head dims differ")
    if tuple(lse.shape) != (hq, lq) or tuple(delta.shape) != (hq, lq):
        raise CpattnError(2, "lse and delta must be [hq, lq]")
    if tuple(dq.shape) != (lq, hq, d) or tuple(dk.shape) != (lk, hkv, d) or tuple(dv.shape) != (lk, hkv, d):
        raise CpattnError(2, "dq must be [lq, hq, d] and dk, dv [lk, hkv, d]")
    if dout.dtype != q.dtype or k.dtype != q.dtype or v.dtype != q.dtype:
        raise CpattnError(3, "q, k, v and dout must share one dtype")
    _pos_len(q_pos, lq, "q_pos")
    _pos_len(k_pos, lk, "k_pos")
    if plan is not None:
        if cu_seqlens is None:
            raise CpattnError(1, "a plan is for calls with documents (cu_seqlens)")
        st = lib.cpattn_varlen_partial_bwd_planned(
            _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(dout, "dout"), _dtype_code(q), lq, lk, hq, hkv, d,
            _dev(q_pos, "q_pos", torch.int32), _dev(k_pos, "k_pos", torch.int32),
            _dev(cu_seqlens, "cu_seqlens", torch.int32), cu_seqlens.numel() - 1, float(softmax_scale),
            _dev(lse, "lse", torch.float32), _dev(delta, "delta", torch.float32), _dev(dq, "dq", torch.float32),
            int(bool(accumulate_dq)), _dev(dk, "dk", torch.float32), _dev(dv, "dv", torch.float32),
            int(bool(accumulate_dkv)), _dev(plan, "plan", torch.int32), plan.numel(), _stream(stream))
        _check(lib, st)
        return
    st = lib.cpattn_partial_bwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(dout, "dout"), _dtype_code(q), lq, lk,
                                hq, hkv, d, _dev(q_pos, "q_pos", torch.int32), _dev(k_pos, "k_pos", torch.int32),
                                int(bool(causal)), _dev(cu_seqlens, "cu_seqlens", torch.int32),
                                0 if cu_seqlens is None else cu_seqlens.numel() - 1, float(softmax_scale),
                                _dev(lse, "lse", torch.float32), _dev(delta, "delta", torch.float32),
                                _dev(dq, "dq", torch.float32), int(bool(accumulate_dq)),
                                _dev(dk, "dk", torch.float32), _dev(dv, "dv", torch.float32),
                                int(bool(accumulate_dkv)), _stream(stream))
    _check(lib, st)


def cpattn_partial_bwd_multi(q, k_blocks, v_blocks, dout, q_pos, k_pos_blocks, lse, delta, dq, dk_blocks, dv_blocks,
                             causal=True, softmax_scale=0.0, accumulate_dq=False, accumulate_dkv=False,
                             cu_seqlens=None, stream=None):
    """Gradients of several present KV blocks in one call, in list order: dq
    (+)= the sum of the blocks' shares, dk_blocks[b], dv_blocks[b] (+)= block
    b's key gradients; see cpattn_partial_bwd_multi in include/cpattn.h."""
    import torch
    lib = load_library()
    n = len(k_blocks)
    if n == 0 or len(v_blocks) != n or len(k_pos_blocks) != n or len(dk_blocks) != n or len(dv_blocks) != n:
        raise CpattnError(5, "k_blocks, v_blocks, k_pos_blocks, dk_blocks and dv_blocks must be non-empty lists "
                             "of one length")
    if q.dim() != 3 or tuple(dout.shape) != tuple(q.shape):
        raise CpattnError(2, "q, dout must be [lq, hq, d]")
    lq, hq, d = q.shape
    if tuple(lse.shape) != (hq, lq) or tuple(delta.shape) != (hq, lq):
        raise CpattnError(2, "lse and delta must be [hq, lq]")
    if tuple(dq.shape) != (lq, hq, d):
        raise CpattnError(2, "dq must be [lq, hq, d]")
    if dout.dtype != q.dtype:
        raise CpattnError(3, "q, k, v and dout must share one dtype")
    hkv = k_blocks[0].shape[1] if k_blocks[0].dim() == 3 else -1
    for k, v, p, dk, dv in zip(k_blocks, v_blocks, k_pos_blocks, dk_blocks, dv_blocks):
        if k.dim() != 3 or k.shape[2] != d or tuple(v.shape) != tuple(k.shape):
            raise CpattnError(2, "each k, v must be [lk, hkv, d] with q's d")
        # (one KV head count for every block: the C ABI sizes each block's rows with it)
        if k.shape[1] != hkv:
            raise CpattnError(2, "every KV block must have the same number of KV heads (%d and %d)" % (hkv, k.shape[1]))
        if tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(k.shape):
            raise CpattnError(2, "each dk, dv must have its k's shape")
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise CpattnError(3, "q, k, v and dout must share one dtype")
        _pos_len(p, k.shape[0], "k_pos")
    _pos_len(q_pos, lq, "q_pos")
    ptrs = ctypes.c_void_p * n
    kp = ptrs(*[_dev(k, "k", q.dtype) for k in k_blocks])
    vp_ = ptrs(*[_dev(v, "v", q.dtype) for v in v_blocks])
    pp = ptrs(*[_dev(p, "k_pos", torch.int32) for p in k_pos_blocks])
    dkp = ptrs(*[_dev(t, "dk", torch.float32) for t in dk_blocks])
    dvp = ptrs(*[_dev(t, "dv", torch.float32) for t in dv_blocks])
    lks = (ctypes.c_int64 * n)(*[int(k.shape[0]) for k in k_blocks])
    st = lib.cpattn_partial_bwd_multi(_dev(q, "q"), ctypes.cast(kp, ctypes.c_void_p),
                                      ctypes.cast(vp_, ctypes.c_void_p), _dev(dout, "dout"), _dtype_code(q), lq,
                                      ctypes.cast(lks, ctypes.c_void_p), n, hq, hkv, d,
                                      _dev(q_pos, "q_pos", torch.int32), ctypes.cast(pp, ctypes.c_void_p),
                                      int(bool(causal)), _dev(cu_seqlens, "cu_seqlens", torch.int32),
                                      0 if cu_seqlens is None else cu_seqlens.numel() - 1, float(softmax_scale),
                                      _dev(lse, "lse", torch.float32), _dev(delta, "delta", torch.float32),
                                      _dev(dq, "dq", torch.float32), int(bool(accumulate_dq)),
                                      ctypes.cast(dkp, ctypes.c_void_p), ctypes.cast(dvp, ctypes.c_void_p),
                                      int(bool(accumulate_dkv)), _stream(stream))
    _check(lib, st)


__all__ = ["cpattn_zigzag_index", "cpattn_partial", "cpattn_varlen_partial", "cpattn_partial_multi",
           "cpattn_partial_workgroups", "cpattn_varlen_plan", "cpattn_bwd_query_workgroups", "cpattn_varlen_bwd_plan",
           "cpattn_merge_lse", "cpattn_bwd_delta", "cpattn_partial_bwd", "cpattn_partial_bwd_multi", "cpattn_version",
           "CpattnError", "load_library", "header_functions"]
