"""CPU fp64 oracle for one context-parallel rank's exact attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product library
(``context_long_sequence_amd``) never imports, links or calls it.

It wraps ``liboracle.so`` (built from ``oracle.c`` by ``oracle/build.py``) with
numpy arrays. Inputs are bf16 bit patterns (``np.uint16``) or ``np.float32``;
all arithmetic is fp64. Functions and the passages they follow:

* ``local_positions`` — contiguous split (PCP page
  "大模型长序列显存优化：PCP与DCP序列并行实战指南", §3.5), zig-zag chunks and the
  literal striped example (zig-zag page "大模型长上下文训练的挑战与突破", §4.2).
* ``attention`` — plain two-pass softmax attention with causal masking by
  global position (FCP page "从固定环到自由拓扑：FCP到底在解决什么", §3.3 and §4.2:
  the blockwise method must equal full attention).
* ``merge`` — the exact combination of two partial results (PCP page §4.2,
  FCP page §3.3).
* ``attention_grad`` — dQ, dK, dV of ``attention`` for a given dO, from the
  definition of softmax attention (the backward that training-time context
  parallelism runs over the same blocks, PCP page §2.3).

Nothing here is parity-unpinned: ``tests/test_oracle.py`` pins every function
(brute force at 50 digits, closed forms, invariants, the pages' literal index
example), and ``tests/test_oracle_mutants.py`` checks that planted mistakes fail
those pins.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

CONTIGUOUS, ZIGZAG, STRIPED = 0, 1, 2
_LAYOUTS = {"contiguous": CONTIGUOUS, "zigzag": ZIGZAG, "striped": STRIPED}

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _dtype_code(a):
    if a.dtype == np.uint16:
        return 0
    if a.dtype == np.float32:
        return 1
    raise TypeError("oracle inputs are bf16 bit patterns (uint16) or float32, got %s" % a.dtype)


class Oracle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path=LIB):
        if not os.path.exists(path):
            from . import build as _b
            _b.build(out=path)
        lib = ctypes.CDLL(path)
        lib.oracle_local_positions.restype = ctypes.c_int64
        lib.oracle_local_positions.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               _i64p, ctypes.c_int32, _i32p, _i32p]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, _i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_double,
                                         _i64p, _i32p, ctypes.c_int64, _f64p, _f64p, _i64p, ctypes.c_int32]
        lib.oracle_softmax_row.restype = ctypes.c_int64
        lib.oracle_softmax_row.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, _i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_double,
                                           ctypes.c_int64, ctypes.c_int32, _f64p]
        lib.oracle_attention_grad.restype = ctypes.c_int
        lib.oracle_attention_grad.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, _i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_double,
                                              _f64p, _i64p, _i32p, ctypes.c_int64, _f64p, _f64p, _f64p, _f64p,
                                              ctypes.c_int32]
        lib.oracle_merge.restype = None
        lib.oracle_merge.argtypes = [ctypes.c_int64, ctypes.c_int32, _f64p, _f64p, _f64p, _f64p, _f64p, _f64p]
        self.lib = lib
        self.path = path

    # -- positions -----------------------------------------------------------
    def local_positions(self, S, cp, rank, layout="zigzag", doc_lens=None):
        """(positions, document starts) of `rank`'s tokens, both int32 ascending."""
        lay = _LAYOUTS[layout] if isinstance(layout, str) else int(layout)
        n_max = S // cp
        pos = np.zeros(n_max, np.int32)
        start = np.zeros(n_max, np.int32)
        docs = None if doc_lens is None else np.ascontiguousarray(doc_lens, np.int64)
        n = self.lib.oracle_local_positions(S, cp, rank, lay, _ptr(docs, _i64p),
                                            0 if docs is None else len(docs),
                                            _ptr(pos, _i32p), _ptr(start, _i32p))
        if n < 0:
            raise ValueError("sequence (or a document) is not divisible as the layout requires")
        return pos[:n], start[:n]

    # -- attention -----------------------------------------------------------
    def attention(self, q, k, v, q_pos=None, k_pos=None, q_start=None, causal=True, scale=None,
                  rows=None, heads=None, n_threads=0):
        """Exact attention of (row, head) pairs; returns (o [n, d], lse [n], n_visible [n]).

        q: [lq, hq, d]; k, v: [lk, hkv, d]. Without rows/heads every pair is
        computed, in order row * hq + head.
        """
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        code = _dtype_code(q)
        assert _dtype_code(k) == code and _dtype_code(v) == code
        lq, hq, d = q.shape
        lk, hkv, d2 = k.shape
        assert v.shape == k.shape and d2 == d
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        qp = None if q_pos is None else np.ascontiguousarray(q_pos, np.int32)
        kp = None if k_pos is None else np.ascontiguousarray(k_pos, np.int32)
        qs = None if q_start is None else np.ascontiguousarray(q_start, np.int32)
        if rows is None:
            r = h = None
            n = lq * hq
        else:
            r = np.ascontiguousarray(rows, np.int64)
            h = np.ascontiguousarray(heads, np.int32)
            assert r.shape == h.shape
            n = len(r)
        o = np.zeros((n, d), np.float64)
        lse = np.zeros(n, np.float64)
        cnt = np.zeros(n, np.int64)
        rc = self.lib.oracle_attention(q.ctypes.data, k.ctypes.data, v.ctypes.data, code, lq, lk, hq, hkv, d,
                                       _ptr(qp, _i32p), _ptr(qs, _i32p), _ptr(kp, _i32p), int(bool(causal)),
                                       float(scale), _ptr(r, _i64p), _ptr(h, _i32p), n,
                                       _ptr(o, _f64p), _ptr(lse, _f64p), _ptr(cnt, _i64p), int(n_threads))
        if rc != 0:
            raise ValueError("oracle_attention rejected its arguments")
        return o, lse, cnt

    def softmax_row(self, q, k, row, head, q_pos=None, k_pos=None, q_start=None, causal=True, scale=None):
        """Softmax weights of one (row, head) over all keys (0 where not visible)."""
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        code = _dtype_code(q)
        lq, hq, d = q.shape
        lk, hkv, _ = k.shape
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        qp = None if q_pos is None else np.ascontiguousarray(q_pos, np.int32)
        kp = None if k_pos is None else np.ascontiguousarray(k_pos, np.int32)
        qs = None if q_start is None else np.ascontiguousarray(q_start, np.int32)
        p = np.zeros(lk, np.float64)
        n = self.lib.oracle_softmax_row(q.ctypes.data, k.ctypes.data, code, lq, lk, hq, hkv, d,
                                        _ptr(qp, _i32p), _ptr(qs, _i32p), _ptr(kp, _i32p), int(bool(causal)),
                                        float(scale), int(row), int(head), _ptr(p, _f64p))
        if n < 0:
            raise ValueError("oracle_softmax_row rejected its arguments")
        return p

    # -- gradients -----------------------------------------------------------
    def attention_grad(self, q, k, v, dout, q_pos=None, k_pos=None, q_start=None, causal=True, scale=None,
                       rows=None, heads=None, n_threads=0):
        """Gradients of ``attention`` for the output gradient dout [lq, hq, d].

        Without rows/heads: returns (dq [lq, hq, d], dk [lk, hkv, d],
        dv [lk, hkv, d], delta [lq, hq]). With rows/heads: (dq [n, d], None,
        None, delta [n]) for those (row, head) pairs only.
        """
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        code = _dtype_code(q)
        assert _dtype_code(k) == code and _dtype_code(v) == code
        lq, hq, d = q.shape
        lk, hkv, _ = k.shape
        dout = np.ascontiguousarray(dout, np.float64)
        assert dout.shape == q.shape
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        qp = None if q_pos is None else np.ascontiguousarray(q_pos, np.int32)
        kp = None if k_pos is None else np.ascontiguousarray(k_pos, np.int32)
        qs = None if q_start is None else np.ascontiguousarray(q_start, np.int32)
        if rows is None:
            r = h = None
            n = lq * hq
            dk = np.zeros((lk, hkv, d), np.float64)
            dv = np.zeros((lk, hkv, d), np.float64)
        else:
            r = np.ascontiguousarray(rows, np.int64)
            h = np.ascontiguousarray(heads, np.int32)
            n = len(r)
            dk = dv = None
        dq = np.zeros((n, d), np.float64)
        delta = np.zeros(n, np.float64)
        rc = self.lib.oracle_attention_grad(q.ctypes.data, k.ctypes.data, v.ctypes.data, code, lq, lk, hq, hkv, d,
                                            _ptr(qp, _i32p), _ptr(qs, _i32p), _ptr(kp, _i32p), int(bool(causal)),
                                            float(scale), _ptr(dout, _f64p), _ptr(r, _i64p), _ptr(h, _i32p), n,
                                            _ptr(dq, _f64p), _ptr(dk, _f64p), _ptr(dv, _f64p), _ptr(delta, _f64p),
                                            int(n_threads))
        if rc != 0:
            raise ValueError("oracle_attention_grad rejected its arguments")
        if rows is None:
            return dq.reshape(lq, hq, d), dk, dv, delta.reshape(lq, hq)
        return dq, None, None, delta

    # -- merge ---------------------------------------------------------------
    def merge(self, o_a, lse_a, o_b, lse_b):
        """fp64 merge of two partial results over disjoint key sets."""
        o_a = np.ascontiguousarray(o_a, np.float64)
        o_b = np.ascontiguousarray(o_b, np.float64)
        lse_a = np.ascontiguousarray(lse_a, np.float64)
        lse_b = np.ascontiguousarray(lse_b, np.float64)
        n = lse_a.size
        d = o_a.size // max(n, 1)
        o = np.empty_like(o_a)
        lse = np.empty_like(lse_a)
        self.lib.oracle_merge(n, d, _ptr(o_a, _f64p), _ptr(lse_a, _f64p), _ptr(o_b, _f64p), _ptr(lse_b, _f64p),
                              _ptr(o, _f64p), _ptr(lse, _f64p))
        return o, lse


_default = None


def get():
    """The oracle built from oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
