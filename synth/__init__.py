"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds no attention arithmetic: only random tensors, their rounding
to bf16, block arrival orders, document lengths, sampled rows, and the table of
workload shapes. Positions (which tokens a rank owns) are NOT computed here:
the product library and the oracle each derive them on their own.

The pages measure on unnamed 7B/13B-class attention layers and on trained
models; no dataset is named, so i.i.d. normal tensors of the pages' shapes
stand in for activations.
"""
from dataclasses import dataclass, field, replace
from concurrent.futures import ThreadPoolExecutor
import math

import numpy as np

# ---------------------------------------------------------------------------
# bf16 helpers (input preparation only)


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# random tensors

_TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "dout": 3}


def normal_tensor(shape, seed, which, block=0, sigma=1.0, dtype="bf16"):
    """N(0,1)*sigma tensor drawn from PCG64 seeded by (seed, which, block).

    Returns uint16 bf16 bits for dtype 'bf16', float32 for 'f32'. Each (tensor,
    block) has its own stream, so blocks can be drawn independently.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TENSOR_IDS[which], block])))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def arrival_order(n_blocks, seed):
    """Seeded permutation of block ids: the order in which KV blocks arrive."""
    return np.random.default_rng(seed).permutation(n_blocks).astype(np.int64)


def doc_lengths(total, lo, hi, multiple, seed):
    """Document lengths log-uniform in [lo, hi], rounded down to `multiple`.

    Drawn until the next one would overflow `total`; the last document takes
    the remainder (which may be shorter than lo).
    """
    rng = np.random.default_rng(seed)
    out = []
    used = 0
    while used < total:
        L = int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L -= L % multiple
        if L <= 0:
            continue
        if used + L > total:
            L = total - used
        out.append(L)
        used += L
    return np.array(out, np.int64)


# ---------------------------------------------------------------------------
# workloads


@dataclass(frozen=True)
class Workload:
    """One rank's share of a context-parallel attention problem.

    block_kind:
      'rank_shares' — KV block b is rank b's share under the same layout;
      'chunks'      — KV block b is the b-th of n_blocks equal contiguous chunks;
      'whole'       — one block holding the whole sequence.
    """
    name: str
    S: int
    cp: int
    rank: int
    layout: str            # 'zigzag' | 'contiguous' | 'striped'
    hq: int
    hkv: int
    d: int
    dtype: str             # 'bf16' | 'f32'
    sigma: float
    block_kind: str
    n_blocks: int
    seed: int
    docs: tuple = None     # (lo, hi) for log-uniform document lengths, or None
    sampled_rows: int = 0  # 0 = every (row, head) is checked
    description: str = ""

    @property
    def lq(self):
        return self.S // self.cp

    def doc_lens(self):
        if self.docs is None:
            return None
        return doc_lengths(self.S, self.docs[0], self.docs[1], 2 * self.cp, self.seed + 500)

    def block_len(self, b):
        if self.block_kind == "whole":
            return self.S
        return self.S // self.n_blocks

    def arrival(self):
        return arrival_order(self.n_blocks, self.seed + 1000)

    def q(self):
        return normal_tensor((self.lq, self.hq, self.d), self.seed, "q", 0, self.sigma, self.dtype)

    def dout(self):
        """Output gradient for the backward: N(0,1), shape and dtype of Q."""
        return normal_tensor((self.lq, self.hq, self.d), self.seed, "dout", 0, 1.0, self.dtype)

    def kv_block(self, b, which):
        return normal_tensor((self.block_len(b), self.hkv, self.d), self.seed, which, b, self.sigma, self.dtype)

    def kv_all(self, which, threads=8):
        """All blocks of K (or V) concatenated in block-id order."""
        with ThreadPoolExecutor(max_workers=threads) as ex:
            parts = list(ex.map(lambda b: self.kv_block(b, which), range(self.n_blocks)))
        return np.concatenate(parts, axis=0)

    def sample_pairs(self, n_pairs=None, chunk=None):
        """(rows, heads) to check, stratified evenly over heads: for every head
        the first and last token of each chunk of `chunk` local tokens (default:
        the rank's two zig-zag halves), plus n_pairs // hq interior tokens drawn
        uniformly from the rest. n_pairs = 0 (and no sampled_rows): every pair."""
        n_pairs = n_pairs or self.sampled_rows
        if not n_pairs:
            r = np.repeat(np.arange(self.lq, dtype=np.int64), self.hq)
            h = np.tile(np.arange(self.hq, dtype=np.int32), self.lq)
            return r, h
        rng = np.random.default_rng(self.seed + 2000)
        chunk = chunk or max(1, self.lq // 2)
        ends = np.array(sorted({e for c0 in range(0, self.lq, chunk) for e in (c0, min(c0 + chunk, self.lq) - 1)}),
                        np.int64)
        interior = np.setdiff1d(np.arange(self.lq, dtype=np.int64), ends)
        per_head = min(max(1, n_pairs // self.hq), len(interior))
        rows, heads = [], []
        for h in range(self.hq):
            extra = rng.choice(interior, size=per_head, replace=False)
            rr = np.unique(np.concatenate([ends, extra.astype(np.int64)]))
            rows.append(rr)
            heads.append(np.full(len(rr), h, np.int32))
        return np.concatenate(rows), np.concatenate(heads)

    def scaled(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "zigzag1k_cp4_h1_d64_f32": Workload("zigzag1k_cp4_h1_d64_f32", S=1024, cp=4, rank=1, layout="zigzag", hq=1, hkv=1, d=64, dtype="f32", sigma=1.0,
                   block_kind="rank_shares", n_blocks=4, seed=1000,
                   description="1 head, d64, fp32, 1024 tokens zig-zag cp4, rank 1: 256 queries vs 4 rank-share "
                               "blocks of 256 in seeded order"),
    "zigzag64k_cp8_h32_d128": Workload("zigzag64k_cp8_h32_d128", S=65536, cp=8, rank=1, layout="zigzag", hq=32, hkv=32, d=128, dtype="bf16", sigma=0.5,
                   block_kind="rank_shares", n_blocks=8, seed=1001,
                   description="7B-class layer, 64K tokens zig-zag cp8, rank 1: 8192 queries x 32 heads, d128, "
                               "vs 8 rank-share blocks of 8192 in seeded order"),
    "contig128k_h16kv2_d64": Workload("contig128k_h16kv2_d64", S=131072, cp=1, rank=0, layout="contiguous", hq=16, hkv=2, d=64, dtype="bf16", sigma=1.0,
                   block_kind="whole", n_blocks=1, seed=1002, sampled_rows=4096,
                   description="Ulysses head share of cp4 with 64 Q / 8 KV heads: 16 Q / 2 KV heads, d64, full "
                               "causal 131072 tokens"),
    "docs128k_zigzag_cp4_h32_d128": Workload("docs128k_zigzag_cp4_h32_d128", S=131072, cp=4, rank=1, layout="zigzag", hq=32, hkv=32, d=128, dtype="bf16", sigma=0.5,
                   block_kind="rank_shares", n_blocks=4, seed=1003, docs=(1024, 32768),
                   description="packed 128K tokens of log-uniform [1K,32K] documents, per-document zig-zag cp4, "
                               "rank 1: 32768 queries x 32 heads, d128, vs 4 rank-share blocks"),
    "zigzag1m_cp8_h32kv8_d128": Workload("zigzag1m_cp8_h32kv8_d128", S=1 << 20, cp=8, rank=1, layout="zigzag", hq=32, hkv=8, d=128, dtype="bf16", sigma=0.5,
                   block_kind="chunks", n_blocks=16, seed=1004, sampled_rows=2048,
                   description="1M tokens zig-zag cp8, rank 1: 131072 queries x 32 Q / 8 KV heads, d128, vs 16 "
                               "chunks of 65536 in seeded order"),
}
