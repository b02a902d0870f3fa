"""One rank's share of context-parallel attention: device-resident inputs and
the per-step driver that feeds KV blocks to the library in arrival order.

Orchestration only — every arithmetic step runs in the HIP kernels behind
the C ABI. This is the loop of the FCP page ("从固定环到自由拓扑：FCP到底在解决
什么", §3.3): each arriving block is folded into the rank's running
(O, LSE) state, in whatever order the blocks arrive.
"""
import numpy as np

from . import (cpattn_bwd_delta, cpattn_merge_lse, cpattn_partial, cpattn_partial_bwd, cpattn_partial_bwd_multi,
               cpattn_partial_multi, cpattn_varlen_bwd_plan, cpattn_varlen_partial, cpattn_varlen_plan,
               cpattn_zigzag_index)


def bits_to_device(a, device="cuda"):
    """numpy uint16 (bf16 bit patterns) or float32 array -> torch tensor on `device`."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def block_positions(S, cp, n_blocks, block_kind, layout, cu_seqlens=None):
    """Global positions of every KV block's tokens, in block-id order (int32
    numpy arrays), all from the library's index builder: rank b's share under
    the workload's layout ('rank_shares'), the b-th of n_blocks equal
    contiguous chunks ('chunks': the contiguous split with cp = n_blocks), or
    the whole sequence ('whole': the contiguous split with cp = 1)."""
    if block_kind == "rank_shares":
        return [cpattn_zigzag_index(S, cp, b, layout, cu_seqlens)[0] for b in range(n_blocks)]
    if block_kind == "chunks":
        return [cpattn_zigzag_index(S, n_blocks, b, "contiguous")[0] for b in range(n_blocks)]
    if block_kind == "whole":
        return [cpattn_zigzag_index(S, 1, 0, "contiguous")[0]]
    raise ValueError(block_kind)


class RankShare:
    """Device tensors of one rank's share and the step that runs every block.

    q [lq, hq, d]; k_blocks / v_blocks: lists of [lk_b, hkv, d]; positions as
    int32 device tensors; cu_seqlens (optional) as an int32 device tensor.
    """

    def __init__(self, q, k_blocks, v_blocks, q_pos, k_pos_blocks, cu_seqlens=None, causal=True, out_dtype=None):
        import torch
        self.q, self.k_blocks, self.v_blocks = q, k_blocks, v_blocks
        self.q_pos, self.k_pos_blocks = q_pos, k_pos_blocks
        self.cu_seqlens = cu_seqlens
        self.causal = causal
        lq, hq, d = q.shape
        self.out_dtype = out_dtype or q.dtype
        self.o = torch.empty((lq, hq, d), dtype=self.out_dtype, device=q.device)
        self.lse = torch.empty((hq, lq), dtype=torch.float32, device=q.device)
        self._o_part = None
        self._lse_part = None
        self.plans = None   # per-block plans of the document calls (plan_blocks)
        self.bwd_plans = None   # and of their gradient calls

    @property
    def n_blocks(self):
        return len(self.k_blocks)

    def plan_blocks(self, q_pos_host, k_pos_host, cu_host):
        """Plans of the document calls (cpattn_varlen_plan, from the host copies
        of the positions), one per block, on the device; used by call_block."""
        import torch
        lq, hq, d = self.q.shape
        hkv = self.k_blocks[0].shape[1]
        dt = "bf16" if self.q.dtype == torch.bfloat16 else "f32"
        self.plans = [torch.from_numpy(cpattn_varlen_plan(q_pos_host, kp, cu_host, hq, hkv, d, dt)).to(self.q.device)
                      for kp in k_pos_host]
        self.bwd_plans = [torch.from_numpy(cpattn_varlen_bwd_plan(q_pos_host, kp, cu_host, hq, hkv)).to(self.q.device)
                          for kp in k_pos_host]

    def call_block(self, b, o, lse, accumulate):
        if self.cu_seqlens is not None:
            cpattn_varlen_partial(self.q, self.k_blocks[b], self.v_blocks[b], self.q_pos, self.k_pos_blocks[b],
                                  self.cu_seqlens, o, lse, accumulate=accumulate,
                                  plan=None if self.plans is None else self.plans[b])
        else:
            cpattn_partial(self.q, self.k_blocks[b], self.v_blocks[b], self.q_pos, self.k_pos_blocks[b], o, lse,
                           causal=self.causal, accumulate=accumulate)

    def call_multi(self, blocks, o, lse, accumulate):
        blocks = list(blocks)
        cpattn_partial_multi(self.q, [self.k_blocks[b] for b in blocks], [self.v_blocks[b] for b in blocks],
                             self.q_pos, [self.k_pos_blocks[b] for b in blocks], o, lse, causal=self.causal,
                             accumulate=accumulate, cu_seqlens=self.cu_seqlens)

    def step(self, order, mode="accumulate"):
        """Fold every block, in `order`, into (self.o, self.lse) and return them.

        mode 'accumulate': the kernel merges each block in its epilogue.
        mode 'merge': each block is written as its own partial, then merged by
        the standalone merge kernel.
        mode 'fused': all blocks in one cpattn_partial_multi call (the state
        stays in registers between blocks).
        """
        import torch
        order = list(order)
        if mode == "fused":
            self.call_multi(order, self.o, self.lse, accumulate=False)
            return self.o, self.lse
        self.call_block(order[0], self.o, self.lse, accumulate=False)
        if mode == "accumulate":
            for b in order[1:]:
                self.call_block(b, self.o, self.lse, accumulate=True)
        elif mode == "merge":
            if self._o_part is None:
                self._o_part = torch.empty_like(self.o)
                self._lse_part = torch.empty_like(self.lse)
            for b in order[1:]:
                self.call_block(b, self._o_part, self._lse_part, accumulate=False)
                cpattn_merge_lse(self.o, self.lse, self._o_part, self._lse_part)
        else:
            raise ValueError(mode)
        return self.o, self.lse

    def backward(self, dout, order, lse=None, mode="blocks"):
        """Gradients of the step: dq [lq, hq, d] and per-block dk, dv [lk_b, hkv, d]
        (float32), with every block's backward run in `order`.

        Uses the merged (self.o, self.lse) of the last forward step (or `lse`):
        D = <dO, O> once, then (mode "blocks") one cpattn_partial_bwd call per
        block, the first writing dq and the others adding to it, or (mode
        "fused") one cpattn_partial_bwd_multi call over the blocks in `order`;
        each block's dk, dv are written. With documents and plans
        (plan_blocks), each per-block call is planned.
        """
        import torch
        lq, hq, d = self.q.shape
        dev = self.q.device
        if getattr(self, "dq", None) is None:
            self.dq = torch.empty((lq, hq, d), dtype=torch.float32, device=dev)
            self.delta = torch.empty((hq, lq), dtype=torch.float32, device=dev)
            self.dk = [torch.empty(k.shape, dtype=torch.float32, device=dev) for k in self.k_blocks]
            self.dv = [torch.empty(k.shape, dtype=torch.float32, device=dev) for k in self.k_blocks]
        lse = self.lse if lse is None else lse
        cpattn_bwd_delta(self.o, dout, self.delta)
        if mode == "fused":
            cpattn_partial_bwd_multi(self.q, [self.k_blocks[b] for b in order], [self.v_blocks[b] for b in order],
                                     dout, self.q_pos, [self.k_pos_blocks[b] for b in order], lse, self.delta,
                                     self.dq, [self.dk[b] for b in order], [self.dv[b] for b in order],
                                     causal=self.causal, cu_seqlens=self.cu_seqlens)
            return self.dq, self.dk, self.dv
        if mode != "blocks":
            raise ValueError("mode must be 'blocks' or 'fused'")
        for i, b in enumerate(order):
            cpattn_partial_bwd(self.q, self.k_blocks[b], self.v_blocks[b], dout, self.q_pos, self.k_pos_blocks[b],
                               lse, self.delta, self.dq, self.dk[b], self.dv[b], causal=self.causal,
                               accumulate_dq=i > 0, accumulate_dkv=False, cu_seqlens=self.cu_seqlens,
                               plan=None if self.bwd_plans is None else self.bwd_plans[b])
        return self.dq, self.dk, self.dv


def share_from_workload(wl, device="cuda", blocks=None, plan=True):
    """Build a RankShare for a synth.Workload: positions from the library's
    index builder, tensors from the seeded generators; with documents (and
    `plan`), the plan of every block's call."""
    import torch
    docs = wl.doc_lens()
    cu = None if docs is None else np.concatenate([[0], np.cumsum(docs)]).astype(np.int32)
    q_pos, _ = cpattn_zigzag_index(wl.S, wl.cp, wl.rank, wl.layout, cu)
    kps = block_positions(wl.S, wl.cp, wl.n_blocks, wl.block_kind, wl.layout, cu)
    blocks = range(wl.n_blocks) if blocks is None else blocks
    kb = [bits_to_device(wl.kv_block(b, "k"), device) for b in blocks]
    vb = [bits_to_device(wl.kv_block(b, "v"), device) for b in blocks]
    kp = [torch.from_numpy(kps[b]).to(device) for b in blocks]
    share = RankShare(bits_to_device(wl.q(), device), kb, vb, torch.from_numpy(q_pos).to(device), kp,
                      None if cu is None else torch.from_numpy(cu).to(device))
    share.q_pos_host = q_pos
    share.k_pos_host = [kps[b] for b in blocks]
    share.cu_host = cu
    if cu is not None and plan:
        share.plan_blocks(q_pos, share.k_pos_host, cu)
    return share
