"""Arrival pipeline on one GPU: KV blocks delivered by a copy stream while the
compute stream folds each arrived block into the rank's (O, LSE) state.

The FCP page ("从固定环到自由拓扑：FCP到底在解决什么") runs the communication and the
attention kernels on separate streams synchronised by events, with the KV cut
into blocks of a few thousand tokens so that both sides keep the pipeline full
(§4.3); it finds 1K-token blocks too fine, one event synchronisation per block
outweighing the overlap, and 8K right (§6.3); and it measures communication
alone, computation alone and the two overlapped before tuning anything (§7).

Here a copy stands in for the network link: from pinned host memory over PCIe
(about the bandwidth of one inter-node link) or from another device buffer (a
fast intra-node link). A block is cut into pieces of at most `chunk` keys; the
pieces pass through a ring of `n_slots` receive buffers on the device. Every
piece is one `cpattn_partial` call, so a piece is a KV block to the library.

Orchestration only: every arithmetic step runs in the HIP kernels behind the
C ABI; the copies are plain stream-ordered memory copies.
"""
from . import cpattn_partial, cpattn_varlen_partial


def split_blocks(block_keys, order, chunk):
    """Arrival schedule of pieces: for each block id in `order` (block b has
    `block_keys[b]` keys), its keys cut into consecutive ranges of at most
    `chunk` keys. Returns [(block, lo, hi), ...] in arrival order; a block
    with no keys contributes one empty piece, so every block is folded in."""
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    pieces = []
    for b in order:
        n = int(block_keys[b])
        if n == 0:
            pieces.append((b, 0, 0))
            continue
        for lo in range(0, n, chunk):
            pieces.append((b, lo, min(lo + chunk, n)))
    return pieces


def plan(n_pieces, n_slots):
    """The two-stream schedule as data.

    Piece i lands in slot i % n_slots. Its copy waits until the kernel of
    piece i - n_slots, the slot's previous user, has finished with it, then
    records arrived[i]; its kernel waits for arrived[i], folds the piece in
    (accumulating from the second piece on) and records free[i]. Kernels run
    in arrival order on the compute stream and copies in arrival order on
    the copy stream. Returns a list of ops, each
    {"kind": "copy" | "kernel", "piece": i, "slot": s, "wait": [...], "record": name,
     "accumulate": bool (kernels)}, in the order a host issues them.
    """
    if n_slots < 1:
        raise ValueError("n_slots must be >= 1")
    ops = []
    for i in range(n_pieces):
        s = i % n_slots
        ops.append({"kind": "copy", "piece": i, "slot": s,
                    "wait": ["free%d" % (i - n_slots)] if i >= n_slots else [], "record": "arrived%d" % i})
        ops.append({"kind": "kernel", "piece": i, "slot": s, "wait": ["arrived%d" % i], "record": "free%d" % i,
                    "accumulate": i > 0})
    return ops


class ArrivalPipeline:
    """Delivers a RankShare's KV blocks piece by piece on a copy stream and
    folds each piece in on a compute stream as soon as it has arrived.

    source "host": the blocks are staged once in pinned host memory and each
    piece is copied host -> device; "device": they are copied device ->
    device from the share's own resident tensors.
    """

    def __init__(self, share, chunk, n_slots=3, source="host"):
        import torch
        if source not in ("host", "device"):
            raise ValueError("source must be 'host' or 'device'")
        self.share, self.chunk, self.n_slots, self.source = share, int(chunk), int(n_slots), source
        k0 = share.k_blocks[0]
        hkv, d = k0.shape[1], k0.shape[2]
        dev = k0.device
        if source == "host":
            self.k_src = [k.cpu().pin_memory() for k in share.k_blocks]
            self.v_src = [v.cpu().pin_memory() for v in share.v_blocks]
            self.p_src = [p.cpu().pin_memory() for p in share.k_pos_blocks]
        else:
            self.k_src, self.v_src, self.p_src = share.k_blocks, share.v_blocks, share.k_pos_blocks
        self.k_slot = [torch.empty((self.chunk, hkv, d), dtype=k0.dtype, device=dev) for _ in range(self.n_slots)]
        self.v_slot = [torch.empty((self.chunk, hkv, d), dtype=k0.dtype, device=dev) for _ in range(self.n_slots)]
        self.p_slot = [torch.empty((self.chunk,), dtype=torch.int32, device=dev) for _ in range(self.n_slots)]
        self.copy_stream = torch.cuda.Stream(device=dev)
        self.compute_stream = torch.cuda.Stream(device=dev)

    def pieces(self, order):
        return split_blocks([k.shape[0] for k in self.share.k_blocks], order, self.chunk)

    def _fold(self, k, v, kp, accumulate, stream):
        sh = self.share
        if sh.cu_seqlens is not None:
            cpattn_varlen_partial(sh.q, k, v, sh.q_pos, kp, sh.cu_seqlens, sh.o, sh.lse, accumulate=accumulate,
                                  stream=stream)
        else:
            cpattn_partial(sh.q, k, v, sh.q_pos, kp, sh.o, sh.lse, causal=sh.causal, accumulate=accumulate,
                           stream=stream)

    def _copy(self, i, piece):
        b, lo, hi = piece
        s = i % self.n_slots
        n = hi - lo
        self.k_slot[s][:n].copy_(self.k_src[b][lo:hi], non_blocking=True)
        self.v_slot[s][:n].copy_(self.v_src[b][lo:hi], non_blocking=True)
        self.p_slot[s][:n].copy_(self.p_src[b][lo:hi], non_blocking=True)

    def run(self, order, start_event=None):
        """The overlapped pipeline; enqueues everything and returns (o, lse)
        (valid once the compute stream has finished)."""
        import torch
        pieces = self.pieces(order)
        events = {}
        cs, ks = self.copy_stream, self.compute_stream
        if start_event is not None:
            cs.wait_event(start_event)
            ks.wait_event(start_event)
        for op in plan(len(pieces), self.n_slots):
            i, s = op["piece"], op["slot"]
            stream = cs if op["kind"] == "copy" else ks
            for w in op["wait"]:
                stream.wait_event(events[w])
            with torch.cuda.stream(stream):
                if op["kind"] == "copy":
                    self._copy(i, pieces[i])
                else:
                    n = pieces[i][2] - pieces[i][1]
                    self._fold(self.k_slot[s][:n], self.v_slot[s][:n], self.p_slot[s][:n], op["accumulate"], ks)
            ev = torch.cuda.Event()
            ev.record(stream)
            events[op["record"]] = ev
        return self.share.o, self.share.lse

    def comm_only(self, order):
        """Only the copies, back to back on the copy stream."""
        import torch
        with torch.cuda.stream(self.copy_stream):
            for i, piece in enumerate(self.pieces(order)):
                self._copy(i, piece)

    def compute_only(self, order):
        """Only the kernels, on the resident device blocks (no copies, no waits)."""
        sh = self.share
        for i, (b, lo, hi) in enumerate(self.pieces(order)):
            self._fold(sh.k_blocks[b][lo:hi], sh.v_blocks[b][lo:hi], sh.k_pos_blocks[b][lo:hi], i > 0,
                       self.compute_stream)

    def measure(self, order, reps=3, warmup=1):
        """Milliseconds per step of communication alone, computation alone and
        the overlapped pipeline (each the mean of `reps` after `warmup`), and
        the share of the shorter side the overlap hid:
        (comm + compute - overlapped) / min(comm, compute)."""
        import torch
        dev = self.share.q.device

        def timed(fn, stream):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize(dev)
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(reps):
                fn()
            t1.record(stream)
            torch.cuda.synchronize(dev)
            return t0.elapsed_time(t1) / reps

        comm = timed(lambda: self.comm_only(order), self.copy_stream)
        compute = timed(lambda: self.compute_only(order), self.compute_stream)

        def overlapped():
            start = torch.cuda.Event()
            start.record(self.compute_stream)
            self.run(order, start_event=start)
            # the next repetition's copies may not overwrite a slot still in use
            self.copy_stream.wait_stream(self.compute_stream)

        both = timed(overlapped, self.compute_stream)
        hidden = (comm + compute - both) / min(comm, compute) if min(comm, compute) > 0 else 0.0
        return {"comm_ms": comm, "compute_ms": compute, "overlapped_ms": both, "hidden": hidden,
                "pieces": len(self.pieces(order)), "chunk": self.chunk, "slots": self.n_slots,
                "source": self.source}
