"""Host-side replay of the global-memory address arithmetic of the gfx950
kernels (partial_fwd.hip, partial_bwd.hip and the tile_io.hpp helpers they
share), for a given launch.

For every workgroup and wave of a launch the replay recomputes what the
kernel computes from its arguments, in the kernel's order: the workgroup
remap, the key-range searches (every probe), the tiles each workgroup
loads, the buffer descriptors (base and record count) of every
range-checked load, the 32-bit offsets every lane passes, and the row and
byte indices of every plain load and store. The per-workgroup decisions are
formed for all workgroups at once (numpy arrays over the grid), and each
access is checked against the extent of the tensor it addresses:

* a raw buffer load (stride 0) reads a lane's bytes only when the lane's
  offset is below the descriptor's record count (the hardware's range
  check; lanes at or past it read zeros without touching memory). The
  record count must be a non-negative 32-bit int (a negative count would be
  a huge unsigned one, and nothing would be range-checked), every offset a
  non-negative 32-bit value, and every byte a lane reads must lie inside
  the tensor. The scalar offset of the direct-to-LDS loads is counted in
  the address but not in the range check, the conservative reading (a lane
  whose own offset is in range is taken to read);
* a plain load or store must lie wholly inside its tensor;
* an index into an int32 array (positions, document offsets) must lie in
  [0, n).

When many descriptors share one set of lane offsets, the lanes that read
are those whose offset is below the record count, so the lowest and highest
byte read follow from the sorted offsets; the check of those two bytes
covers every lane.

It also checks the launch-level invariants the kernels rely on: the remap
is a permutation of the grid, and the values that decide barrier counts
(the workgroup's tile range, its early exit) agree between its waves.

The replay models the committed sources; when those change, so must it.
Test infrastructure: nothing in the library imports it.
"""
from functools import lru_cache

import numpy as np

LANES = np.arange(64, dtype=np.int64)
INT32_MAX = (1 << 31) - 1
U32 = 1 << 32


class AccessError(AssertionError):
    pass


class Mem:
    """Extents (bytes) of the tensors one launch addresses, and the checks."""

    def __init__(self, **sizes):
        self.size = dict(sizes)
        self.stats = {}

    def _note(self, kind, name, n, lo, hi, count=0):
        s = self.stats.setdefault((kind, name), {"n": 0, "lo": None, "hi": None, "max_count": 0})
        s["n"] += int(n)
        if lo is not None:
            s["lo"] = lo if s["lo"] is None else min(s["lo"], lo)
            s["hi"] = hi if s["hi"] is None else max(s["hi"], hi)
        s["max_count"] = max(s["max_count"], int(count))

    def _extent(self, what, name, lo, hi):
        if lo < 0 or hi > self.size[name]:
            raise AccessError("%s %s: bytes [%d, %d) outside [0, %d)" % (what, name, lo, hi, self.size[name]))

    def buffer(self, name, base, count, voff, width, what=""):
        """Raw buffer loads: descriptor bases `base` (byte offsets from the start
        of tensor `name`, scalar offsets included) and record counts `count`
        (bytes), shape [n]; lane offsets `voff`, either [lanes] (shared by every
        descriptor) or [n, lanes]; `width` bytes a lane."""
        base = np.atleast_1d(np.asarray(base, np.int64))
        count = np.broadcast_to(np.asarray(count, np.int64), base.shape)
        voff = np.asarray(voff, np.int64)
        if base.size == 0:
            return
        if count.min() < 0 or count.max() > INT32_MAX:
            raise AccessError("%s %s: record count %d .. %d is not a non-negative int" % (
                what, name, count.min(), count.max()))
        if voff.size and (voff.min() < 0 or voff.max() >= U32):
            raise AccessError("%s %s: lane offset %d .. %d out of 32 bits" % (what, name, voff.min(), voff.max()))
        if voff.ndim == 1:
            vs = np.sort(voff)
            k = np.searchsorted(vs, count, side="left")  # lanes whose offset is below the count
            live = k > 0
            if not live.any():
                self._note("buffer", name, base.size, None, None, count.max())
                return
            lo = int((base[live] + vs[0]).min())
            hi = int((base[live] + vs[k[live] - 1]).max()) + width
        else:
            live = voff < count[:, None]
            if not live.any():
                self._note("buffer", name, base.size, None, None, count.max())
                return
            addr = base[:, None] + voff
            lo = int(addr[live].min())
            hi = int(addr[live].max()) + width
        self._extent(what, name, lo, hi)
        self._note("buffer", name, base.size, lo, hi, count.max())

    def plain(self, name, byte_off, width, what=""):
        """Plain (unchecked) global loads or stores of `width` bytes at each offset."""
        off = np.asarray(byte_off, np.int64)
        if off.size == 0:
            return
        lo, hi = int(off.min()), int(off.max()) + width
        self._extent(what, name, lo, hi)
        self._note("plain", name, off.size, lo, hi)

    def index(self, name, idx, what=""):
        """int32 element reads a[idx]."""
        self.plain(name, np.asarray(idx, np.int64) * 4, 4, what)

    @staticmethod
    def lds(off, width, limit, what=""):
        off = np.asarray(off, np.int64)
        if off.size and (off.min() < 0 or off.max() + width > limit):
            raise AccessError("%s: LDS bytes [%d, %d) outside [0, %d)" % (what, off.min(), off.max() + width, limit))

    def summary(self):
        out = []
        for (kind, name), s in sorted(self.stats.items()):
            out.append("%s %s: %d accesses, bytes [%s, %s) of %d%s" % (
                kind, name, s["n"], s["lo"], s["hi"], self.size[name],
                ", max record count %d" % s["max_count"] if kind == "buffer" else ""))
        return out


def xcd_remap(bid, n):
    x, slot = bid & 7, bid >> 3
    q, rem = n >> 3, n & 7
    return x * q + np.minimum(x, rem) + slot


def check_remap(n):
    """The workgroup remap is a permutation of [0, n)."""
    if n == 0:
        return
    got = np.sort(xcd_remap(np.arange(n, dtype=np.int64), n))
    if not np.array_equal(got, np.arange(n)):
        raise AccessError("workgroup remap is not a permutation of %d ids" % n)


def clamp_rows(n, hi):
    return np.minimum(np.maximum(n, 0), hi)


def ragged_ranges(starts, lengths):
    """Concatenation of arange(s, s + n) for each (s, n), and the entry each came from."""
    lengths = np.asarray(lengths, np.int64)
    owner = np.repeat(np.arange(lengths.size), lengths)
    first = np.cumsum(lengths) - lengths
    return np.asarray(starts, np.int64)[owner] + np.arange(lengths.sum()) - first[owner], owner


# ---------------------------------------------------------------------------
# searches (device_common.hpp)

class Searches:
    """Wave-cooperative upper bounds (every lane's probe checked) and the
    per-lane binary searches over document offsets. A search is a pure
    function of (array, n, x): its probes are checked the first time and the
    result reused."""

    def __init__(self, mem, arrays):
        self.mem = mem
        self.arrays = arrays  # name -> int32 numpy array
        self.wave = lru_cache(maxsize=None)(self._wave)
        self.upper = lru_cache(maxsize=None)(self._upper)
        self.start = lru_cache(maxsize=None)(self._doc_start)
        self.end = lru_cache(maxsize=None)(self._doc_end)

    def _wave(self, name, n, x):
        a = self.arrays[name]
        lo, hi = 0, n
        while lo < hi:
            step = (hi - lo + 63) >> 6
            first = lo + LANES * step
            probe = first < hi
            idx = np.where(probe, np.minimum(first + step, hi) - 1, lo)
            self.mem.index(name, idx, "wave search")  # every lane's index, probing or not
            c = int((probe & (a[idx] <= x)).sum())
            seg = lo + c * step
            if seg >= hi:
                lo = hi
            else:
                hi = min(seg + step, hi) - 1
                lo = seg
        return lo

    def _upper(self, name, n, x):
        a = self.arrays[name]
        lo, hi = 0, n
        while lo < hi:
            mid = (lo + hi) >> 1
            self.mem.index(name, mid, "binary search")
            if a[mid] <= x:
                lo = mid + 1
            else:
                hi = mid
        return lo

    def _doc_start(self, cu, n_seqs, x):
        idx = max(self.upper(cu, n_seqs + 1, x) - 1, 0)
        self.mem.index(cu, idx, "doc_start")
        return int(self.arrays[cu][idx])

    def _doc_end(self, cu, n_seqs, x):
        idx = self.upper(cu, n_seqs + 1, x)
        if idx <= n_seqs:
            self.mem.index(cu, idx, "doc_end")
            return int(self.arrays[cu][idx])
        return INT32_MAX

    @staticmethod
    def _many(fn, xs):
        xs = np.asarray(xs, np.int64)
        u, inv = np.unique(xs, return_inverse=True)
        return np.array([fn(int(x)) for x in u], np.int64)[inv].reshape(xs.shape)

    def wave_upper_bound(self, name, n, xs):
        return self._many(lambda x: self.wave(name, int(n), x), xs)

    def doc_start(self, cu, n_seqs, xs):
        return self._many(lambda x: self.start(cu, int(n_seqs), x), xs)

    def doc_end(self, cu, n_seqs, xs):
        return self._many(lambda x: self.end(cu, int(n_seqs), x), xs)


# ---------------------------------------------------------------------------
# tile staging (tile_io.hpp) for the partial-attention kernel

class FwdCfg:
    NW = 8  # waves sharing a tile's loads

    def __init__(self, in_bf16, D):
        self.bf16 = in_bf16
        self.D = D
        self.esz = 2 if in_bf16 else 4
        self.NB = (4 if D == 64 else 2) if in_bf16 else 1
        self.BK = 32 * self.NB
        self.row_bytes = D * self.esz
        self.tile_bytes = self.BK * self.row_bytes
        self.n_inst = self.tile_bytes // 1024
        self.rpi = 1024 // self.row_bytes
        self.NQ = D // 16 if in_bf16 else D // 2
        self.NDT = D // 32
        assert self.n_inst % self.NW == 0 and (self.NW * self.rpi) % 16 == 0

    def swz(self, row, is_v):
        if self.bf16:
            if is_v:
                return ((row & 3) << 2) if self.D == 128 else (((row >> 1) & 1) << 2)
            return (row & 15) if self.D == 128 else ((row >> 1) & 7)
        return row & 15

    def lane_voff(self, wave, row_stride, is_v):
        lr = (LANES * 16) // self.row_bytes
        pc = ((LANES * 16) % self.row_bytes) >> 4
        row = wave * self.rpi + lr
        chunk = pc ^ self.swz(row, is_v)
        if chunk.max() >= self.row_bytes // 16:
            raise AccessError("swizzled chunk leaves the row")
        return lr * row_stride + chunk * 16


def load_tile(mem, c, tensor, head_base, row_stride, r0, lk, wave, is_v):
    """Direct-to-LDS loads of K or V tiles: one wave's instructions, for
    workgroups with first rows r0[n], head offsets head_base[n]."""
    r0 = np.atleast_1d(np.asarray(r0, np.int64))
    head_base = np.broadcast_to(np.asarray(head_base, np.int64), r0.shape)
    base = head_base + r0 * row_stride
    rows = lk - r0
    if r0.size and rows.min() <= 0:
        # the helper assumes a tile that starts inside the block (its tail
        # branch forms the count from rows - 1)
        raise AccessError("load_tile asked for a tile at or past the block's end")
    full = rows >= c.BK
    voff0 = c.lane_voff(wave, row_stride, is_v)
    lr = (LANES * 16) // c.row_bytes
    for it in range(c.n_inst // c.NW):
        inst = wave + c.NW * it
        mem.lds(inst * 1024 + LANES * 16, 16, c.tile_bytes, "load_tile")
        if full.any():
            mem.buffer(tensor, base[full] + inst * c.rpi * row_stride, (c.BK - 1) * row_stride + c.row_bytes, voff0,
                       16, "load_tile")
        if (~full).any():
            rt = rows[~full][:, None]
            row = inst * c.rpi + lr
            rc = np.where(row < rt, row, rt - 1)
            voff = voff0 + (rc - lr) * row_stride
            mem.buffer(tensor, base[~full], (rows[~full] - 1) * row_stride + c.row_bytes, voff, 16,
                       "load_tile (tail)")


def load_positions(mem, src, r0, lk, wave, BK=64):
    E = BK // FwdCfg.NW
    r0 = np.atleast_1d(np.asarray(r0, np.int64))
    rows = np.minimum(lk - r0, BK)
    if r0.size and rows.min() <= 0:
        raise AccessError("load_positions asked for positions at or past the block's end")
    issuing = LANES[LANES < E]  # the load sits under `lane < E`
    e = E * wave + (issuing & (E - 1))
    idx = np.where(e < rows[:, None], e, rows[:, None] - 1)
    mem.buffer(src, r0 * 4, rows * 4, idx * 4, 4, "load_positions")
    mem.lds(E * wave * 4 + issuing * 4, 4, BK * 4, "load_positions")


def fetch_tiles(mem, c, tensor, head_base, row_stride, r0s, lims, wave, is_v):
    """Register-staged fetches (fetch_tile) of tiles with first rows r0s and key limits lims."""
    r0s = np.asarray(r0s, np.int64)
    rows = clamp_rows(np.asarray(lims, np.int64) - r0s, c.BK)
    voff0 = c.lane_voff(wave, row_stride, is_v)
    for it in range(c.n_inst // c.NW):
        voff = voff0 + (wave + c.NW * it) * c.rpi * row_stride
        mem.buffer(tensor, head_base + r0s * row_stride, rows * row_stride, voff, 16, "fetch_tile")
        mem.lds((wave + c.NW * it) * 1024 + LANES * 16, 16, c.tile_bytes, "commit_tile")


def fetch_positions(mem, src, r0s, lims, wave, BK=64):
    E = BK // FwdCfg.NW
    r0s = np.asarray(r0s, np.int64)
    if src is None:  # null source: an empty range
        rows, src = np.zeros_like(r0s), "null"
    else:
        rows = clamp_rows(np.asarray(lims, np.int64) - r0s, BK)
    mem.buffer(src, r0s * 4, rows * 4, (E * wave + (LANES & (E - 1))) * 4, 4, "fetch_positions")


# ---------------------------------------------------------------------------
# partial-attention kernel (partial_fwd.hip)

def fwd_workgroups(lq, hq, hkv):
    """Workgroups of one forward launch (8 waves: query heads of one KV group x 32-row blocks)."""
    G = hq // hkv
    g_wg = 8 if G % 8 == 0 else 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    r_wg = 8 // g_wg
    return ((lq + 32 * r_wg - 1) // (32 * r_wg)) * (hq // g_wg)


PLAN_REC = 48  # int32 per workgroup in a document call's plan
PLAN_TILE, PLAN_KB, PLAN_KE, PLAN_SLAST, PLAN_SFIRST, PLAN_FLO, PLAN_FHI, PLAN_FLAGS = 0, 1, 2, 4, 12, 20, 28, 36


def replay_forward(mem, sr, *, lq, hq, hkv, D, in_bf16, out_bf16, causal, accumulate, blocks, varlen=False,
                   n_seqs=0, multi=False, plan=None):
    """One launch of the partial-attention kernel. blocks: list of
    (k tensor, v tensor, k_pos array name, lk) — one for a single-block call.
    Tensors: 'q', 'o', 'lse', 'q_pos', 'cu' (and 'wg_plan' with `plan`, the
    int32 records of a planned document call: the kernel reads its record
    instead of searching, and clamps every addressing value from it into
    range, as modelled here, so the tiles it loads stay inside the block
    whatever the plan holds). Returns the K/V tiles loaded."""
    c = FwdCfg(in_bf16, D)
    G = hq // hkv
    g_wg = 8 if G % 8 == 0 else 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    r_wg = 8 // g_wg
    n_qtiles = (lq + 32 * r_wg - 1) // (32 * r_wg)
    n_wg = n_qtiles * (hq // g_wg)
    if n_wg <= 0:
        return 0
    check_remap(n_wg)
    planned = plan is not None and varlen and not multi
    if planned:
        # every workgroup id reads its record's tile and key range, and each
        # wave its own entries
        bid = np.arange(n_wg, dtype=np.int64)
        mem.index("wg_plan", (bid[:, None] * PLAN_REC + np.array([PLAN_TILE, PLAN_KB, PLAN_KE])).ravel(), "plan")
        for f in (PLAN_SLAST, PLAN_SFIRST, PLAN_FLO, PLAN_FHI, PLAN_FLAGS):
            mem.index("wg_plan", (bid[:, None] * PLAN_REC + f + np.arange(8)).ravel(), "plan, per wave")
        # one grid row per workgroup id, computing its record's (clamped)
        # tile: a plan that repeats a tile is replayed as it runs
        recs = np.asarray(plan, np.int64).reshape(n_wg, PLAN_REC)
    deep = False  # (two-ahead staging sets are no longer used)
    osz = 2 if out_bf16 else 4
    row_stride = hkv * D * c.esz
    li, g = LANES & 31, LANES >> 5
    qp = sr.arrays.get("q_pos")

    # grid: [workgroup, wave] (lanes on a last axis where they differ)
    L = np.arange(n_wg, dtype=np.int64)[:, None]
    if planned:
        L = np.clip(recs[:, PLAN_TILE], 0, n_wg - 1)[:, None]
    w = np.arange(8, dtype=np.int64)[None, :]
    hgrp = L // n_qtiles
    qt = n_qtiles - 1 - L % n_qtiles
    wg_r0 = qt * 32 * r_wg
    wg_r1 = np.minimum(wg_r0 + 32 * r_wg, lq)
    h = hgrp * g_wg + w % g_wg
    hk = h // G
    r0 = wg_r0 + 32 * (w // g_wg)
    r1 = np.minimum(r0 + 32, lq)
    active = r0 < lq
    wg_r0, wg_r1 = np.broadcast_to(wg_r0, r0.shape), np.broadcast_to(wg_r1, r0.shape)
    qi = np.minimum(r0[..., None] + li, lq - 1)
    row_valid = active[..., None] & (r0[..., None] + li < lq)
    wave_id = np.broadcast_to(w, r0.shape)

    if causal:
        mem.index("q_pos", qi, "q_pos[qi]")
    s_wg = s_wave = np.zeros(r0.shape, np.int64)
    if planned:
        per_lane = recs[:, PLAN_FLAGS:PLAN_FLAGS + 8] & 1
        across = per_lane.astype(bool)
        if across.any():
            sr.doc_start("cu", n_seqs, qp[qi[across]])
    elif varlen and causal:
        i_first = np.where(active, r0, wg_r1 - 1)
        i_last = np.where(active, r1 - 1, wg_r1 - 1)
        mem.index("q_pos", np.stack([wg_r0, i_first, i_last]))
        d0 = sr.wave_upper_bound("cu", n_seqs + 1, qp[wg_r0])
        d1 = sr.wave_upper_bound("cu", n_seqs + 1, qp[i_first])
        d2 = sr.wave_upper_bound("cu", n_seqs + 1, qp[i_last])
        j0, j1, j2 = np.where(d0 > 0, d0 - 1, 0), np.where(d1 > 0, d1 - 1, 0), np.where(d2 > 0, d2 - 1, 0)
        mem.index("cu", np.stack([j0, j1, j2]))
        s_wg, s_wave = sr.arrays["cu"][j0].astype(np.int64), sr.arrays["cu"][j2].astype(np.int64)
        across = d2 > d1 + 1  # a wave across three or more documents: per-lane starts
        if across.any():
            sr.doc_start("cu", n_seqs, qp[qi[across]])

    q_loaded = np.zeros(r0.shape, bool)
    seen = np.zeros(r0.shape, bool)
    exited = np.zeros(r0.shape, bool)
    tiles = 0
    for (kt, vt, kp, lk) in blocks:
        kbase = hk * D * c.esz
        alive = ~exited
        if planned:
            p_kb = np.broadcast_to(np.clip(recs[:, PLAN_KB], 0, lk)[:, None], r0.shape)
            p_ke = np.broadcast_to(np.clip(recs[:, PLAN_KE], 0, lk)[:, None], r0.shape)
            none = ~(p_ke > p_kb)
        elif causal and lk > 0:
            mem.index(kp, [0, lk - 1], "kpos[0], kpos[lk - 1]")  # (a single-block call reads them first)
            mem.index("q_pos", wg_r1 - 1)
            none = sr.arrays[kp][0] > qp[wg_r1 - 1]
            k_first, k_last = int(sr.arrays[kp][0]), int(sr.arrays[kp][lk - 1])
        else:
            none = np.full(r0.shape, causal and lk == 0)
        skip = alive & (none | (lk <= 0))
        if not multi and accumulate:
            exited |= skip
        act = alive & ~skip
        need_q = act & ~q_loaded
        for ks in range(c.NQ):
            if in_bf16:
                mem.plain("q", ((qi * hq + h[..., None]) * D + 16 * ks + 8 * g)[need_q] * 2, 16, "load_q")
            else:
                mem.plain("q", ((qi * hq + h[..., None]) * D + 2 * ks + g)[need_q] * 4, 4, "load_q")
        q_loaded |= act
        psrc = kp if causal else kt  # non-causal: the same instruction reads the key tensor

        def load_first(sel, kt0, n_avail):
            for wv in range(8):
                m = sel & (wave_id == wv)
                if not m.any():
                    continue
                t0, na, hb = kt0[m], n_avail[m], kbase[m]
                load_tile(mem, c, kt, hb, row_stride, t0 * c.BK, lk, wv, False)
                load_positions(mem, psrc, t0 * c.BK, lk, wv, c.BK)
                m1, m2 = na > 1, na > 2
                load_tile(mem, c, kt, hb[m1], row_stride, (t0[m1] + 1) * c.BK, lk, wv, False)
                load_positions(mem, psrc, (t0[m1] + 1) * c.BK, lk, wv, c.BK)
                load_tile(mem, c, vt, hb, row_stride, t0 * c.BK, lk, wv, True)
                load_tile(mem, c, kt, hb[m2], row_stride, (t0[m2] + 2) * c.BK, lk, wv, False)
                load_positions(mem, psrc, (t0[m2] + 2) * c.BK, lk, wv, c.BK)
                load_tile(mem, c, vt, hb[m1], row_stride, (t0[m1] + 1) * c.BK, lk, wv, True)

        early = not varlen or planned
        zeros = np.zeros(r0.shape, np.int64)
        if planned:
            load_first(act, p_kb // c.BK, (p_ke + c.BK - 1) // c.BK - p_kb // c.BK)
        elif early:
            load_first(act, zeros, zeros + (lk + c.BK - 1) // c.BK)
        kb, ke = zeros, zeros + lk
        if planned:
            kb, ke = p_kb.astype(np.int64), p_ke.astype(np.int64)
        elif causal and act.any():
            q_lo_i = np.where(active, r0, wg_r1 - 1)
            mem.index("q_pos", np.stack([wg_r1 - 1, q_lo_i])[:, act])
            wq_hi = qp[wg_r1 - 1].astype(np.int64)
            q_lo = qp[q_lo_i].astype(np.int64)
            ke, kb = ke.copy(), kb.copy()
            # searches whose answer the block's first or last key gives run over an empty range
            s_ke = act & ~(k_last <= wq_hi)
            ke[s_ke] = sr.wave_upper_bound(kp, lk, wq_hi[s_ke])
            sr.wave_upper_bound(kp, lk, q_lo[act & ~(k_last <= q_lo)])
            if varlen:
                s_kb = act & ~(k_first >= s_wg)
                kb[s_kb] = sr.wave_upper_bound(kp, lk, s_wg[s_kb] - 1)
                sr.wave_upper_bound(kp, lk, s_wave[act & ~(k_first >= s_wave)] - 1)
        kt_begin = kb // c.BK
        nt = np.where(ke > kb, (ke + c.BK - 1) // c.BK - kt_begin, 0)
        if not (np.all(kt_begin == kt_begin[:, :1]) and np.all(nt == nt[:, :1])):
            raise AccessError("waves of a workgroup disagree on its tile range")
        go = act & (nt > 0)
        seen |= go
        tiles += int(nt[:, 0][go[:, 0]].sum())
        if not early:
            load_first(go, kt_begin, nt)
        # ring fetches of group j = {K(j+1) and its positions, V(j)}:
        # j = 2 .. nt-1 (issued when j < nt); at d 64 (bf16) j = 2 and 3 .. nt+2, unconditionally
        for wv in range(8):
            m = go & (wave_id == wv)
            if not m.any():
                continue
            n_e, kb_e, hb_e = nt[m], kt_begin[m], kbase[m]
            if deep:
                j3, own3 = ragged_ranges(np.full(n_e.shape, 3), n_e)  # 3 .. nt+2
                js, own = np.concatenate([np.full(n_e.shape, 2), j3]), np.concatenate([np.arange(n_e.size), own3])
                klim = np.where(js + 1 < n_e[own], lk, 0)
                vlim = np.where(js < n_e[own], lk, 0)
            else:
                js, own = ragged_ranges(np.full(n_e.shape, 2), np.maximum(n_e - 2, 0))
                klim = vlim = np.full(js.shape, lk)
            j0 = (kb_e[own] + js) * c.BK
            fetch_tiles(mem, c, kt, hb_e[own], row_stride, j0 + c.BK, klim, wv, False)
            fetch_positions(mem, kp if causal else None, j0 + c.BK, klim, wv, c.BK)
            fetch_tiles(mem, c, vt, hb_e[own], row_stride, j0, vlim, wv, True)

    # epilogue (workgroups that left early, and accumulating ones that saw nothing, write nothing)
    ep = ~exited & ~(~seen & accumulate)
    lane_ep = ep[..., None] & row_valid
    lse_off = (h[..., None] * lq + r0[..., None] + li) * 4
    if accumulate:
        mem.plain("lse", lse_off[lane_ep], 4, "lse (stored)")
    if out_bf16:
        RS, CH = D * 2 + 16, D * 2 // 16
        RPP = 64 // CH
        n_rows = np.where(active, np.minimum(32, lq - r0), 0)
        prow, pchunk = LANES // CH, LANES % CH
        for ps in range(32 // RPP):
            row = ps * RPP + prow
            ok = ep[..., None] & (row < n_rows[..., None])
            off = ((r0[..., None] * hq + h[..., None]) * D + row * hq * D + pchunk * 8) * 2
            mem.plain("o", off[ok], 16, "o rows")
            mem.lds(row * RS + pchunk * 16, 16, c.tile_bytes, "o staging")
        for dt in range(c.NDT):
            for rr in range(4):
                mem.lds(li * RS + (32 * dt + 8 * rr + 4 * g) * 2, 8, c.tile_bytes, "o staging")
    else:
        for dt in range(c.NDT):
            for rr in range(4):
                dv = 32 * dt + 8 * rr + 4 * g
                mem.plain("o", (((r0[..., None] + li) * hq + h[..., None]) * D + dv)[lane_ep] * osz, 16, "o")
    mem.plain("lse", lse_off[lane_ep & (g == 0)], 4, "lse")
    return tiles


# ---------------------------------------------------------------------------
# gradient kernels (partial_bwd.hip)

def replay_delta(mem, *, lq, hq, D, o_esz, do_esz, chunk=1 << 22):
    LPP = D // 8
    n = lq * hq
    total = (n * LPP + 255) // 256 * 256
    for t0 in range(0, total, chunk):
        t = np.arange(t0, min(t0 + chunk, total), dtype=np.int64)
        pair = t // LPP
        sub = (t % 256) % LPP
        ok = pair < n
        base = pair[ok] * D + 8 * sub[ok]
        mem.plain("o", base * o_esz, 8 * o_esz, "delta: o")
        mem.plain("dout", base * do_esz, 8 * do_esz, "delta: dout")
        wr = ok & (sub == 0)
        mem.plain("delta", ((pair[wr] % hq) * lq + pair[wr] // hq) * 4, 4, "delta")


def bwd_off(row, chunk, D):
    """LDS byte offset of 16-byte chunk `chunk` of row `row` of a gradient-kernel tile."""
    if D == 128:
        swz = ((row & 3) << 2) | ((row >> 2) & 3)
    else:
        swz = (((row >> 1) & 1) << 2) | ((row >> 2) & 3)
    return row * 2 * D + ((chunk ^ swz) << 4)


def staged_store_offsets(first_rows, n_rows, heads, head, D):
    """Byte offsets of the 16-byte stores of store_rows_lds (partial_bwd.hip) for
    waves whose first rows are first_rows [..., waves], into a float32
    [n_rows][heads][D] tensor at head `head` (broadcast against first_rows);
    LDS offsets checked against the 32 x D/2-float stage."""
    dtp = D // 64
    pcols = 32 * dtp
    chk = pcols // 4
    rb = pcols * 4
    rpi = 64 // chk
    li, g = LANES & 31, LANES >> 5
    rl, cl = LANES // chk, LANES % chk
    for dt in range(dtp):
        for rr in range(4):
            c = 8 * dt + 2 * rr + g
            Mem.lds(li * rb + ((c ^ (li & (chk - 1))) << 4), 16, 32 * rb, "staged store write")
    first = np.asarray(first_rows, np.int64)[..., None]
    head = np.asarray(head, np.int64)[..., None]
    n_valid = np.minimum(32, n_rows - first)
    out = []
    for ps in range(2):
        for k in range(32 // rpi):
            row = k * rpi + rl
            Mem.lds(row * rb + ((cl ^ (row & (chk - 1))) << 4), 16, 32 * rb, "staged store read")
            ok = np.broadcast_to(row < n_valid, np.broadcast(first, head, row).shape)
            off = (((first + row) * heads + head) * D + ps * pcols + 4 * cl) * 4
            out.append(np.broadcast_to(off, ok.shape)[ok])
    return np.concatenate(out)


def _bwd_keys(mem, sr, names, *, lq, lk, hq, hkv, D, causal, varlen, n_seqs):
    """The key kernel's workgroups of one block (block tensors named in `names`)."""
    G = hq // hkv
    kchunks = D // 8
    tb = 32 * 2 * D
    li, g = LANES & 31, LANES >> 5
    NQ = D // 16
    kpa = sr.arrays.get(names["k_pos"])
    # ---- key kernel: workgroup = 128 keys of one KV head ----
    if lk > 0:
        n_tiles = (lk + 127) // 128
        n_wg = n_tiles * hkv
        check_remap(n_wg)
        U, FT = tb // 16, 256
        NU = 2 * U // FT
        q_stride = hq * D * 2
        L = np.arange(n_wg, dtype=np.int64)
        hk = L // n_tiles
        wg_j0 = (L % n_tiles) * 128
        wg_j1 = np.minimum(wg_j0 + 128, lk)
        i_lo, i_hi = np.zeros(n_wg, np.int64), np.full(n_wg, lq, np.int64)
        if causal:
            mem.index(names["k_pos"], wg_j0, "k_pos[wg_j0]")
            i_lo = sr.wave_upper_bound("q_pos", lq, kpa[wg_j0].astype(np.int64) - 1)
            if varlen:
                mem.index(names["k_pos"], wg_j1 - 1)
                i_hi = sr.wave_upper_bound("q_pos", lq, sr.doc_end("cu", n_seqs, kpa[wg_j1 - 1]) - 1)
        nqt = np.where(i_hi > i_lo, (i_hi - i_lo + 31) // 32, 0)
        n_it = G * nqt
        # the consumers fetch tiles 0, 1, 2 before the loop, then tile k+3 in phase k = 0 .. n_it
        its, own = ragged_ranges(np.zeros(n_wg), n_it + 4)
        live = its < n_it[own]
        nq = np.maximum(nqt[own], 1)
        hh = hk[own] * G + np.where(live, its // nq, 0)
        i0 = np.where(live, i_lo[own] + 32 * (its % nq), lq)
        rows = clamp_rows(lq - i0, 32)
        ct = np.arange(FT, dtype=np.int64)
        for u in range(NU):
            unit = ct + FT * u
            is_o = unit >= U
            for wv in range(4):  # consumer wave 4 + wv: threads 64wv .. 64wv+63 of ct
                lanes = slice(64 * wv, 64 * wv + 64)
                if is_o[lanes].min() != is_o[lanes].max():
                    raise AccessError("a fetch unit is not wave-uniform in its tensor")
            lu = np.where(is_o, unit - U, unit)
            voff = (lu // kchunks) * q_stride + (lu % kchunks) * 16
            for name, sel in (("q", ~is_o), ("dout", is_o)):
                if sel.any():
                    mem.buffer(name, hh * D * 2 + i0 * q_stride, rows * q_stride, voff[sel], 16, "dkv fetch")
            mem.lds(bwd_off(lu // kchunks, lu % kchunks, D), 16, tb, "dkv commit")
        lo = hh * lq + i0
        for wave in range(4, 8):
            mine = rows if wave == 4 else np.zeros_like(rows)
            mem.buffer("lse", lo * 4, mine * 4, LANES * 4, 4, "dkv lse")
            mem.buffer("delta", lo * 4, mine * 4, LANES * 4, 4, "dkv delta")
            mem.buffer("q_pos" if causal else "null", i0 * 4 if causal else 0 * i0, mine * 4 if causal else 0 * mine,
                       LANES * 4, 4, "dkv q_pos")
        # each wave's 32 keys: producers read K, V rows and positions; consumers store dK, dV
        kw = np.arange(4, dtype=np.int64)[None, :]
        j0 = wg_j0[:, None] + 32 * kw
        kj = np.minimum(j0[..., None] + li, lk - 1)
        key_valid = j0[..., None] + li < lk
        hk3 = hk[:, None, None]
        for ks in range(NQ):
            off = ((kj * hkv + hk3) * D + 8 * g + 16 * ks) * 2
            mem.plain(names["k"], off, 16, "dkv kreg")
            mem.plain(names["v"], off, 16, "dkv vreg")
        if causal:
            mem.index(names["k_pos"], kj, "k_pos[kj]")
            mem.index(names["k_pos"], np.minimum(j0 + 31, lk - 1), "dkv wave's last key")
            if varlen:
                sr.doc_end("cu", n_seqs, kpa[kj])
        # dK, dV leave through LDS (store_rows_lds): rows j0 + row, whole lines
        off = staged_store_offsets(j0, lk, hkv, hk[:, None], D)
        mem.plain(names["dk"], off, 16, "dk")
        mem.plain(names["dv"], off, 16, "dv")



def _bwd_query(mem, sr, blocks, *, lq, hq, hkv, D, causal, varlen, n_seqs, acc_dq, multi, order=None):
    """The query kernel over `blocks` (a list of (names, lk)): a single-block
    call (multi False, one block) or a multi-block call, whose workgroups walk
    the blocks in order and store dQ once. `order`: a planned call's plan (the
    logical tile of each workgroup, read with plain loads and clamped into
    range), or None for the default order."""
    G = hq // hkv
    kchunks = D // 8
    tb = 32 * 2 * D
    li, g = LANES & 31, LANES >> 5
    NQ = D // 16
    qp = sr.arrays.get("q_pos")
    n_tiles = (lq + 127) // 128
    n_wg = n_tiles * hq
    check_remap(n_wg)
    kv_stride = hkv * D * 2
    if order is None:
        L = np.arange(n_wg, dtype=np.int64)   # (the default order is a permutation: every tile once)
    else:
        order = np.asarray(order, np.int64)
        if order.shape != (n_wg,):
            raise AccessError("a plan of %d entries for %d workgroups" % (len(order), n_wg))
        mem.index("dq_plan", np.arange(n_wg), "dq plan")
        L = np.clip(order, 0, n_wg - 1)
    h = L // n_tiles
    hk = h // G
    wg_r0 = (n_tiles - 1 - L % n_tiles) * 128
    wg_r1 = np.minimum(wg_r0 + 128, lq)
    r0 = wg_r0[:, None] + 32 * np.arange(4, dtype=np.int64)[None, :]
    qi = np.minimum(r0[..., None] + li, lq - 1)
    row_valid = r0[..., None] + li < lq
    h3 = h[:, None, None]
    for ks in range(NQ):
        off = ((qi * hq + h3) * D + 8 * g + 16 * ks) * 2
        mem.plain("q", off, 16, "dq qreg")
        mem.plain("dout", off, 16, "dq dreg")
    mem.index("lse", h3 * lq + qi, "dq lse")
    mem.index("delta", (h3 * lq + qi)[row_valid], "dq delta")
    if causal:
        mem.index("q_pos", qi, "dq q_pos")
        mem.index("q_pos", np.minimum(r0, lq - 1), "dq wave's first row")
        if varlen:
            sr.doc_start("cu", n_seqs, qp[qi])
    seen = np.zeros(n_wg, bool)
    for names, lk in blocks:
        kpn = names["k_pos"]
        kpa = sr.arrays.get(kpn)
        if multi and lk == 0:
            continue  # the block is skipped before any read of it
        kb, ke = np.zeros(n_wg, np.int64), np.full(n_wg, lk, np.int64)
        if causal:
            mem.index("q_pos", np.stack([wg_r1 - 1, wg_r0]))
            ke = sr.wave_upper_bound(kpn, lk, qp[wg_r1 - 1])
            if varlen:
                kb = sr.wave_upper_bound(kpn, lk, sr.doc_start("cu", n_seqs, qp[wg_r0]) - 1)
        nt = np.where(ke > kb, (ke - kb + 31) // 32, 0)
        if (multi or acc_dq) and lk > 0 and causal:
            mem.index(kpn, [0], "k_pos[0]")
        seen |= nt > 0
        ts, own = ragged_ranges(np.zeros(n_wg), nt)  # fetch(0), then fetch(t+1) for t + 1 < nt
        j0 = kb[own] + 32 * ts
        rows = clamp_rows(lk - j0, 32)
        tid = np.arange(256, dtype=np.int64)
        for u in range(D // 64):
            unit = tid + 256 * u
            voff = (unit // kchunks) * kv_stride + (unit % kchunks) * 16
            mem.buffer(names["k"], hk[own] * D * 2 + j0 * kv_stride, rows * kv_stride, voff, 16, "dq fetch k")
            mem.buffer(names["v"], hk[own] * D * 2 + j0 * kv_stride, rows * kv_stride, voff, 16, "dq fetch v")
            mem.lds(bwd_off(unit // kchunks, unit % kchunks, D), 16, tb, "dq commit")
        if causal and ts.size:
            idx = j0[:, None] + np.arange(32)
            mem.index(kpn, idx[idx < lk], "dq k_pos")
    writes = ~(~seen & bool(acc_dq))  # accumulating workgroups that see nothing leave dQ alone
    mem.plain("dq", staged_store_offsets(r0[writes], lq, hq, h[writes][:, None], D), 16, "dq")


BWD_NAMES = {"k": "k", "v": "v", "k_pos": "k_pos", "dk": "dk", "dv": "dv"}


def replay_backward(mem, sr, *, lq, lk, hq, hkv, D, causal, varlen=False, n_seqs=0, acc_dq=False, acc_dkv=False,
                    dq_order=None):
    """One cpattn_partial_bwd call (cpattn_varlen_partial_bwd_planned with
    `dq_order`, its plan, in tensor 'dq_plan'): the key kernel, then the query
    kernel. Tensors: 'q', 'dout', 'k', 'v', 'lse', 'delta', 'q_pos', 'k_pos',
    'cu', 'dq', 'dk', 'dv'."""
    if lk > 0:
        _bwd_keys(mem, sr, BWD_NAMES, lq=lq, lk=lk, hq=hq, hkv=hkv, D=D, causal=causal, varlen=varlen,
                  n_seqs=n_seqs)
    if lq > 0:
        _bwd_query(mem, sr, [(BWD_NAMES, lk)], lq=lq, hq=hq, hkv=hkv, D=D, causal=causal, varlen=varlen,
                   n_seqs=n_seqs, acc_dq=acc_dq, multi=False, order=dq_order)


def bwd_block_names(b):
    return {"k": "k%d" % b, "v": "v%d" % b, "k_pos": "kp%d" % b, "dk": "dk%d" % b, "dv": "dv%d" % b}


def replay_backward_multi(mem, sr, *, lq, lks, hq, hkv, D, causal, varlen=False, n_seqs=0, acc_dq=False):
    """One cpattn_partial_bwd_multi call over blocks b = 0 .. len(lks)-1 (block
    b's tensors 'k<b>', 'v<b>', 'kp<b>', 'dk<b>', 'dv<b>'; the rest as in
    replay_backward): the key kernel's grid over every block's workgroups,
    then the query kernel walking the blocks."""
    n = len(lks)
    wg_end = np.cumsum([(lk + 127) // 128 * hkv for lk in lks]).astype(np.int64)
    total = int(wg_end[-1])
    if total >= 1 << 31:
        raise AccessError("key-kernel grid too large")
    # each workgroup's block: the first b (b + 1 < n) with bid < wg_end[b]
    bid = np.arange(total, dtype=np.int64)
    blk = np.zeros(total, np.int64)
    for b in range(n - 1):
        blk += bid >= wg_end[b]
    local = bid - np.where(blk > 0, wg_end[np.maximum(blk - 1, 0)], 0)
    for b in range(n):
        n_wg = (lks[b] + 127) // 128 * hkv
        mine = np.sort(local[blk == b])
        if not np.array_equal(mine, np.arange(n_wg)):
            raise AccessError("block %d's workgroups are not exactly 0 .. %d" % (b, n_wg - 1))
        if lks[b] > 0:
            _bwd_keys(mem, sr, bwd_block_names(b), lq=lq, lk=lks[b], hq=hq, hkv=hkv, D=D, causal=causal,
                      varlen=varlen, n_seqs=n_seqs)
    if lq > 0:
        _bwd_query(mem, sr, [(bwd_block_names(b), lks[b]) for b in range(n)], lq=lq, hq=hq, hkv=hkv, D=D,
                   causal=causal, varlen=varlen, n_seqs=n_seqs, acc_dq=acc_dq, multi=True)


def f32_off(row, chunk):
    """LDS byte offset of 16-byte chunk `chunk` of row `row` of a float32 gradient-kernel tile (without the row base)."""
    return (chunk ^ (row & 15)) << 4


def replay_backward_f32(mem, sr, *, lq, lk, hq, hkv, D, causal, varlen=False, n_seqs=0):
    """One cpattn_partial_bwd call with float32 inputs (partial_bwd_f32.hip):
    the key kernel, then the query kernel. Tensors as in replay_backward."""
    G = hq // hkv
    row_bytes = 4 * D
    kchunks = D // 4
    tb = 32 * row_bytes
    units = tb // 16 // 256
    li, g = LANES & 31, LANES >> 5
    NK, NDT = D // 2, D // 32
    qp, kpa = sr.arrays.get("q_pos"), sr.arrays.get("k_pos")
    tid = np.arange(256, dtype=np.int64)
    for u in range(units):
        unit = tid + 256 * u
        mem.lds((unit // kchunks) * row_bytes + f32_off(unit // kchunks, unit % kchunks), 16, tb, "f32 commit")
    for col in range(D):
        mem.lds(np.arange(32) * row_bytes + f32_off(np.arange(32), col >> 2) + ((col & 3) << 2), 4, tb, "f32 at")
    # ---- key kernel: workgroup = 128 keys (32 per wave) of one KV head ----
    if lk > 0:
        n_tiles = (lk + 127) // 128
        n_wg = n_tiles * hkv
        check_remap(n_wg)
        q_stride = hq * D * 4
        L = np.arange(n_wg, dtype=np.int64)
        hk = L // n_tiles
        wg_j0 = (L % n_tiles) * 128
        wg_j1 = np.minimum(wg_j0 + 128, lk)
        i_lo, i_hi = np.zeros(n_wg, np.int64), np.full(n_wg, lq, np.int64)
        if causal:
            mem.index("k_pos", wg_j0, "k_pos[wg_j0]")
            i_lo = sr.wave_upper_bound("q_pos", lq, kpa[wg_j0].astype(np.int64) - 1)
            if varlen:
                mem.index("k_pos", wg_j1 - 1)
                i_hi = sr.wave_upper_bound("q_pos", lq, sr.doc_end("cu", n_seqs, kpa[wg_j1 - 1]) - 1)
        nqt = np.where(i_hi > i_lo, (i_hi - i_lo + 31) // 32, 0)
        n_it = G * nqt
        its, own = ragged_ranges(np.zeros(n_wg), n_it)  # fetch(0), then fetch(it + 1) for it + 1 < n_it
        nq = np.maximum(nqt[own], 1)
        hh = hk[own] * G + its // nq
        i0 = i_lo[own] + 32 * (its % nq)
        rows = clamp_rows(lq - i0, 32)
        for u in range(units):
            unit = tid + 256 * u
            voff = (unit // kchunks) * q_stride + (unit % kchunks) * 16
            for name in ("q", "dout"):
                mem.buffer(name, hh * D * 4 + i0 * q_stride, rows * q_stride, voff, 16, "dkv f32 fetch")
        r = i0[:, None] + np.arange(32)
        ok = r < lq
        mem.index("lse", (hh[:, None] * lq + r)[ok], "dkv f32 lse")
        mem.index("delta", (hh[:, None] * lq + r)[ok], "dkv f32 delta")
        if causal:
            mem.index("q_pos", r[ok], "dkv f32 q_pos")
        j0 = wg_j0[:, None] + 32 * np.arange(4, dtype=np.int64)[None, :]
        kj = np.minimum(j0[..., None] + li, lk - 1)
        key_valid = j0[..., None] + li < lk
        hk3 = hk[:, None, None]
        for ks in range(NK):
            off = ((kj * hkv + hk3) * D + 2 * ks + g) * 4
            mem.plain("k", off, 4, "dkv f32 kreg")
            mem.plain("v", off, 4, "dkv f32 vreg")
        if causal:
            mem.index("k_pos", kj, "k_pos[kj]")
            if varlen:
                sr.doc_end("cu", n_seqs, kpa[kj])
        for dt in range(NDT):
            for rr in range(4):
                off = (((kj * hkv + hk3) * D + 32 * dt + 8 * rr + 4 * g) * 4)[key_valid]
                mem.plain("dk", off, 16, "dk")
                mem.plain("dv", off, 16, "dv")
    # ---- query kernel: workgroup = 128 rows (32 per wave) of one query head ----
    if lq > 0:
        n_tiles = (lq + 127) // 128
        n_wg = n_tiles * hq
        check_remap(n_wg)
        kv_stride = hkv * D * 4
        L = np.arange(n_wg, dtype=np.int64)
        h = L // n_tiles
        hk = h // G
        wg_r0 = (n_tiles - 1 - L % n_tiles) * 128
        wg_r1 = np.minimum(wg_r0 + 128, lq)
        r0 = wg_r0[:, None] + 32 * np.arange(4, dtype=np.int64)[None, :]
        qi = np.minimum(r0[..., None] + li, lq - 1)
        row_valid = r0[..., None] + li < lq
        h3 = h[:, None, None]
        for ks in range(NK):
            off = ((qi * hq + h3) * D + 2 * ks + g) * 4
            mem.plain("q", off, 4, "dq f32 qreg")
            mem.plain("dout", off, 4, "dq f32 dreg")
        mem.index("lse", h3 * lq + qi, "dq lse")
        mem.index("delta", (h3 * lq + qi)[row_valid], "dq delta")
        if causal:
            mem.index("q_pos", qi, "dq q_pos")
            mem.index("q_pos", np.minimum(r0, lq - 1), "dq wave's first row")
            if varlen:
                sr.doc_start("cu", n_seqs, qp[qi])
        for dt in range(NDT):
            for rr in range(4):
                off = (((qi * hq + h3) * D + 32 * dt + 8 * rr + 4 * g) * 4)[row_valid]
                mem.plain("dq", off, 16, "dq")
        kb, ke = np.zeros(n_wg, np.int64), np.full(n_wg, lk, np.int64)
        if causal:
            mem.index("q_pos", np.stack([wg_r1 - 1, wg_r0]))
            ke = sr.wave_upper_bound("k_pos", lk, qp[wg_r1 - 1])
            if varlen:
                kb = sr.wave_upper_bound("k_pos", lk, sr.doc_start("cu", n_seqs, qp[wg_r0]) - 1)
        nt = np.where(ke > kb, (ke - kb + 31) // 32, 0)
        ts, own = ragged_ranges(np.zeros(n_wg), nt)
        j0 = kb[own] + 32 * ts
        rows = clamp_rows(lk - j0, 32)
        for u in range(units):
            unit = tid + 256 * u
            voff = (unit // kchunks) * kv_stride + (unit % kchunks) * 16
            mem.buffer("k", hk[own] * D * 4 + j0 * kv_stride, rows * kv_stride, voff, 16, "dq f32 fetch k")
            mem.buffer("v", hk[own] * D * 4 + j0 * kv_stride, rows * kv_stride, voff, 16, "dq f32 fetch v")
        if causal and ts.size:
            idx = j0[:, None] + np.arange(32)
            mem.index("k_pos", idx[idx < lk], "dq k_pos")
