"""Python handle over the C++ host block manager (``pa_bm_*`` in include/pa.h)."""
from __future__ import annotations

import ctypes as C

import numpy as np

from ._lib import BmStats, check, lib


def _ptr(a: np.ndarray, ctype):
    """Address of a contiguous array of `ctype` elements (the C arguments are
    c_void_p; the element type is checked here).  Read from the array
    interface: `ndarray.ctypes` builds a helper object on every access."""
    assert a.dtype.itemsize == C.sizeof(ctype) and a.flags.c_contiguous
    return a.__array_interface__["data"][0]


class BlockManager:
    """Free pool, block tables, reference counts and copy-on-write planning."""

    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        self._h = C.c_void_p()
        fo = None
        if free_order is not None:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if fo.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
        check(lib().pa_bm_create(num_blocks, block_size,
                                 _ptr(fo, C.c_int32) if fo is not None else None,
                                 C.byref(self._h)), "pa_bm_create")
        self.num_blocks, self.block_size = num_blocks, block_size
        self._step_fn = None
        self._step_out = (C.c_int32(0), C.c_int32(0))
        self._step_ref = (C.byref(self._step_out[0]), C.byref(self._step_out[1]))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and lib is not None:
            lib().pa_bm_destroy(h)
            self._h = None

    def add_seq(self, seq_id: int, num_tokens: int) -> np.ndarray:
        slots = np.empty(max(num_tokens, 0), dtype=np.int64)
        check(lib().pa_bm_add_seq(self._h, seq_id, num_tokens, _ptr(slots, C.c_int64)),
              "pa_bm_add_seq")
        return slots

    def fork(self, parent: int, child: int):
        check(lib().pa_bm_fork(self._h, parent, child), "pa_bm_fork")

    def extend(self, seq_id: int, num_tokens: int):
        slots = np.empty(max(num_tokens, 0), dtype=np.int64)
        pairs = np.empty((1, 2), dtype=np.int32)
        n = C.c_int32(0)
        check(lib().pa_bm_extend(self._h, seq_id, num_tokens, _ptr(slots, C.c_int64),
                                 _ptr(pairs, C.c_int32), C.byref(n)), "pa_bm_extend")
        return slots, pairs[:n.value].copy()

    def append_slots(self, seq_ids):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        slots = np.empty(len(ids), dtype=np.int64)
        pairs = np.empty((max(len(ids), 1), 2), dtype=np.int32)
        n = C.c_int32(0)
        check(lib().pa_bm_append_slots(self._h, _ptr(ids, C.c_int64), len(ids),
                                       _ptr(slots, C.c_int64), _ptr(pairs, C.c_int32),
                                       C.byref(n)), "pa_bm_append_slots")
        return slots, pairs[:n.value].copy()

    def step(self, seq_ids, capacity: int = 0):
        """One decode step's host work (pa_bm_step): reserve one position per
        sequence and export the tables after it.  capacity: table row length
        to try first (grown and retried when a table is longer).  Returns
        (slots, cow pairs [n][2], tables [n][blocks needed], lens).

        The outputs are views of one fresh int32 block, laid out
        slots (int64) | lens | pairs | tables, so a call reads one address
        from numpy (each read costs about a microsecond) and the arrays stay
        valid after later calls."""
        ids = seq_ids if (isinstance(seq_ids, np.ndarray) and seq_ids.dtype == np.int64
                          and seq_ids.flags.c_contiguous) else \
            np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        cap = max(int(capacity), 1)
        f = self._step_fn
        if f is None:
            f = self._step_fn = lib().pa_bm_step
        ncow, need = self._step_out
        pi = _ptr(ids, C.c_int64)
        npair = max(n, 1)
        o_lens, o_pairs = 2 * n, 3 * n                    # int32 offsets
        o_tab = o_pairs + 2 * npair
        while True:
            blk = np.empty(o_tab + n * cap, dtype=np.int32)
            a = blk.__array_interface__["data"][0]     # 16-byte aligned: slots first
            st = f(self._h, pi, n, cap, a, a + 4 * o_pairs, self._step_ref[0], a + 4 * o_tab,
                   a + 4 * o_lens, self._step_ref[1])
            if st != 0 and need.value > cap:
                cap = need.value                    # nothing changed: retry with room
                continue
            check(st, "pa_bm_step")
            break
        nb = max(need.value, 1)
        tables = blk[o_tab:].reshape(n, cap)
        if nb != cap:
            tables = np.ascontiguousarray(tables[:, :nb])
        slots = blk[:o_lens].view(np.int64)
        lens = blk[o_lens:o_pairs]
        pairs = blk[o_pairs:o_tab].reshape(npair, 2)[:ncow.value]
        return slots, pairs, tables, lens

    def free_seq(self, seq_id: int):
        check(lib().pa_bm_free_seq(self._h, seq_id), "pa_bm_free_seq")

    def reorder(self, old_ids, new_ids, parents):
        """Beam step: new_ids[j] continues old_ids[parents[j]] (fork unless the
        same id); old ids not among new_ids are released."""
        o = np.ascontiguousarray(old_ids, dtype=np.int64)
        n = np.ascontiguousarray(new_ids, dtype=np.int64)
        p = np.ascontiguousarray(parents, dtype=np.int32)
        if p.shape != n.shape:
            raise ValueError("one parent per new id")
        check(lib().pa_bm_reorder(self._h, _ptr(o, C.c_int64), len(o), _ptr(n, C.c_int64),
                                  _ptr(p, C.c_int32), len(n)), "pa_bm_reorder")

    def release_before(self, seq_id: int, first_pos: int) -> int:
        """Sliding window: drop the blocks wholly before first_pos (entries -> -1)."""
        n = C.c_int32(0)
        check(lib().pa_bm_release_before(self._h, seq_id, int(first_pos), C.byref(n)),
              "pa_bm_release_before")
        return int(n.value)

    def block_tables(self, seq_ids, max_blocks: int):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((len(ids), max_blocks), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        check(lib().pa_bm_block_tables(self._h, _ptr(ids, C.c_int64), len(ids), max_blocks,
                                       _ptr(tables, C.c_int32), _ptr(lens, C.c_int32)),
              "pa_bm_block_tables")
        return tables, lens

    def seq_len(self, seq_id: int) -> int:
        v = C.c_int32()
        check(lib().pa_bm_seq_len(self._h, seq_id, C.byref(v)), "pa_bm_seq_len")
        return v.value

    def refcount(self, block: int) -> int:
        v = C.c_int32()
        check(lib().pa_bm_refcount(self._h, block, C.byref(v)), "pa_bm_refcount")
        return v.value

    def stats(self) -> dict:
        s = BmStats()
        check(lib().pa_bm_stats(self._h, C.byref(s)), "pa_bm_stats")
        return {f: getattr(s, f) for f, _ in BmStats._fields_ if f != "reserved"}
