"""Python handle over the C++ host block manager (``pa_bm_*`` in include/pa.h)."""
from __future__ import annotations

import ctypes as C

import numpy as np

from ._lib import BmStats, check, lib


def _ptr(a: np.ndarray, ctype):
    """Address of a contiguous array of `ctype` elements (the C arguments are
    c_void_p; the element type is checked here)."""
    assert a.dtype.itemsize == C.sizeof(ctype) and a.flags.c_contiguous
    return a.ctypes.data


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
