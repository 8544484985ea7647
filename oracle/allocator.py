"""Reference model of the KV block manager (host side).

What the pages fix:

* KV memory is a pool of same-size physical blocks (e.g. 16 tokens); each
  request sees its tokens as consecutive logical blocks and a block table maps
  logical to physical blocks, with no need for contiguity (page 1, section
  「PagedAttentionの解決策」; page 3, section 「用語解説」, entries on logical /
  physical blocks and the block table).
* Generated tokens fill the last block; one new block is taken each time a
  block's 16 slots are used up (page 2, section 「OSの知恵をGPUへ…」, first bullet;
  page 3, section 「KV キャッシュマネージャ」).
* A finished request hands its blocks back to the pool (page 3, section
  「KV キャッシュマネージャ」).
* Forked sequences (parallel sampling, beam search) share blocks by reference
  count without copying; a shared block is duplicated only when a write must
  land in it (page 2, third bullet of the same section; page 3, sections
  「用語解説」 (Copy-on-Write) and 「並列サンプリングやビームサーチでの共有」).

Readings taken where the pages are silent (the C++ block manager makes the
same choices so tables compare bit for bit):

* free list is a LIFO stack; a fresh pool hands blocks out in ``free_order``;
* a released block is pushed when its count reaches zero, in table order;
* the writer copies when the target block's count is above one, and the last
  remaining holder writes in place;
* batched reservations are all-or-nothing: if the batch needs more blocks
  than are free nothing changes;
* slot = physical_block * block_size + position % block_size.

Beam search and parallel sampling (page 3, section
「並列サンプリングやビームサーチでの共有」): ``reorder`` continues each new
sequence from a parent of the previous step by fork, then frees the dropped
ones; the next write into a shared last block copies it.

Sliding window (page 1, jisaku.com glossary, section
「他のKVキャッシュ最適化との組み合わせ」: with a sliding window, blocks that
have left the window can be released to save memory on long contexts):
``release_before(sid, first_pos)`` drops the sequence's blocks whose every
slot lies before ``first_pos``.  Reading: their table entries become -1, so
position p still maps to entry p // block_size; a dropped block is pushed on
the free list when its count reaches zero, in table order, like ``free_seq``.
"""
from __future__ import annotations

import numpy as np

OK, INVALID_ARG, UNSUPPORTED, OUT_OF_BLOCKS, UNKNOWN_SEQ, SEQ_EXISTS = 0, 1, 2, 3, 4, 5


class AllocError(Exception):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


class AllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError(INVALID_ARG, "num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError(INVALID_ARG, "free_order must be a permutation of [0, N)")
        self.N = num_blocks
        self.bs = block_size
        self.free = list(reversed(order))       # pop() yields free_order[0] first
        self.ref = np.zeros(num_blocks, dtype=np.int64)
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}

    # -- helpers -----------------------------------------------------------
    def _seq(self, sid):
        if sid not in self.tables:
            raise AllocError(UNKNOWN_SEQ, f"unknown sequence {sid}")
        return self.tables[sid]

    def _pop(self):
        b = self.free.pop()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _needs(self, sid, n, ref_delta):
        """Blocks needed to write positions [len, len+n) of sid (CoW included)."""
        L, table = self.lens[sid], self.tables[sid]
        need = 0
        if n == 0:
            return 0
        if L % self.bs != 0:
            tail = table[L // self.bs]
            if self.ref[tail] + ref_delta.get(tail, 0) > 1:
                need += 1
                ref_delta[tail] = ref_delta.get(tail, 0) - 1
        # positions p in [L, L+n) with p % bs == 0 start a new block
        first = -(-L // self.bs) * self.bs
        if first < L + n:
            need += (L + n - 1 - first) // self.bs + 1
        return need

    def _write(self, sid, n):
        """Reserve positions [len, len+n) of sid; returns (slots, cow_pairs)."""
        L, table = self.lens[sid], self.tables[sid]
        slots, cows = [], []
        for p in range(L, L + n):
            if p % self.bs == 0:
                table.append(self._pop())
            else:
                blk = table[p // self.bs]
                if self.ref[blk] > 1:
                    new = self._pop()
                    self.ref[blk] -= 1
                    cows.append((blk, new))
                    table[p // self.bs] = new
            slots.append(table[p // self.bs] * self.bs + p % self.bs)
        self.lens[sid] = L + n
        return slots, cows

    # -- API ---------------------------------------------------------------
    def add_seq(self, sid: int, n: int):
        if sid in self.tables:
            raise AllocError(SEQ_EXISTS, f"sequence {sid} exists")
        if n < 0:
            raise AllocError(INVALID_ARG, "negative token count")
        need = -(-n // self.bs)
        if need > len(self.free):
            raise AllocError(OUT_OF_BLOCKS, "out of blocks")
        self.tables[sid], self.lens[sid] = [], 0
        slots, cows = self._write(sid, n)
        assert not cows
        return np.array(slots, dtype=np.int64)

    def fork(self, parent: int, child: int):
        table = self._seq(parent)
        if child in self.tables:
            raise AllocError(SEQ_EXISTS, f"sequence {child} exists")
        for b in table:
            if b >= 0:
                self.ref[b] += 1
        self.tables[child] = list(table)
        self.lens[child] = self.lens[parent]

    def extend(self, sid: int, n: int):
        self._seq(sid)
        if n < 0:
            raise AllocError(INVALID_ARG, "negative token count")
        if self._needs(sid, n, {}) > len(self.free):
            raise AllocError(OUT_OF_BLOCKS, "out of blocks")
        slots, cows = self._write(sid, n)
        return np.array(slots, dtype=np.int64), np.array(cows, dtype=np.int32).reshape(-1, 2)

    def append_slots(self, sids):
        sids = [int(s) for s in sids]
        for s in sids:
            self._seq(s)
        if len(set(sids)) != len(sids):
            raise AllocError(INVALID_ARG, "duplicate sequence in batch")
        delta, need = {}, 0
        for s in sids:
            need += self._needs(s, 1, delta)
        if need > len(self.free):
            raise AllocError(OUT_OF_BLOCKS, "out of blocks")
        slots, cows = [], []
        for s in sids:
            sl, cw = self._write(s, 1)
            slots += sl
            cows += cw
        return np.array(slots, dtype=np.int64), np.array(cows, dtype=np.int32).reshape(-1, 2)

    def free_seq(self, sid: int):
        table = self._seq(sid)
        for b in table:
            if b < 0:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[sid]
        del self.lens[sid]

    def reorder(self, old_ids, new_ids, parents):
        """Beam search / parallel sampling step: sequence new_ids[j] continues
        old_ids[parents[j]].  A new id equal to its parent's id keeps that
        sequence; any other new id is a fork of the parent (shared blocks,
        no copy); then every old id that is not among new_ids is freed.
        Forks come before frees, so a block shared by a dropped parent and
        its children is never released.  All-or-nothing: ids are checked
        first (unknown old id, repeated old or new id, parent index out of
        range, new id already live and not its own parent)."""
        old_ids = [int(x) for x in old_ids]
        new_ids = [int(x) for x in new_ids]
        parents = [int(p) for p in parents]
        if len(parents) != len(new_ids):
            raise AllocError(INVALID_ARG, "one parent per new id")
        if len(set(old_ids)) != len(old_ids) or len(set(new_ids)) != len(new_ids):
            raise AllocError(INVALID_ARG, "repeated id")
        for o in old_ids:
            self._seq(o)
        for n, p in zip(new_ids, parents):
            if not 0 <= p < len(old_ids):
                raise AllocError(INVALID_ARG, "parent index out of range")
            if n != old_ids[p] and n in self.tables:
                raise AllocError(SEQ_EXISTS, f"sequence {n} exists")
        for n, p in zip(new_ids, parents):
            if n != old_ids[p]:
                self.fork(old_ids[p], n)
        keep = set(new_ids)
        for o in old_ids:
            if o not in keep:
                self.free_seq(o)

    def release_before(self, sid: int, first_pos: int) -> int:
        """Drops the blocks of sid whose 16 slots all lie before first_pos
        (clamped to the length); returns the number of entries dropped."""
        table = self._seq(sid)
        if first_pos < 0:
            raise AllocError(INVALID_ARG, "negative position")
        f = min(int(first_pos), self.lens[sid])
        n = 0
        for k in range(f // self.bs):            # block k covers [k*bs, (k+1)*bs)
            b = table[k]
            if b < 0:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
            table[k] = -1
            n += 1
        return n

    def seq_len(self, sid: int) -> int:
        self._seq(sid)
        return self.lens[sid]

    def block_tables(self, sids, max_blocks: int):
        out = np.full((len(sids), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(sids), dtype=np.int32)
        for i, s in enumerate(sids):
            t = self._seq(int(s))
            if len(t) > max_blocks:
                raise AllocError(INVALID_ARG, "table longer than max_blocks")
            out[i, :len(t)] = t
            lens[i] = self.lens[int(s)]
        return out, lens

    def stats(self):
        used = int((self.ref > 0).sum())
        return {
            "num_blocks": self.N,
            "free_blocks": len(self.free),
            "used_blocks": used,
            "shared_blocks": int((self.ref > 1).sum()),
            "tokens": int(sum(self.lens.values())),
            "slack_slots": int(sum(len(t) * self.bs - self.lens[s]
                                   for s, t in self.tables.items())),
        }

    def check_invariants(self):
        """Counts equal table references; free and referenced blocks partition the pool."""
        cnt = np.zeros(self.N, dtype=np.int64)
        for t in self.tables.values():
            for b in t:
                if b >= 0:
                    cnt[b] += 1
        assert np.array_equal(cnt, self.ref)
        free = set(self.free)
        assert len(free) == len(self.free)
        assert all(self.ref[b] == 0 for b in free)
        assert len(free) + int((self.ref > 0).sum()) == self.N
