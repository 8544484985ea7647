"""Pins for the sliding-window pieces of the oracle: the window release of
the allocator model (hand-worked tables and free list, fork counts,
invariants) and windowed decode (brute force over the last W token rows,
W >= L reduces to full attention, W = 1 returns the last V row exactly,
reuse of released blocks changes nothing)."""
import numpy as np
import pytest

from oracle import AllocatorModel, bits_of, decode_ref, dense_ref, run_case, to_f64
from oracle.allocator import AllocError
from workloads.configs import custom_case, small_case, windowed


def test_release_before_hand_example():
    am = AllocatorModel(10, 16, free_order=[3, 7, 1, 5, 0, 2, 4, 6, 8, 9])
    am.add_seq(1, 100)                       # 7 blocks: 3 7 1 5 0 2 4 (last holds 4 tokens)
    assert am.tables[1] == [3, 7, 1, 5, 0, 2, 4]
    # positions 0..39 leave the window: blocks 0 (0..15) and 1 (16..31) are
    # wholly before 40, block 2 (32..47) is not
    assert am.release_before(1, 40) == 2
    assert am.tables[1] == [-1, -1, 1, 5, 0, 2, 4]
    assert am.free == [9, 8, 6, 3, 7]        # pushed in table order; pop() takes 7 first
    assert am.seq_len(1) == 100
    # the next write still lands in the last block, then a new block at 112
    slots, cows = am.extend(1, 13)
    assert slots[0] == 4 * 16 + 4 and slots[-1] == 7 * 16 + 0 and len(cows) == 0
    assert am.tables[1][-1] == 7
    # releasing again is a no-op for dropped entries; a clamp at the length
    assert am.release_before(1, 40) == 0
    # clamped to the length 113: blocks 2..6 go (block 7 holds position 112)
    assert am.release_before(1, 10 ** 6) == 5
    assert am.tables[1] == [-1] * 7 + [7]
    am.check_invariants()


def test_release_clamps_to_full_blocks_below_the_length():
    am = AllocatorModel(8, 16)
    am.add_seq(5, 40)                        # blocks 0, 1 full, block 2 holds 8 tokens
    assert am.release_before(5, 1000) == 2   # clamp to 40: only blocks wholly below 40
    assert am.tables[5] == [-1, -1, 2]
    with pytest.raises(AllocError):
        am.release_before(5, -1)
    am.check_invariants()


def test_release_with_forks_keeps_shared_blocks():
    am = AllocatorModel(8, 16)
    am.add_seq(1, 48)
    am.fork(1, 2)
    assert am.release_before(2, 32) == 2     # child drops its references only
    assert am.tables[1] == [0, 1, 2] and am.tables[2] == [-1, -1, 2]
    assert list(am.ref[:3]) == [1, 1, 2] and len(am.free) == 5
    assert am.release_before(1, 16) == 1     # last holder of block 0: back to the pool
    assert am.free[-1] == 0
    am.fork(2, 3)                            # a fork shares only live blocks
    assert am.tables[3] == [-1, -1, 2] and am.ref[2] == 3
    am.free_seq(2)
    am.free_seq(3)
    am.free_seq(1)
    assert len(am.free) == 8
    am.check_invariants()


def test_random_ops_with_releases_keep_invariants():
    rng = np.random.default_rng(7)
    am = AllocatorModel(64, 16, free_order=rng.permutation(64))
    live = []
    for step in range(400):
        op = rng.integers(5)
        try:
            if op == 0 or not live:
                sid = step
                am.add_seq(sid, int(rng.integers(0, 60)))
                live.append(sid)
            elif op == 1:
                s = live[rng.integers(len(live))]
                am.release_before(s, int(rng.integers(0, am.seq_len(s) + 20)))
            elif op == 2:
                s = live[rng.integers(len(live))]
                am.fork(s, 10_000 + step)
                live.append(10_000 + step)
            elif op == 3:
                s = live[rng.integers(len(live))]
                am.extend(s, int(rng.integers(0, 20)))
            else:
                s = live.pop(rng.integers(len(live)))
                am.free_seq(s)
        except AllocError:
            pass
        am.check_invariants()
        st = am.stats()
        assert st["slack_slots"] >= 0


@pytest.mark.parametrize("W", [1, 5, 16, 17, 33, 64])
def test_windowed_decode_is_dense_attention_over_the_last_w_rows(W):
    case = windowed(custom_case(3, "bf16", [1, 20, 40, 70, 100], 8, 2, 32), W)
    ref = run_case(case)
    for i in range(case.num_seqs):
        L = int(case.lens[i])
        rws = case.rows[int(case.batch[i])][max(0, L - W):L]
        want = dense_ref(bits_of(case.q[i], "bf16"), bits_of(case.k_tok[rws], "bf16"),
                         bits_of(case.v_tok[rws], "bf16"), "bf16")
        assert np.abs(ref["out"][i] - want).max() <= 1e-12


def test_window_one_returns_the_new_token_value():
    case = windowed(custom_case(4, "f32", [3, 17, 32, 33], 4, 4, 16), 1)
    ref = run_case(case)
    for i in range(case.num_seqs):
        row = case.rows[int(case.batch[i])][int(case.lens[i]) - 1]
        v = to_f64(bits_of(case.v_tok[row], "f32"), "f32")          # [Hkv][D]
        assert np.array_equal(ref["out"][i], v)


def test_window_at_least_the_length_is_full_attention():
    base = small_case("llama3_8b_bf16")
    full = run_case(base)["out"]
    wide = run_case(windowed(base, int(base.lens.max()), reuse=False))["out"]
    assert np.array_equal(full, wide)


def test_released_blocks_are_reused_and_nothing_changes():
    base = custom_case(5, "bf16", [100, 300, 257], 8, 2, 32)
    a = windowed(base, 64, reuse=False)
    b = windowed(base, 64, reuse=True)
    ra, rb = run_case(a), run_case(b)
    # with reuse the new sequences took the released blocks...
    released = set(int(x) for i in range(3)
                   for x in set(run_case(base, decode=False)["tables"][i].tolist()) -
                   set(ra["tables"][i].tolist()) if x >= 0)
    assert released and rb["setup_stats"]["used_blocks"] > ra["setup_stats"]["used_blocks"]
    assert not np.array_equal(ra["k_pool"], rb["k_pool"])
    # ...and the windowed outputs are identical
    assert np.array_equal(ra["out"], rb["out"])
    assert (ra["tables"][:, :2] == -1).all()
