"""Pins for beam-search bookkeeping in the oracle: the reorder op of the
allocator model (hand-worked tables, counts and free list; all-or-nothing
errors; invariants over random beam histories) and the beam workload's
final decode against dense attention over each beam's own token history
(no pool, no table, no sharing)."""
import numpy as np
import pytest

from oracle import AllocatorModel, bits_of, dense_ref, run_case
from oracle.allocator import AllocError
from workloads.configs import beam_case


def test_reorder_hand_example():
    am = AllocatorModel(8, 16)
    am.add_seq(0, 20)                        # blocks 0, 1
    am.fork(0, 1)
    am.fork(0, 2)
    am.extend(1, 1)                          # copy of block 1 -> 2 (pair (1, 2))
    assert am.tables[1] == [0, 2] and list(am.ref[:3]) == [3, 2, 1]
    # new beams: 0 (keeps), 5 (child of 0), 2 (keeps); beam 1 dropped
    am.reorder([0, 1, 2], [0, 5, 2], [0, 0, 2])
    assert sorted(am.tables) == [0, 2, 5]
    assert am.tables[5] == [0, 1] and list(am.ref[:3]) == [3, 3, 0]
    assert am.free[-1] == 2                  # block 2 (beam 1's copy) back on top
    am.check_invariants()


@pytest.mark.parametrize("args,code", [
    (([0, 9], [0], [0]), "unknown"),         # unknown old id
    (([0, 0], [0], [0]), "repeat"),          # repeated old id
    (([0], [3, 3], [0, 0]), "repeat"),       # repeated new id
    (([0], [3], [1]), "range"),              # parent index out of range
    (([0], [1], [0]), "exists"),             # new id live, not its own parent
])
def test_reorder_errors_change_nothing(args, code):
    am = AllocatorModel(8, 16)
    am.add_seq(0, 20)
    am.add_seq(1, 5)
    before = ({k: list(v) for k, v in am.tables.items()}, list(am.ref), list(am.free))
    with pytest.raises(AllocError):
        am.reorder(*args)
    assert ({k: list(v) for k, v in am.tables.items()}, list(am.ref), list(am.free)) == before


@pytest.mark.parametrize("seed,P,K,plen,steps", [(1, 2, 4, 40, 20), (2, 3, 3, 17, 35),
                                                 (3, 1, 8, 16, 16)])
def test_beam_decode_is_dense_attention_over_each_history(seed, P, K, plen, steps):
    case = beam_case(seed, "bf16", P, K, plen, steps, 8, 2, 32)
    ref = run_case(case)
    for i, sid in enumerate(case.batch.tolist()):
        rws = case.rows[sid]
        assert len(rws) == case.lens[i] == plen + steps + 1
        want = dense_ref(bits_of(case.q[i], "bf16"), bits_of(case.k_tok[rws], "bf16"),
                         bits_of(case.v_tok[rws], "bf16"), "bf16")
        assert np.abs(ref["out"][i] - want).max() <= 1e-12


def test_beam_history_shares_blocks_and_keeps_invariants():
    case = beam_case(4, "bf16", 4, 4, 64, 40, 8, 2, 32)
    am = AllocatorModel(case.num_blocks, 16, case.free_order)
    from oracle.run import run_script
    run_script(am, case.script, case.rows)
    am.check_invariants()
    st = am.stats()
    unshared = sum(-(-int(L - 1) // 16) for L in case.lens)     # before the step's token
    assert st["used_blocks"] < unshared
    assert st["shared_blocks"] > 0
    # every prompt's first blocks are still shared by its beams' common prefix
    tables = [am.tables[s] for s in case.batch.tolist()]
    for p in range(4):
        firsts = {t[0] for t in tables[4 * p:4 * p + 4]}
        assert len(firsts) == 1
