"""GPU parity of pa_decode_step_shared: prefixes shared by groups of
sequences (forks: parallel samples, beams) attended once per group, the rest
by the even split, folded by the merge.  The result is the attention of
pa_decode_step (page 3, abeam.tech review, sections
「並列サンプリングやビームサーチでの共有」 and 「よくある質問」), so the
oracle is decode_ref; pools, tables, slots and copies bit for bit."""
import numpy as np
import pytest
import torch

from oracle import run_case
from tests.gpu_helpers import (CODED_TOL, NAN_BITS, REG_TOL, TOL, max_err, require_gpu,
                               run_gpu_step, say)
from workloads import make_case, small_case
from workloads.configs import Case, beam_case, position_coded

pytestmark = pytest.mark.gpu


def _check(case, got, ref, tol):
    plan = got["plan"]
    assert np.array_equal(plan.tables, ref["tables"])
    assert np.array_equal(plan.slots, ref["step_slots"])
    assert np.array_equal(plan.cows, ref["step_cows"].reshape(-1, 2))
    assert np.array_equal(got["k_pool"], ref["k_pool"]), "K pool differs"
    assert np.array_equal(got["v_pool"], ref["v_pool"]), "V pool differs"
    err = max_err(got["out"], ref["out"])
    pre, rows, start, mg = got["shared"]
    say(f"  {case.name}: {len(start) - 1} groups (largest {mg}), "
        f"max |gpu - oracle| = {err:.3e}")
    assert err <= tol
    return len(start) - 1


@pytest.mark.parametrize("parked", [True, False], ids=["parked_forks", "literal"])
@pytest.mark.parametrize("coded", [False, True], ids=["random", "coded"])
def test_small_parallel_sampling(parked, coded):
    case = small_case("cow_parallel_bf16", parked_forks=parked)
    if coded:
        case = position_coded(case, seed=11)
    say(f"[shared] {case.name} parked={parked}")
    ref = run_case(case, pool_fill=NAN_BITS["bf16"])
    got = run_gpu_step(case, shared=2)
    assert _check(case, got, ref, CODED_TOL if coded else REG_TOL["bf16"]) == 2


@pytest.mark.parametrize("seed,dtype,P,K,plen,steps,hq,hkv,d", [
    (1, "bf16", 2, 4, 40, 20, 32, 8, 128),
    (3, "f16", 1, 8, 100, 16, 8, 8, 128),
    (4, "bf16", 4, 4, 100, 40, 16, 4, 64),
    (5, "bf16", 3, 5, 300, 12, 64, 8, 128),
    (6, "f16", 2, 6, 200, 30, 12, 4, 128),
])
def test_beam_histories(seed, dtype, P, K, plen, steps, hq, hkv, d):
    """Beams share their prompt and often later blocks; groups form by first
    block, with the prefix common to all beams of a prompt."""
    case = beam_case(seed, dtype, P, K, plen, steps, hq, hkv, d)
    say(f"[shared] {case.name}")
    ref = run_case(case, pool_fill=NAN_BITS[dtype])
    got = run_gpu_step(case, shared=1)
    assert _check(case, got, ref, REG_TOL[dtype]) >= 1


@pytest.mark.parametrize("prompt_len,hq,hkv,d,dtype", [
    (16, 32, 8, 128, "bf16"),     # one shared block: three of four prefix pieces empty
    (40, 32, 8, 128, "bf16"),
    (100, 8, 8, 128, "f16"),      # one query head per KV head (one-wave workgroups)
    (300, 12, 4, 64, "bf16"),     # three per KV head, D = 64
    (520, 64, 4, 128, "bf16"),    # sixteen per KV head
    (700, 32, 8, 64, "f16"),
])
def test_prefix_pieces_over_short_and_long_prompts(prompt_len, hq, hkv, d, dtype):
    """Prompts forked into samples with tails of up to 1200 tokens: the long
    contexts make the prefix pass cut each shared prefix into several key
    ranges, some empty when the prompt holds only a block or two."""
    from workloads.configs import _parallel_sampling
    rng = np.random.default_rng(prompt_len)
    case = _parallel_sampling("pieces", 7 + prompt_len, dtype, 3, 4, prompt_len, 1200, hq, hkv,
                              d, "cpu", parked_forks=True, rng=rng)
    say(f"[shared pieces] prompt {prompt_len} Hq={hq} Hkv={hkv} D={d} {dtype} "
        f"max L={int(case.lens.max())}")
    ref = run_case(case, pool_fill=NAN_BITS[dtype])
    got = run_gpu_step(case, shared=1)
    assert _check(case, got, ref, REG_TOL[dtype]) == 3
    coded = position_coded(case, seed=prompt_len)
    ref = run_case(coded, pool_fill=NAN_BITS[dtype])
    got = run_gpu_step(coded, shared=1)
    _check(coded, got, ref, CODED_TOL)


def test_no_group_equals_plain_step_bit_for_bit():
    """A batch whose sequences share nothing: no prefix pass, and the rest is
    pa_decode_step on the even split, bit for bit."""
    case = small_case("llama3_8b_bf16")
    say("[shared] no groups")
    a = run_gpu_step(case, shared=1)
    assert len(a["shared"][2]) == 1
    b = run_gpu_step(case, partition_size=-1)
    assert np.array_equal(a["out"], b["out"])


def test_shared_close_to_plain_step():
    """Same inputs through pa_decode_step and pa_decode_step_shared: only the
    order of the fp32 sums differs."""
    case = small_case("cow_parallel_bf16")
    a = run_gpu_step(case, shared=2)
    b = run_gpu_step(case, partition_size=-1)
    assert max_err(a["out"], b["out"]) <= 1e-4


def _rerun(got, case, pre, rows, start, mg, workspace=None):
    """pa_decode_step_shared again on the step's state (the append rewrites
    the same slots with the same values) with a given plan."""
    pk = require_gpu()
    cache, plan = got["cache"], got["plan"]
    out = torch.empty(got["out"].shape, device="cuda")
    nr = torch.as_tensor(case.new_rows(), device="cuda")
    k_tok, v_tok = case.k_tok.cuda(), case.v_tok.cuda()
    pk.ops.decode_step_shared(out, got["q"], cache.k_pool, cache.v_pool,
                              k_tok.index_select(0, nr), v_tok.index_select(0, nr),
                              plan.d_slots, plan.d_tables, plan.d_lens, plan.max_context_len,
                              pre, rows, start, mg, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_inconsistent_plans_give_nan_rows_only_where_inconsistent():
    """The device checks of the plan: a prefix length that is not a whole
    number of blocks, one that differs from the group's, a nonzero prefix
    for a sequence in no group, and a group whose first member's length is
    unusable each give NaN rows for exactly the sequences concerned; every
    other row is the step's result.  The same workspace serves every call,
    so rows stamped by an earlier call are not taken for this call's."""
    require_gpu()
    case = small_case("cow_parallel_bf16", parked_forks=False)
    got = run_gpu_step(case, shared=2)
    good = got["out"]
    pre, rows, start, mg = got["shared"]
    assert len(start) == 3
    g0 = [int(r) for r in rows[int(start[0]):int(start[1])]]
    g1 = [int(r) for r in rows[int(start[1]):int(start[2])]]
    lens = got["plan"].lens
    ws = require_gpu().ops.decode_shared_workspace(case.num_seqs, case.num_q_heads,
                                                   case.num_kv_heads, case.head_dim,
                                                   got["plan"].max_context_len, got["q"].dtype)

    def run(p=pre, r=rows, s=start):
        return _rerun(got, case, p, r, s, mg, workspace=ws)

    def expect(o, nan_rows):
        for i in range(case.num_seqs):
            if i in nan_rows:
                assert np.isnan(o[i]).all(), f"row {i} should be NaN"
            else:
                assert not np.isnan(o[i]).any(), f"row {i} should be finite"
                assert max_err(o[i], good[i]) <= 1e-4
    say(f"[shared checks] groups {g0} {g1}, lens {list(lens)}")
    expect(run(), set())
    bad = pre.clone(); bad[g0[1]] = 8                       # not whole blocks
    expect(run(p=bad), {g0[1]})
    bad = pre.clone(); bad[g0[2]] = 32                      # differs from the group's 64
    expect(run(p=bad), {g0[2]})
    bad = pre.clone(); bad[g0[0]] = 8                       # the group's own length unusable
    expect(run(p=bad), set(g0))
    # group 1 left out of the plan, its members' prefixes kept: no pass
    # attended them in this call
    expect(run(r=rows[:len(g0)].contiguous(), s=start[:2].contiguous()), set(g1))
    # a sequence with a nonzero prefix that is not a member, beside a good plan
    expect(run(r=torch.cat([rows[:len(g0) - 1], rows[len(g0):]]).contiguous(),
               s=torch.tensor([0, len(g0) - 1, len(rows) - 1], dtype=torch.int32,
                              device="cuda")), {g0[-1]})
    # the whole plan again on the same workspace
    expect(run(), set())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kw", [{}, {"parked_forks": False}], ids=["parked_forks", "literal"])
@pytest.mark.parametrize("coded", [False, True], ids=["random", "coded"])
def test_full_size_parallel_sampling_every_row(kw, coded):
    """The copy-on-write workload at full size (32 prompts of 1024 tokens x 8
    samples): 32 groups sharing 64 blocks; every row against the oracle and
    every sequence's K/V gathered bit-exact."""
    from tests.test_gpu_fullsize import check_every_gather, check_every_row, check_plan
    require_gpu()
    case = make_case("cow_parallel_bf16", device="cuda", **kw)
    if coded:
        case = position_coded(case, seed=12)
    say(f"[shared full size] {case.name} {kw}")
    got = run_gpu_step(case, pools=False, shared=4)
    check_plan(case, got)
    pre, rows, start, mg = got["shared"]
    assert len(start) - 1 == 32 and mg == 8 and set(pre.cpu().tolist()) == {1024}
    check_every_row(case, got["out"], CODED_TOL if coded else REG_TOL["bf16"], case.name)
    check_every_gather(case, got)


def _shared_inputs():
    pk = require_gpu()
    case = small_case("cow_parallel_bf16", parked_forks=False)
    got = run_gpu_step(case, shared=2)
    cache, plan = got["cache"], got["plan"]
    nr = torch.as_tensor(case.new_rows(), device="cuda")
    k_new = case.k_tok.cuda().index_select(0, nr).contiguous()
    v_new = case.v_tok.cuda().index_select(0, nr).contiguous()
    return pk, case, got, cache, plan, k_new, v_new


def test_shared_step_on_a_side_stream_matches_the_default_stream():
    """The call on a caller's side stream (workspace allocated for that
    stream): the library forks its prefix pass from that stream and joins it
    back before the merge; the rows equal the default-stream call's bit for
    bit."""
    pk, case, got, cache, plan, k_new, v_new = _shared_inputs()
    pre, rows, start, mg = got["shared"]
    ref = torch.empty(got["out"].shape, device="cuda")
    pk.ops.decode_step_shared(ref, got["q"], cache.k_pool, cache.v_pool, k_new, v_new,
                              plan.d_slots, plan.d_tables, plan.d_lens, plan.max_context_len,
                              pre, rows, start, mg)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = torch.empty(got["out"].shape, device="cuda")
        pk.ops.decode_step_shared(out, got["q"], cache.k_pool, cache.v_pool, k_new, v_new,
                                  plan.d_slots, plan.d_tables, plan.d_lens,
                                  plan.max_context_len, pre, rows, start, mg, stream=side)
    side.synchronize()
    assert torch.equal(out, ref)


def test_shared_step_captured_in_a_graph_replays_like_the_eager_call():
    """The step captured into a HIP graph (the prefix pass's fork and join are
    captured as event nodes) and replayed three times, with eager work and
    synchronisations between the replays: every replay's rows equal the
    eager call's bit for bit."""
    pk, case, got, cache, plan, k_new, v_new = _shared_inputs()
    pre, rows, start, mg = got["shared"]
    B, Hq, D = got["out"].shape
    ws = pk.ops.decode_shared_workspace(B, Hq, case.num_kv_heads, D, plan.max_context_len,
                                        got["q"].dtype)
    eager = torch.empty((B, Hq, D), device="cuda")
    pk.ops.decode_step_shared(eager, got["q"], cache.k_pool, cache.v_pool, k_new, v_new,
                              plan.d_slots, plan.d_tables, plan.d_lens, plan.max_context_len,
                              pre, rows, start, mg, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty((B, Hq, D), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pk.ops.decode_step_shared(out, got["q"], cache.k_pool, cache.v_pool, k_new, v_new,
                                  plan.d_slots, plan.d_tables, plan.d_lens,
                                  plan.max_context_len, pre, rows, start, mg, workspace=ws,
                                  stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        ws.zero_()                                   # no stale partial or stamp helps
        junk = torch.randn(1 << 16, device="cuda") * (i + 1)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        del junk
    # The plan edited in place between replays (the graph keeps its buffers):
    # group 1 emptied.  Its members keep their prefix lengths, but no prefix
    # pass writes their rows in this replay; the rows an earlier replay wrote
    # carry the same epoch (fixed at capture) and must not be taken: their
    # stamps were cleared by the merge that read them, so these rows are NaN.
    g1 = [int(r) for r in rows[int(start[1]):int(start[2])]]
    start[2] = start[1]
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    o, e = out.cpu().numpy(), eager.cpu().numpy()
    for i in range(B):
        if i in g1:
            assert np.isnan(o[i]).all(), f"row {i}"
        else:
            assert np.array_equal(o[i], e[i]), f"row {i}"
