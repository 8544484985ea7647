"""GPU parity of beam-search bookkeeping: multi-step beam histories (reorder,
fork, free, one-token appends with copy-on-write) replayed through the C++
block manager and the device ops, against the oracle on NaN-poisoned pools
(tables, slots, copy pairs and whole pools bit for bit; the final step's
outputs element by element), and the multi-layer copy bit for bit."""
import numpy as np
import pytest
import torch

from oracle import bits_of, copy_ref, run_case
from tests.gpu_helpers import (CODED_TOL, NAN_BITS, REG_TOL, TOL, max_err, require_gpu,
                               run_gpu_step, say)
from workloads.configs import beam_case

pytestmark = pytest.mark.gpu


def _check(case, got, ref):
    plan = got["plan"]
    assert np.array_equal(plan.tables, ref["tables"])
    assert np.array_equal(plan.slots, ref["step_slots"])
    assert np.array_equal(plan.cows, ref["step_cows"].reshape(-1, 2))
    assert np.array_equal(got["k_pool"], ref["k_pool"]), "K pool differs"
    assert np.array_equal(got["v_pool"], ref["v_pool"]), "V pool differs"
    err = max_err(got["out"], ref["out"])
    say(f"  {case.name}: {len(plan.cows)} step copies, max |gpu - oracle| = {err:.3e}")
    assert err <= TOL[case.dtype]
    assert err <= REG_TOL[case.dtype], "beyond the regression bar"


@pytest.mark.parametrize("seed,dtype,P,K,plen,steps,hq,hkv,d", [
    (1, "bf16", 2, 4, 40, 20, 32, 8, 128),
    (2, "bf16", 3, 3, 17, 35, 8, 2, 64),
    (3, "f16", 1, 8, 16, 16, 8, 8, 128),
    (4, "bf16", 4, 4, 100, 40, 16, 4, 128),
])
@pytest.mark.parametrize("fused,ps", [(True, 0), (False, 0), (True, 64)])
def test_beam_histories_match_oracle(seed, dtype, P, K, plen, steps, hq, hkv, d, fused, ps):
    case = beam_case(seed, dtype, P, K, plen, steps, hq, hkv, d)
    say(f"[beam] {case.name} fused={fused} P={ps}")
    ref = run_case(case, pool_fill=NAN_BITS[dtype])
    got = run_gpu_step(case, partition_size=ps, fused=fused)
    _check(case, got, ref)
    st = got["cache"].bm.stats()
    assert st["shared_blocks"] > 0


def test_copy_blocks_layers_bitexact():
    """Copy pairs applied to 4 layers' pools with distinct contents in one
    launch, against the oracle's block copy per layer; out-of-range pairs skip."""
    pk = require_gpu()
    N, H, D, layers = 40, 4, 128, 4
    g = torch.Generator(device="cuda").manual_seed(5)
    ks, vs = [], []
    for _ in range(layers):
        k, v = pk.ops.new_pools(N, H, D, torch.bfloat16, "cuda")
        k.copy_(torch.randn(k.shape, generator=g, device="cuda"))
        v.copy_(torch.randn(v.shape, generator=g, device="cuda"))
        ks.append(k)
        vs.append(v)
    before = [(bits_of(k, "bf16"), bits_of(v, "bf16")) for k, v in zip(ks, vs)]
    pairs = np.array([[3, 7], [11, 2], [5, 39], [0, 20], [N + 4, 1], [6, -1]], dtype=np.int32)
    pk.ops.copy_blocks_layers(ks, vs, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    for l_ in range(layers):
        kb, vb = before[l_]
        copy_ref(kb, vb, pairs[:4])
        assert np.array_equal(bits_of(ks[l_], "bf16"), kb), l_
        assert np.array_equal(bits_of(vs[l_], "bf16"), vb), l_


@pytest.mark.timeout(900)
@pytest.mark.parametrize("coded", [False, True], ids=["random", "position_coded"])
def test_beam_search_at_scale_every_beam(coded):
    """64 beams (16 prompts x 4) of Llama-3-8B heads after 64 beam steps on
    1024-token prompts, poisoned pools: bookkeeping bit-exact against the
    oracle's, every beam's output against dense attention over its own
    history, and every beam's K/V gathered bit-exact."""
    from tests.test_gpu_fullsize import check_every_gather, check_every_row
    from workloads.configs import position_coded
    require_gpu()
    case = beam_case(6, "bf16", 16, 4, 1024, 64, 32, 8, 128, device="cuda")
    if coded:
        case = position_coded(case, seed=6)
    say(f"[beam at scale] {case.name}: {len(case.script)} set-up ops")
    ref = run_case(case, with_pools=False)
    got = run_gpu_step(case, pools=False)
    plan = got["plan"]
    assert np.array_equal(plan.tables, ref["tables"])
    assert np.array_equal(plan.slots, ref["step_slots"])
    assert np.array_equal(plan.cows, ref["step_cows"].reshape(-1, 2))
    st = got["cache"].bm.stats()
    unshared = sum(-(-int(L) // 16) for L in case.lens)
    say(f"  blocks used {st['used_blocks']} vs {unshared} unshared; "
        f"{len(plan.cows)} copies in the step")
    assert st["used_blocks"] < unshared / 3
    check_every_row(case, got["out"], CODED_TOL if coded else REG_TOL["bf16"], case.name)
    check_every_gather(case, got)
