"""GPU parity of sliding-window decode (pa_decode_window, pa_decode_step_window)
against the oracle's windowed decode_ref, on NaN-poisoned pools whose
out-of-window blocks were released with pa_bm_release_before and then
rewritten by other sequences (so a kernel that read them would be caught)."""
import numpy as np
import pytest
import torch

from oracle import run_case
from oracle.run import oracle_sequence_out
from tests.gpu_helpers import NAN_BITS, REG_TOL, TOL, max_err, require_gpu, run_gpu_step, say
from workloads import make_case, small_case
from workloads.configs import custom_case, windowed

pytestmark = pytest.mark.gpu


@pytest.fixture
def kernel(request):
    """Runs the test on the matrix-core ("auto") or plain-FMA ("generic")
    decode kernels (pa_set_decode_kernel), restoring the default after."""
    pk = require_gpu()
    prev = pk.ops.set_decode_kernel(request.param)
    yield request.param
    pk.ops.set_decode_kernel(prev)


def _check(case, got, ref):
    plan = got["plan"]
    assert np.array_equal(plan.tables, ref["tables"])
    assert np.array_equal(plan.slots, ref["step_slots"])
    assert np.array_equal(got["k_pool"], ref["k_pool"]), "K pool differs"
    assert np.array_equal(got["v_pool"], ref["v_pool"]), "V pool differs"
    err = max_err(got["out"], ref["out"])
    say(f"  {case.name}: max |gpu - oracle| = {err:.3e}")
    assert err <= TOL[case.dtype]
    assert err <= REG_TOL[case.dtype], "beyond the regression bar"


@pytest.mark.parametrize("kernel", ["auto", "generic"], indirect=True)
@pytest.mark.parametrize("name,W,ps", [("llama3_8b_bf16", 100, 0), ("llama3_8b_bf16", 300, 256),
                                       ("llama3_8b_bf16", 17, 64),
                                       ("cow_parallel_bf16", 64, 0),
                                       ("long_context_bf16", 512, 512),
                                       ("long_context_bf16", 700, 0)])
@pytest.mark.parametrize("fused", [True, False])
def test_small_configs_windowed(name, W, ps, fused, kernel):
    case = windowed(small_case(name), W)
    say(f"[window] {case.name} P={ps} fused={fused} kernel={kernel}")
    ref = run_case(case, pool_fill=NAN_BITS[case.dtype])
    assert (ref["tables"] == -1).any()          # some blocks were released
    got = run_gpu_step(case, partition_size=ps, fused=fused)
    _check(case, got, ref)


EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 600]


@pytest.mark.parametrize("kernel", ["auto", "generic"], indirect=True)
@pytest.mark.parametrize("dtype,hq,hkv,d,ps", [("bf16", 32, 8, 128, 0), ("f16", 16, 4, 64, 0),
                                              ("bf16", 8, 8, 128, 64), ("f32", 8, 2, 64, 0),
                                              ("bf16", 12, 4, 128, 16), ("f16", 6, 3, 64, -1),
                                              ("bf16", 64, 8, 128, 0), ("f16", 14, 2, 64, 64),
                                              ("bf16", 32, 2, 64, -1), ("f16", 96, 8, 128, 256)])
@pytest.mark.parametrize("W", [1, 15, 16, 17, 64, 250])
def test_edge_windows(dtype, hq, hkv, d, ps, W, kernel):
    case = windowed(custom_case(71, dtype, EDGE_LENS, hq, hkv, d, partition_size=ps), W)
    say(f"[window edge] {dtype} Hq={hq} Hkv={hkv} D={d} P={ps} W={W} kernel={kernel}")
    ref = run_case(case, pool_fill=NAN_BITS[dtype])
    got = run_gpu_step(case)
    _check(case, got, ref)


@pytest.mark.parametrize("kernel", ["generic"], indirect=True)
def test_plain_fma_kernel_takes_large_groups(kernel):
    case = windowed(custom_case(72, "bf16", [40, 300, 129], 32, 2, 64), 50)
    ref = run_case(case, pool_fill=NAN_BITS["bf16"])
    _check(case, run_gpu_step(case), ref)


def test_window_covering_everything_equals_plain_decode():
    pk = require_gpu()
    case = small_case("llama3_8b_bf16")
    got = run_gpu_step(case)
    plan, cache = got["plan"], got["cache"]
    out = torch.empty(got["out"].shape, device="cuda")
    pk.ops.decode(out, got["q"], cache.k_pool, cache.v_pool, plan.d_tables, plan.d_lens,
                  plan.max_context_len, window=plan.max_context_len)
    assert np.array_equal(out.cpu().numpy(), got["out"])


@pytest.mark.timeout(900)
def test_full_size_long_context_window_every_row():
    """The long-context workload (16 sequences of 32K-131K tokens) with a
    4096-token window, in the bench's configuration (the library's default
    split, poisoned pools): every table bit-exact, only the window's blocks
    resident, every row against the oracle, every window gathered bit-exact."""
    from tests.test_gpu_fullsize import check_every_gather, check_every_row
    require_gpu()
    case = windowed(make_case("long_context_bf16", device="cuda"), 4096, reuse=False)
    say(f"[window full-size] {case.name}")
    ref = run_case(case, with_pools=False)
    got = run_gpu_step(case, partition_size=0, pools=False)
    assert np.array_equal(got["plan"].tables, ref["tables"])
    # only the window's blocks stay resident: at most 4096/16 + 1 per sequence
    st = got["cache"].bm.stats()
    assert st["used_blocks"] == ref["stats"]["used_blocks"] <= 16 * (4096 // 16 + 1)
    check_every_row(case, got["out"], REG_TOL["bf16"], "long context W=4096")
    check_every_gather(case, got)
