"""Full-size parity in the bench's launch configuration: every output row of
every workload against the fp64 oracle, and every sequence's K/V gathered
through its block table bit for bit against its own token rows.

Two kinds of values run through the same steps:

* the workloads' own random values: each row within the oracle contract
  (1e-2 for 16-bit pools) and within the recorded regression bar REG_TOL;
* position-coded values (workloads.configs.position_coded): each row is an
  exact mean of stored 0/64 entries, so a dropped, doubled or misplaced token
  anywhere in a context of up to 131072 tokens moves some element by at least
  64 / L, far above CODED_TOL, which is what rounding alone leaves.

The paging contract these check: the result is that of attention over the
contiguous cache (page 3, abeam.tech review, section 「よくある質問」; page 4,
pro-knowledge-base FAQ), and appended and copied blocks hold exactly the
tokens written (page 3, sections 「KV キャッシュマネージャ」 and
「並列サンプリングやビームサーチでの共有」)."""
import numpy as np
import pytest
import torch

from oracle import bits_of, run_case
from oracle.quant import quantize_ref
from oracle.run import oracle_sequence_out
from tests.gpu_helpers import CODED_TOL, REG_TOL, TOL, max_err, require_gpu, run_gpu_step, say
from workloads import make_case
from workloads.configs import custom_case, position_coded, windowed

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

FULL = [("llama3_8b_bf16", {}), ("opt13b_fp16", {}), ("cow_parallel_bf16", {}),
        ("cow_parallel_bf16", {"parked_forks": False}), ("long_context_bf16", {})]
FULL_IDS = ["llama3_8b", "opt13b", "cow_parked_forks", "cow_literal", "long_context"]
INT_VIEW = {"bf16": torch.int16, "f16": torch.int16, "f32": torch.int32}


def check_plan(case, got):
    """Slots, copy-on-write pairs, tables and lengths bit-exact against the
    oracle's allocator model."""
    ref = run_case(case, with_pools=False)
    plan = got["plan"]
    assert np.array_equal(plan.slots, ref["step_slots"])
    assert np.array_equal(plan.cows, ref["step_cows"].reshape(-1, 2))
    assert np.array_equal(plan.tables, ref["tables"])
    assert np.array_equal(plan.lens, ref["lens"])
    return ref


def check_every_row(case, out, tol, label):
    """Every (sequence, head) row against the oracle's fp64 output computed
    straight from the sequence's token rows (no pool, no table)."""
    worst, at = 0.0, -1
    for i in range(case.num_seqs):
        err = max_err(out[i], oracle_sequence_out(case, i))
        if err > worst:
            worst, at = err, i
    say(f"  {label}: {case.num_seqs} rows, max |gpu - oracle| = {worst:.3e} "
        f"(seq {at}, L={case.lens[at] if at >= 0 else '-'}; bar {tol:.1e})")
    assert worst <= tol, (label, worst, at)
    return worst


def check_every_gather(case, got):
    """Each sequence's attended positions gathered through its table
    (pa_gather_kv) equal its token rows bit for bit: the appends, the
    copy-on-write copies and the step's write all landed where the table
    says, and nothing overwrote them."""
    pk = require_gpu()
    cache, plan = got["cache"], got["plan"]
    cd = getattr(case, "cache_dtype", None)
    W = getattr(case, "window", 0)
    for i in range(case.num_seqs):
        L = int(case.lens[i])
        if L == 0:
            continue
        f = max(0, L - W) if W else 0
        kg, vg = pk.ops.gather_kv(cache.k_pool, cache.v_pool, plan.d_tables[i:i + 1].contiguous(),
                                  plan.d_lens[i:i + 1].contiguous(), L)
        kg = kg[0, :, f:L].transpose(0, 1).contiguous()     # [L - f][Hkv][D]
        vg = vg[0, :, f:L].transpose(0, 1).contiguous()
        idx = torch.as_tensor(case.rows[int(case.batch[i])][f:L], device="cuda")
        kt, vt = case.k_tok.index_select(0, idx), case.v_tok.index_select(0, idx)
        if cd is None:
            iv = INT_VIEW[case.dtype]
            assert torch.equal(kg.view(iv), kt.view(iv)), f"K of sequence {i}"
            assert torch.equal(vg.view(iv), vt.view(iv)), f"V of sequence {i}"
        else:
            want_k = quantize_ref(bits_of(kt, case.dtype), case.dtype, cd, case.k_scale)
            want_v = quantize_ref(bits_of(vt, case.dtype), case.dtype, cd, case.v_scale)
            assert np.array_equal(bits_of(kg, cd), want_k), f"K codes of sequence {i}"
            assert np.array_equal(bits_of(vg, cd), want_v), f"V codes of sequence {i}"
    say(f"  {case.num_seqs} sequences' K/V gathered bit-exact")


def _run_full(case, label, tol, **kw):
    say(f"[full size] {label}: B={case.num_seqs} sum L={int(case.lens.sum())} "
        f"Hq={case.num_q_heads} Hkv={case.num_kv_heads} {case.kv_dtype} {kw}")
    got = run_gpu_step(case, pools=False, **kw)
    check_plan(case, got)
    err = check_every_row(case, got["out"], tol, label)
    return got, err


@pytest.mark.parametrize("name,kw", FULL, ids=FULL_IDS)
def test_full_size_every_row_and_sequence(name, kw):
    """Random values, the workload's own launch configuration (the even split;
    512-token partitions for the long contexts): every row within the contract
    and the regression bar, every sequence's K/V bit-exact."""
    require_gpu()
    case = make_case(name, device="cuda", **kw)
    got, err = _run_full(case, f"{name} {kw}", REG_TOL[case.dtype])
    assert err <= TOL[case.dtype]
    check_every_gather(case, got)


@pytest.mark.parametrize("name,kw", [("tiny_fp32", {})] + FULL, ids=["tiny"] + FULL_IDS)
def test_full_size_position_coded(name, kw):
    """Position-coded values on every workload at full size: each row an exact
    mean, so one token dropped, doubled or read from the wrong block or offset
    anywhere fails."""
    require_gpu()
    case = position_coded(make_case(name, device="cuda", **kw))
    got, _ = _run_full(case, f"{name} coded {kw}", CODED_TOL if case.dtype != "f32" else 1e-5)
    check_every_gather(case, got)


@pytest.mark.parametrize("kernel", ["auto", "generic"])
@pytest.mark.parametrize("ps,fused", [(-1, True), (-1, "phased"), (-1, False), (16, True),
                                      (64, True), (256, False), (512, True), (2048, True)])
def test_llama_position_coded_every_partitioning(ps, fused, kernel):
    """The Llama-3-8B batch, position-coded, on the even split and on fixed
    partitions from one block to a whole context, fused and unfused steps,
    matrix-core and plain-FMA kernels: every piece boundary exercised."""
    pk = require_gpu()
    prev = pk.ops.set_decode_kernel(kernel)
    try:
        case = position_coded(make_case("llama3_8b_bf16", device="cuda"), seed=1)
        _run_full(case, f"llama coded P={ps} fused={fused} kernel={kernel}", CODED_TOL,
                  partition_size=ps, fused=fused)
    finally:
        pk.ops.set_decode_kernel(prev)


@pytest.mark.parametrize("q_heads", [64, 96, 128])
def test_llama_more_heads_position_coded(q_heads):
    """8, 12 and 16 query heads per KV head (two to four head groups per K/V
    load) on the Llama-3-8B lengths, position-coded, plus random values."""
    require_gpu()
    case = make_case("llama3_8b_bf16", device="cuda", q_heads=q_heads)
    _run_full(case, f"llama Hq={q_heads}", REG_TOL["bf16"])
    _run_full(position_coded(case, seed=2), f"llama Hq={q_heads} coded", CODED_TOL)


@pytest.mark.parametrize("ps", [-1, 16, 512])
def test_one_context_in_many_pieces_position_coded(ps):
    """One 100 000-token context with one KV head cut into hundreds (even
    split) to thousands (16-token partitions) of pieces."""
    require_gpu()
    case = position_coded(custom_case(52, "bf16", [100000], 4, 1, 128, partition_size=ps,
                                      device="cuda"), seed=3)
    _run_full(case, f"100k context coded P={ps}", CODED_TOL)


@pytest.mark.parametrize("cache_dtype", ["fp8", "i8"])
def test_quantized_llama_position_coded(cache_dtype):
    """8-bit pools (scales 1: codes 0 and +-64 are exact in both formats),
    position-coded, fused step; the codes of every sequence bit-exact."""
    from dataclasses import replace
    require_gpu()
    base = position_coded(make_case("llama3_8b_bf16", device="cuda"), seed=4)
    case = replace(base, cache_dtype=cache_dtype, k_scale=1.0, v_scale=1.0)
    got, _ = _run_full(case, f"llama coded {cache_dtype} pools", CODED_TOL)
    check_every_gather(case, got)


@pytest.mark.parametrize("W", [4096, 1000])
def test_long_context_window_position_coded(W):
    """The long-context batch with a sliding window and its out-of-window
    blocks released: position-coded rows exact over the window."""
    require_gpu()
    case = position_coded(windowed(make_case("long_context_bf16", device="cuda"), W,
                                   reuse=False), seed=5)
    got, _ = _run_full(case, f"long context W={W} coded", CODED_TOL)
    check_every_gather(case, got)
