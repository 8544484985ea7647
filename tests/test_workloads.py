"""The synthetic workloads: deterministic per seed, and shaped as specified."""
import numpy as np
import torch

from oracle import run_case
from workloads import make_case, small_case
from workloads.configs import CONFIG_NAMES


def test_deterministic_per_seed():
    a, b = small_case("llama3_8b_bf16"), small_case("llama3_8b_bf16")
    assert np.array_equal(a.lens, b.lens) and np.array_equal(a.free_order, b.free_order)
    assert torch.equal(a.k_tok, b.k_tok) and torch.equal(a.q, b.q)
    c = small_case("llama3_8b_bf16", seed=999)
    assert not torch.equal(a.k_tok[:10], c.k_tok[:10])


def test_tiny_config_shape():
    c = make_case("tiny_fp32")
    assert list(c.lens) == [1, 15, 16, 37] and c.num_blocks == 16
    assert (c.num_q_heads, c.num_kv_heads, c.head_dim, c.dtype) == (4, 4, 64, "f32")
    assert sorted(c.free_order.tolist()) == list(range(16))


def test_llama_config_structure_without_values():
    # lengths and pool only (values are drawn too, but at 150M elements; keep them)
    c = make_case("llama3_8b_bf16")
    assert c.num_seqs == 64 and c.lens.min() >= 256 and c.lens.max() <= 2048
    need = sum(-(-int(L) // 16) for L in c.lens)
    assert c.num_blocks == int(np.ceil(1.2 * need))
    assert c.k_tok.dtype == torch.bfloat16 and c.k_tok.shape == (int(c.lens.sum()), 8, 128)


def test_small_cases_all_build_and_run():
    for n in CONFIG_NAMES:
        c = small_case(n)
        r = run_case(c, with_pools=False)
        assert np.array_equal(r["lens"], c.lens)


def test_cow_case_parked_forks_force_copies():
    c = small_case("cow_parallel_bf16")
    r = run_case(c, with_pools=False)
    assert len(r["step_cows"]) == c.notes["parked_forks"]
    lit = small_case("cow_parallel_bf16", parked_forks=False)
    assert len(run_case(lit, with_pools=False)["step_cows"]) == 0


def test_position_coded_values_name_their_row_and_head():
    """The V code of a position-coded case reads back as (token row, KV head);
    K and q hold only 0 and +-64, with q's pattern set by h % 4."""
    from workloads.configs import CODE_UNIT, position_coded
    c = position_coded(small_case("opt13b_fp16"))
    R, H, D = c.v_tok.shape
    nb, gb = c.notes["position_coded"]["row_bits"], c.notes["position_coded"]["head_bits"]
    v = c.v_tok.to(torch.float64).numpy() / CODE_UNIT
    assert set(np.unique(v).tolist()) <= {0.0, 1.0}
    rows = (v[:, :, :nb] * (1 << np.arange(nb))).sum(-1)
    heads = (v[:, :, nb:nb + gb] * (1 << np.arange(gb))).sum(-1)
    assert np.array_equal(rows, np.repeat(np.arange(R)[:, None], H, 1))
    assert np.array_equal(heads, np.repeat(np.arange(H)[None, :], R, 0))
    assert not v[:, :, nb + gb:].any()
    k = c.k_tok.to(torch.float64).numpy()
    assert set(np.unique(k).tolist()) <= {-CODE_UNIT, 0.0, CODE_UNIT} and not k[:, :, 2:].any()
    assert (k[:, :, 0] > 0).any() and (k[:, :, 0] < 0).any() and (k[:, :, 1] > 0).any()
    q = c.q.to(torch.float64).numpy()
    for h in range(c.num_q_heads):
        want = np.zeros(D)
        if h % 4 == 0:
            want[0] = CODE_UNIT
        elif h % 4 == 1:
            want[0] = -CODE_UNIT
        elif h % 4 == 2:
            want[1] = CODE_UNIT
        assert np.array_equal(q[:, h], np.repeat(want[None], c.num_seqs, 0))
    # same structure as the case it codes
    base = small_case("opt13b_fp16")
    assert np.array_equal(c.lens, base.lens) and c.script == base.script
