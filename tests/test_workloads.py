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
