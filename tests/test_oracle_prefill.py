"""Pins for the prefill / chunked-prefill oracle (oracle/prefill.py), each
against something other than the function itself: the decode oracle (one
query token), torch's scaled_dot_product_attention in fp64 with the causal
mask (a library routine over the contiguous K/V), explicit token loops over
the unpaged token rows, the prefix property of causal attention, and
invariance under the physical placement of the blocks."""
import numpy as np
import pytest
import torch

from oracle import bits_of, decode_ref, run_case, to_f64
from oracle.cache import gather_ref
from oracle.prefill import prefill_ref
from workloads.configs import prefill_case


def _setup(seed, dtype, lens, qlens, hq, hkv, d):
    case, q, qs = prefill_case(seed, dtype, lens, qlens, hq, hkv, d)
    ref = run_case(case, decode=False)
    return case, bits_of(q, dtype), qs, ref


def test_one_query_token_is_the_decode_step():
    case, _, _, ref = _setup(1, "bf16", [1, 17, 40, 100], [1, 1, 1, 1], 8, 2, 64)
    qb = bits_of(case.q, "bf16")                       # the decode step's q rows
    qs = np.arange(5)
    got = prefill_ref(qb, ref["k_pool"], ref["v_pool"], ref["tables"], ref["lens"], qs, "bf16")
    want = decode_ref(qb, ref["k_pool"], ref["v_pool"], ref["tables"], ref["lens"], "bf16")
    assert np.abs(got - want).max() <= 1e-12


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 8, 2, 64), ("f32", 4, 4, 32),
                                            ("f16", 6, 3, 64)])
@pytest.mark.parametrize("L,n", [(37, 37), (70, 21), (16, 1), (33, 32)])
def test_matches_torch_sdpa_with_causal_mask(dtype, hq, hkv, d, L, n):
    case, qb, qs, ref = _setup(2, dtype, [L], [n], hq, hkv, d)
    got = prefill_ref(qb, ref["k_pool"], ref["v_pool"], ref["tables"], ref["lens"], qs, dtype)
    K, V = gather_ref(ref["k_pool"], ref["v_pool"], ref["tables"][0], L, 16)   # [Hkv][L][D]
    G = hq // hkv
    k = torch.from_numpy(to_f64(K, dtype)).repeat_interleave(G, 0)[None]      # [1][Hq][L][D]
    v = torch.from_numpy(to_f64(V, dtype)).repeat_interleave(G, 0)[None]
    qq = torch.from_numpy(to_f64(qb, dtype)).permute(1, 0, 2)[None]            # [1][Hq][n][D]
    mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]     # [n][L]
    want = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=mask)
    want = want[0].permute(1, 0, 2).numpy()
    assert np.abs(got - want).max() <= 1e-12


def test_brute_force_token_loops():
    """Explicit sums over the generator's token rows in logical order (no
    pool, no table, no matrix products)."""
    lens, qlens = [5, 19, 3], [5, 4, 2]
    case, qb, qs, ref = _setup(3, "bf16", lens, qlens, 4, 2, 16)
    got = prefill_ref(qb, ref["k_pool"], ref["v_pool"], ref["tables"], ref["lens"], qs, "bf16")
    q = to_f64(qb, "bf16")
    K = to_f64(bits_of(case.k_tok, "bf16"), "bf16")
    V = to_f64(bits_of(case.v_tok, "bf16"), "bf16")
    for b, (L, n) in enumerate(zip(lens, qlens)):
        rows = case.rows[case.batch[b]]
        for i in range(n):
            p = L - n + i
            for h in range(4):
                g = h // 2
                s = [0.25 * sum(q[qs[b] + i, h, e] * K[rows[t], g, e] for e in range(16))
                     for t in range(p + 1)]
                mx = max(s)
                w = [np.exp(x - mx) for x in s]
                num = sum(w[t] * V[rows[t], g] for t in range(p + 1))
                assert np.abs(got[qs[b] + i, h] - num / sum(w)).max() <= 1e-12


def test_each_row_is_decode_over_its_prefix():
    """Causal attention of the token at position p equals the decode step of
    the same sequence cut at length p + 1, with that token's query."""
    L = 45
    case, qb, qs, ref = _setup(4, "f16", [L], [L], 8, 4, 32)
    got = prefill_ref(qb, ref["k_pool"], ref["v_pool"], ref["tables"], ref["lens"], qs, "f16")
    for p in (0, 1, 15, 16, 17, 31, 44):
        want = decode_ref(qb[p:p + 1], ref["k_pool"], ref["v_pool"], ref["tables"],
                          np.array([p + 1]), "f16")
        assert np.abs(got[p] - want[0]).max() <= 1e-12


def test_invariant_under_block_placement():
    """The same tokens stored in other physical blocks give bit-identical output."""
    lens, qlens = [40, 70], [12, 70]
    case, qb, qs, ref = _setup(5, "bf16", lens, qlens, 8, 2, 32)
    a = prefill_ref(qb, ref["k_pool"], ref["v_pool"], ref["tables"], ref["lens"], qs, "bf16")
    perm = np.random.default_rng(9).permutation(ref["k_pool"].shape[0])
    kp = np.empty_like(ref["k_pool"])
    vp = np.empty_like(ref["v_pool"])
    kp[perm] = ref["k_pool"]
    vp[perm] = ref["v_pool"]
    tables = np.where(ref["tables"] >= 0, perm[np.maximum(ref["tables"], 0)], -1)
    b = prefill_ref(qb, kp, vp, tables, ref["lens"], qs, "bf16")
    assert np.array_equal(a, b)


def test_empty_chunk_rows():
    """A sequence with no query tokens contributes no rows."""
    case, qb, qs, ref = _setup(6, "bf16", [20, 30], [0, 3], 4, 4, 16)
    got = prefill_ref(qb, ref["k_pool"], ref["v_pool"], ref["tables"], ref["lens"], qs, "bf16")
    assert got.shape == (3, 4, 16) and np.isfinite(got).all()
