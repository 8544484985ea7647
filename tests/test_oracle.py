"""Pins for the CPU oracle: values fixed by the pages, by mathematics, or by a
library routine — never by the oracle itself."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (AllocatorModel, append_ref, bits_of, decode_ref, dense_ref, gather_ref,
                    k_offset, new_pools, partitioned_ref, run_case, to_f64, v_offset)
from oracle.run import oracle_sequence_out
from workloads import make_case, small_case
from workloads.configs import Case, custom_case, CONFIG_NAMES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- widening --
def test_bf16_widening_known_bits():
    # bf16 = top 16 bits of binary32: sign, 8-bit exponent (bias 127), 7 mantissa bits.
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    want = np.array([1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127,
                     0.0, -0.0])
    got = to_f64(bits, "bf16")
    assert np.array_equal(got, want)
    assert np.signbit(got[-1])
    assert math.isinf(to_f64(np.array([0x7F80], np.uint16), "bf16")[0])
    # and agrees with torch's own bf16 -> fp64 conversion
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    assert np.array_equal(t.numpy(), got)


def test_f16_f32_widening_known_bits():
    assert np.array_equal(to_f64(np.array([0x3C00, 0x0001, 0xC400], np.uint16), "f16"),
                          [1.0, 2.0 ** -24, -4.0])
    assert np.array_equal(to_f64(np.array([0x3F800000, 0x00000001], np.uint32), "f32"),
                          [1.0, 2.0 ** -149])


def test_bits_roundtrip_matches_torch_values():
    x = torch.randn(257)
    for dt, td in (("bf16", torch.bfloat16), ("f16", torch.float16), ("f32", torch.float32)):
        t = x.to(td)
        assert np.array_equal(to_f64(bits_of(t, dt), dt), t.to(torch.float64).numpy())


# ---------------------------------------------------------- worked example --
def test_worked_example_100_tokens():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_100_tokens.json")))
    prefix = g["table_prefix"]
    rest = [b for b in range(16) if b not in prefix]
    am = AllocatorModel(16, g["block_size"], prefix + rest)
    slots = am.add_seq(0, g["num_tokens"])
    table = am.tables[0]
    assert table[:3] == prefix
    assert len(table) == g["num_logical_blocks"]
    assert g["num_tokens"] - (len(table) - 1) * g["block_size"] == g["tokens_in_last_block"]
    assert am.stats()["slack_slots"] == g["slack_slots"] <= 15
    for p, s in g["position_to_slot"].items():
        assert slots[int(p)] == s


# ------------------------------------------------------------------ layout --
# Offsets enumerated by hand from the layout statement (bs = 16, x = 16 / elt):
#   K: (((b*H + h)*(D/x) + d//x)*bs + t)*x + d%x
#   V: (((b*H + h)*(bs/x) + t//x)*D + d)*x + t%x
LAYOUT_CASES = [
    # dtype, H, D, (b, h, t, d), K offset, V offset
    ("bf16", 2, 16, (1, 1, 3, 10), 922, 851),   # K: ((3*2+1)*16+3)*8+2 ; V: ((3*2+0)*16+10)*8+3
    ("bf16", 2, 16, (0, 0, 1, 0), 8, 1),        # K: (0*16+1)*8         ; V: 0*8+1
    ("bf16", 2, 16, (0, 0, 0, 8), 128, 64),     # K: ((0*2+1)*16+0)*8   ; V: (0*16+8)*8
    ("bf16", 2, 16, (2, 0, 15, 15), 1279, 1279),  # both: last element of tile (4*256 - 1 + 256)
    ("f32", 1, 8, (1, 0, 2, 5), 201, 150),      # K: ((1*2+1)*16+2)*4+1 ; V: ((1*4+0)*8+5)*4+2
    ("bf16", 2, 16, (0, 1, 4, 3), 291, 284),    # K: ((1*2+0)*16+4)*8+3 ; V: ((1*2+0)*16+3)*8+4
    ("bf16", 2, 16, (1, 0, 9, 12), 716, 737),   # K: ((2*2+1)*16+9)*8+4 ; V: ((2*2+1)*16+12)*8+1
    ("bf16", 2, 16, (0, 0, 11, 0), 88, 131),    # K: (0*16+11)*8+0      ; V: ((0*2+1)*16+0)*8+3
    ("f32", 1, 8, (0, 0, 6, 1), 25, 38),        # K: (0*16+6)*4+1       ; V: ((0*4+1)*8+1)*4+2
]


@pytest.mark.parametrize("dtype,H,D,idx,ko,vo", LAYOUT_CASES)
def test_layout_offsets_and_append(dtype, H, D, idx, ko, vo):
    b, h, t, d = idx
    x = 4 if dtype == "f32" else 8
    assert k_offset(b, h, t, d, H, D, 16, x) == ko
    assert v_offset(b, h, t, d, H, D, 16, x) == vo
    kp, vp = new_pools(4, H, D, 16, dtype)
    bd = kp.dtype
    tok = np.array([[[1000 + 100 * hh + dd for dd in range(D)] for hh in range(H)]], dtype=bd)
    append_ref(kp, vp, tok, tok + 7, [b * 16 + t], 16)
    assert kp.reshape(-1)[ko] == 1000 + 100 * h + d
    assert vp.reshape(-1)[vo] == 1000 + 100 * h + d + 7
    assert int((kp != 0).sum()) == H * D and int((vp != 0).sum()) == H * D


# ---------------------------------------------- paged == unpaged (brute force) --
def _dense_seq(case, i):
    sid, L = int(case.batch[i]), int(case.lens[i])
    rws = case.rows[sid][:L]
    return dense_ref(bits_of(case.q[i], case.dtype), bits_of(case.k_tok[rws], case.dtype),
                     bits_of(case.v_tok[rws], case.dtype), case.dtype)


def test_tiny_config_paged_equals_bruteforce():
    case = make_case("tiny_fp32")
    res = run_case(case)
    assert list(case.lens) == [1, 15, 16, 37]
    for i in range(case.num_seqs):
        np.testing.assert_allclose(res["out"][i], _dense_seq(case, i), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", [n for n in CONFIG_NAMES if n != "tiny_fp32"])
def test_small_configs_paged_equals_bruteforce(name):
    case = small_case(name)
    res = run_case(case)
    for i in range(case.num_seqs):
        ref = oracle_sequence_out(case, i)
        np.testing.assert_allclose(res["out"][i], ref, rtol=0, atol=1e-12)
    # the slow explicit-loop brute force on two sequences
    for i in (0, case.num_seqs - 1):
        np.testing.assert_allclose(res["out"][i], _dense_seq(case, i), rtol=0, atol=1e-12)


def test_torch_sdpa_fp64_matches():
    case = custom_case(7, "bf16", [40, 1, 129], 8, 2, 64)
    res = run_case(case)
    G = 4
    for i in range(case.num_seqs):
        L = int(case.lens[i])
        rws = case.rows[i][:L]
        k = torch.from_numpy(to_f64(bits_of(case.k_tok[rws], "bf16"), "bf16"))  # [L][Hkv][D]
        v = torch.from_numpy(to_f64(bits_of(case.v_tok[rws], "bf16"), "bf16"))
        q = torch.from_numpy(to_f64(bits_of(case.q[i], "bf16"), "bf16"))        # [Hq][D]
        k = k.permute(1, 0, 2).repeat_interleave(G, dim=0)[None]                 # [1][Hq][L][D]
        v = v.permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q[None, :, None, :], k, v)
        np.testing.assert_allclose(res["out"][i], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


# -------------------------------------------------------------- invariances --
def _with(case, **changes):
    d = dict(case.__dict__)
    d.update(changes)
    return Case(**d)


def test_physical_permutation_invariance_bitexact():
    case = small_case("llama3_8b_bf16")
    a = run_case(case)
    rng = np.random.default_rng(5)
    b = run_case(_with(case, free_order=rng.permutation(case.num_blocks).astype(np.int32)))
    assert not np.array_equal(a["tables"], b["tables"])
    assert np.array_equal(a["out"], b["out"])


def test_cow_shared_equals_duplicated_bitexact():
    case = small_case("cow_parallel_bf16")
    shared = run_case(case)
    assert len(shared["step_cows"]) == case.notes["parked_forks"] > 0
    dup_script = [("add", int(s), int(L) - 1) for s, L in zip(case.batch, case.lens)]
    need = sum(-(-int(L) // 16) for L in case.lens)
    dup = run_case(_with(case, script=dup_script, num_blocks=need,
                         free_order=np.arange(need, dtype=np.int32)))
    assert len(dup["step_cows"]) == 0
    assert shared["stats"]["used_blocks"] < dup["stats"]["used_blocks"]
    assert np.array_equal(shared["out"], dup["out"])


def test_gqa_identical_queries_identical_outputs():
    case = custom_case(3, "bf16", [77, 5], 8, 2, 64)
    q = case.q.clone()
    q[:, 1] = q[:, 0]          # heads 0 and 1 share KV head 0
    res = run_case(_with(case, q=q))
    assert np.array_equal(res["out"][:, 0], res["out"][:, 1])


def test_gqa_equals_mha_with_replicated_kv():
    case = custom_case(4, "f16", [50, 17, 3], 8, 2, 64)
    gqa = run_case(case)
    mha = _with(case, num_kv_heads=8, k_tok=case.k_tok.repeat_interleave(4, dim=1),
                v_tok=case.v_tok.repeat_interleave(4, dim=1))
    np.testing.assert_allclose(run_case(mha)["out"], gqa["out"], rtol=0, atol=1e-13)


# ------------------------------------------------------------- closed forms --
def _dyadic_case(seed, lens, hq=4, hkv=2, d=64):
    """fp32 case whose values are multiples of 1/256 in [-4, 4], so shifts and
    doublings used below are exact in fp32."""
    case = custom_case(seed, "f32", lens, hq, hkv, d)
    f = lambda t: torch.round(t.float().clamp(-4, 4) * 256) / 256  # noqa: E731
    return _with(case, q=f(case.q), k_tok=f(case.k_tok), v_tok=f(case.v_tok))


def test_single_token_returns_its_value_exactly():
    case = custom_case(11, "bf16", [1, 1, 1], 8, 2, 128)
    out = run_case(case)["out"]
    for i in range(3):
        v = to_f64(bits_of(case.v_tok[case.rows[i][0]], "bf16"), "bf16")   # [Hkv][D]
        assert np.array_equal(out[i], np.repeat(v, 4, axis=0))


def test_zero_query_gives_mean_of_values():
    case = _dyadic_case(12, [33, 16])
    case = _with(case, q=torch.zeros_like(case.q))
    out = run_case(case)["out"]
    for i in range(2):
        V = case.v_tok[case.rows[i]].double().numpy()          # [L][Hkv][D]
        np.testing.assert_allclose(out[i], np.repeat(V.mean(0), 2, axis=0), rtol=0, atol=1e-13)


def test_constant_values_give_that_constant():
    case = _dyadic_case(13, [40, 9])
    c = torch.round(torch.randn(case.v_tok.shape[1:]) * 64) / 64
    case = _with(case, v_tok=c.expand_as(case.v_tok).contiguous())
    out = run_case(case)["out"]
    np.testing.assert_allclose(out, np.broadcast_to(np.repeat(c.double().numpy(), 2, 0),
                                                    out.shape), rtol=0, atol=1e-13)


def test_key_shift_value_shift_and_scaling():
    case = _dyadic_case(14, [45, 18, 2])
    base = run_case(case)["out"]
    u = torch.round(torch.randn(case.k_tok.shape[1:]) * 64) / 64        # same u for every token
    shifted_k = run_case(_with(case, k_tok=case.k_tok + u))["out"]
    np.testing.assert_allclose(shifted_k, base, rtol=0, atol=1e-12)
    c = torch.round(torch.randn(case.v_tok.shape[1:]) * 64) / 64
    shifted_v = run_case(_with(case, v_tok=case.v_tok + c))["out"]
    np.testing.assert_allclose(shifted_v, base + np.repeat(c.double().numpy(), 2, 0)[None],
                               rtol=0, atol=1e-12)
    doubled = run_case(_with(case, v_tok=case.v_tok * 2))["out"]
    assert np.array_equal(doubled, 2 * base)


def test_empty_sequence_gives_zero_row():
    kp, vp = new_pools(2, 1, 64, 16, "f32")
    q = bits_of(torch.randn(1, 2, 64), "f32")
    out = decode_ref(q, kp, vp, np.full((1, 1), -1, np.int32), np.array([0]), "f32")
    assert np.array_equal(out, np.zeros((1, 2, 64)))


# ---------------------------------------------------------------- partitions --
@pytest.mark.parametrize("psize", [16, 64, 512, 4096])
def test_partitioned_merge_equals_single_pass(psize):
    case = small_case("long_context_bf16")
    res = run_case(case)
    part = partitioned_ref(bits_of(case.q, "bf16"), res["k_pool"], res["v_pool"],
                           res["tables"], res["lens"], "bf16", psize)
    np.testing.assert_allclose(part, res["out"], rtol=0, atol=1e-12)


def test_merge_partials_closed_form():
    # two partitions, one token each: the merge must give the two-token softmax average
    m = np.array([0.3, -1.2])
    l = np.array([1.0, 1.0])
    acc = np.array([[2.0, 0.0], [0.0, 4.0]])
    w = np.exp([0.3, -1.2])
    want = (w[0] * acc[0] + w[1] * acc[1]) / w.sum()
    np.testing.assert_allclose(oracle.merge_partials(m, l, acc), want, rtol=1e-15)


def test_gather_walks_table_in_logical_order():
    kp, vp = new_pools(8, 1, 8, 16, "f32")
    table = [5, 2, 7]
    toks = np.arange(40 * 8, dtype=np.uint32).reshape(40, 1, 8) + 1
    slots = [table[p // 16] * 16 + p % 16 for p in range(40)]
    append_ref(kp, vp, toks, toks, slots, 16)
    K, V = gather_ref(kp, vp, table, 40, 16)
    assert np.array_equal(K[0], toks[:, 0]) and np.array_equal(V[0], toks[:, 0])


# ------------------------------------------------- peaked-softmax closed form --
@pytest.mark.parametrize("name", ["llama3_8b_bf16", "opt13b_fp16", "cow_parallel_bf16"])
def test_position_coded_rows_are_means_of_marked_rows(name):
    """Softmax limit: scores of 0 or +-4096/sqrt(D) put weight e^-362 or less
    on every row below a head's top score, so each row of decode_ref is, to
    far below 1e-12, the plain mean of the V rows with the top score (all rows
    when q = 0).  The means are computed here by explicit set sums over the
    token rows, with no softmax and no pool."""
    from workloads.configs import position_coded
    c = position_coded(small_case(name))
    ref = run_case(c)
    G = c.num_q_heads // c.num_kv_heads
    K = c.k_tok.to(torch.float64).numpy()
    V = c.v_tok.to(torch.float64).numpy()
    q = c.q.to(torch.float64).numpy()
    for i, (sid, L) in enumerate(zip(c.batch.tolist(), c.lens.tolist())):
        rws = c.rows[sid][:L]
        for h in range(c.num_q_heads):
            g = h // G
            dots = [float(np.dot(q[i, h], K[r, g])) for r in rws]
            top = max(dots)
            chosen = [r for r, s in zip(rws, dots) if s == top]
            want = sum(V[r, g] for r in chosen) / len(chosen)
            assert np.abs(ref["out"][i, h] - want).max() < 1e-12
