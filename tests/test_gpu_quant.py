"""GPU parity of the quantized (8-bit) cache: the encoding append bit for bit
against the oracle's quantize_ref over every finite bf16 / fp16 value and
hand-made fp32 ties, and decode over the codes (pa_decode_quant,
pa_decode_step_quant) element by element against decode_ref on pools
poisoned with a code the append never writes."""
import numpy as np
import pytest
import torch

from oracle import bits_of, run_case
from oracle.cache import append_ref, gather_ref, new_pools
from oracle.quant import quantize_ref
from oracle.run import oracle_sequence_out
from tests.gpu_helpers import CODE_TORCH, NAN_BITS, TOL, max_err, require_gpu, run_gpu_step, say
from workloads.configs import custom_case, make_case, position_coded, quantized, small_case

pytestmark = pytest.mark.gpu
FMTS = ["fp8", "i8"]


def _append_both(fmt, src, k_vals, v_vals, k_scale, v_scale):
    """GPU pools after cache_append_quant of tokens [T][H][D] into slots 0..T-1,
    and the oracle's pools for the same writes."""
    pk = require_gpu()
    T, H, D = k_vals.shape
    N = -(-T // 16)
    kp, vp = pk.ops.new_pools(N, H, D, CODE_TORCH[fmt], "cuda",
                              fill=-128 if fmt == "i8" else float("nan"))
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    pk.ops.cache_append_quant(kp, vp, k_vals.cuda(), v_vals.cuda(), slots, k_scale, v_scale)
    torch.cuda.synchronize()
    okp, ovp = new_pools(N, H, D, 16, fmt, fill=NAN_BITS[fmt])
    append_ref(okp, ovp, quantize_ref(bits_of(k_vals, src), src, fmt, k_scale),
               quantize_ref(bits_of(v_vals, src), src, fmt, v_scale), np.arange(T), 16)
    return bits_of(kp, fmt), bits_of(vp, fmt), okp, ovp


def _as_tokens(flat: torch.Tensor, H=2, D=128):
    n = flat.numel()
    T = -(-n // (H * D))
    pad = torch.zeros(T * H * D - n, dtype=flat.dtype)
    return torch.cat([flat, pad]).reshape(T, H, D)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("scale", [1.0, 0.0371, 3.0, 1.0 / 448, 2.0 ** -6])
def test_encode_every_finite_bf16(fmt, scale):
    bits = np.arange(1 << 16, dtype=np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    vals = torch.from_numpy(bits[finite].view(np.int16).copy()).view(torch.bfloat16)
    k = _as_tokens(vals)
    v = k.flip(0).contiguous()
    say(f"[quant append] {fmt} bf16 scale={scale}: {int(finite.sum())} values")
    gk, gv, ok, ov = _append_both(fmt, "bf16", k, v, scale, scale * 0.75)
    assert np.array_equal(gk, ok), np.flatnonzero(gk.ravel() != ok.ravel())[:10]
    assert np.array_equal(gv, ov)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_every_finite_fp16(fmt):
    bits = np.arange(1 << 16, dtype=np.uint16)
    finite = (bits & 0x7C00) != 0x7C00
    vals = torch.from_numpy(bits[finite].view(np.int16).copy()).view(torch.float16)
    k = _as_tokens(vals)
    say(f"[quant append] {fmt} fp16: {int(finite.sum())} values")
    gk, gv, ok, ov = _append_both(fmt, "f16", k, k, 0.5, 1.0 / 3.0)
    assert np.array_equal(gk, ok)
    assert np.array_equal(gv, ov)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_fp32_ties_and_extremes(fmt):
    """Exact midpoints between neighbouring codes (ties to even), saturation,
    signed zeros, and random fp32 values, at scale 1 (y = x exactly)."""
    if fmt == "fp8":
        from oracle.numerics import E4M3_TABLE
        pos = torch.from_numpy(E4M3_TABLE[:0x7F].copy())
        mids = ((pos[1:] + pos[:-1]) / 2).float()
    else:
        mids = torch.arange(-127, 127, dtype=torch.float32) + 0.5
    g = torch.Generator().manual_seed(8)
    extra = torch.tensor([0.0, -0.0, 448.0, -448.0, 460.0, 464.0, 470.0, 1e6, -1e6, 126.5,
                          127.4, 127.5, 128.0, -127.5, 2.0 ** -10, -(2.0 ** -10), 1e-30])
    vals = torch.cat([mids, -mids, extra, torch.randn(40000, generator=g) * 40,
                      torch.randn(4000, generator=g) * 0.01]).float()
    k = _as_tokens(vals)
    say(f"[quant append] {fmt} fp32 ties: {vals.numel()} values")
    gk, gv, ok, ov = _append_both(fmt, "f32", k, k, 1.0, 1.0)
    assert np.array_equal(gk, ok)
    assert np.array_equal(gv, ov)


def _oracle_poisoned(case):
    return run_case(case, pool_fill=NAN_BITS[case.kv_dtype])


def _compare_full(case, ref, got, tol=TOL["bf16"]):
    plan = got["plan"]
    assert np.array_equal(plan.tables, ref["tables"])
    assert np.array_equal(plan.cows, ref["step_cows"].reshape(-1, 2))
    assert np.array_equal(got["k_pool"], ref["k_pool"]), "K pool differs"
    assert np.array_equal(got["v_pool"], ref["v_pool"]), "V pool differs"
    err = max_err(got["out"], ref["out"])
    say(f"  {case.name}: max |gpu - oracle| = {err:.3e} (tol {tol})")
    assert err <= tol


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name", ["llama3_8b_bf16", "cow_parallel_bf16", "long_context_bf16"])
@pytest.mark.parametrize("fused,ps", [(True, 0), (False, 0), (True, 64), (False, 256)])
def test_small_configs_match_oracle(fmt, name, fused, ps):
    case = quantized(small_case(name), fmt)
    say(f"[quant decode] {case.name} fused={fused} P={ps}")
    ref = _oracle_poisoned(case)
    got = run_gpu_step(case, partition_size=ps, fused=fused)
    _compare_full(case, ref, got)


EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 1023, 1025]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("hq,hkv,d,ps", [(32, 8, 128, 0), (16, 4, 64, 0), (8, 8, 128, 512),
                                         (12, 4, 128, 16), (6, 3, 64, -1), (2, 1, 128, 256),
                                         (64, 8, 128, 0), (40, 8, 64, 256), (14, 2, 128, -1),
                                         (96, 8, 128, 0), (32, 2, 64, -1), (26, 2, 128, 128)])
def test_edge_lengths_and_shapes(fmt, hq, hkv, d, ps):
    case = quantized(custom_case(61, "bf16", EDGE_LENS, hq, hkv, d, partition_size=ps,
                                 boost_prob=0.02), fmt)
    say(f"[quant edge] {fmt} Hq={hq} Hkv={hkv} D={d} P={ps}")
    ref = _oracle_poisoned(case)
    got = run_gpu_step(case)
    _compare_full(case, ref, got)


# Position-coded steps over 8-bit pools on the even split: 0 and 64 are
# codes of both formats (64 maps to the largest code), so every row is a
# mean of stored V rows and one dropped, doubled or misplaced token moves
# some element by at least 64 / L (1.6e-2 here).  The V scale 64 / 448 (or
# 64 / 127) is not exact in fp32: a decoded 64 is off by up to 3e-6, and the
# fp32 division by the row sum and the scaling add a few ulps of values near
# 64 (7.6e-6 each): 6e-5 bounds that.  The cut charges 8-bit range starts
# differently from 16-bit ones; these batches cross many range starts.
CODED_TOL_8BIT = 6e-5
SPLIT_LENS_CODED = {
    "many_short": list(np.random.default_rng(5).integers(1, 41, size=300)),
    "mixed": [33] * 7 + [4000, 1, 17, 2500],
}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("lens", list(SPLIT_LENS_CODED), ids=list(SPLIT_LENS_CODED))
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (28, 4, 64)])
def test_even_split_position_coded(fmt, lens, hq, hkv, d):
    case = quantized(position_coded(custom_case(57, "bf16", SPLIT_LENS_CODED[lens], hq, hkv, d,
                                                partition_size=-1)), fmt)
    say(f"[quant split coded] {fmt} {lens} Hq={hq} Hkv={hkv} D={d}")
    ref = _oracle_poisoned(case)
    got = run_gpu_step(case)
    _compare_full(case, ref, got, CODED_TOL_8BIT)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("ps", [0, 256])
def test_bad_inputs_give_nan_or_zero_rows(fmt, ps):
    pk = require_gpu()
    case = quantized(custom_case(62, "bf16", [40, 300, 700, 20, 33], 8, 2, 128), fmt)
    say(f"[quant errors] {fmt} P={ps}")
    got = run_gpu_step(case, partition_size=ps)
    cache, plan = got["cache"], got["plan"]
    tables = plan.d_tables.clone()
    tables[1, 5] = case.num_blocks + 7
    tables[2, 0] = -3
    lens = plan.d_lens.clone()
    lens[3] = plan.max_context_len + 1
    lens[4] = 0
    out = torch.full(got["out"].shape, 7.0, device="cuda")
    pk.ops.decode_quant(out, got["q"], cache.k_pool, cache.v_pool, tables, lens,
                        plan.max_context_len, case.k_scale, case.v_scale, partition_size=ps)
    o = out.cpu().numpy()
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all() and np.isnan(o[3]).all()
    assert np.array_equal(o[0], got["out"][0])
    assert np.array_equal(o[4], np.zeros_like(o[4]))


@pytest.mark.parametrize("fmt", FMTS)
def test_single_token_context_is_the_scaled_code(fmt):
    """L = 1: softmax weight 1, out = v_scale * code exactly (one fp32 product)."""
    case = quantized(custom_case(63, "bf16", [1, 1, 1], 8, 2, 64), fmt)
    ref = run_case(case)
    got = run_gpu_step(case)
    assert np.array_equal(got["out"].astype(np.float64),
                          ref["out"].astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("fmt", FMTS)
def test_gather_and_copy_move_codes_bit_for_bit(fmt):
    pk = require_gpu()
    case = quantized(small_case("cow_parallel_bf16"), fmt)
    ref = _oracle_poisoned(case)
    got = run_gpu_step(case)
    assert len(got["plan"].cows) > 0            # the step copied shared blocks
    cache, plan = got["cache"], got["plan"]
    kg, vg = pk.ops.gather_kv(cache.k_pool, cache.v_pool, plan.d_tables, plan.d_lens,
                              plan.max_context_len)
    kg, vg = bits_of(kg, fmt), bits_of(vg, fmt)
    for b in range(case.num_seqs):
        L = int(case.lens[b])
        K, V = gather_ref(ref["k_pool"], ref["v_pool"], ref["tables"][b], L, 16)
        assert np.array_equal(kg[b, :, :L], K) and np.array_equal(vg[b, :, :L], V)
        assert not kg[b, :, L:].any() and not vg[b, :, L:].any()


@pytest.mark.parametrize("fmt", FMTS)
def test_full_size_llama3_8b_sampled(fmt):
    """Llama-3-8B-shaped batch at full size over an 8-bit cache, in the
    bench's launch configuration; sampled rows against the oracle."""
    require_gpu()
    case = quantized(make_case("llama3_8b_bf16", device="cuda"), fmt)
    say(f"[quant full-size] {case.name}")
    ref = run_case(case, with_pools=False)
    got = run_gpu_step(case, poison=False)
    assert np.array_equal(got["plan"].tables, ref["tables"])
    rng = np.random.default_rng(17)
    picks = sorted(set([0, case.num_seqs - 1, int(np.argmax(case.lens))] +
                       [int(i) for i in rng.choice(case.num_seqs, 2, replace=False)]))
    for i in picks:
        want = oracle_sequence_out(case, i)
        err = max_err(got["out"][i], want)
        say(f"  seq {i} L={case.lens[i]}: max err {err:.3e}")
        assert err <= TOL["bf16"]
    assert not np.isnan(got["out"]).any()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("hq,hkv,ps", [(32, 8, 0), (32, 8, 256), (8, 2, -1), (8, 8, 64),
                                       (64, 8, 0), (48, 8, 256)])
def test_step_slot_cases_match_append_then_decode(fmt, hq, hkv, ps):
    """pa_decode_step_quant (new tokens encoded inside the attention and merge
    kernels) == pa_cache_append_quant then pa_decode_quant, for the table's
    slot, -1 (no write) and a slot in a block no table references."""
    pk = require_gpu()
    case = quantized(custom_case(82, "bf16", [40, 300, 700, 20, 33, 129], hq, hkv, 128,
                                 partition_size=ps), fmt)
    say(f"[quant step slots] {fmt} Hq={hq} Hkv={hkv} P={ps}")
    dev = torch.device("cuda")
    k_tok, v_tok = case.k_tok.to(dev), case.v_tok.to(dev)
    caches = []
    for _ in range(2):
        c = pk.PagedKVCache(case.num_blocks, hkv, 128, torch.bfloat16, dev,
                            free_order=case.free_order,
                            fill=-128 if fmt == "i8" else float("nan"),
                            cache_dtype=CODE_TORCH[fmt], k_scale=case.k_scale,
                            v_scale=case.v_scale)
        c.replay(case.script, case.rows, k_tok, v_tok)
        caches.append((c, c.plan_step(case.batch)))
    (c1, p1), (c2, p2) = caches
    unused = sorted(set(range(case.num_blocks)) - set(p1.tables[p1.tables >= 0].tolist()))
    slots = p1.d_slots.clone()
    slots[1] = -1
    slots[3] = unused[0] * 16 + 5
    nr = torch.as_tensor(case.new_rows(), device=dev)
    k_new, v_new = k_tok.index_select(0, nr), v_tok.index_select(0, nr)
    q = case.q.to(dev)
    o1 = torch.empty(q.shape, dtype=torch.float32, device=dev)
    o2 = torch.empty_like(o1)
    pk.ops.decode_step_quant(o1, q, c1.k_pool, c1.v_pool, k_new, v_new, slots, p1.d_tables,
                             p1.d_lens, p1.max_context_len, case.k_scale, case.v_scale,
                             partition_size=ps)
    pk.ops.cache_append_quant(c2.k_pool, c2.v_pool, k_new, v_new, slots, case.k_scale,
                              case.v_scale)
    pk.ops.decode_quant(o2, q, c2.k_pool, c2.v_pool, p2.d_tables, p2.d_lens,
                        p2.max_context_len, case.k_scale, case.v_scale, partition_size=ps)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(c1.k_pool, fmt), bits_of(c2.k_pool, fmt))
    assert np.array_equal(bits_of(c1.v_pool, fmt), bits_of(c2.v_pool, fmt))
    a, b = o1.cpu().numpy(), o2.cpu().numpy()
    keep = list(range(case.num_seqs))
    if fmt == "fp8":
        # sequences 1 and 3: their last position is never written (NaN codes)
        for i in (1, 3):
            assert np.isnan(a[i]).all() and np.isnan(b[i]).all()
        keep = [i for i in keep if i not in (1, 3)]
    assert max_err(a[keep], b[keep]) <= 1e-4


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("ps", [0, 64])
def test_every_code_value_widened_exactly(fmt, ps):
    """K and V rows made of every finite code value of the format (E4M3: the
    254 non-NaN codes, subnormals and -0 included; INT8: -127 .. 127), at
    scale 1 so that each value is its own code: decode over them against the
    oracle, which widens each code from its field layout.  A code widened to
    the wrong bf16 value moves some output by far more than the bar."""
    from dataclasses import replace
    if fmt == "fp8":
        vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
        vals = vals[~torch.isnan(vals)]
    else:
        vals = torch.arange(-127, 128, dtype=torch.float32)
    case = custom_case(64, "bf16", [300, 257, 64, 511], 32, 8, 128, partition_size=ps,
                       q_std=2.0 / float(vals.abs().max()))
    g = torch.Generator().manual_seed(65)
    R, H, D = case.k_tok.shape
    idx_k = torch.randint(0, len(vals), (R, H, D), generator=g)
    idx_v = torch.randint(0, len(vals), (R, H, D), generator=g)
    # every value appears in every (head, 64-dim tile) somewhere in K and V
    flat = torch.arange(R * H * D) % len(vals)
    idx_k.view(-1)[: len(flat)] = flat[torch.randperm(len(flat), generator=g)]
    k_tok = vals[idx_k].to(torch.bfloat16)
    v_tok = vals[idx_v].to(torch.bfloat16)
    case = replace(case, k_tok=k_tok, v_tok=v_tok, cache_dtype=fmt, k_scale=1.0, v_scale=1.0,
                   name=f"every_code_{fmt}")
    say(f"[quant every code] {fmt} P={ps}: {len(vals)} values")
    ref = _oracle_poisoned(case)
    got = run_gpu_step(case)
    _compare_full(case, ref, got)
