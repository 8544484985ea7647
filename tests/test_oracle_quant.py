"""Pins for the quantized-cache oracle (oracle/quant.py and the 8-bit code
formats in oracle/numerics.py), each against something other than the
function itself: hand-decoded codes of the OCP E4M3 layout and of two's
complement bytes, torch's own float8_e4m3fn conversion (a library routine),
hand-rounded ties, closed-form error bounds of rounding, hand-enumerated
offsets of the 1-byte pool layout, and brute force over the token rows."""
import numpy as np
import pytest
import torch

from oracle import bits_of, decode_ref, run_case, to_f64
from oracle.cache import append_ref, gather_ref, new_pools
from oracle.quant import dequantize_ref, inv_scale_f32, quantize_ref, scaled_f32
from workloads.configs import custom_case, quantized, small_case


def _bf16_bits(vals):
    return bits_of(torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16), "bf16")


# -- code formats --------------------------------------------------------------

@pytest.mark.parametrize("code,val", [(0x38, 1.0), (0x40, 2.0), (0xC0, -2.0), (0x7E, 448.0),
                                      (0xFE, -448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
                                      (0x08, 2.0 ** -6), (0x39, 1.125), (0x00, 0.0)])
def test_e4m3_hand_values(code, val):
    assert to_f64(np.array([code], np.uint8), "fp8")[0] == val


def test_e4m3_special_codes():
    v = to_f64(np.array([0x80, 0x7F, 0xFF], np.uint8), "fp8")
    assert v[0] == 0.0 and np.signbit(v[0])
    assert np.isnan(v[1]) and np.isnan(v[2])


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = to_f64(codes, "fp8")
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(mine[ok], lib[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(lib[ok]))


def test_i8_codes():
    v = to_f64(np.array([0x00, 0x01, 0x7F, 0x80, 0x81, 0xFF], np.uint8), "i8")
    assert list(v) == [0, 1, 127, -128, -127, -1]


# -- quantization ----------------------------------------------------------------

def test_i8_hand_rounding():
    # scale 0.5: y = 2x; ties round to even; clamp to +-127
    x = _bf16_bits([1.0, 0.25, 0.75, 1.25, -1.25, 100.0, -100.0, 0.0, 3.0])
    got = quantize_ref(x, "bf16", "i8", 0.5).view(np.int8)
    assert list(got) == [2, 0, 2, 2, -2, 127, -127, 0, 6]


def test_reciprocal_scale_is_rounded_to_fp32():
    # 1/0.1f rounds to exactly 10.0f; 1/3f rounds to 0x3EAAAAAB
    assert inv_scale_f32(0.1) == np.float32(10.0)
    assert inv_scale_f32(3.0).view(np.uint32) == 0x3EAAAAAB
    # y = fp32(x * inv): 1 * fp32(1/3) stays the rounded reciprocal
    y = scaled_f32(_bf16_bits([1.0]), "bf16", 3.0)
    assert y[0] == np.float32(1.0) / np.float32(3.0)


@pytest.mark.parametrize("y,code", [
    (1.0625, 0x38),            # between 1.0 (0x38) and 1.125 (0x39): tie, even code
    (1.1875, 0x3A),            # between 1.125 and 1.25: tie, even code 0x3A
    (1.06, 0x38), (1.07, 0x39), (1.1, 0x39),
    (2.0 ** -10, 0x00),        # half the smallest subnormal: tie with zero
    (-(2.0 ** -10), 0x80),     # ... keeps its sign
    (3 * 2.0 ** -10, 0x02),    # between 2^-9 (0x01) and 2^-8 (0x02): tie, even
    (448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE),
    (-0.0, 0x80), (240.0, 0x77), (248.0, 0x78),   # 240 = 1.875*2^7; 248 ties 240/256
])
def test_e4m3_hand_rounding(y, code):
    # scale 1: the product is y itself (y is exact in bf16 or fp32 here)
    x = np.array([np.float32(y)]).view(np.uint32)
    assert quantize_ref(x, "f32", "fp8", 1.0)[0] == code


def test_e4m3_rounding_matches_torch_in_range():
    """torch's float8_e4m3fn cast (round to nearest even) of clamp(y, +-448)."""
    g = torch.Generator().manual_seed(3)
    y = torch.cat([torch.randn(20000, generator=g) * s for s in (0.01, 1.0, 30.0, 300.0)])
    mids = (torch.from_numpy(to_f64(np.arange(0x7E, dtype=np.uint8), "fp8")) +
            torch.from_numpy(to_f64(np.arange(1, 0x7F, dtype=np.uint8), "fp8"))) / 2
    y = torch.cat([y, mids.float(), -mids.float()])
    xb = y.numpy().view(np.uint32)
    mine = quantize_ref(xb, "f32", "fp8", 1.0)
    lib = y.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, lib)


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
def test_rounding_error_bounds(fmt):
    """|code*s - x| <= s/2 (i8, in range) and <= 2^-4 |x| (fp8, normal range):
    half a step of the grid the value lands on."""
    g = torch.Generator().manual_seed(4)
    x = (torch.randn(50000, generator=g) * 2).to(torch.bfloat16)
    xb = bits_of(x, "bf16")
    xv = to_f64(xb, "bf16")
    s = float(np.abs(xv).max()) / (127.0 if fmt == "i8" else 448.0)
    s32 = float(np.float32(s))
    back = dequantize_ref(quantize_ref(xb, "bf16", fmt, s), fmt, s)
    err = np.abs(back - xv)
    if fmt == "i8":
        assert (err <= 0.5 * s32 * (1 + 1e-6)).all()
    else:
        normal = np.abs(xv) / s32 >= 2.0 ** -6
        assert (err[normal] <= 2.0 ** -4 * np.abs(xv[normal]) * (1 + 1e-6)).all()
        assert (err[~normal] <= 2.0 ** -10 * s32 * (1 + 1e-6)).all()


# -- 1-byte pool layout ----------------------------------------------------------

def test_one_byte_pool_offsets_by_hand():
    """x = 16: K (b, h, t, d) at (((b*H + h)*(D/16) + d//16)*16 + t)*16 + d%16,
    V at (((b*H + h)*1 + 0)*D + d)*16 + t; offsets enumerated by hand."""
    H, D = 2, 32
    kp, vp = new_pools(3, H, D, 16, "fp8")
    assert kp.shape == (3, H, 2, 16, 16) and vp.shape == (3, H, 1, D, 16)
    k_new = np.zeros((1, H, D), np.uint8)
    v_new = np.zeros((1, H, D), np.uint8)
    k_new[0, 1, 17] = 0xAB
    v_new[0, 1, 17] = 0xCD
    append_ref(kp, vp, k_new, v_new, [2 * 16 + 3], 16)     # block 2, token 3
    # K: (((2*2 + 1)*2 + 1)*16 + 3)*16 + 1 = 11*16*16 + 3*16 + 1 = 2865
    assert np.flatnonzero(kp.ravel()).tolist() == [2865]
    # V: ((2*2 + 1)*32 + 17)*16 + 3 = 177*16 + 3 = 2835
    assert np.flatnonzero(vp.ravel()).tolist() == [2835]
    K, V = gather_ref(kp, vp, np.array([0, 2]), 20, 16)
    assert K[1, 19, 17] == 0xAB and V[1, 19, 17] == 0xCD


# -- attention over a quantized cache --------------------------------------------

@pytest.mark.parametrize("fmt", ["i8", "fp8"])
def test_quantized_decode_brute_force(fmt):
    """Explicit token loops over the dequantized token rows (no pool, no table)."""
    case = quantized(custom_case(7, "bf16", [5, 19, 33], 4, 2, 16), fmt)
    ref = run_case(case)
    q = to_f64(bits_of(case.q, "bf16"), "bf16")
    K = dequantize_ref(quantize_ref(bits_of(case.k_tok, "bf16"), "bf16", fmt, case.k_scale),
                       fmt, case.k_scale)
    V = dequantize_ref(quantize_ref(bits_of(case.v_tok, "bf16"), "bf16", fmt, case.v_scale),
                       fmt, case.v_scale)
    for b, L in enumerate(case.lens):
        rows = case.rows[case.batch[b]][:L]
        for h in range(4):
            s = [0.25 * sum(q[b, h, e] * K[r, h // 2, e] for e in range(16)) for r in rows]
            w = np.exp(np.array(s) - max(s))
            want = sum(w[t] * V[rows[t], h // 2] for t in range(L)) / w.sum()
            assert np.abs(ref["out"][b, h] - want).max() <= 1e-12


@pytest.mark.parametrize("fmt", ["i8", "fp8"])
def test_quantized_pools_hold_codes_of_the_rows(fmt):
    case = quantized(small_case("cow_parallel_bf16"), fmt)
    ref = run_case(case, decode=False)
    assert ref["k_pool"].dtype == np.uint8
    for b in range(case.num_seqs):
        L = int(case.lens[b])
        K, V = gather_ref(ref["k_pool"], ref["v_pool"], ref["tables"][b], L, 16)
        rows = case.rows[case.batch[b]][:L]
        kc = quantize_ref(bits_of(case.k_tok[rows], "bf16"), "bf16", fmt, case.k_scale)
        vc = quantize_ref(bits_of(case.v_tok[rows], "bf16"), "bf16", fmt, case.v_scale)
        assert np.array_equal(K, kc.transpose(1, 0, 2))
        assert np.array_equal(V, vc.transpose(1, 0, 2))


@pytest.mark.parametrize("fmt,bound", [("i8", 0.03), ("fp8", 0.25)])
def test_quantized_decode_stays_near_full_precision(fmt, bound):
    """The accuracy side of the trade-off: on unit-normal K/V the outputs over
    the 8-bit cache stay within a small absolute distance of the bf16 ones
    (E4M3 keeps 3 mantissa bits: up to 1/16 relative per element, so about
    0.2 on the largest |V| of about 4; a dropped scale would be off by orders
    of magnitude)."""
    base = small_case("llama3_8b_bf16")
    full = run_case(base)["out"]
    q8 = run_case(quantized(base, fmt))["out"]
    err = np.abs(q8 - full).max()
    assert 1e-4 < err <= bound, err
