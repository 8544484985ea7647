"""pa_cache_append and pa_cache_append_quant over the slot patterns that
decide between whole-chunk and element-wise writes: runs that fill whole
token groups (a prompt, a prefill chunk), runs that start or end inside a
group, reversed and interleaved runs, gaps and skipped slots.  Pools are
NaN-poisoned and compared bit for bit with the oracle's append (page 3,
abeam.tech review, section 「KV キャッシュマネージャ」: new tokens fill the
sequence's last block), so a whole-chunk write that touched a slot it should
not have shows up."""
import numpy as np
import pytest
import torch

from oracle import append_ref, bits_of, new_pools
from tests.gpu_helpers import NAN_BITS, require_gpu, say

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
NB = 64


def _patterns():
    r = np.random.default_rng(5)
    run = lambda a, n: list(range(a, a + n))  # noqa: E731
    perm = r.permutation(NB)
    return {
        "prompt_512": run(16 * 7, 512),                 # whole blocks, block-aligned
        "mid_group_start": run(16 * 3 + 3, 100),        # starts and ends inside groups
        "reversed": run(16 * 5, 40)[::-1],              # right slots, wrong order
        "two_interleaved": [x for p in zip(run(16 * 9, 48), run(16 * 20 + 5, 48)) for x in p],
        "gap_in_group": run(16 * 11, 5) + [-1] + run(16 * 11 + 6, 30),
        "skipped_inside": run(16 * 30, 7) + [10**9] + run(16 * 30 + 8, 24),
        "shuffled_blocks": [16 * int(b) + t for b in perm[:6] for t in range(16)],
        "one_token": [16 * 40 + 9],
        "group_cut_by_end": run(16 * 41, 13),
    }


PATTERNS = _patterns()


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("pattern", list(PATTERNS))
def test_append_patterns_bit_exact(dtype, pattern):
    pk = require_gpu()
    slots = PATTERNS[pattern]
    H, D = 4, 128 if dtype != "f32" else 64
    say(f"[append] {pattern} {dtype} T={len(slots)}")
    k, v = pk.ops.new_pools(NB, H, D, TORCH[dtype], "cuda", fill=float("nan"))
    g = torch.Generator().manual_seed(len(slots))
    kn = torch.randn(len(slots), H, D, generator=g).to(TORCH[dtype]).cuda()
    vn = torch.randn(len(slots), H, D, generator=g).to(TORCH[dtype]).cuda()
    pk.ops.cache_append(k, v, kn, vn, torch.tensor(slots, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    kp, vp = new_pools(NB, H, D, 16, dtype, fill=NAN_BITS[dtype])
    ok = [s if 0 <= s < NB * 16 else -1 for s in slots]
    append_ref(kp, vp, bits_of(kn, dtype), bits_of(vn, dtype), ok, 16)
    assert np.array_equal(bits_of(k, dtype), kp), "K pool"
    assert np.array_equal(bits_of(v, dtype), vp), "V pool"


@pytest.mark.parametrize("cache_dtype", ["fp8", "i8"])
@pytest.mark.parametrize("pattern", ["prompt_512", "mid_group_start", "reversed", "gap_in_group",
                                     "shuffled_blocks", "group_cut_by_end"])
def test_quant_append_one_call_equals_token_by_token(cache_dtype, pattern):
    """The quantizing append in one call (whole blocks of 16 codes written as
    whole chunks) equals the same tokens appended one call per token (every
    write element-wise), code for code."""
    pk = require_gpu()
    slots = PATTERNS[pattern]
    H, D = 4, 128
    cd = {"fp8": torch.float8_e4m3fn, "i8": torch.int8}[cache_dtype]
    say(f"[append quant] {pattern} {cache_dtype}")
    g = torch.Generator().manual_seed(3)
    kn = torch.randn(len(slots), H, D, generator=g).to(torch.bfloat16).cuda()
    vn = torch.randn(len(slots), H, D, generator=g).to(torch.bfloat16).cuda()
    st = torch.tensor(slots, dtype=torch.int64, device="cuda")
    pools = []
    for per_token in (False, True):
        k, v = pk.ops.new_pools(NB, H, D, cd, "cuda", fill=-128 if cache_dtype == "i8" else float("nan"))
        if per_token:
            for i in range(len(slots)):
                pk.ops.cache_append_quant(k, v, kn[i:i + 1], vn[i:i + 1], st[i:i + 1], 0.05, 0.04)
        else:
            pk.ops.cache_append_quant(k, v, kn, vn, st, 0.05, 0.04)
        torch.cuda.synchronize()
        pools.append((bits_of(k, cache_dtype), bits_of(v, cache_dtype)))
    assert np.array_equal(pools[0][0], pools[1][0]), "K codes"
    assert np.array_equal(pools[0][1], pools[1][1]), "V codes"


def test_raw_byte_append_whole_blocks():
    """8-bit pools through the raw byte append (16 codes per chunk): a whole
    block appended in order, beside a partial one, bit for bit."""
    pk = require_gpu()
    H, D = 2, 64
    slots = list(range(16 * 4, 16 * 6)) + list(range(16 * 8 + 2, 16 * 8 + 9))
    k, v = pk.ops.new_pools(NB, H, D, torch.int8, "cuda", fill=-128)
    g = torch.Generator().manual_seed(9)
    kn = torch.randint(-127, 128, (len(slots), H, D), generator=g, dtype=torch.int8).cuda()
    vn = torch.randint(-127, 128, (len(slots), H, D), generator=g, dtype=torch.int8).cuda()
    pk.ops.cache_append(k, v, kn, vn, torch.tensor(slots, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    kp, vp = new_pools(NB, H, D, 16, "i8", fill=NAN_BITS["i8"])
    append_ref(kp, vp, bits_of(kn, "i8"), bits_of(vn, "i8"), slots, 16)
    assert np.array_equal(bits_of(k, "i8"), kp) and np.array_equal(bits_of(v, "i8"), vp)
