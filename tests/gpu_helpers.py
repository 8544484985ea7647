"""Shared helpers for the GPU tests: run one workload step through the C ABI
and collect everything the oracle comparison needs."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

# canonical NaN bit patterns torch writes for fill_(nan): the oracle pools are
# poisoned with the same bits so whole pools compare bit for bit
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0,
            # 8-bit pools: E4M3's NaN code; INT8 has no NaN, -128 is a code the
            # quantizing append never writes (it clamps to +-127)
            "fp8": 0x7F, "i8": 0x80}
CODE_TORCH = {"fp8": torch.float8_e4m3fn, "i8": torch.int8}
TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
# Regression bar of the random-value runs with 16-bit pools, kept beside the
# 1e-2 contract.  The kernels accumulate in fp32 and feed P . V with P split
# into a high and a low 16-bit part (|p - hi - lo| <= 2^-16 |p|), so each
# weight carries a relative error below 2^-16; numerator and denominator then
# move by at most that fraction of max |v| (about 6 for unit normals at these
# sizes): 1.8e-4 if every rounding had the same sign.  The roundings are
# unbiased and average out: measured on MI355X the largest decode error over
# every test, full sizes included, is 1.9e-5.  1e-4 keeps 5x of room and sits
# below what one dropped or doubled token of a 2048-token context does to a
# row (5.7e-4 in the median).
REG_TOL = {"f32": 1e-5, "f16": 1e-4, "bf16": 1e-4}
# Position-coded runs (workloads.configs.position_coded): every row is an
# exact mean of 0/64 entries, so the only error left is the final division
# and scaling (a few fp32 ulps of values below 64); one dropped, doubled or
# misplaced token moves some element by at least 64 / L >= 4.8e-4 for
# contexts up to 131072 tokens.
CODED_TOL = 2e-5


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import paged_kv_cache_212_amd as pk
    pk.lib()          # raises if the HIP library is not built
    return pk


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu_step(case, partition_size=None, poison=True, max_blocks=None, fused=True,
                 pools=True, shared=None):
    """Replays the case's set-up and runs one step on the GPU.

    Returns dict(plan=StepPlan, out=np fp32, k_pool/v_pool=np bits (only with
    ``pools``), cache=PagedKVCache).  shared=m: pa_decode_step_shared with the
    shared-prefix plan of the step (groups sharing at least m blocks).
    """
    pk = require_gpu()
    from oracle import bits_of  # test side only: stored-bit views for comparison
    dev = torch.device("cuda")
    td = case.k_tok.dtype
    cd = getattr(case, "cache_dtype", None)
    fill = (-128 if cd == "i8" else float("nan")) if poison else 0
    cache = pk.PagedKVCache(case.num_blocks, case.num_kv_heads, case.head_dim, td, dev,
                            free_order=case.free_order, fill=fill,
                            cache_dtype=CODE_TORCH.get(cd), k_scale=case.k_scale,
                            v_scale=case.v_scale)
    k_tok, v_tok = case.k_tok.to(dev), case.v_tok.to(dev)
    cache.replay(case.script, case.rows, k_tok, v_tok)
    plan = cache.plan_step(case.batch, max_blocks)
    nr = torch.as_tensor(case.new_rows(), device=dev)
    k_new, v_new = k_tok.index_select(0, nr), v_tok.index_select(0, nr)
    q = case.q.to(dev)
    ps = case.partition_size if partition_size is None else partition_size
    sp = cache.shared_plan(plan, shared) if shared else None
    out = cache.step(plan, q, k_new, v_new, partition_size=ps, fused=fused,
                     window=getattr(case, "window", 0), shared=sp)
    torch.cuda.synchronize()
    res = {"plan": plan, "out": out.cpu().numpy(), "cache": cache, "q": q, "shared": sp}
    if pools:
        res["k_pool"] = bits_of(cache.k_pool, case.kv_dtype)
        res["v_pool"] = bits_of(cache.v_pool, case.kv_dtype)
    return res


def max_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert not np.isnan(a).any(), "NaN in GPU output"
    return float(np.abs(a - b).max()) if a.size else 0.0
