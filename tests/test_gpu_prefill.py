"""GPU parity of pa_prefill (attention of a chunk of query tokens per sequence
over the paged cache) against the oracle's prefill_ref, element by element,
on NaN-poisoned pools (unwritten slots must never reach the output)."""
import numpy as np
import pytest
import torch

from oracle import bits_of, run_case
from oracle.prefill import prefill_ref
from tests.gpu_helpers import NAN_BITS, REG_TOL, TOL, max_err, require_gpu, run_gpu_step, say
from workloads.configs import prefill_case

pytestmark = pytest.mark.gpu


def _run(seed, dtype, lens, qlens, hq, hkv, d, max_qlen=None, tables_hook=None, **kw):
    pk = require_gpu()
    case, q, qs = prefill_case(seed, dtype, lens, qlens, hq, hkv, d, **kw)
    got = run_gpu_step(case)                       # set-up + step: all lens[b] tokens cached
    plan, cache = got["plan"], got["cache"]
    dev = torch.device("cuda")
    qd = q.to(dev)
    T = qd.shape[0]
    out = torch.full((T, hq, d), 7.0, dtype=torch.float32, device=dev)
    tables = plan.d_tables.clone()
    lens_d = plan.d_lens.clone()
    qs_d = torch.as_tensor(qs, dtype=torch.int32, device=dev)
    if tables_hook is not None:
        tables_hook(tables, lens_d, qs_d)
    mq = int(max(qlens)) if max_qlen is None else max_qlen
    pk.ops.prefill(out, qd, cache.k_pool, cache.v_pool, tables, lens_d, qs_d,
                   plan.max_context_len, mq)
    torch.cuda.synchronize()
    return case, q, qs, out.cpu().numpy()


def _oracle(case, q, qs, dtype):
    ref = run_case(case, decode=False, pool_fill=NAN_BITS[dtype])
    return prefill_ref(bits_of(q, dtype), ref["k_pool"], ref["v_pool"], ref["tables"],
                       ref["lens"], qs, dtype)


CASES = [
    # dtype, lens, qlens, hq, hkv, d
    ("bf16", [37, 16, 1, 100], [37, 16, 1, 100], 8, 2, 64),            # full prefill
    ("bf16", [300, 70, 513], [17, 64, 129], 32, 8, 128),               # chunked prefill
    ("f16", [200, 33, 5], [1, 1, 1], 8, 8, 128),                       # one token: decode
    ("f16", [15, 17, 31, 33, 255, 256, 257], [15, 1, 16, 32, 200, 255, 3], 16, 2, 64),
    ("bf16", [1024, 2000], [512, 1000], 12, 4, 128),
    ("bf16", [64, 48], [0, 48], 8, 1, 128),                             # empty chunk
]


@pytest.mark.parametrize("dtype,lens,qlens,hq,hkv,d", CASES)
def test_prefill_matches_oracle(dtype, lens, qlens, hq, hkv, d):
    say(f"[prefill] {dtype} lens={lens} qlens={qlens} Hq={hq} Hkv={hkv} D={d}")
    case, q, qs, got = _run(11, dtype, lens, qlens, hq, hkv, d)
    want = _oracle(case, q, qs, dtype)
    err = max_err(got, want)
    say(f"  max |gpu - oracle| = {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_peaked_scores_match_oracle(dtype):
    """1% of the key vectors scaled x8 (as in the long-context workload): the
    scores span a wide range, so the running max moves by large steps and the
    kernel's accumulator rescaling is exercised."""
    say(f"[prefill] peaked scores {dtype}")
    case, q, qs, got = _run(13, dtype, [1500, 700, 2048], [1500, 300, 512], 32, 8, 128,
                            boost_prob=0.01)
    want = _oracle(case, q, qs, dtype)
    err = max_err(got, want)
    say(f"  max |gpu - oracle| = {err:.3e}")
    assert err <= TOL[dtype]


def test_prefill_one_token_matches_decode():
    """A one-token chunk per sequence is the decode step: pa_prefill against
    pa_decode on the same cache and query rows."""
    pk = require_gpu()
    say("[prefill] one-token chunks vs pa_decode")
    lens = [40, 300, 17, 1]
    case, q, qs, got = _run(12, "bf16", lens, [1] * 4, 32, 8, 128)
    dec = run_gpu_step(case)
    # decode with the prefill query rows on the same cache state
    plan, cache = dec["plan"], dec["cache"]
    out = torch.empty(4, 32, 128, device="cuda")
    pk.ops.decode(out, q.to("cuda"), cache.k_pool, cache.v_pool, plan.d_tables, plan.d_lens,
                  plan.max_context_len)
    torch.cuda.synchronize()
    assert max_err(got, out.cpu().numpy()) <= 1e-5


def test_prefill_bad_inputs_give_nan_rows_or_none():
    say("[prefill] bad table entry, over-long chunk, broken query offsets")
    lens, qlens = [40, 90, 33, 20], [10, 20, 5, 4]

    def hook(tables, lens_d, qs_d):
        tables[0, 1] = 10 ** 6                  # entry outside the pool
        lens_d[1] = 10 ** 5                     # longer than the declared bound
        qs_d[3] = 99                            # sequence 2: 35 > 33 tokens of chunk...
        qs_d[4] = 39                            # ...and sequence 3: offsets out of order

    case, q, qs, got = _run(13, "bf16", lens, qlens, 8, 2, 64, tables_hook=hook)
    assert np.isnan(got[0:10]).all()                     # sequence 0
    assert np.isnan(got[10:30]).all()                    # sequence 1
    # sequences 2 (rows 30..34 by its own offsets, now 30..98: out of bounds) and
    # 3 (offsets 99 > 39): nothing written
    assert np.all(got[30:39] == 7.0)


@pytest.mark.timeout(900)
def test_prefill_full_size_every_row():
    """The bench's chunked prefill at full size (16 sequences of 2048 tokens,
    Llama-3-8B heads, the last 512 tokens as the chunk, shuffled blocks,
    poisoned pools): every query row of every head against the oracle."""
    say("[prefill] full-size chunked prefill, every row")
    B, L, n = 16, 2048, 512
    case, q, qs, got = _run(21, "bf16", [L] * B, [n] * B, 32, 8, 128, device="cuda")
    want = _oracle(case, q, qs, "bf16")
    err = max_err(got, want)
    say(f"  {B * n} query rows x 32 heads: max |gpu - oracle| = {err:.3e}")
    assert err <= REG_TOL["bf16"]
