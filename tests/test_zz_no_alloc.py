"""pa_decode_step_noalloc (partials in the library's fixed device array, no
allocation) against pa_decode_step with a caller workspace: bit-identical
rows and pools, and both within the oracle bars, on two calls in a row, the
second with a smaller batch."""
import numpy as np
import pytest
import torch

from oracle import bits_of
from oracle.run import oracle_sequence_out
from tests.gpu_helpers import REG_TOL, TOL, max_err, require_gpu, say
from workloads import make_case, small_case

pytestmark = pytest.mark.gpu


def _prepared(case):
    pk = require_gpu()
    dev = torch.device("cuda")
    k_tok, v_tok = case.k_tok.to(dev), case.v_tok.to(dev)
    caches = []
    for _ in range(2):
        c = pk.PagedKVCache(case.num_blocks, case.num_kv_heads, case.head_dim, k_tok.dtype, dev,
                            free_order=case.free_order, fill=float("nan"))
        c.replay(case.script, case.rows, k_tok, v_tok)
        caches.append((c, c.plan_step(case.batch)))
    nr = torch.as_tensor(case.new_rows(), device=dev)
    return caches, case.q.to(dev), k_tok.index_select(0, nr), v_tok.index_select(0, nr)


@pytest.mark.parametrize("ps", [0, 256])
def test_noalloc_step_equals_workspace_step(ps):
    pk = require_gpu()
    for case in (make_case("llama3_8b_bf16", device="cuda"), small_case("llama3_8b_bf16")):
        say(f"[no-alloc] {case.name} B={case.num_seqs} P={ps}")
        caches, q, k_new, v_new = _prepared(case)
        (c1, p1), (c2, p2) = caches
        o1 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        o2 = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda")
        pk.ops.decode_step(o1, q, c1.k_pool, c1.v_pool, k_new, v_new, p1.d_slots, p1.d_tables,
                           p1.d_lens, p1.max_context_len, partition_size=ps)
        pk.ops.decode_step_noalloc(o2, q, c2.k_pool, c2.v_pool, k_new, v_new, p2.d_slots,
                                   p2.d_tables, p2.d_lens, p2.max_context_len, partition_size=ps)
        torch.cuda.synchronize()
        a, b = o1.cpu().numpy(), o2.cpu().numpy()
        assert np.array_equal(a, b), "rows differ from the workspace step"
        assert np.array_equal(bits_of(c1.k_pool, case.dtype), bits_of(c2.k_pool, case.dtype))
        assert np.array_equal(bits_of(c1.v_pool, case.dtype), bits_of(c2.v_pool, case.dtype))
        worst = max(max_err(b[i], oracle_sequence_out(case, i)) for i in range(case.num_seqs))
        say(f"  bit-identical to pa_decode_step; max |gpu - oracle| = {worst:.3e}")
        assert worst <= TOL[case.dtype] and worst <= REG_TOL[case.dtype]
