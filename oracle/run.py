"""One decode step of a workload, end to end on the oracle side.

Replays the set-up script on ``AllocatorModel``, fills the pools with the
token rows, then performs the step: reserve one slot per batch sequence
(copy-on-write pairs included), copy the pairs' blocks, write the new tokens,
and attend.  The order copy -> append -> attend follows from the pages: a
shared block is duplicated before the write that needs it (page 3, section
「並列サンプリングやビームサーチでの共有」), and the new token's key/value are
part of the context it attends to (the context length counts it).
"""
from __future__ import annotations

import numpy as np
import torch

from .allocator import AllocatorModel
from .attention import decode_ref
from .cache import append_ref, copy_ref, new_pools
from .numerics import bits_of, to_f64
from .quant import dequantize_ref, quantize_ref


def run_script(am: AllocatorModel, script, rows, on_write=None, on_copy=None):
    """Replay set-up ops; report each (slots, token rows) write and CoW pairs."""
    for op in script:
        kind = op[0]
        if kind == "add":
            _, sid, n = op
            slots = am.add_seq(sid, n)
            if on_write is not None and n:
                on_write(slots, rows[sid][:n])
        elif kind == "extend":
            _, sid, n = op
            start = am.seq_len(sid)
            slots, cows = am.extend(sid, n)
            if on_copy is not None and len(cows):
                on_copy(cows)
            if on_write is not None and n:
                on_write(slots, rows[sid][start:start + n])
        elif kind == "fork":
            am.fork(op[1], op[2])
        elif kind == "free":
            am.free_seq(op[1])
        elif kind == "release":
            am.release_before(op[1], op[2])
        elif kind == "reorder":
            am.reorder(op[1], op[2], op[3])
        else:
            raise ValueError(op)


def run_case(case, with_pools=True, decode=True, pool_fill=0):
    """Oracle results for one decode step.

    Returns a dict with tables, lens, step slots, step CoW pairs, and (when
    requested) the final pools (stored bits) and the fp64 output [B][Hq][D].
    ``pool_fill`` is the bit pattern unused pool slots start with.
    """
    am = AllocatorModel(case.num_blocks, case.block_size, case.free_order)
    res = {}
    cd = getattr(case, "cache_dtype", None)
    if with_pools:
        kp, vp = new_pools(case.num_blocks, case.num_kv_heads, case.head_dim, case.block_size,
                           cd or case.dtype, fill=pool_fill)
        kb = bits_of(case.k_tok, case.dtype)
        vb = bits_of(case.v_tok, case.dtype)
        if cd is not None:
            # a quantized cache stores the codes of the token rows
            kb = quantize_ref(kb, case.dtype, cd, case.k_scale)
            vb = quantize_ref(vb, case.dtype, cd, case.v_scale)

        def on_write(slots, rws):
            append_ref(kp, vp, kb[rws], vb[rws], slots, case.block_size)

        def on_copy(pairs):
            copy_ref(kp, vp, pairs)
    else:
        on_write = on_copy = None
    run_script(am, case.script, case.rows, on_write, on_copy)
    res["setup_stats"] = am.stats()
    slots, cows = am.append_slots(case.batch)
    res["step_slots"], res["step_cows"] = slots, cows
    if with_pools:
        copy_ref(kp, vp, cows)
        nr = case.new_rows()
        append_ref(kp, vp, kb[nr], vb[nr], slots, case.block_size)
    mb = max(1, max(-(-int(L) // case.block_size) for L in case.lens))
    tables, lens = am.block_tables(case.batch, mb)
    assert np.array_equal(lens, case.lens)
    res["tables"], res["lens"], res["stats"] = tables, lens, am.stats()
    res["allocator"] = am
    if with_pools:
        res["k_pool"], res["v_pool"] = kp, vp
        if decode:
            res["out"] = decode_ref(bits_of(case.q, case.dtype), kp, vp, tables, lens,
                                    cd or case.dtype, case.scale, case.block_size,
                                    q_dtype=case.dtype, k_scale=case.k_scale,
                                    v_scale=case.v_scale, window=getattr(case, "window", 0))
    return res


def oracle_sequence_out(case, i):
    """fp64 output [Hq][D] for batch entry i, straight from its token rows.

    Used for sampled checks at full size: no pool and no table, only the
    sequence's K/V in logical order and the attention definition.
    """
    sid, L = int(case.batch[i]), int(case.lens[i])
    Hq, D = case.num_q_heads, case.head_dim
    if L == 0:
        return np.zeros((Hq, D))
    W = getattr(case, "window", 0)
    rws = case.rows[sid][max(0, L - W) if W else 0:L]     # a window keeps the last W
    idx = torch.as_tensor(rws, device=case.k_tok.device)
    K = to_f64(bits_of(case.k_tok.index_select(0, idx), case.dtype), case.dtype)  # [L][Hkv][D]
    V = to_f64(bits_of(case.v_tok.index_select(0, idx), case.dtype), case.dtype)
    cd = getattr(case, "cache_dtype", None)
    if cd is not None:
        K = dequantize_ref(quantize_ref(bits_of(case.k_tok.index_select(0, idx), case.dtype),
                                        case.dtype, cd, case.k_scale), cd, case.k_scale)
        V = dequantize_ref(quantize_ref(bits_of(case.v_tok.index_select(0, idx), case.dtype),
                                        case.dtype, cd, case.v_scale), cd, case.v_scale)
    q = to_f64(bits_of(case.q[i], case.dtype), case.dtype)                         # [Hq][D]
    G = Hq // case.num_kv_heads
    out = np.empty((Hq, D))
    for h in range(Hq):
        s = case.scale * (K[:, h // G, :] @ q[h])
        w = np.exp(s - s.max())
        out[h] = (w @ V[:, h // G, :]) / w.sum()
    return out
