"""Attention of a chunk of query tokens over a paged KV cache (prefill and
chunked prefill), in fp64.  TEST INFRASTRUCTURE ONLY (see the package header).

Sequence b holds L = lens[b] tokens in its blocks, the last n_b of which are
the chunk being processed: the prompt itself (n_b = L, prefill), a slice of a
long prompt on top of an already cached prefix (chunked prefill), or one
generated token (n_b = 1, the decode step).  Query row query_start[b] + i is
the token at position p = L - n_b + i; it attends causally, to positions
0 .. p of its own sequence, with GQA head mapping h -> h // G:

    s_t   = scale * sum_d q[row,h,d] * K_b[g,t,d]          t in [0, p]
    out   = sum_t exp(s_t - max s) * V_b[g,t,:] / sum_t exp(s_t - max s)

Sources (sections named by their headings): the prompt's tokens fill a
sequence's blocks like generated ones and attention reads them through the
block table (page 3, abeam.tech review, 「KV キャッシュマネージャ」 and
「モデル構造ではなくサービング基盤の変更」); the same review names the
prompt (prefill) phase as a separate stage whose optimisation came after the
paper (「今後注目すべき方向性」, 「限界」).  The pages give no formula for it: the
causal form above is the standard self-attention of a decoder over its own
prefix, and with n_b = 1 it is the decode step of ``decode_ref``.
"""
from __future__ import annotations

import numpy as np

from .cache import gather_ref
from .numerics import to_f64


def prefill_ref(q_bits, k_pool, v_pool, tables, lens, query_start, dtype, scale=None, bs=16):
    """q_bits [T][Hq][D] (T = query_start[-1]); pools of stored bits; tables
    [B][MB]; lens [B]; query_start [B+1] non-decreasing with
    query_start[b+1] - query_start[b] <= lens[b].

    Returns out [T][Hq][D] fp64.
    """
    T, Hq, D = q_bits.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    q = to_f64(q_bits, dtype)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    qs = np.asarray(query_start, dtype=np.int64)
    for b in range(len(lens)):
        L = int(lens[b])
        n = int(qs[b + 1] - qs[b])
        if n == 0:
            continue
        Kb, Vb = gather_ref(k_pool, v_pool, tables[b], L, bs)
        Kb, Vb = to_f64(Kb, dtype), to_f64(Vb, dtype)
        r0 = int(qs[b])
        pos = L - n + np.arange(n)            # position of each query token
        # key t is visible to the query at position p when t <= p (causal)
        visible = np.arange(L)[None, :] <= pos[:, None]          # [n][L]
        for h in range(Hq):
            g = h // G
            s = scale * (q[r0:r0 + n, h] @ Kb[g].T)                # [n][L]
            s = np.where(visible, s, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))           # 0 where not visible
            out[r0:r0 + n, h] = (w / w.sum(axis=1, keepdims=True)) @ Vb[g]
    return out
