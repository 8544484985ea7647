"""Decode attention over a paged KV cache, in fp64.

For one decode step of sequence b with context length L, query head h reads
key/value head g = h // G (G = Hq / Hkv consecutive query heads per KV head):

    s_t   = scale * sum_d q[b,h,d] * K_b[g,t,d]          t in [0, L)
    out   = sum_t exp(s_t - max s) * V_b[g,t,:] / sum_t exp(s_t - max s)

with K_b, V_b the sequence's cache reassembled in logical order through its
block table.  The pages state that paging changes only where K/V live and how
the kernel reads them, not the result (page 3, sections
「モデル構造ではなくサービング基盤の変更」 and 「よくある質問」; page 4, FAQ on
accuracy); the formula is standard scaled dot-product attention for one query.
Tokens at positions >= L never contribute; L = 0 yields a zero row.

``partitioned_ref`` splits the context into fixed-size partitions and merges
them with the log-sum-exp combine; it equals ``decode_ref`` up to fp64
rounding and pins the merge algebra the long-context path relies on.
"""
from __future__ import annotations

import numpy as np

from .cache import gather_ref
from .numerics import to_f64


def _softmax_row(s):
    m = s.max()
    e = np.exp(s - m)
    return e / e.sum()


def decode_ref(q_bits, k_pool, v_pool, tables, lens, dtype, scale=None, bs=16, q_dtype=None,
               k_scale=1.0, v_scale=1.0, window=0):
    """q_bits [B][Hq][D]; pools of stored bits; tables int [B][MB]; lens [B].

    ``dtype`` is the pools' dtype, ``q_dtype`` that of q (default: the same).
    A quantized cache ("i8"/"fp8" codes) holds K = code * k_scale and
    V = code * v_scale (scales taken as fp32); the attention is the formula
    above over those values.  ``window`` W > 0: sliding-window attention over
    the last W positions only, t in [max(0, L - W), L) (page 1, section
    「他のKVキャッシュ最適化との組み合わせ」, SWA; the span is this reading).
    Returns out [B][Hq][D] fp64.
    """
    B, Hq, D = q_bits.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    q = to_f64(q_bits, dtype if q_dtype is None else q_dtype)
    ks, vs = float(np.float32(k_scale)), float(np.float32(v_scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        first = max(0, L - window) if window else 0
        Kb, Vb = gather_ref(k_pool, v_pool, tables[b], L, bs, first)
        Kb, Vb = to_f64(Kb, dtype) * ks, to_f64(Vb, dtype) * vs
        for h in range(Hq):
            g = h // G
            s = scale * (Kb[g] @ q[b, h])            # [L]
            out[b, h] = _softmax_row(s) @ Vb[g]
    return out


def dense_ref(q_bits, k_rows_bits, v_rows_bits, dtype, scale=None):
    """Brute force for one sequence straight from its token rows (no pool, no table).

    q_bits [Hq][D]; k_rows_bits/v_rows_bits [L][Hkv][D] in logical order.
    Written as explicit sums over tokens so it shares nothing with decode_ref.
    """
    Hq, D = q_bits.shape
    L, Hkv, _ = k_rows_bits.shape
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    q = to_f64(q_bits, dtype)
    K = to_f64(k_rows_bits, dtype)
    V = to_f64(v_rows_bits, dtype)
    out = np.zeros((Hq, D), dtype=np.float64)
    if L == 0:
        return out
    for h in range(Hq):
        g = h // G
        s = np.array([scale * float(np.sum(q[h] * K[t, g])) for t in range(L)])
        w = np.exp(s - s.max())
        num = np.zeros(D)
        for t in range(L):
            num += w[t] * V[t, g]
        out[h] = num / w.sum()
    return out


def merge_partials(m, l, acc):
    """Log-sum-exp combine of per-partition (max, sum, unnormalised acc).

    m, l: [P]; acc: [P][D].  out = sum_p e^{m_p-M} acc_p / sum_p e^{m_p-M} l_p.
    """
    M = np.max(m)
    w = np.exp(m - M)
    return (w[:, None] * acc).sum(0) / (w * l).sum()


def partitioned_ref(q_bits, k_pool, v_pool, tables, lens, dtype, partition_size,
                    scale=None, bs=16):
    """Same output as decode_ref, computed partition by partition then merged."""
    B, Hq, D = q_bits.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    q = to_f64(q_bits, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        Kb, Vb = gather_ref(k_pool, v_pool, tables[b], L, bs)
        Kb, Vb = to_f64(Kb, dtype), to_f64(Vb, dtype)
        starts = list(range(0, L, partition_size))
        for h in range(Hq):
            g = h // G
            ms, ls, accs = [], [], []
            for p0 in starts:
                p1 = min(L, p0 + partition_size)
                s = scale * (Kb[g, p0:p1] @ q[b, h])
                m = s.max()
                e = np.exp(s - m)
                ms.append(m)
                ls.append(e.sum())
                accs.append(e @ Vb[g, p0:p1])
            out[b, h] = merge_partials(np.array(ms), np.array(ls), np.array(accs))
    return out
