"""Paged KV pools: layout, token append, block copy, and the table walk.

Layout (a choice of this library; the pages describe blocks and tables but no
byte layout).  With ``x = 16 / element_bytes`` (4 for fp32, 8 for fp16/bf16,
16 for the 8-bit code formats):

* K pool: ``[num_blocks][num_kv_heads][head_dim / x][block_size][x]`` —
  element (block b, head h, in-block token t, dim d) sits at
  ``(((b*H + h)*(D/x) + d//x)*bs + t)*x + d%x``;
* V pool: ``[num_blocks][num_kv_heads][block_size / x][head_dim][x]`` —
  element (b, h, t, d) sits at ``(((b*H + h)*(bs/x) + t//x)*D + d)*x + t%x``
  (each dim row holds x consecutive tokens).

A token at logical position p of a sequence lives in physical block
``table[p // bs]`` at in-block offset ``p % bs`` (page 1, section
「PagedAttentionの解決策」; page 3, section 「用語解説」, block table entry).
Pools here hold raw stored bits (uint16 for fp16/bf16, uint32 for fp32, uint8
for the 8-bit codes of a quantized cache; see quant.py for how codes are made).
"""
from __future__ import annotations

import numpy as np

from .numerics import bits_dtype


def x_of(dtype: str) -> int:
    """Elements per 16 bytes."""
    return 16 // np.dtype(bits_dtype(dtype)).itemsize


def k_offset(b, h, t, d, H, D, bs, x):
    """Flat element index of K(b, h, t, d) in the K pool."""
    return (((b * H + h) * (D // x) + d // x) * bs + t) * x + d % x


def v_offset(b, h, t, d, H, D, bs, x):
    """Flat element index of V(b, h, t, d) in the V pool."""
    return (((b * H + h) * (bs // x) + t // x) * D + d) * x + t % x


def new_pools(num_blocks, H, D, bs, dtype, fill=0):
    x = x_of(dtype)
    bd = bits_dtype(dtype)
    k = np.full((num_blocks, H, D // x, bs, x), fill, dtype=bd)
    v = np.full((num_blocks, H, bs // x, D, x), fill, dtype=bd)
    return k, v


def _k_token(k_pool, b, t):
    """[H][D] view order of K for in-block token t of block b."""
    H, Dx, bs, x = k_pool.shape[1:]
    return k_pool[b, :, :, t, :].reshape(H, Dx * x)


def append_ref(k_pool, v_pool, k_new_bits, v_new_bits, slots, bs):
    """Write token i's K/V (all heads) into slot ``slots[i]``; slot -1 skips.

    k_new_bits/v_new_bits: [T][H][D] stored bits.  Pure bit moves.
    """
    H, Dx, _, x = k_pool.shape[1:]
    D = Dx * x
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        b, t = int(s) // bs, int(s) % bs
        k_pool[b, :, :, t, :] = k_new_bits[i].reshape(H, Dx, x)
        v_pool[b, :, t // x, :, t % x] = v_new_bits[i].reshape(H, D)


def copy_ref(k_pool, v_pool, pairs):
    """For each (src, dst) in order: whole block dst := block src, K and V, all heads."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]


def gather_ref(k_pool, v_pool, table, L, bs, first=0):
    """Logically contiguous K and V of positions [first, L) of one sequence:
    two arrays [H][L - first][D] of bits (every block used must be in the table)."""
    H, Dx, _, x = k_pool.shape[1:]
    D = Dx * x
    pos = np.arange(first, L, dtype=np.int64)
    L = L - first
    blk = np.asarray(table, dtype=np.int64)[pos // bs]     # physical block of position p
    if (blk < 0).any():
        raise ValueError("position reached through a released table entry")
    off = pos % bs                                           # token inside that block
    K = k_pool[blk, :, :, off, :]                            # [L][H][D/x][x]
    V = v_pool[blk, :, off // x, :, off % x]                 # [L][H][D]
    K = np.ascontiguousarray(K.reshape(L, H, D).transpose(1, 0, 2))
    V = np.ascontiguousarray(V.transpose(1, 0, 2))
    return K, V
