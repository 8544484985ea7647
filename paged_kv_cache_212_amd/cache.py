"""A paged KV cache on one GPU: device pools plus the host block manager, and
one decode step through the library (reserve -> copy-on-write -> append ->
attend)."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import ops
from .block_manager import BlockManager

BLOCK_SIZE = ops.BLOCK_SIZE


@dataclass
class StepPlan:
    """Host-side reservation for one decode step, with device copies of its arrays."""
    seq_ids: np.ndarray
    slots: np.ndarray          # int64 [B]
    cows: np.ndarray           # int32 [n][2]
    tables: np.ndarray         # int32 [B][max_blocks]
    lens: np.ndarray           # int32 [B]
    max_context_len: int
    d_slots: torch.Tensor
    d_cows: torch.Tensor
    d_tables: torch.Tensor
    d_lens: torch.Tensor


class PagedKVCache:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 device="cuda", free_order=None, fill=None, cache_dtype=None, k_scale=1.0,
                 v_scale=1.0):
        """dtype: the dtype of the K/V rows written and of q.  cache_dtype
        (torch.float8_e4m3fn or torch.int8): a quantized cache whose pools hold
        codes with K = code * k_scale, V = code * v_scale (q, k/v rows: bf16)."""
        self.bm = BlockManager(num_blocks, BLOCK_SIZE, free_order)
        self._table_cap = 1          # table row length tried first by plan_step
        if cache_dtype is not None and cache_dtype not in ops.CODE_DTYPES:
            raise ValueError("cache_dtype must be torch.float8_e4m3fn or torch.int8")
        self.cache_dtype = cache_dtype
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.k_pool, self.v_pool = ops.new_pools(num_blocks, num_kv_heads, head_dim,
                                                 cache_dtype or dtype, device, fill)
        self.num_blocks, self.num_kv_heads, self.head_dim = num_blocks, num_kv_heads, head_dim
        self.dtype, self.device = dtype, torch.device(device)

    def _d(self, a: np.ndarray) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.device)

    # -- sequence set-up ----------------------------------------------------
    def write(self, slots: np.ndarray, k: torch.Tensor, v: torch.Tensor):
        if not len(slots):
            return
        if self.cache_dtype is not None:
            ops.cache_append_quant(self.k_pool, self.v_pool, k.contiguous(), v.contiguous(),
                                   self._d(slots.astype(np.int64)), self.k_scale, self.v_scale)
        else:
            ops.cache_append(self.k_pool, self.v_pool, k.contiguous(), v.contiguous(),
                             self._d(slots.astype(np.int64)))

    def copy(self, pairs: np.ndarray):
        if len(pairs):
            ops.copy_blocks(self.k_pool, self.v_pool, self._d(pairs.astype(np.int32)))

    def add_seq(self, seq_id: int, k: torch.Tensor, v: torch.Tensor):
        slots = self.bm.add_seq(seq_id, k.shape[0])
        self.write(slots, k, v)
        return slots

    def extend(self, seq_id: int, k: torch.Tensor, v: torch.Tensor):
        slots, cows = self.bm.extend(seq_id, k.shape[0])
        self.copy(cows)
        self.write(slots, k, v)
        return slots, cows

    def fork(self, parent: int, child: int):
        self.bm.fork(parent, child)

    def free(self, seq_id: int):
        self.bm.free_seq(seq_id)

    def replay(self, script, rows, k_tok: torch.Tensor, v_tok: torch.Tensor):
        """Runs set-up ops ("add", sid, n) / ("extend", sid, n) / ("fork", p, c) /
        ("free", sid) / ("release", sid, first_pos) / ("reorder", old, new,
        parents); written tokens are
        rows[sid][pos] of k_tok / v_tok."""
        for op in script:
            if op[0] == "add":
                _, sid, n = op
                idx = torch.as_tensor(rows[sid][:n], device=k_tok.device)
                self.add_seq(sid, k_tok.index_select(0, idx), v_tok.index_select(0, idx))
            elif op[0] == "extend":
                _, sid, n = op
                start = self.bm.seq_len(sid)
                idx = torch.as_tensor(rows[sid][start:start + n], device=k_tok.device)
                self.extend(sid, k_tok.index_select(0, idx), v_tok.index_select(0, idx))
            elif op[0] == "fork":
                self.fork(op[1], op[2])
            elif op[0] == "free":
                self.free(op[1])
            elif op[0] == "release":
                self.bm.release_before(op[1], op[2])
            elif op[0] == "reorder":
                self.bm.reorder(op[1], op[2], op[3])
            else:
                raise ValueError(op)

    # -- decode step ----------------------------------------------------------
    def plan_step(self, seq_ids, max_blocks: int | None = None) -> StepPlan:
        """Reserve one position per sequence and export the tables (host work)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        if max_blocks is None:
            # one call: reserve, then export tables as long as the longest
            slots, cows, tables, lens = self.bm.step(ids, self._table_cap)
            self._table_cap = max(self._table_cap, tables.shape[1])
        else:
            slots, cows = self.bm.append_slots(ids)
            tables, lens = self.bm.block_tables(ids, max_blocks)
        return StepPlan(ids, slots, cows, tables, lens, int(lens.max(initial=0)),
                        self._d(slots), self._d(cows.reshape(-1, 2)), self._d(tables),
                        self._d(lens))

    def shared_plan(self, plan: StepPlan, min_shared_blocks: int = 4):
        """Groups of the step's sequences that share a prefix of blocks
        (pa_shared_prefix_plan on the step's tables), on the device:
        (prefix_len, group_rows, group_start, max_group)."""
        pre, rows, start, mg = ops.shared_prefix_plan(plan.tables, plan.lens, min_shared_blocks)
        return self._d(pre), self._d(rows), self._d(start), mg

    def step(self, plan: StepPlan, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
             out: torch.Tensor | None = None, scale=None, partition_size: int = 0,
             workspace=None, stream=None, fused=True, window: int = 0, shared=None):
        """Copy-on-write, append the new tokens, then decode attention (all on device).

        fused: True -> one pa_decode_step call; "phased" -> pa_decode_step_partial
        then pa_decode_step_merge; False -> pa_cache_append then pa_decode.  A
        quantized cache: pa_decode_step_quant (fused) or pa_cache_append_quant
        then pa_decode_quant (False).  window > 0: sliding-window attention
        (pa_decode_step_window, or pa_cache_append then pa_decode_window).
        shared: a shared_plan(...) result: pa_decode_step_shared, each shared
        prefix attended once per group (fp16/bf16 pools, fused step)."""
        if plan.cows.shape[0]:
            ops.copy_blocks(self.k_pool, self.v_pool, plan.d_cows, stream)
        if out is None:
            # from the launch stream's pool of the caching allocator: memory
            # freed by work on another stream is not handed to this launch
            # before that work is done
            if stream is None:
                out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
            else:
                with torch.cuda.stream(stream):
                    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if shared is not None:
            if window or self.cache_dtype is not None or fused is not True:
                raise ValueError("shared prefixes take the fused step over fp16/bf16 pools")
            pre, rows, start, mg = shared
            ops.decode_step_shared(out, q, self.k_pool, self.v_pool, k_new, v_new, plan.d_slots,
                                   plan.d_tables, plan.d_lens, plan.max_context_len, pre, rows,
                                   start, mg, scale, workspace, stream)
            return out
        if window:
            # sliding window: fused step, or append then windowed decode
            if self.cache_dtype is not None:
                raise ValueError("a sliding window takes fp32/fp16/bf16 pools")
            if fused:
                ops.decode_step(out, q, self.k_pool, self.v_pool, k_new, v_new, plan.d_slots,
                                plan.d_tables, plan.d_lens, plan.max_context_len, scale,
                                partition_size, workspace, stream, window=window)
            else:
                ops.cache_append(self.k_pool, self.v_pool, k_new, v_new, plan.d_slots, stream)
                ops.decode(out, q, self.k_pool, self.v_pool, plan.d_tables, plan.d_lens,
                           plan.max_context_len, scale, partition_size, workspace, stream,
                           window=window)
            return out
        if self.cache_dtype is not None:
            if fused:
                ops.decode_step_quant(out, q, self.k_pool, self.v_pool, k_new, v_new,
                                      plan.d_slots, plan.d_tables, plan.d_lens,
                                      plan.max_context_len, self.k_scale, self.v_scale, scale,
                                      partition_size, workspace, stream)
            else:
                ops.cache_append_quant(self.k_pool, self.v_pool, k_new, v_new, plan.d_slots,
                                       self.k_scale, self.v_scale, stream)
                ops.decode_quant(out, q, self.k_pool, self.v_pool, plan.d_tables, plan.d_lens,
                                 plan.max_context_len, self.k_scale, self.v_scale, scale,
                                 partition_size, workspace, stream)
            return out
        if fused == "phased":
            B, Hq, D = q.shape
            if workspace is None:
                workspace = ops.decode_workspace(B, Hq, self.num_kv_heads, D,
                                                 plan.max_context_len, partition_size, q.dtype,
                                                 q.device, stream)
            ops.decode_step(out, q, self.k_pool, self.v_pool, k_new, v_new, plan.d_slots,
                            plan.d_tables, plan.d_lens, plan.max_context_len, scale,
                            partition_size, workspace, stream, phase="partial")
            ops.decode_step(out, q, self.k_pool, self.v_pool, k_new, v_new, plan.d_slots,
                            plan.d_tables, plan.d_lens, plan.max_context_len, scale,
                            partition_size, workspace, stream, phase="merge")
        elif fused:
            ops.decode_step(out, q, self.k_pool, self.v_pool, k_new, v_new, plan.d_slots,
                            plan.d_tables, plan.d_lens, plan.max_context_len, scale,
                            partition_size, workspace, stream)
        else:
            ops.cache_append(self.k_pool, self.v_pool, k_new, v_new, plan.d_slots, stream)
            ops.decode(out, q, self.k_pool, self.v_pool, plan.d_tables, plan.d_lens,
                       plan.max_context_len, scale, partition_size, workspace, stream)
        return out
