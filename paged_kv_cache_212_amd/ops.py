"""Device operations on torch tensors, forwarded to the C ABI.

torch provides device memory and the current HIP stream; each function checks
shapes and dtypes, then passes raw pointers to the library.  Nothing here
computes.
"""
from __future__ import annotations

import ctypes as C

import torch

from ._lib import (PA_BF16, PA_F16, PA_F32, PA_FP8_E4M3, PA_INT8, PA_KERNEL_AUTO,
                   PA_KERNEL_GENERIC, check, lib)

BLOCK_SIZE = 16
_DT = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
       torch.float8_e4m3fn: PA_FP8_E4M3, torch.int8: PA_INT8}
# pool dtypes of a quantized cache: 8-bit codes, value = code * the pool's scale
CODE_DTYPES = (torch.float8_e4m3fn, torch.int8)


def pa_dtype(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported KV dtype {t}")
    return _DT[t]


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def new_pools(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
              device="cuda", fill=None):
    """K pool [N][Hkv][D/x][16][x] and V pool [N][Hkv][16/x][D][x] (x = 16 bytes / element)."""
    x = 16 // torch.empty((), dtype=dtype).element_size()
    k = torch.empty((num_blocks, num_kv_heads, head_dim // x, BLOCK_SIZE, x), dtype=dtype,
                    device=device)
    v = torch.empty((num_blocks, num_kv_heads, BLOCK_SIZE // x, head_dim, x), dtype=dtype,
                    device=device)
    if fill is not None:
        k.fill_(fill)
        v.fill_(fill)
    return k, v


def _pool_dims(k_pool: torch.Tensor, v_pool: torch.Tensor):
    N, H = k_pool.shape[0], k_pool.shape[1]
    D = v_pool.shape[3] if v_pool.dim() == 5 else -1
    x = 16 // k_pool.element_size()
    if k_pool.shape != (N, H, D // x, BLOCK_SIZE, x) or \
            v_pool.shape != (N, H, BLOCK_SIZE // x, D, x) or k_pool.dtype != v_pool.dtype:
        raise ValueError("k_pool/v_pool shapes or dtypes do not match the pool layout")
    if k_pool.numel() != v_pool.numel():
        raise ValueError("k_pool and v_pool sizes differ")
    return N, H, D


def cache_append(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None):
    """Write k_new/v_new [T][Hkv][D] into slots slot_mapping [T] (int64, -1 = skip)."""
    N, H, D = _pool_dims(k_pool, v_pool)
    T = k_new.shape[0]
    if k_new.shape != (T, H, D) or v_new.shape != (T, H, D) or k_new.dtype != k_pool.dtype \
            or v_new.dtype != k_pool.dtype:
        raise ValueError("k_new/v_new must be [T][Hkv][D] in the pool dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    check(lib().pa_cache_append(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                _dev(slot_mapping, "slot_mapping"), T, N, H, D, BLOCK_SIZE,
                                pa_dtype(k_pool.dtype), _stream(stream)), "pa_cache_append")


def cache_append_quant(k_pool, v_pool, k_new, v_new, slot_mapping, k_scale, v_scale,
                       stream=None):
    """Encode k_new/v_new [T][Hkv][D] (fp32/fp16/bf16) into the 8-bit codes of
    a quantized pool (float8_e4m3fn or int8) at slots slot_mapping [T]:
    code = round(x / scale) as pa_cache_append_quant defines it."""
    N, H, D = _pool_dims(k_pool, v_pool)
    if k_pool.dtype not in CODE_DTYPES:
        raise ValueError("cache_append_quant needs a float8_e4m3fn or int8 pool")
    T = k_new.shape[0]
    if k_new.shape != (T, H, D) or v_new.shape != (T, H, D) or k_new.dtype != v_new.dtype \
            or k_new.dtype in CODE_DTYPES:
        raise ValueError("k_new/v_new must be [T][Hkv][D] in fp32, fp16 or bf16")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    check(lib().pa_cache_append_quant(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                      _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                      _dev(slot_mapping, "slot_mapping"), T, N, H, D, BLOCK_SIZE,
                                      pa_dtype(k_pool.dtype), pa_dtype(k_new.dtype),
                                      float(k_scale), float(v_scale), _stream(stream)),
          "pa_cache_append_quant")


def copy_blocks(k_pool, v_pool, block_pairs, stream=None):
    """block dst := block src for each row (src, dst) of block_pairs (int32 [n][2])."""
    N, H, D = _pool_dims(k_pool, v_pool)
    n = block_pairs.shape[0]
    if n == 0:
        return
    if block_pairs.dtype != torch.int32 or block_pairs.shape != (n, 2):
        raise ValueError("block_pairs must be int32 [n][2]")
    check(lib().pa_copy_blocks(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                               _dev(block_pairs, "block_pairs"), n, N, H, D, BLOCK_SIZE,
                               pa_dtype(k_pool.dtype), _stream(stream)), "pa_copy_blocks")


def copy_blocks_layers(k_pools, v_pools, block_pairs, stream=None):
    """block dst := block src in every layer's pools (lists of pool tensors of
    one shape and dtype), one launch (pa_copy_blocks_layers)."""
    if len(k_pools) != len(v_pools) or not k_pools:
        raise ValueError("one K and one V pool per layer")
    N, H, D = _pool_dims(k_pools[0], v_pools[0])
    for kp, vp in zip(k_pools, v_pools):
        if _pool_dims(kp, vp) != (N, H, D) or kp.dtype != k_pools[0].dtype:
            raise ValueError("all layers' pools must have one shape and dtype")
        _dev(kp, "k_pool")
        _dev(vp, "v_pool")
    n = block_pairs.shape[0]
    if n == 0:
        return
    if block_pairs.dtype != torch.int32 or block_pairs.shape != (n, 2):
        raise ValueError("block_pairs must be int32 [n][2]")
    dev = k_pools[0].device
    kptr = torch.tensor([t.data_ptr() for t in k_pools], dtype=torch.int64, device=dev)
    vptr = torch.tensor([t.data_ptr() for t in v_pools], dtype=torch.int64, device=dev)
    check(lib().pa_copy_blocks_layers(kptr.data_ptr(), vptr.data_ptr(), len(k_pools),
                                      _dev(block_pairs, "block_pairs"), n, N, H, D, BLOCK_SIZE,
                                      pa_dtype(k_pools[0].dtype), _stream(stream)),
          "pa_copy_blocks_layers")
    if stream is not None:   # the pointer arrays stay valid until the copy has run
        kptr.record_stream(stream)
        vptr.record_stream(stream)


_KERNELS = {"auto": PA_KERNEL_AUTO, "generic": PA_KERNEL_GENERIC}


def set_decode_kernel(kernel: str) -> str:
    """Kernel family of the fp16/bf16 decode calls (pa_set_decode_kernel):
    "auto" (matrix cores) or "generic" (plain FMAs).  Returns the previous
    choice.  Change it only between calls: it also sizes the workspace."""
    if kernel not in _KERNELS:
        raise ValueError(f"kernel must be one of {sorted(_KERNELS)}")
    prev = int(lib().pa_set_decode_kernel(_KERNELS[kernel]))
    return {v: k for k, v in _KERNELS.items()}[prev]


def decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          partition_size, dtype) -> int:
    return int(lib().pa_decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              max_context_len, partition_size,
                                              pa_dtype(dtype)))


def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                           partition_size, dtype) -> int:
    return int(lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                               max_context_len, partition_size,
                                               pa_dtype(dtype)))


def decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                     partition_size, dtype, device="cuda", stream=None):
    """Workspace tensor for the decode calls.  With ``stream`` (a
    torch.cuda.Stream) the memory comes from that stream's pool of torch's
    caching allocator, so once the tensor is dropped it is handed out again
    only to work ordered after the calls made on ``stream``."""
    n = decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                               partition_size, dtype)
    if stream is None:
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


EVEN_SPLIT = -1   # partition_size value selecting the even split of the batch's work


def decode(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale=None,
           partition_size=0, workspace=None, stream=None, phase="both", window=0):
    """out [B][Hq][D] float32 = paged decode attention of q [B][Hq][D].

    partition_size: > 0 fixed partitions, 0 library default, EVEN_SPLIT (-1).
    phase: "both" (pa_decode), "partial" (pa_decode_partial) or "merge"
    (pa_decode_merge).  window > 0: sliding-window attention over the last
    `window` positions (pa_decode_window; phase "both" only)."""
    fn = {"both": "pa_decode", "partial": "pa_decode_partial", "merge": "pa_decode_merge"}[phase]
    if window:
        if phase != "both":
            raise ValueError("a sliding window runs both phases in one call")
        return _decode_window(out, q, k_pool, v_pool, block_tables, context_lens,
                              max_context_len, scale, window, partition_size, workspace, stream)
    N, H, D = _pool_dims(k_pool, v_pool)
    B, Hq = q.shape[0], q.shape[1]
    if q.shape != (B, Hq, D) or q.dtype != k_pool.dtype:
        raise ValueError("q must be [B][Hq][D] in the pool dtype")
    if out.shape != (B, Hq, D) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [B][Hq][D]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    scale = D ** -0.5 if scale is None else float(scale)
    if workspace is None:
        workspace = decode_workspace(B, Hq, H, D, max_context_len, partition_size, q.dtype,
                                     q.device, stream)
    check(getattr(lib(), fn)(_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
                          _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables"),
                          _dev(context_lens, "context_lens"), B, Hq, H, D, BLOCK_SIZE, N,
                          block_tables.shape[1], int(max_context_len), scale,
                          int(partition_size), pa_dtype(q.dtype), _dev(workspace, "workspace"),
                          workspace.numel() * workspace.element_size(), _stream(stream)),
          fn)
    return out


def _check_decode_args(out, q, k_pool, block_tables, context_lens, D, q_dtype):
    B, Hq = q.shape[0], q.shape[1]
    if q.shape != (B, Hq, D) or q.dtype != q_dtype:
        raise ValueError(f"q must be [B][Hq][D] in {q_dtype}")
    if out.shape != (B, Hq, D) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [B][Hq][D]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    return B, Hq


def decode_quant(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, k_scale,
                 v_scale, scale=None, partition_size=0, workspace=None, stream=None):
    """Decode attention over a quantized cache (pa_decode_quant): q bf16
    [B][Hq][D], pools of float8_e4m3fn or int8 codes with K = code * k_scale,
    V = code * v_scale."""
    N, H, D = _pool_dims(k_pool, v_pool)
    if k_pool.dtype not in CODE_DTYPES:
        raise ValueError("decode_quant needs a float8_e4m3fn or int8 pool")
    B, Hq = _check_decode_args(out, q, k_pool, block_tables, context_lens, D, torch.bfloat16)
    scale = D ** -0.5 if scale is None else float(scale)
    if workspace is None:
        workspace = decode_workspace(B, Hq, H, D, max_context_len, partition_size,
                                     k_pool.dtype, q.device, stream)
    check(lib().pa_decode_quant(_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
                                _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables"),
                                _dev(context_lens, "context_lens"), B, Hq, H, D, BLOCK_SIZE, N,
                                block_tables.shape[1], int(max_context_len), scale,
                                int(partition_size), pa_dtype(k_pool.dtype), float(k_scale),
                                float(v_scale), _dev(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream)),
          "pa_decode_quant")
    return out


def decode_step_quant(out, q, k_pool, v_pool, k_new, v_new, slot_mapping, block_tables,
                      context_lens, max_context_len, k_scale, v_scale, scale=None,
                      partition_size=0, workspace=None, stream=None):
    """Encode each sequence's new token (bf16 rows of k_new/v_new) into its slot
    and decode over the quantized cache, in one call (pa_decode_step_quant)."""
    N, H, D = _pool_dims(k_pool, v_pool)
    if k_pool.dtype not in CODE_DTYPES:
        raise ValueError("decode_step_quant needs a float8_e4m3fn or int8 pool")
    B, Hq = _check_decode_args(out, q, k_pool, block_tables, context_lens, D, torch.bfloat16)
    if k_new.shape != (B, H, D) or v_new.shape != (B, H, D) or \
            k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise ValueError("k_new/v_new must be bf16 [B][Hkv][D]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (B,):
        raise ValueError("slot_mapping must be int64 [B]")
    scale = D ** -0.5 if scale is None else float(scale)
    if workspace is None:
        workspace = decode_workspace(B, Hq, H, D, max_context_len, partition_size,
                                     k_pool.dtype, q.device, stream)
    check(lib().pa_decode_step_quant(_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
                                     _dev(v_pool, "v_pool"), _dev(k_new, "k_new"),
                                     _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping"),
                                     _dev(block_tables, "block_tables"),
                                     _dev(context_lens, "context_lens"), B, Hq, H, D,
                                     BLOCK_SIZE, N, block_tables.shape[1], int(max_context_len),
                                     scale, int(partition_size), pa_dtype(k_pool.dtype),
                                     float(k_scale), float(v_scale),
                                     _dev(workspace, "workspace"),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream)),
          "pa_decode_step_quant")
    return out


def _decode_window(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale,
                   window, partition_size, workspace, stream):
    N, H, D = _pool_dims(k_pool, v_pool)
    if k_pool.dtype in CODE_DTYPES:
        raise ValueError("sliding-window decode takes fp32/fp16/bf16 pools")
    B, Hq = _check_decode_args(out, q, k_pool, block_tables, context_lens, D, k_pool.dtype)
    scale = D ** -0.5 if scale is None else float(scale)
    if workspace is None:
        workspace = decode_workspace(B, Hq, H, D, max_context_len, partition_size, q.dtype,
                                     q.device, stream)
    check(lib().pa_decode_window(_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
                                 _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables"),
                                 _dev(context_lens, "context_lens"), B, Hq, H, D, BLOCK_SIZE, N,
                                 block_tables.shape[1], int(max_context_len), scale,
                                 int(window), int(partition_size), pa_dtype(q.dtype),
                                 _dev(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
          "pa_decode_window")
    return out


def decode_step(out, q, k_pool, v_pool, k_new, v_new, slot_mapping, block_tables,
                context_lens, max_context_len, scale=None, partition_size=0, workspace=None,
                stream=None, phase="both", window=0):
    """Append each sequence's new token (row b of k_new/v_new, slot slot_mapping[b]) and
    decode, in one call (pa_decode_step).

    phase: "both" (pa_decode_step), or "partial" then "merge"
    (pa_decode_step_partial, pa_decode_step_merge; same arguments and workspace).
    window > 0: sliding-window attention (pa_decode_step_window; phase "both")."""
    fn = {"both": "pa_decode_step", "partial": "pa_decode_step_partial",
          "merge": "pa_decode_step_merge"}[phase]
    if window and phase != "both":
        raise ValueError("a sliding window runs both phases in one call")
    if window:
        fn = "pa_decode_step_window"
    N, H, D = _pool_dims(k_pool, v_pool)
    B, Hq = q.shape[0], q.shape[1]
    if q.shape != (B, Hq, D) or q.dtype != k_pool.dtype:
        raise ValueError("q must be [B][Hq][D] in the pool dtype")
    if k_new.shape != (B, H, D) or v_new.shape != (B, H, D) or k_new.dtype != k_pool.dtype \
            or v_new.dtype != k_pool.dtype:
        raise ValueError("k_new/v_new must be [B][Hkv][D] in the pool dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (B,):
        raise ValueError("slot_mapping must be int64 [B]")
    if out.shape != (B, Hq, D) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [B][Hq][D]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    scale = D ** -0.5 if scale is None else float(scale)
    if workspace is None:
        workspace = decode_workspace(B, Hq, H, D, max_context_len, partition_size, q.dtype,
                                     q.device, stream)
    win = (int(window),) if window else ()
    check(getattr(lib(), fn)(_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
                             _dev(v_pool, "v_pool"), _dev(k_new, "k_new"),
                             _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping"),
                             _dev(block_tables, "block_tables"),
                             _dev(context_lens, "context_lens"), B, Hq, H, D, BLOCK_SIZE, N,
                             block_tables.shape[1], int(max_context_len), scale, *win,
                             int(partition_size), pa_dtype(q.dtype),
                             _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream(stream)),
          fn)
    return out


def decode_step_noalloc(out, q, k_pool, v_pool, k_new, v_new, slot_mapping, block_tables,
                        context_lens, max_context_len, scale=None, partition_size=0,
                        stream=None):
    """pa_decode_step without a workspace (pa_decode_step_noalloc): the
    partials go to the library's fixed device array; nothing is allocated,
    here or in the library.  Calls that overlap on one device race."""
    N, H, D = _pool_dims(k_pool, v_pool)
    B, Hq = _check_decode_args(out, q, k_pool, block_tables, context_lens, D, k_pool.dtype)
    if k_new.shape != (B, H, D) or v_new.shape != (B, H, D) or k_new.dtype != k_pool.dtype \
            or v_new.dtype != k_pool.dtype:
        raise ValueError("k_new/v_new must be [B][Hkv][D] in the pool dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (B,):
        raise ValueError("slot_mapping must be int64 [B]")
    scale = D ** -0.5 if scale is None else float(scale)
    check(lib().pa_decode_step_noalloc(_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
                                       _dev(v_pool, "v_pool"), _dev(k_new, "k_new"),
                                       _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping"),
                                       _dev(block_tables, "block_tables"),
                                       _dev(context_lens, "context_lens"), B, Hq, H, D,
                                       BLOCK_SIZE, N, block_tables.shape[1],
                                       int(max_context_len), scale, int(partition_size),
                                       pa_dtype(q.dtype), _stream(stream)),
          "pa_decode_step_noalloc")
    return out


def shared_prefix_plan(tables, lens, min_shared_blocks=4):
    """Host plan of pa_shared_prefix_plan over the step's tables (numpy int32
    [n][max_blocks]) and lengths ([n]): returns (prefix_len [n], group_rows
    [rows], group_start [groups + 1], max_group) as numpy int32 arrays."""
    import numpy as np
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    n = int(lens.shape[0])
    if tables.ndim != 2 or tables.shape[0] != n:
        raise ValueError("tables must be [n][max_blocks]")
    prefix = np.zeros(n, dtype=np.int32)
    rows = np.zeros(max(n, 1), dtype=np.int32)
    start = np.zeros(n + 1, dtype=np.int32)
    ng, mg = C.c_int32(0), C.c_int32(0)
    check(lib().pa_shared_prefix_plan(tables.ctypes.data, lens.ctypes.data, n, tables.shape[1],
                                      BLOCK_SIZE, int(min_shared_blocks), prefix.ctypes.data,
                                      rows.ctypes.data, start.ctypes.data, C.byref(ng),
                                      C.byref(mg)), "pa_shared_prefix_plan")
    return prefix, rows[:int(start[ng.value])].copy(), start[:ng.value + 1].copy(), mg.value


def decode_shared_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                            dtype, device="cuda", stream=None):
    n = int(lib().pa_decode_shared_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                   max_context_len, pa_dtype(dtype)))
    if stream is None:
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def decode_step_shared(out, q, k_pool, v_pool, k_new, v_new, slot_mapping, block_tables,
                       context_lens, max_context_len, prefix_len, group_rows, group_start,
                       max_group_size, scale=None, workspace=None, stream=None):
    """pa_decode_step with prefixes shared by groups of sequences attended once
    per group (pa_decode_step_shared); prefix_len [B], group_rows [rows] and
    group_start [groups + 1] are device int32 tensors from shared_prefix_plan."""
    N, H, D = _pool_dims(k_pool, v_pool)
    B, Hq = _check_decode_args(out, q, k_pool, block_tables, context_lens, D, k_pool.dtype)
    if k_new.shape != (B, H, D) or v_new.shape != (B, H, D) or k_new.dtype != k_pool.dtype \
            or v_new.dtype != k_pool.dtype:
        raise ValueError("k_new/v_new must be [B][Hkv][D] in the pool dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (B,):
        raise ValueError("slot_mapping must be int64 [B]")
    for t, name in ((prefix_len, "prefix_len"), (group_rows, "group_rows"),
                    (group_start, "group_start")):
        if t.dtype != torch.int32 or t.dim() != 1:
            raise ValueError(f"{name} must be a 1-D int32 tensor")
    if prefix_len.shape != (B,):
        raise ValueError("prefix_len must be int32 [B]")
    ng = group_start.shape[0] - 1
    if ng < 0:
        raise ValueError("group_start must hold num_groups + 1 offsets")
    scale = D ** -0.5 if scale is None else float(scale)
    if workspace is None:
        workspace = decode_shared_workspace(B, Hq, H, D, max_context_len, q.dtype, q.device,
                                            stream)
    gr = _dev(group_rows, "group_rows") if group_rows.numel() else None
    gs = _dev(group_start, "group_start")
    check(lib().pa_decode_step_shared(_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
                                      _dev(v_pool, "v_pool"), _dev(k_new, "k_new"),
                                      _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping"),
                                      _dev(block_tables, "block_tables"),
                                      _dev(context_lens, "context_lens"),
                                      _dev(prefix_len, "prefix_len"), gr, gs, ng,
                                      int(group_rows.numel()), int(max_group_size), B, Hq, H, D,
                                      BLOCK_SIZE, N, block_tables.shape[1],
                                      int(max_context_len), scale, pa_dtype(q.dtype),
                                      _dev(workspace, "workspace"),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "pa_decode_step_shared")
    return out


def prefill(out, q, k_pool, v_pool, block_tables, context_lens, query_start, max_context_len,
            max_query_len, scale=None, stream=None):
    """out [T][Hq][D] float32 = causal attention of the query rows q [T][Hq][D]
    over the paged cache (pa_prefill): rows query_start[b] .. query_start[b+1]-1
    are the last tokens of sequence b, whose context_lens[b] tokens are in the
    pool already."""
    N, H, D = _pool_dims(k_pool, v_pool)
    T, Hq = q.shape[0], q.shape[1]
    B = context_lens.shape[0]
    if q.shape != (T, Hq, D) or q.dtype != k_pool.dtype:
        raise ValueError("q must be [T][Hq][D] in the pool dtype")
    if out.shape != (T, Hq, D) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [T][Hq][D]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.dim() != 1:
        raise ValueError("context_lens must be int32 [B]")
    if query_start.dtype != torch.int32 or query_start.shape != (B + 1,):
        raise ValueError("query_start must be int32 [B + 1]")
    scale = D ** -0.5 if scale is None else float(scale)
    check(lib().pa_prefill(_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
                           _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables"),
                           _dev(context_lens, "context_lens"), _dev(query_start, "query_start"),
                           B, T, Hq, H, D, BLOCK_SIZE, N, block_tables.shape[1],
                           int(max_context_len), int(max_query_len), scale, pa_dtype(q.dtype),
                           _stream(stream)), "pa_prefill")
    return out


def gather_kv(k_pool, v_pool, block_tables, context_lens, max_context_len, stream=None):
    """Contiguous K, V [B][Hkv][max_context_len][D] reassembled through the tables."""
    N, H, D = _pool_dims(k_pool, v_pool)
    B = block_tables.shape[0]
    k_out = torch.empty((B, H, max_context_len, D), dtype=k_pool.dtype, device=k_pool.device)
    v_out = torch.empty_like(k_out)
    check(lib().pa_gather_kv(_dev(k_out, "k_out"), _dev(v_out, "v_out"), _dev(k_pool, "k_pool"),
                             _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables"),
                             _dev(context_lens, "context_lens"), B, H, D, BLOCK_SIZE, N,
                             block_tables.shape[1], int(max_context_len),
                             pa_dtype(k_pool.dtype), _stream(stream)), "pa_gather_kv")
    return k_out, v_out
