"""Synthetic decode-step workloads.

Each ``Case`` describes one decode step over a batch of sequences whose earlier
tokens already sit in a paged KV cache:

* ``script``: set-up operations to replay on a block manager before the step,
  ``("add", sid, n)``, ``("fork", parent, child)``, ``("extend", sid, n)``,
  ``("free", sid)``.  ``add``/``extend`` write the next ``n`` logical positions
  of ``sid`` with the token rows ``rows[sid][pos]``.
* the step itself: every sequence of ``batch`` reserves one more position
  (``lens[b] - 1``), writes token row ``rows[sid][lens[b] - 1]`` there, then
  attends with ``q[b]`` over all ``lens[b]`` positions.

Context lengths therefore count the new token (append first, then attend).

Random draws: a NumPy ``default_rng(seed)`` draws the structure in the order
lengths -> pool permutation -> (long-context key mask) -> (sample tails); a
``torch.Generator`` seeded from the same seed draws q, then K, then V as
float32 normals, rounded once (round-to-nearest-even) into the KV dtype.  All
consumers read the same stored bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
import math

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "i8": 1}
CODE_MAX = {"i8": 127.0, "fp8": 448.0}     # largest code magnitude of the 8-bit formats

CONFIG_NAMES = ("tiny_fp32", "llama3_8b_bf16", "opt13b_fp16", "cow_parallel_bf16",
                "long_context_bf16")


@dataclass
class Case:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray          # int32 [N]: order in which a fresh pool hands out blocks
    script: list                    # set-up ops (see module docstring)
    batch: np.ndarray               # int64 [B]: sequence ids decoded in this step
    lens: np.ndarray                # int32 [B]: context length after the step's append
    rows: dict                      # sid -> int64 [len]: token row of every logical position
    q: torch.Tensor                 # [B][Hq][D] in the KV dtype
    k_tok: torch.Tensor             # [R][Hkv][D] in the KV dtype
    v_tok: torch.Tensor             # [R][Hkv][D] in the KV dtype
    partition_size: int = 0         # 0 = let the library choose
    notes: dict = field(default_factory=dict)
    # quantized cache: pools hold 8-bit codes ("i8" / "fp8") of the token rows
    # (which stay in ``dtype``, as do q and the step's new tokens), K = code *
    # k_scale, V = code * v_scale.  None: pools hold ``dtype`` itself.
    cache_dtype: str | None = None
    k_scale: float = 1.0
    v_scale: float = 1.0
    # sliding window: the step attends the last `window` positions (0 = all)
    window: int = 0

    @property
    def kv_dtype(self) -> str:
        """dtype of the pools' elements."""
        return self.cache_dtype or self.dtype

    @property
    def num_seqs(self) -> int:
        return int(self.batch.shape[0])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elt_bytes(self) -> int:
        return ELT_BYTES[self.kv_dtype]

    def attended_lens(self) -> np.ndarray:
        """Positions each sequence attends: L, or min(L, window) with a window."""
        L = self.lens.astype(np.int64)
        return np.minimum(L, self.window) if self.window else L

    def kv_bytes(self) -> int:
        """Logical K+V bytes one decode step reads: sum(attended) * Hkv * 2 * D * elt."""
        return int(self.attended_lens().sum()) * self.num_kv_heads * 2 * \
            self.head_dim * self.elt_bytes

    def new_rows(self) -> np.ndarray:
        """Token row written by this step's append, per batch entry."""
        return np.array([self.rows[int(s)][int(L) - 1] for s, L in zip(self.batch, self.lens)],
                        dtype=np.int64)


def quantized(case: Case, cache_dtype: str) -> Case:
    """The same workload over a quantized cache: per-pool scales calibrated on
    the drawn token rows (largest |value| maps to the format's largest code,
    computed in fp32)."""
    if cache_dtype not in CODE_MAX:
        raise KeyError(cache_dtype)
    amax_k = float(case.k_tok.abs().max().float())
    amax_v = float(case.v_tok.abs().max().float())
    ks = float(np.float32(amax_k) / np.float32(CODE_MAX[cache_dtype]))
    vs = float(np.float32(amax_v) / np.float32(CODE_MAX[cache_dtype]))
    name = case.name.rsplit("_", 1)[0] + "_" + cache_dtype + "kv"
    return replace(case, name=name, cache_dtype=cache_dtype, k_scale=ks, v_scale=vs)


def beam_case(seed: int, dtype: str, n_prompts: int, beams: int, prompt_len: int, steps: int,
              hq: int, hkv: int, d: int, device="cpu", *, pool_factor: float = 1.3) -> Case:
    """Beam search over ``steps`` decode steps, then one more step as the
    case's step.  Each prompt is written once and forked into ``beams``
    sequences; at every later step each beam picks a parent among its
    prompt's beams of the previous step (seeded draws with replacement,
    sorted), a parent's first child keeps its id, the others are forks under
    fresh ids, and parents without children are freed (op ``("reorder", old,
    new, parents)``); then every beam appends one token (op ``("extend",
    sid, 1)``, with the copy-on-write of a shared last block).  Every
    (step, beam) token has a row of its own; a beam's rows are its parent's
    plus its new one."""
    rng = np.random.default_rng(seed)
    script, rows = [], {}
    R = n_prompts * prompt_len
    next_row = R
    live = []                                         # per prompt: beam ids
    next_id = 0
    for p in range(n_prompts):
        pid = 10_000_000 + p
        rows[pid] = np.arange(p * prompt_len, (p + 1) * prompt_len, dtype=np.int64)
        script.append(("add", pid, prompt_len))
        ids = []
        for _ in range(beams):
            script.append(("fork", pid, next_id))
            rows[next_id] = rows[pid]
            ids.append(next_id)
            next_id += 1
        script.append(("free", pid))
        live.append(ids)
    for t in range(steps + 1):
        if t > 0:                                    # reorder, then append
            for p in range(n_prompts):
                old = live[p]
                parents = np.sort(rng.integers(0, beams, size=beams))
                new, seen = [], set()
                for par in parents.tolist():
                    if par not in seen:
                        seen.add(par)
                        new.append(old[par])
                    else:
                        new.append(next_id)
                        rows[next_id] = rows[old[par]]
                        next_id += 1
                script.append(("reorder", list(old), list(new), parents.tolist()))
                live[p] = new
        for p in range(n_prompts):
            for sid in live[p]:
                rows[sid] = np.concatenate([rows[sid], [next_row]])
                next_row += 1
                if t < steps:
                    script.append(("extend", sid, 1))
    batch = np.array([sid for ids in live for sid in ids], dtype=np.int64)
    lens = np.array([len(rows[s]) for s in batch.tolist()], dtype=np.int32)
    # blocks: prompts once, then at most one new block per beam per 16 steps
    # plus one copy per beam per step
    need = n_prompts * -(-prompt_len // 16) + n_prompts * beams * (steps + 2) * 2
    num_blocks = int(math.ceil(pool_factor * need))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    B = len(batch)
    q, k, v = _draw_values(seed, (B, hq, d), (next_row, hkv, d), dtype, device)
    notes = {"prompts": n_prompts, "beams": beams, "steps": steps}
    return Case(f"beam_{dtype}_{n_prompts}x{beams}_p{prompt_len}_s{steps}", dtype, hq, hkv, d, 16,
                num_blocks, free_order, script, batch, lens, rows, q, k, v, 0, notes)


def windowed(case: Case, window: int, reuse: bool = True) -> Case:
    """The same step with sliding-window attention over the last ``window``
    positions.  Before the step each batch sequence releases the blocks wholly
    before its window start L - window; with ``reuse``, one new sequence per
    releasing sequence then takes as many blocks (so those blocks hold other
    tokens when the step runs).  The new sequences reuse existing token rows
    and are not decoded."""
    if window <= 0:
        raise ValueError("window must be positive")
    script = list(case.script)
    rows = dict(case.rows)
    extra = []
    for sid, L in zip(case.batch.tolist(), case.lens.tolist()):
        first = max(0, int(L) - window)
        script.append(("release", int(sid), first))
        # blocks wholly before `first` among the L - 1 cached positions
        nrel = min(first, int(L) - 1) // case.block_size
        if reuse and nrel:
            extra.append((300_000 + int(sid), nrel * case.block_size, int(sid)))
    for new_sid, n, src in extra:
        rows[new_sid] = case.rows[src][:n]
        script.append(("add", new_sid, n))
    name = f"{case.name}_w{window}"
    return replace(case, name=name, script=script, rows=rows, window=int(window))


def _draw_values(seed: int, nq: tuple, nkv: tuple, dtype: str, device, q_std: float = 1.0,
                 key_boost=None):
    """q, K, V as float32 normals (in that order), rounded once to ``dtype``."""
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * seed + 17)
    td = TORCH_DTYPE[dtype]
    q = torch.randn(nq, generator=g, device=device, dtype=torch.float32)
    if q_std != 1.0:
        q.mul_(q_std)
    q = q.to(td)
    k = torch.randn(nkv, generator=g, device=device, dtype=torch.float32)
    if key_boost is not None:
        # key_boost: bool [R][Hkv]; the chosen key vectors are multiplied by 8
        # (a power of two, so the rounded value is the rounded original x 8).
        kb = torch.as_tensor(key_boost, device=device)
        k[kb] *= 8.0
    k = k.to(td)
    v = torch.randn(nkv, generator=g, device=device, dtype=torch.float32).to(td)
    return q, k, v


def _pool_size(lens, block_size, extra_blocks=0, factor=1.2):
    need = int(sum(-(-int(L) // block_size) for L in lens)) + extra_blocks
    return int(math.ceil(factor * need))


def _independent(name, seed, dtype, lens, hq, hkv, d, device, *, num_blocks=None,
                 q_std=1.0, boost_prob=0.0, partition_size=0, bs=16, rng=None):
    """Batch of unrelated sequences; sequence b has id b and cached lens[b]-1 tokens."""
    lens = np.asarray(lens, dtype=np.int32)
    if num_blocks is None:
        num_blocks = _pool_size(lens, bs)
    free_order = rng.permutation(num_blocks).astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(lens.astype(np.int64))])
    R = int(offs[-1])
    boost = None
    if boost_prob > 0:
        boost = rng.random((R, hkv)) < boost_prob
    q, k, v = _draw_values(seed, (len(lens), hq, d), (R, hkv, d), dtype, device, q_std, boost)
    rows = {b: np.arange(offs[b], offs[b + 1], dtype=np.int64) for b in range(len(lens))}
    script = [("add", b, int(lens[b]) - 1) for b in range(len(lens))]
    notes = {}
    if boost is not None:
        notes["boosted_keys"] = int(boost.sum())
    return Case(name, dtype, hq, hkv, d, bs, int(num_blocks), free_order, script,
                np.arange(len(lens), dtype=np.int64), lens, rows, q, k, v,
                partition_size, notes)


def _parallel_sampling(name, seed, dtype, n_prompts, n_samples, prompt_len, tail_max, hq, hkv,
                       d, device, *, parked_forks=True, bs=16, rng=None):
    """Prompts shared by n_samples forks each, plus a private tail per sample.

    With ``parked_forks`` each sample whose last block is partly filled is forked
    once more into a parked sequence that is never decoded, so that block is
    shared (reference count 2) when the step writes into it and must be copied
    first.  Without it no step write lands on a shared block.
    """
    tails = rng.integers(0, tail_max + 1, size=n_prompts * n_samples)
    B = n_prompts * n_samples
    lens = (prompt_len + tails + 1).astype(np.int32)
    # unique token rows: every prompt once, then every sample's tail (+ new token)
    prompt_base = np.arange(n_prompts, dtype=np.int64) * prompt_len
    tail_sizes = tails + 1
    tail_base = n_prompts * prompt_len + np.concatenate([[0], np.cumsum(tail_sizes)[:-1]])
    R = int(n_prompts * prompt_len + tail_sizes.sum())
    rows, script = {}, []
    parent_id = lambda p: 100_000 + p  # noqa: E731
    parked_id = lambda s: 200_000 + s  # noqa: E731
    for p in range(n_prompts):
        pid = parent_id(p)
        rows[pid] = prompt_base[p] + np.arange(prompt_len, dtype=np.int64)
        script.append(("add", pid, prompt_len))
        for s in range(n_samples):
            sid = p * n_samples + s
            rows[sid] = np.concatenate([rows[pid], tail_base[sid] +
                                        np.arange(tail_sizes[sid], dtype=np.int64)])
            script.append(("fork", pid, sid))
        script.append(("free", pid))
    n_parked = 0
    for sid in range(B):
        if tails[sid] > 0:
            script.append(("extend", sid, int(tails[sid])))
        if parked_forks and (prompt_len + tails[sid]) % bs != 0:
            script.append(("fork", sid, parked_id(sid)))
            n_parked += 1
    unique_blocks = n_prompts * (-(-prompt_len // bs)) + int(
        sum(-(-int(L) // bs) - prompt_len // bs for L in lens))
    num_blocks = int(math.ceil(1.2 * (unique_blocks + n_parked)))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    q, k, v = _draw_values(seed, (B, hq, d), (R, hkv, d), dtype, device)
    notes = {"parked_forks": n_parked, "tails": tails, "unique_blocks": unique_blocks}
    return Case(name, dtype, hq, hkv, d, bs, num_blocks, free_order, script,
                np.arange(B, dtype=np.int64), lens, rows, q, k, v, 0, notes)


def make_case(name: str, seed: int | None = None, device="cpu", **kw) -> Case:
    """One of the five decode workloads at full size.  q_heads (Llama-3-8B
    shape only): the number of query heads over the same 8 KV heads and
    lengths (default 32)."""
    idx = CONFIG_NAMES.index(name) + 1
    seed = idx if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "tiny_fp32":
        # 4 sequences, contexts {1,15,16,37}, 4 heads, D=64, pool of 16 blocks.
        return _independent(name, seed, "f32", [1, 15, 16, 37], 4, 4, 64, device,
                            num_blocks=16, rng=rng)
    if name == "llama3_8b_bf16":
        lens = rng.integers(256, 2048 + 1, size=64)
        return _independent(name, seed, "bf16", lens, kw.get("q_heads", 32), 8, 128, device,
                            rng=rng)
    if name == "opt13b_fp16":
        z = rng.standard_normal(256)
        lens = np.clip(np.rint(600.0 * np.exp(0.9 * z)), 16, 2048).astype(np.int64)
        return _independent(name, seed, "f16", lens, 40, 40, 128, device, q_std=0.5, rng=rng)
    if name == "cow_parallel_bf16":
        return _parallel_sampling(name, seed, "bf16", 32, 8, 1024, 512, 32, 8, 128, device,
                                  parked_forks=kw.get("parked_forks", True), rng=rng)
    if name == "long_context_bf16":
        lens = rng.integers(32768, 131072 + 1, size=16)
        return _independent(name, seed, "bf16", lens, 32, 8, 128, device, boost_prob=0.01,
                            partition_size=512, rng=rng)
    raise KeyError(name)


def small_case(name: str, seed: int | None = None, device="cpu", **kw) -> Case:
    """Reduced versions of the five workloads: same head shapes, dtypes and
    length structure, sized so the fp64 oracle finishes in well under a second,
    while still spanning several blocks, several partitions and ragged tails."""
    idx = CONFIG_NAMES.index(name) + 1
    seed = 100 + idx if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "tiny_fp32":
        return make_case(name, seed=1, device=device)
    if name == "llama3_8b_bf16":
        lens = np.concatenate([[1, 16, 17, 32], rng.integers(1, 600, size=4)])
        return _independent(name, seed, "bf16", lens, 32, 8, 128, device, rng=rng)
    if name == "opt13b_fp16":
        z = rng.standard_normal(8)
        lens = np.clip(np.rint(60.0 * np.exp(0.9 * z)), 1, 400).astype(np.int64)
        return _independent(name, seed, "f16", lens, 40, 40, 128, device, q_std=0.5, rng=rng)
    if name == "cow_parallel_bf16":
        return _parallel_sampling(name, seed, "bf16", 2, 4, 64, 40, 32, 8, 128, device,
                                  parked_forks=kw.get("parked_forks", True), rng=rng)
    if name == "long_context_bf16":
        lens = rng.integers(1100, 2600, size=3)
        return _independent(name, seed, "bf16", lens, 32, 8, 128, device, boost_prob=0.05,
                            partition_size=512, rng=rng)
    raise KeyError(name)


def custom_case(seed, dtype, lens, hq, hkv, d, device="cpu", *, num_blocks=None,
                partition_size=0, q_std=1.0, boost_prob=0.0, pool_factor=1.2) -> Case:
    """Free-form batch of independent sequences (edge cases, sweeps)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    if num_blocks is None:
        num_blocks = max(1, _pool_size(lens, 16, factor=pool_factor))
    return _independent(f"custom_{dtype}_{hq}x{hkv}x{d}", seed, dtype, lens, hq, hkv, d, device,
                        num_blocks=num_blocks, q_std=q_std, boost_prob=boost_prob,
                        partition_size=partition_size, rng=rng)


def prefill_case(seed, dtype, lens, qlens, hq, hkv, d, device="cpu", *, num_blocks=None,
                 pool_factor=1.2, boost_prob=0.0):
    """Seeded inputs for attending a chunk of query tokens per sequence
    (prefill, chunked prefill): the decode case of the same sequences, whose
    set-up and step append leave all lens[b] tokens in the cache, plus query
    rows q [T][hq][d] for the last qlens[b] positions of each sequence and
    their row offsets query_start [B+1] (T = query_start[-1]).  boost_prob:
    as in custom_case (key vectors scaled x8 with that probability).

    Returns (case, q, query_start)."""
    lens = np.asarray(lens, dtype=np.int64)
    qlens = np.asarray(qlens, dtype=np.int64)
    if qlens.shape != lens.shape or (qlens < 0).any() or (qlens > lens).any():
        raise ValueError("qlens must be in [0, lens] per sequence")
    case = custom_case(seed, dtype, lens, hq, hkv, d, device, num_blocks=num_blocks,
                       pool_factor=pool_factor, boost_prob=boost_prob)
    query_start = np.zeros(len(lens) + 1, dtype=np.int64)
    query_start[1:] = np.cumsum(qlens)
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * seed + 29)
    q = torch.randn((int(query_start[-1]), hq, d), generator=g, device=device,
                    dtype=torch.float32).to(TORCH_DTYPE[dtype])
    return case, q, query_start


CODE_UNIT = 64.0   # the magnitude of every non-zero entry of a position-coded case


def position_coded(case: Case, seed: int = 0, mark_prob: float = 1.0 / 16) -> Case:
    """The same step (lengths, set-up, tables, pool) with q, K and V replaced
    by exact patterns of 0 and +-64, so that every output row is a plain
    average of stored V rows and a dropped, doubled or misplaced token
    changes it by far more than rounding does.

    * V: row r, KV head g holds 64 * bit i of r in dim i (i < bits of the
      largest row) and 64 * bit j of g in the next dims; other dims 0.  A V
      row thus names its token row and head.
    * K: zero, except that with probability ``mark_prob`` each (row, head)
      gets +64 in dim 0 ("set A"), else with the same probability -64 in dim
      0 ("set B"), and independently +64 in dim 1 ("set C").
    * q: query head h gets, by h % 4: +64 e_0, -64 e_0, +64 e_1, or 0.

    Scores are then 0 or +-4096 * scale, so a head's weights are 1 on its
    marked rows and underflow to 0 elsewhere (all rows when none is marked,
    and always for q = 0): each output row is the mean of a set of V rows,
    sums of 0/64 entries that fp32 holds exactly.  Marks are drawn with a
    seeded torch.Generator on the case's device.
    """
    dev = case.k_tok.device
    R, Hkv, D = case.k_tok.shape
    td = case.k_tok.dtype
    nbits = max(1, int(R - 1).bit_length())
    gbits = max(1, int(Hkv - 1).bit_length())
    if nbits + gbits > D or D < 2:
        raise ValueError("head_dim too small for the row code")
    r = torch.arange(R, device=dev, dtype=torch.int64)
    g = torch.arange(Hkv, device=dev, dtype=torch.int64)
    v = torch.zeros((R, Hkv, D), device=dev, dtype=torch.float32)
    for i in range(nbits):
        v[:, :, i] = ((r >> i) & 1).to(torch.float32)[:, None] * CODE_UNIT
    for j in range(gbits):
        v[:, :, nbits + j] = ((g >> j) & 1).to(torch.float32)[None, :] * CODE_UNIT
    gen = torch.Generator(device=dev)
    gen.manual_seed(7_919 * seed + 3)
    u0 = torch.rand((R, Hkv), generator=gen, device=dev)
    u1 = torch.rand((R, Hkv), generator=gen, device=dev)
    k = torch.zeros((R, Hkv, D), device=dev, dtype=torch.float32)
    k[:, :, 0] = torch.where(u0 < mark_prob, CODE_UNIT,
                             torch.where(u0 < 2 * mark_prob, -CODE_UNIT, 0.0))
    k[:, :, 1] = torch.where(u1 < mark_prob, CODE_UNIT, 0.0)
    B, Hq, _ = case.q.shape
    q = torch.zeros((B, Hq, D), device=case.q.device, dtype=torch.float32)
    kind = torch.arange(Hq, device=case.q.device) % 4
    q[:, kind == 0, 0] = CODE_UNIT
    q[:, kind == 1, 0] = -CODE_UNIT
    q[:, kind == 2, 1] = CODE_UNIT
    notes = dict(case.notes)
    notes["position_coded"] = {"row_bits": nbits, "head_bits": gbits, "mark_prob": mark_prob}
    return replace(case, name=case.name + "_coded", q=q.to(td), k_tok=k.to(td), v_tok=v.to(td),
                   notes=notes)
