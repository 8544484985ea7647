"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/pa.h declares, validates arguments before any launch, and its
C++ block manager reproduces the oracle's allocator model bit for bit."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import paged_kv_cache_212_amd as pk
from paged_kv_cache_212_amd._lib import (PA_ERR_INVALID_ARG, PA_ERR_OUT_OF_BLOCKS,
                                         PA_ERR_SEQ_EXISTS, PA_ERR_UNKNOWN_SEQ,
                                         PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_BF16, PA_F16,
                                         PA_FP8_E4M3, PA_INT8,
                                         PA_F32, SIGNATURES)
from oracle import AllocatorModel, AllocError
from oracle import allocator as om
from tests.test_allocator_model import random_ops

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 18
    h = pk.lib()
    for n in names:
        assert hasattr(h, n), n
        assert n in SIGNATURES, f"binding lacks {n}"
    assert set(SIGNATURES) == set(names)
    assert b"gfx950" in h.pa_version()


def test_device_calls_reject_bad_scalars_without_launching():
    h = pk.lib()
    nul = None
    # block size, head dim, dtype, G and workspace checks all happen before any launch
    assert h.pa_decode(nul, nul, nul, nul, nul, nul, 1, 8, 2, 128, 32, 10, 4, 64, 0.1, 0,
                       PA_BF16, nul, 0, nul) == PA_ERR_UNSUPPORTED
    assert h.pa_decode(nul, nul, nul, nul, nul, nul, 1, 8, 2, 96, 16, 10, 4, 64, 0.1, 0,
                       PA_BF16, nul, 0, nul) == PA_ERR_UNSUPPORTED
    assert h.pa_decode(nul, nul, nul, nul, nul, nul, 1, 8, 3, 128, 16, 10, 4, 64, 0.1, 0,
                       PA_BF16, nul, 0, nul) == PA_ERR_INVALID_ARG
    assert h.pa_decode(nul, nul, nul, nul, nul, nul, 1, 64, 2, 128, 16, 10, 4, 64, 0.1, 0,
                       PA_BF16, nul, 0, nul) == PA_ERR_UNSUPPORTED
    assert h.pa_decode(nul, nul, nul, nul, nul, nul, 1, 8, 2, 128, 16, 10, 4, 64, 0.1, 24,
                       PA_BF16, nul, 0, nul) == PA_ERR_INVALID_ARG
    assert h.pa_decode(nul, nul, nul, nul, nul, nul, 1, 8, 2, 128, 16, 10, 4, 64, -1.0, 0,
                       PA_BF16, nul, 0, nul) == PA_ERR_INVALID_ARG
    assert h.pa_decode(nul, nul, nul, nul, nul, nul, 1, 8, 2, 128, 16, 10, 4, 64, 0.1, 0,
                       7, nul, 0, nul) == PA_ERR_INVALID_ARG
    # valid scalars but NULL device pointers: rejected, still no launch
    assert h.pa_decode(nul, nul, nul, nul, nul, nul, 1, 8, 2, 128, 16, 10, 4, 64, 0.1, 0,
                       PA_BF16, nul, 0, nul) == PA_ERR_INVALID_ARG
    assert b"NULL" in h.pa_last_error()
    # multi-partition case without workspace (pointers are fake but never dereferenced)
    fake = C.c_void_p(1 << 20)
    assert h.pa_decode(fake, fake, fake, fake, fake, fake, 2, 8, 2, 128, 16, 10, 400, 6000, 0.1,
                       512, PA_BF16, nul, 0, nul) == PA_ERR_WORKSPACE
    assert h.pa_decode_step_partial(nul, nul, nul, nul, nul, nul, nul, nul, nul, 1, 8, 2, 128,
                                    16, 10, 4, 64, 0.1, 0, PA_BF16, nul, 0,
                                    nul) == PA_ERR_INVALID_ARG
    assert h.pa_decode_step_merge(nul, nul, nul, nul, nul, nul, nul, nul, nul, 1, 8, 2, 128,
                                  16, 10, 4, 64, 0.1, 0, PA_BF16, nul, 0,
                                  nul) == PA_ERR_INVALID_ARG
    assert h.pa_cache_append(nul, nul, nul, nul, nul, 4, 10, 8, 128, 16, PA_BF16,
                             nul) == PA_ERR_INVALID_ARG
    assert h.pa_cache_append(nul, nul, nul, nul, nul, 0, 10, 8, 128, 16, PA_BF16, nul) == 0
    assert h.pa_copy_blocks(nul, nul, nul, 3, 10, 8, 128, 8, PA_F16, nul) == PA_ERR_UNSUPPORTED
    assert h.pa_copy_blocks(nul, nul, nul, 0, 10, 8, 128, 16, PA_F16, nul) == 0
    assert h.pa_gather_kv(nul, nul, nul, nul, nul, nul, 2, 8, 128, 16, 10, 4, 64, PA_F32,
                          nul) == PA_ERR_INVALID_ARG


def test_quantized_cache_calls_reject_bad_arguments_without_launching():
    h = pk.lib()
    nul = None

    def dq(dt=PA_FP8_E4M3, hq=8, hkv=2, ks=0.1, vs=0.1, fn=h.pa_decode_quant):
        return fn(nul, nul, nul, nul, nul, nul, 1, hq, hkv, 128, 16, 10, 4, 64, 0.1, 0, dt, ks,
                  vs, nul, 0, nul)
    assert dq(dt=PA_BF16) == PA_ERR_INVALID_ARG          # not an 8-bit pool
    assert dq(hq=34) == PA_ERR_UNSUPPORTED                # G = 17 > 16
    assert dq(hq=32) == PA_ERR_INVALID_ARG                # G = 16: NULL pointers
    assert dq(ks=0.0) == PA_ERR_INVALID_ARG
    assert dq(vs=float("inf")) == PA_ERR_INVALID_ARG
    assert dq() == PA_ERR_INVALID_ARG                     # valid scalars, NULL pointers
    assert b"NULL" in h.pa_last_error()
    assert dq(dt=PA_INT8) == PA_ERR_INVALID_ARG
    # 8-bit pools are not accepted by the 16-bit entry points
    assert h.pa_decode(nul, nul, nul, nul, nul, nul, 1, 8, 2, 128, 16, 10, 4, 64, 0.1, 0,
                       PA_INT8, nul, 0, nul) == PA_ERR_INVALID_ARG
    assert b"pa_decode_quant" in h.pa_last_error()
    assert h.pa_decode_step_quant(nul, nul, nul, nul, nul, nul, nul, nul, nul, 1, 8, 2, 128, 16,
                                  10, 4, 64, 0.1, 0, PA_INT8, 0.1, 0.1, nul, 0,
                                  nul) == PA_ERR_INVALID_ARG

    def aq(cd=PA_FP8_E4M3, sd=PA_BF16, ks=0.1, vs=0.1, n=4):
        return h.pa_cache_append_quant(nul, nul, nul, nul, nul, n, 10, 8, 128, 16, cd, sd, ks, vs,
                                       nul)
    assert aq(cd=PA_BF16) == PA_ERR_INVALID_ARG
    assert aq(sd=PA_INT8) == PA_ERR_INVALID_ARG
    assert aq(ks=-1.0) == PA_ERR_INVALID_ARG
    assert aq() == PA_ERR_INVALID_ARG                     # NULL pointers
    assert aq(n=0) == 0
    # byte moves accept the 8-bit dtypes
    assert h.pa_cache_append(nul, nul, nul, nul, nul, 0, 10, 8, 128, 16, PA_INT8, nul) == 0
    assert h.pa_copy_blocks(nul, nul, nul, 0, 10, 8, 128, 16, PA_FP8_E4M3, nul) == 0
    # queries: the even split by default; G > 16 invalid
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, 0, PA_FP8_E4M3) == 0
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, 512, PA_INT8) == 512
    assert h.pa_decode_partition_size(64, 128, 8, 128, 2048, 0, PA_INT8) == 0
    assert h.pa_decode_partition_size(64, 136, 8, 128, 2048, 0, PA_INT8) == -1
    assert h.pa_decode_workspace_bytes(64, 32, 8, 128, 2048, 0, PA_INT8) == \
        h.pa_decode_workspace_bytes(64, 32, 8, 128, 2048, 0, PA_BF16)


def test_window_calls_reject_bad_arguments_without_launching():
    h = pk.lib()
    nul = None

    def dw(window=64, hq=8, hkv=2, dt=PA_BF16):
        return h.pa_decode_window(nul, nul, nul, nul, nul, nul, 1, hq, hkv, 128, 16, 10, 4, 64,
                                  0.1, window, 0, dt, nul, 0, nul)
    assert dw(window=-1) == PA_ERR_INVALID_ARG
    assert dw(hq=68, hkv=4) == PA_ERR_UNSUPPORTED        # G = 17 > 16
    assert dw(hq=64, hkv=4) == PA_ERR_INVALID_ARG        # G = 16: NULL pointers
    assert dw(dt=PA_INT8) == PA_ERR_INVALID_ARG          # 8-bit pools: pa_decode_quant
    assert dw() == PA_ERR_INVALID_ARG                    # valid scalars, NULL pointers
    assert dw(window=0) == PA_ERR_INVALID_ARG            # window 0: the plain decode's checks
    assert h.pa_decode_step_window(nul, nul, nul, nul, nul, nul, nul, nul, nul, 1, 8, 2, 128,
                                   16, 10, 4, 64, 0.1, 16, 0, PA_BF16, nul, 0,
                                   nul) == PA_ERR_INVALID_ARG
    bm = pk.BlockManager(8, 16)
    bm.add_seq(1, 40)
    assert bm.release_before(1, 1000) == 2
    with pytest.raises(pk.PAError):
        bm.release_before(1, -5)
    with pytest.raises(pk.PAError):
        bm.release_before(2, 5)
    assert bm.block_tables([1], 3)[0].tolist() == [[-1, -1, 2]]


def test_beam_calls_reject_bad_arguments_without_launching():
    h = pk.lib()
    nul = None
    # multi-layer copy: scalar checks before any launch
    assert h.pa_copy_blocks_layers(nul, nul, 4, nul, 3, 10, 8, 128, 16, 9, nul) == \
        PA_ERR_INVALID_ARG                                       # unknown dtype
    assert h.pa_copy_blocks_layers(nul, nul, 4, nul, 3, 10, 8, 128, 8, PA_BF16, nul) == \
        PA_ERR_UNSUPPORTED                                       # block size 8
    assert h.pa_copy_blocks_layers(nul, nul, -1, nul, 3, 10, 8, 128, 16, PA_BF16, nul) == \
        PA_ERR_INVALID_ARG
    assert h.pa_copy_blocks_layers(nul, nul, 4, nul, 3, 10, 8, 128, 16, PA_BF16, nul) == \
        PA_ERR_INVALID_ARG                                       # NULL pointers
    assert h.pa_copy_blocks_layers(nul, nul, 4, nul, 0, 10, 8, 128, 16, PA_BF16, nul) == 0
    assert h.pa_copy_blocks_layers(nul, nul, 0, nul, 3, 10, 8, 128, 16, PA_INT8, nul) == 0
    # reorder: all-or-nothing
    bm = pk.BlockManager(8, 16)
    bm.add_seq(0, 20)
    bm.add_seq(1, 3)
    before = (bm.stats(), bm.block_tables([0, 1], 2))
    for args in (([0, 9], [0], [0]), ([0, 0], [0], [0]), ([0], [3, 3], [0, 0]),
                 ([0], [3], [1]), ([0], [1], [0])):
        with pytest.raises(pk.PAError):
            bm.reorder(*args)
        after = (bm.stats(), bm.block_tables([0, 1], 2))
        assert after[0] == before[0] and np.array_equal(after[1][0], before[1][0])
    bm.reorder([0, 1], [0, 7], [0, 0])                          # 7 forks 0, 1 is dropped
    assert bm.block_tables([0, 7], 2)[0].tolist() == [[0, 1], [0, 1]]
    assert bm.refcount(0) == 2 and bm.refcount(2) == 0


def test_prefill_rejects_bad_scalars_without_launching():
    h = pk.lib()
    nul = None
    args = lambda **kw: [kw.get(k, v) for k, v in (  # noqa: E731
        ("out", nul), ("q", nul), ("kp", nul), ("vp", nul), ("tab", nul), ("lens", nul),
        ("qs", nul), ("B", 2), ("T", 8), ("Hq", 8), ("Hkv", 2), ("D", 128), ("bs", 16),
        ("N", 10), ("MB", 4), ("ctx", 64), ("mq", 8), ("scale", 0.1), ("dt", PA_BF16),
        ("st", nul))]
    assert h.pa_prefill(*args(dt=PA_F32)) == PA_ERR_UNSUPPORTED
    assert h.pa_prefill(*args(D=96)) == PA_ERR_UNSUPPORTED
    assert h.pa_prefill(*args(bs=8)) == PA_ERR_UNSUPPORTED
    assert h.pa_prefill(*args(Hkv=3)) == PA_ERR_INVALID_ARG
    assert h.pa_prefill(*args(scale=-1.0)) == PA_ERR_INVALID_ARG
    assert h.pa_prefill(*args(mq=-1)) == PA_ERR_INVALID_ARG
    assert h.pa_prefill(*args()) == PA_ERR_INVALID_ARG          # NULL pointers
    assert h.pa_prefill(*args(T=0)) == 0                          # nothing to do


def test_stream_read_rejects_bad_buffers():
    h = pk.lib()
    assert h.pa_stream_read(None, 16, C.c_void_p(16), None) == PA_ERR_INVALID_ARG
    assert h.pa_stream_read(C.c_void_p(16), 24, C.c_void_p(16), None) == PA_ERR_INVALID_ARG
    assert h.pa_stream_read(C.c_void_p(8), 16, C.c_void_p(16), None) == PA_ERR_INVALID_ARG
    assert h.pa_stream_read(C.c_void_p(16), 0, C.c_void_p(16), None) == 0


def test_timing_hook_arguments():
    h = pk.lib()
    assert h.pa_time_next_attention(None, C.c_void_p(16)) == PA_ERR_INVALID_ARG
    assert h.pa_time_next_attention(C.c_void_p(16), None) == PA_ERR_INVALID_ARG
    assert h.pa_time_next_attention(None, None) == 0      # disarm


def test_workspace_and_partition_queries():
    h = pk.lib()
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, 0, PA_BF16) == 0     # default: split
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, 0, PA_F32) == 256    # fp32 default
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, -1, PA_BF16) == 0    # even split
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, -1, PA_F32) == 256   # fixed on fp32
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, -2, PA_BF16) == -1
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, 256, PA_BF16) == 256
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, 100, PA_BF16) == -1
    # up to 16 query heads per KV head: the even split by default (one to
    # four head groups per K/V load on the matrix cores)
    assert h.pa_decode_partition_size(64, 64, 8, 128, 2048, 0, PA_BF16) == 0
    assert h.pa_decode_partition_size(64, 40, 8, 64, 2048, 0, PA_F16) == 0
    assert h.pa_decode_partition_size(64, 128, 8, 128, 2048, 0, PA_F16) == 0
    assert h.pa_decode_partition_size(64, 136, 8, 128, 2048, 0, PA_F16) == -1
    # the even split counts the batch's work in 32 bits (below 2^30 ticks:
    # 8 per 4-block unit plus at most 12 per (sequence, KV head) range).
    # Beyond that the default falls back to fixed partitions and an explicit
    # even split is refused, with no workspace size.
    units = lambda ctx: (-(-ctx // 16) + 3) // 4  # noqa: E731
    assert 65535 * 64 * (12 + 8 * units(131072)) >= 1 << 30
    assert h.pa_decode_partition_size(65535, 64, 64, 128, 131072, 0, PA_BF16) == 256
    assert h.pa_decode_partition_size(65535, 64, 64, 128, 131072, -1, PA_BF16) == -1
    assert h.pa_decode_partition_size(65535, 64, 64, 128, 131072, -1, PA_FP8_E4M3) == -1
    assert h.pa_decode_workspace_bytes(65535, 64, 64, 128, 131072, -1, PA_BF16) == 0
    assert h.pa_decode_workspace_bytes(65535, 64, 64, 128, 131072, 0, PA_BF16) > 0
    assert 16 * 8 * (12 + 8 * units(131072)) < 1 << 30     # the long-context batch fits
    assert h.pa_decode_partition_size(16, 32, 8, 128, 131072, -1, PA_BF16) == 0
    # max_context_len near the int32 limit: the plan's arithmetic is 64-bit
    assert h.pa_decode_partition_size(1, 1, 1, 128, 2**31 - 1, 0, PA_BF16) == 0
    assert h.pa_decode_partition_size(1, 1, 1, 128, 2**31 - 1, 256, PA_BF16) == 256
    # one partition -> no workspace
    assert h.pa_decode_workspace_bytes(4, 8, 2, 64, 256, 512, PA_F32) == 0
    # 3 partitions of 512: m, l and acc rows, each region 256-byte aligned
    rows = 4 * 8 * 3
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert h.pa_decode_workspace_bytes(4, 8, 2, 64, 1100, 512, PA_F32) == \
        2 * al(rows * 4) + al(rows * 64 * 4) + al(4 * 2 * 4)


def _c_apply(bm, op):
    try:
        if op[0] == "add":
            return ("ok", bm.add_seq(op[1], op[2]).tolist())
        if op[0] == "fork":
            bm.fork(op[1], op[2])
            return ("ok",)
        if op[0] == "extend":
            s, c = bm.extend(op[1], op[2])
            return ("ok", s.tolist(), c.tolist())
        if op[0] == "append":
            s, c = bm.append_slots(op[1])
            return ("ok", s.tolist(), c.tolist())
        if op[0] == "free":
            bm.free_seq(op[1])
            return ("ok",)
        if op[0] == "release":
            return ("ok", bm.release_before(op[1], op[2]))
        if op[0] == "reorder":
            bm.reorder(op[1], op[2], op[3])
            return ("ok",)
    except pk.PAError as e:
        return ("err", e.code)


_CODE = {om.OUT_OF_BLOCKS: PA_ERR_OUT_OF_BLOCKS, om.UNKNOWN_SEQ: PA_ERR_UNKNOWN_SEQ,
         om.SEQ_EXISTS: PA_ERR_SEQ_EXISTS, om.INVALID_ARG: PA_ERR_INVALID_ARG}


@pytest.mark.parametrize("seed", range(8))
def test_cpp_block_manager_matches_model(seed):
    from tests.test_allocator_model import apply_model
    ops_, N = random_ops(seed, n_ops=500, num_blocks=80)
    order = np.random.default_rng(seed + 50).permutation(N)
    am = AllocatorModel(N, 16, order)
    bm = pk.BlockManager(N, 16, order)
    live = set()
    n_err = 0
    for op in ops_:
        want = apply_model(am, op)
        got = _c_apply(bm, op)
        if want[0] == "err":
            n_err += 1
            assert got == ("err", _CODE[want[1]]), (op, want, got)
        else:
            assert got == want, op
            if op[0] in ("add", "fork"):
                live.add(op[-1] if op[0] == "fork" else op[1])
            if op[0] == "free":
                live.discard(op[1])
        st = bm.stats()
        ms = am.stats()
        for k in ("num_blocks", "free_blocks", "used_blocks", "shared_blocks", "tokens",
                  "slack_slots"):
            assert st[k] == ms[k], (k, op)
    ids = sorted(am.tables)
    mb = max([1] + [len(t) for t in am.tables.values()])
    t_c, l_c = bm.block_tables(ids, mb)
    t_m, l_m = am.block_tables(ids, mb)
    assert np.array_equal(t_c, t_m) and np.array_equal(l_c, l_m)
    for b in range(N):
        assert bm.refcount(b) == am.ref[b]


def test_cpp_block_manager_errors_and_atomicity():
    bm = pk.BlockManager(4, 16)
    bm.add_seq(1, 48)
    bm.add_seq(2, 15)
    before = (bm.stats(), bm.block_tables([1, 2], 4))
    with pytest.raises(pk.PAError) as e:
        bm.append_slots([2, 1])
    assert e.value.code == PA_ERR_OUT_OF_BLOCKS
    after = (bm.stats(), bm.block_tables([1, 2], 4))
    assert before[0] == after[0] and all(np.array_equal(a, b) for a, b in
                                         zip(before[1], after[1]))
    with pytest.raises(pk.PAError) as e:
        bm.append_slots([2, 2])
    assert e.value.code == PA_ERR_INVALID_ARG
    with pytest.raises(pk.PAError) as e:
        bm.add_seq(1, 1)
    assert e.value.code == PA_ERR_SEQ_EXISTS
    with pytest.raises(pk.PAError) as e:
        bm.free_seq(9)
    assert e.value.code == PA_ERR_UNKNOWN_SEQ
    with pytest.raises(pk.PAError):
        pk.BlockManager(4, 16, [0, 1, 1, 2])
    with pytest.raises(pk.PAError):
        bm.block_tables([1], 2)          # seq 1 has 3 blocks


def test_cpp_worked_example_100_tokens():
    bm = pk.BlockManager(16, 16, [3, 7, 1] + [b for b in range(16) if b not in (3, 7, 1)])
    slots = bm.add_seq(0, 100)
    t, l = bm.block_tables([0], 8)
    assert t[0, :3].tolist() == [3, 7, 1] and (t[0] >= 0).sum() == 7 and l[0] == 100
    assert [slots[p] for p in (0, 15, 16, 20, 31, 32, 35, 47)] == [48, 63, 112, 116, 127, 16, 19,
                                                                   31]
    assert bm.stats()["slack_slots"] == 12


def test_cpp_replays_workload_scripts_like_model():
    from workloads import small_case
    from workloads.configs import CONFIG_NAMES
    for name in CONFIG_NAMES:
        case = small_case(name)
        am = AllocatorModel(case.num_blocks, 16, case.free_order)
        bm = pk.BlockManager(case.num_blocks, 16, case.free_order)
        for op in case.script:
            if op[0] == "add":
                assert np.array_equal(am.add_seq(op[1], op[2]), bm.add_seq(op[1], op[2]))
            elif op[0] == "extend":
                a, b = am.extend(op[1], op[2]), bm.extend(op[1], op[2])
                assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
            elif op[0] == "fork":
                am.fork(op[1], op[2])
                bm.fork(op[1], op[2])
            else:
                am.free_seq(op[1])
                bm.free_seq(op[1])
        a, b = am.append_slots(case.batch), bm.append_slots(case.batch)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        mb = max(-(-int(L) // 16) for L in case.lens)
        ta, la = am.block_tables(case.batch, mb)
        tb, lb = bm.block_tables(case.batch, mb)
        assert np.array_equal(ta, tb) and np.array_equal(la, lb)


def test_decode_kernel_choice_is_an_explicit_setting():
    """The plain-FMA switch is set through pa_set_decode_kernel, not read from
    the environment: it changes the plan pa_decode_partition_size reports
    (even split 0 on the matrix cores, 256-token partitions on plain FMAs),
    returns the previous choice and rejects unknown values unchanged."""
    h = pk.lib()
    os.environ["PA_DECODE_KERNEL"] = "generic"       # no longer consulted
    try:
        assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, 0, PA_BF16) == 0
    finally:
        del os.environ["PA_DECODE_KERNEL"]
    assert pk.ops.set_decode_kernel("generic") == "auto"
    try:
        assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, 0, PA_BF16) == 256
        ws_generic = h.pa_decode_workspace_bytes(64, 32, 8, 128, 2048, 0, PA_BF16)
        assert h.pa_set_decode_kernel(7) == 1       # unknown: unchanged, reported
        assert b"unknown kernel" in h.pa_last_error()
    finally:
        assert pk.ops.set_decode_kernel("auto") == "generic"
    assert h.pa_decode_partition_size(64, 32, 8, 128, 2048, 0, PA_BF16) == 0
    assert h.pa_decode_workspace_bytes(64, 32, 8, 128, 2048, 0, PA_BF16) != ws_generic
    with pytest.raises(ValueError):
        pk.ops.set_decode_kernel("fast")


def test_noalloc_step_rejects_sizes_beyond_its_scratch_before_any_device_call():
    """pa_decode_step_noalloc checks the partials it needs against its fixed
    64 MiB array before touching the device: 16 contexts of 131072 tokens on
    the even split need more, and are refused with PA_ERR_WORKSPACE (NULL
    pointers: nothing was launched); bad scalars still get their own error."""
    h = pk.lib()
    nul = None
    need = h.pa_decode_workspace_bytes(16, 32, 8, 128, 131072, -1, PA_BF16)
    assert need > 64 << 20
    assert h.pa_decode_step_noalloc(nul, nul, nul, nul, nul, nul, nul, nul, nul, 16, 32, 8, 128,
                                    16, 100, 8192, 131072, 0.1, -1, PA_BF16,
                                    nul) == PA_ERR_WORKSPACE
    assert b"static scratch" in h.pa_last_error()
    assert h.pa_decode_step_noalloc(nul, nul, nul, nul, nul, nul, nul, nul, nul, 16, 32, 8, 96,
                                    16, 100, 8192, 2048, 0.1, -1, PA_BF16,
                                    nul) == PA_ERR_UNSUPPORTED


def _check_shared_plan(tables, lens, prefix, rows, start, mg, min_blocks=4):
    """Properties every shared-prefix plan must have (host logic)."""
    n = len(lens)
    seen = set()
    assert start[0] == 0 and np.all(np.diff(start) >= 2)
    assert mg == (int(np.diff(start).max()) if len(start) > 1 else 0)
    firsts = []
    for g in range(len(start) - 1):
        mem = rows[start[g]:start[g + 1]].tolist()
        assert mem == sorted(mem) and not seen & set(mem)
        seen |= set(mem)
        P = int(prefix[mem[0]]) // 16
        assert P >= min_blocks and all(int(prefix[i]) == 16 * P for i in mem)
        for i in mem:
            assert 16 * P < lens[i]                          # the member keeps its own tail
            assert np.array_equal(tables[i, :P], tables[mem[0], :P]) and (tables[i, :P] >= 0).all()
        # maximal: the cap is reached, or the next entries differ among members
        cap = min((int(lens[i]) - 1) // 16 for i in mem)
        if P < cap:
            assert len(set(int(tables[i, P]) for i in mem)) > 1 or int(tables[mem[0], P]) < 0
        firsts.append(int(tables[mem[0], 0]))
    assert len(firsts) == len(set(firsts))                  # one group per first block
    for i in range(n):
        if i not in seen:
            assert prefix[i] == 0
    # sequences that start with a grouped first block are in that group
    for i in range(n):
        if lens[i] > 16 * min_blocks and int(tables[i, 0]) in firsts:
            assert i in seen


def test_shared_prefix_plan_groups_parallel_samples_by_prompt():
    from workloads import small_case
    case = small_case("cow_parallel_bf16")                 # 2 prompts of 64 tokens x 4 samples
    ref = om_run(case)
    tables, lens = ref["tables"], ref["lens"]
    prefix, rows, start, mg = pk.ops.shared_prefix_plan(tables, lens, min_shared_blocks=2)
    _check_shared_plan(tables, lens, prefix, rows, start, mg, 2)
    assert len(start) - 1 == 2 and mg == 4
    assert set(prefix.tolist()) == {64}                     # the whole block-aligned prompt


def om_run(case):
    from oracle import run_case
    return run_case(case, with_pools=False)


@pytest.mark.parametrize("seed", range(6))
def test_shared_prefix_plan_properties_on_random_fork_trees(seed):
    rng = np.random.default_rng(seed)
    am = AllocatorModel(4000, 16, rng.permutation(4000).astype(np.int32))
    ids = []
    for p in range(int(rng.integers(1, 6))):
        root = 1000 * p
        am.add_seq(root, int(rng.integers(1, 300)))
        ids.append(root)
        for c in range(int(rng.integers(0, 5))):
            parent = int(rng.choice(ids))
            child = root + c + 1
            am.fork(parent, child)
            if rng.random() < 0.7:
                am.extend(child, int(rng.integers(0, 80)))
            ids.append(child)
    batch = [i for i in ids if am.seq_len(i) > 0]
    rng.shuffle(batch)
    am.append_slots(batch)
    mb = max(-(-am.seq_len(i) // 16) for i in batch)
    tables, lens = am.block_tables(batch, mb)
    for mn in (1, 2, 4):
        prefix, rows, start, mg = pk.ops.shared_prefix_plan(tables, lens, min_shared_blocks=mn)
        _check_shared_plan(tables, lens, prefix, rows, start, mg, mn)


def test_shared_prefix_plan_rejects_bad_arguments():
    h = pk.lib()
    ng, mg = C.c_int32(), C.c_int32()
    assert h.pa_shared_prefix_plan(None, None, -1, 4, 16, 1, None, None, None, C.byref(ng),
                                   C.byref(mg)) == PA_ERR_INVALID_ARG
    assert h.pa_shared_prefix_plan(None, None, 3, 4, 16, 1, None, None, None, C.byref(ng),
                                   C.byref(mg)) == PA_ERR_INVALID_ARG
    assert h.pa_shared_prefix_plan(None, None, 3, 4, 16, 0, None, None, None, C.byref(ng),
                                   C.byref(mg)) == PA_ERR_INVALID_ARG


def test_decode_step_shared_rejects_bad_arguments_before_any_launch():
    """pa_decode_step_shared checks its scalars on the host, before the
    prefix pass or any other device call: an unsupported dtype, a scale that
    is not positive and finite, inconsistent group counts, a missing prefix
    array, a short workspace."""
    from paged_kv_cache_212_amd._lib import PA_F32
    h = pk.lib()
    nul = None

    def call(dtype=PA_BF16, scale=0.088, groups=1, rows=2, max_group=2, B=4, prefix=nul,
             ws=nul, ws_bytes=0):
        return h.pa_decode_step_shared(nul, nul, nul, nul, nul, nul, nul, nul, nul, prefix, nul,
                                       nul, groups, rows, max_group, B, 32, 8, 128, 16, 64, 8,
                                       100, scale, dtype, ws, ws_bytes, nul)
    assert call(dtype=PA_F32) == PA_ERR_UNSUPPORTED
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert call(scale=bad) == PA_ERR_INVALID_ARG
    assert call(groups=1, rows=1) == PA_ERR_INVALID_ARG          # a group of one
    assert call(groups=2, rows=3) == PA_ERR_INVALID_ARG          # fewer than 2 per group
    assert call(groups=1, rows=2, max_group=3) == PA_ERR_INVALID_ARG
    assert call(rows=5) == PA_ERR_INVALID_ARG                    # more rows than sequences
    assert call() == PA_ERR_INVALID_ARG                          # no prefix array
    need = h.pa_decode_shared_workspace_bytes(4, 32, 8, 128, 100, PA_BF16)
    assert need > 0
    fake = C.c_void_p(256)                                       # never dereferenced
    assert call(groups=0, rows=0, max_group=0, prefix=fake, ws=fake,
                ws_bytes=need - 1) == PA_ERR_WORKSPACE


@pytest.mark.parametrize("seed", range(6))
def test_pa_bm_step_matches_model_append_then_tables(seed):
    """pa_bm_step against the allocator model over random op sequences: each
    batch reservation goes through the one-call step (starting from a random,
    often too small, table width, so the grow-and-retry path runs), and its
    slots, copy pairs, tables and lengths equal the model's append_slots then
    block_tables; failures give the model's error code and change nothing."""
    from tests.test_allocator_model import apply_model
    ops_, N = random_ops(seed + 100, n_ops=400, num_blocks=80)
    order = np.random.default_rng(seed + 7).permutation(N)
    am = AllocatorModel(N, 16, order)
    bm = pk.BlockManager(N, 16, order)
    rng = np.random.default_rng(seed)
    steps = 0
    for op in ops_:
        if op[0] != "append":
            want, got = apply_model(am, op), _c_apply(bm, op)
            assert (got == ("err", _CODE[want[1]])) if want[0] == "err" else got == want, op
            continue
        ids = list(op[1])
        want = apply_model(am, op)
        before = bm.stats()
        try:
            s, c, t, l = bm.step(ids, int(rng.integers(0, 4)))
            got = ("ok", s.tolist(), c.tolist())
        except pk.PAError as e:
            got = ("err", e.code)
        if want[0] == "err":
            assert got == ("err", _CODE[want[1]]), (op, want, got)
            assert bm.stats() == before
            continue
        assert got == want, op
        steps += 1
        mb = max([1] + [len(am.tables[i]) for i in ids])
        t_m, l_m = am.block_tables(ids, mb)
        assert t.shape == t_m.shape and np.array_equal(t, t_m) and np.array_equal(l, l_m)
    assert steps > 10


def test_pa_bm_step_width_and_argument_errors_change_nothing():
    h = pk.lib()
    bm = pk.BlockManager(8, 16)
    bm.add_seq(1, 32)                       # the step needs a third block
    bm.add_seq(2, 5)
    n = 2
    ids = np.array([1, 2], dtype=np.int64)
    slots = np.empty(n, np.int64)
    pairs = np.empty((n, 2), np.int32)
    tables = np.empty((n, 2), np.int32)
    lens = np.empty(n, np.int32)
    ncow, need = C.c_int32(0), C.c_int32(0)
    before = bm.stats()
    st = h.pa_bm_step(bm._h, ids.ctypes.data, n, 2, slots.ctypes.data, pairs.ctypes.data,
                      C.byref(ncow), tables.ctypes.data, lens.ctypes.data, C.byref(need))
    assert st == PA_ERR_INVALID_ARG and need.value == 3 and bm.stats() == before
    dup = np.array([2, 2], dtype=np.int64)
    wide = np.empty((n, 4), np.int32)
    st = h.pa_bm_step(bm._h, dup.ctypes.data, n, 4, slots.ctypes.data, pairs.ctypes.data,
                      C.byref(ncow), wide.ctypes.data, lens.ctypes.data, C.byref(need))
    assert st == PA_ERR_INVALID_ARG and bm.stats() == before
    unknown = np.array([1, 9], dtype=np.int64)
    st = h.pa_bm_step(bm._h, unknown.ctypes.data, n, 4, slots.ctypes.data, pairs.ctypes.data,
                      C.byref(ncow), wide.ctypes.data, lens.ctypes.data, C.byref(need))
    assert st == PA_ERR_UNKNOWN_SEQ and bm.stats() == before
    assert h.pa_bm_step(bm._h, ids.ctypes.data, n, 4, None, None, None, None, None,
                        C.byref(need)) == PA_ERR_INVALID_ARG
    s, c, t, l = bm.step(ids, 1)
    assert t.shape == (2, 3) and l.tolist() == [33, 6] and s.tolist()[1] == t[1, 0] * 16 + 5


def test_bm_step_outputs_stay_valid_across_calls():
    """BlockManager.step returns views of one fresh block per call: the arrays
    of an earlier step keep their values after later steps, have the dtypes
    and shapes of the C outputs, and agree with append_slots/block_tables on a
    replica manager."""
    a = pk.BlockManager(64, 16)
    b = pk.BlockManager(64, 16)
    for m in (a, b):
        m.add_seq(1, 31)
        m.add_seq(2, 16)
        m.fork(1, 3)
    ids = np.array([1, 2, 3], dtype=np.int64)
    first = a.step(ids, 1)
    kept = [x.copy() for x in first]
    s_b, c_b = b.append_slots(ids)
    t_b, l_b = b.block_tables(ids, first[2].shape[1])
    for _ in range(5):
        a.step(ids, 4)
    for x, y in zip(first, kept):
        assert np.array_equal(x, y)
    s, c, t, l = first
    assert s.dtype == np.int64 and l.dtype == np.int32 and t.dtype == np.int32
    assert c.dtype == np.int32 and c.ndim == 2 and c.shape[1] == 2
    assert t.flags.c_contiguous and s.flags.c_contiguous
    assert np.array_equal(s, s_b) and np.array_equal(c, c_b)
    assert np.array_equal(t, t_b) and np.array_equal(l, l_b)
