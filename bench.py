#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV cache on one MI355X.

A step is one pass of the whole device path over one batch: copy-on-write block
copies (when the step's reservation produced any), then pa_decode_step: the
attention kernel, which attends the batch's new tokens from k_new/v_new, then
the merge kernel, which combines the partials and writes the new tokens into
their slots.  The headline pass times the steps alone (events on the stream
before and after the K steps); a second pass attaches two HIP events to each
attention kernel's own dispatch to time that kernel (the events add a few
microseconds per step, so that pass is not the headline).
The host reservation (slots, copy pairs, block tables) is done by the C++
block manager before the timed region, and the same step is replayed every
iteration (append and copy are idempotent, so every replay does the full work).
Each iteration uses the next of ``--layers`` identical pool copies, as the
layers of a model would, so that no pool is re-read before the others have
streamed through the 256 MB memory-side cache.

Prints one JSON line.  ``value`` is KV bytes read per step / step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV GB/s (% of HBM peak) + µs/step, Llama-3-8B shape"
# metric label of every other workload (the headline metric is the Llama-3-8B one)
WORKLOAD_LABEL = {
    "llama3_8b_bf16": "Llama-3-8B shape",
    "opt13b_fp16": "OPT-13B shape (MHA, 40 heads, fp16)",
    "cow_parallel_bf16": "Llama-3-8B heads, parallel sampling with shared prompt blocks",
    "long_context_bf16": "Llama-3-8B heads, long contexts (32K-131K tokens)",
    "tiny_fp32": "tiny fp32 case",
}


def metric_for(workload: str, variant: str = "") -> str:
    if workload == "llama3_8b_bf16" and not variant:
        return METRIC
    label = WORKLOAD_LABEL.get(workload, workload)
    return ("paged decode attention KV GB/s (% of HBM peak) + µs/step, " + label
            + (f", {variant}" if variant else ""))
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_212_amd", "csrc", "pa_decode.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="llama3_8b_bf16")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--cow-literal", action="store_true",
                    help="cow_parallel_bf16 read literally: block-aligned prompts, no parked "
                         "forks, so the step makes no copy-on-write copy")
    ap.add_argument("--shared-prefix", type=int, default=0, metavar="M",
                    help="prefixes shared by groups of sequences (forks of one prompt) of at "
                         "least M blocks are attended once per group: one "
                         "pa_decode_step_shared per step, planned on the host before the "
                         "timed region (0 = off)")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--q-heads", type=int, default=0,
                    help="llama3_8b_bf16 with this many query heads over its 8 KV heads "
                         "(e.g. 64: 8 query heads per KV head)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU-oracle baseline (0 = skip)")
    ap.add_argument("--mode", choices=("phased", "separate", "step"), default="step",
                    help="step: one pa_decode_step call (the attention kernel with the new "
                         "tokens fused in, then the merge kernel, which writes them); "
                         "phased: pa_decode_step_partial then pa_decode_step_merge; "
                         "separate: pa_cache_append, pa_decode_partial, pa_decode_merge.  "
                         "The attention kernel's dispatch is timed in a second pass")
    ap.add_argument("--prefill", action="store_true",
                    help="measure pa_prefill instead (chunked prefill, Llama-3-8B heads: "
                         "16 sequences of 2048 tokens, the last 512 as the chunk)")
    ap.add_argument("--kv-cache", choices=("fp8", "i8"), default=None,
                    help="quantized cache: the same workload with 8-bit K/V codes (FP8 E4M3 "
                         "or INT8, per-pool scales); one pa_decode_step_quant per step "
                         "(attention kernel with the new tokens encoded in, timed; merge)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: the step attends the last W positions; the "
                         "sequences first release their out-of-window blocks "
                         "(pa_bm_release_before); one pa_decode_step_window per step")
    ap.add_argument("--beam", action="store_true",
                    help="measure a beam-search loop instead (16 prompts x 4 beams, "
                         "reorder + copy-on-write over --beam-layers layers + decode per layer)")
    ap.add_argument("--beam-layers", type=int, default=8)
    ap.add_argument("--no-events", action="store_true",
                    help="skip the second pass, which times each attention kernel with "
                         "events attached to its dispatch")
    ap.add_argument("--record-traffic", nargs=4, default=None,
                    metavar=("WORKLOAD", "RUN_DIR", "CALIB_DIR", "KERNEL"),
                    help="store the HBM traffic of KERNEL (a substring of its name) for "
                         "WORKLOAD in profiles/decode_traffic.json, from rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE csv runs RUN_DIR/FETCH_SIZE and "
                         "RUN_DIR/WRITE_SIZE of this script, scaled by the same counters over "
                         "--copy-calibration runs in CALIB_DIR/FETCH_SIZE and "
                         "CALIB_DIR/WRITE_SIZE, then exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB elementwise copy 5 times (reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_calibration():
    """A plain fp32 elementwise copy of known size: reads 1 GiB, writes 1 GiB per launch."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": n * 4,
                      "copy_calibration_bytes_written_per_launch": n * 4, "launches": 5}))


def counter_per_dispatch(run_dir: str, counter: str, kernel: str):
    """Mean over the dispatches of kernels whose name contains `kernel` of a
    rocprofv3 --pmc counter (csv output, summed over its instances), and the
    dispatch count."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} samples for kernels matching {kernel!r} in {run_dir}")
    return sum(per.values()) / len(per), len(per)


def record_traffic(workload, run_dir, calib_dir, kernel):
    """HBM bytes per launch of `kernel` for `workload`: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) scaled by what they read for the copy
    calibration's known 1 GiB read and 1 GiB written per launch."""
    cf, _ = counter_per_dispatch(os.path.join(calib_dir, "FETCH_SIZE"), "FETCH_SIZE", "Unary")
    cw, _ = counter_per_dispatch(os.path.join(calib_dir, "WRITE_SIZE"), "WRITE_SIZE", "Unary")
    fetch_scale, write_scale = (1 << 30) / (cf * 1024), (1 << 30) / (cw * 1024)
    f, n = counter_per_dispatch(os.path.join(run_dir, "FETCH_SIZE"), "FETCH_SIZE", kernel)
    w, _ = counter_per_dispatch(os.path.join(run_dir, "WRITE_SIZE"), "WRITE_SIZE", kernel)
    rd, wr = f * 1024 * fetch_scale, w * 1024 * write_scale
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        t = {}
    t[workload] = {"kernel_src_sha256_16": kernel_src_hash(), "kernel": kernel,
                   "hbm_bytes_per_launch": int(round(rd + wr)), "read_bytes": int(round(rd)),
                   "write_bytes": int(round(wr)), "fetch_scale": fetch_scale,
                   "write_scale": write_scale, "fetch_kib_per_dispatch": round(f, 1),
                   "write_kib_per_dispatch": round(w, 1), "dispatches": n}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(dict(sorted(t.items())), fh, indent=1)
        fh.write("\n")
    print(json.dumps({workload: t[workload]}))


def kernel_src_hash() -> str:
    """Hash of the decode kernels' source with comments and whitespace removed,
    so that only a change to the code itself invalidates stored counters."""
    src = open(DECODE_SRC, encoding="utf-8").read()
    src = re.sub(r"//[^\n]*", "", src)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return hashlib.sha256(" ".join(src.split()).encode()).hexdigest()[:16]


def traffic_for(workload: str):
    """HBM bytes per partition launch from committed rocprofv3 counters, if they
    were taken on the current decode kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_src_sha256_16") != kernel_src_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def stream_read_context(torch, dev):
    """Context figure: the chip's streaming-read bandwidth on the same GPU
    (pa_stream_read over a 2 GiB buffer, 5 timed passes after 2 warm-up)."""
    from paged_kv_cache_212_amd._lib import check, lib
    n = 2 << 30
    x = torch.ones(n // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        check(lib().pa_stream_read(x.data_ptr(), n, sink.data_ptr(), s), "pa_stream_read")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        check(lib().pa_stream_read(x.data_ptr(), n, sink.data_ptr(), s), "pa_stream_read")
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x
    torch.cuda.empty_cache()
    return {"gbs": round(gbs, 1), "how": "pa_stream_read over a 2 GiB buffer"}


def cpu_baseline(case, budget_s: float):
    """The fp64 oracle on the same step: copy pairs, append, decode_ref.

    Sample: whole decode steps over the full batch, repeated while the time
    budget lasts (at least one)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import append_ref, bits_of, copy_ref, decode_ref, quantize_ref, run_case
    cores = len(os.sched_getaffinity(0))
    cd = case.cache_dtype
    with threadpool_limits(limits=cores):
        ref = run_case(case, decode=False)               # set-up state (not timed)
        kp, vp = ref["k_pool"], ref["v_pool"]
        nr = case.new_rows()
        kb, vb = bits_of(case.k_tok[nr], case.dtype), bits_of(case.v_tok[nr], case.dtype)
        qb = bits_of(case.q, case.dtype)
        times, t_end = [], time.perf_counter() + budget_s
        while not times or time.perf_counter() < t_end:
            t0 = time.perf_counter()
            copy_ref(kp, vp, ref["step_cows"])
            if cd is None:
                append_ref(kp, vp, kb, vb, ref["step_slots"], case.block_size)
            else:     # quantizing append of the new tokens
                append_ref(kp, vp, quantize_ref(kb, case.dtype, cd, case.k_scale),
                           quantize_ref(vb, case.dtype, cd, case.v_scale), ref["step_slots"],
                           case.block_size)
            decode_ref(qb, kp, vp, ref["tables"], ref["lens"], case.kv_dtype, case.scale,
                       case.block_size, q_dtype=case.dtype, k_scale=case.k_scale,
                       v_scale=case.v_scale, window=case.window)
            times.append(time.perf_counter() - t0)
    sec = float(np.mean(times))
    return {"value": round(case.kv_bytes() / sec / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "s_per_step": round(sec, 3),
            "sample": f"{len(times)} full decode step(s) of the same workload (all "
                      f"{case.num_seqs} sequences: copy pairs, append, fp64 decode_ref)"}


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak (no sparsity)


def prefill_bench(args):
    """Chunked prefill over the paged cache: B = 16 sequences of L = 2048
    tokens (Llama-3-8B heads, bf16, shuffled blocks), whose last n = 512 tokens
    are the chunk.  One call = one pa_prefill launch; value = causal-attention
    flops (4*D per attended (query, key, head)) per second."""
    import numpy as np
    import torch

    import paged_kv_cache_212_amd as pk
    from workloads.configs import prefill_case

    B, L, n, Hq, Hkv, D = 16, 2048, 512, 32, 8, 128
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    case, q, qs = prefill_case(21, "bf16", [L] * B, [n] * B, Hq, Hkv, D, device=dev)
    cache = pk.PagedKVCache(case.num_blocks, Hkv, D, torch.bfloat16, dev,
                            free_order=case.free_order, fill=0.0)
    cache.replay(case.script, case.rows, case.k_tok, case.v_tok)
    plan = cache.plan_step(case.batch)
    nr = torch.as_tensor(case.new_rows(), device=dev)
    pk.ops.cache_append(cache.k_pool, cache.v_pool, case.k_tok.index_select(0, nr).contiguous(),
                        case.v_tok.index_select(0, nr).contiguous(), plan.d_slots)
    layers = [(cache.k_pool, cache.v_pool)] + [(cache.k_pool.clone(), cache.v_pool.clone())
                                               for _ in range(args.layers - 1)]
    qs_d = torch.as_tensor(qs, dtype=torch.int32, device=dev)
    out = torch.empty((q.shape[0], Hq, D), dtype=torch.float32, device=dev)

    def call(i):
        kp, vp = layers[i % len(layers)]
        pk.ops.prefill(out, q, kp, vp, plan.d_tables, plan.d_lens, qs_d, plan.max_context_len, n)

    steps = max(1, args.steps // 10)
    for i in range(max(2, args.warmup // 10)):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    attended = B * sum(L - n + i + 1 for i in range(n))        # (query, key) pairs per head
    flops = 4 * D * Hq * attended
    tflops = flops / (us * 1e-6) / 1e12
    kv_unique = B * L * Hkv * 2 * D * 2
    res = {"metric": "paged chunked-prefill attention TFLOP/s, Llama-3-8B shape",
           "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
           "us_per_call": round(us, 2), "higher_is_better": True, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": f"chunked prefill: B={B} sequences of L={L} tokens, last "
                                  f"n={n} as the chunk, Hq={Hq}, Hkv={Hkv}, D={D}, block 16",
                      "query_tokens": B * n, "attended_pairs_per_head": attended,
                      "layers_rotated": args.layers},
           "kv_unique_bytes": kv_unique,
           "roofline": {"kernel": "prefill_pp_kernel (pa_prefill)", "bound": "mfma",
                        "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": None}}
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = prefill_cpu_baseline(case, q, qs, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def beam_bench(args):
    """Beam search over the paged cache: 16 prompts of 1024 tokens x 4 beams
    (64 sequences, Llama-3-8B heads, bf16), --beam-layers layers of pools.
    A step is: host bookkeeping (draw parents, pa_bm_reorder, pa_bm_step: the
    slot reservation and table export written straight into a pinned buffer,
    one upload), pa_copy_blocks_layers over every layer, then
    one pa_decode_step per layer (new token appended, attention, merge).
    Reported: µs per step (wall, synchronised each step as a sampler would),
    the device part, the copy kernel against HBM, and blocks in use against
    the same beams without sharing."""
    import ctypes as C

    import numpy as np
    import torch

    import paged_kv_cache_212_amd as pk
    from paged_kv_cache_212_amd._lib import check, lib
    from paged_kv_cache_212_amd.ops import pa_dtype

    P, K, plen, Hq, Hkv, D = 16, 4, 1024, 32, 8, 128
    nl = args.beam_layers
    B = P * K
    steps, warmup = min(args.steps, 128), min(args.warmup, 16)
    total_steps = warmup + steps
    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    rng = np.random.default_rng(31)
    N = P * (plen // 16) + B * (total_steps // 16 + 3) * 2 + 64
    bm = pk.BlockManager(N, 16, rng.permutation(N).astype(np.int32))
    g = torch.Generator(device=dev).manual_seed(31)
    pools = [pk.ops.new_pools(N, Hkv, D, torch.bfloat16, dev, fill=0) for _ in range(nl)]
    ids = []
    for p in range(P):
        pid = 1_000_000 + p
        slots = bm.add_seq(pid, plen)
        d_slots = torch.from_numpy(slots.astype(np.int64)).to(dev)
        for kp, vp in pools:
            kk = torch.randn((plen, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
            vv = torch.randn((plen, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
            pk.ops.cache_append(kp, vp, kk, vv, d_slots)
        for k in range(K):
            bm.fork(pid, p * K + k)
            ids.append(p * K + k)
        bm.free_seq(pid)
    next_id = B
    q = [torch.randn((B, Hq, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(nl)]
    k_new = [torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(nl)]
    v_new = [torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(nl)]
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    maxL = plen + total_steps + 1
    MB = -(-maxL // 16)
    ws = pk.ops.decode_workspace(B, Hq, Hkv, D, maxL, 0, torch.bfloat16, dev)
    kptr = torch.tensor([kp.data_ptr() for kp, _ in pools], dtype=torch.int64, device=dev)
    vptr = torch.tensor([vp.data_ptr() for _, vp in pools], dtype=torch.int64, device=dev)
    L = lib()
    stream = torch.cuda.current_stream().cuda_stream
    dt = pa_dtype(torch.bfloat16)
    block_bytes = Hkv * 16 * D * 2
    host_us, cpp_us, wall_us, dev_us, copy_us, ncopies = [], [], [], [], [], []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    # one pinned staging buffer and one upload per step: slots (int64), then
    # the int32 copy pairs, tables and lengths
    n32 = 2 * B + B * MB + B
    stage = torch.empty(B * 8 + n32 * 4, dtype=torch.uint8, pin_memory=True)
    d_stage = torch.empty_like(stage, device=dev)
    st_base = stage.data_ptr()
    st_lens = stage.numpy()[B * 8 + (2 * B + B * MB) * 4:].view(np.int32)   # lengths written
    f_bm_step = L.pa_bm_step
    ncow, need = C.c_int32(0), C.c_int32(0)
    base = np.arange(P)[:, None] * K
    import gc
    gc.disable()        # no collector pauses inside the timed host work
    for t in range(total_steps):
        w0 = time.perf_counter()
        # parents per prompt: sorted draws with replacement; a parent's first
        # child keeps its id, later children get fresh ids
        par = np.sort(rng.integers(0, K, size=(P, K)), axis=1)
        first = np.ones((P, K), dtype=bool)
        first[:, 1:] = par[:, 1:] != par[:, :-1]
        parents = (base + par).ravel()
        old = np.asarray(ids, dtype=np.int64)
        new = old[parents].copy()
        nfresh = int((~first).sum())
        new[~first.ravel()] = np.arange(next_id, next_id + nfresh)
        next_id += nfresh
        c0 = time.perf_counter()
        bm.reorder(old, new, parents)
        ids = np.ascontiguousarray(new)
        # pa_bm_step writes slots, copy pairs, tables (row stride MB) and
        # lengths straight into the pinned staging buffer
        check(f_bm_step(bm._h, ids.__array_interface__["data"][0], B, MB, st_base,
                        st_base + B * 8, C.byref(ncow), st_base + B * 8 + 2 * B * 4,
                        st_base + B * 8 + (2 * B + B * MB) * 4, C.byref(need)), "pa_bm_step")
        c1 = time.perf_counter()
        nc = ncow.value
        d_stage.copy_(stage, non_blocking=True)
        d_i32 = d_stage[B * 8:].view(torch.int32)
        d_slots = d_stage[:B * 8].view(torch.int64)
        d_cows = d_i32[:2 * B]
        d_tables = d_i32[2 * B:2 * B + B * MB]
        d_lens = d_i32[2 * B + B * MB:]
        h1 = time.perf_counter()
        ev[0].record()
        ev[1].record()
        if nc:
            check(L.pa_copy_blocks_layers(kptr.data_ptr(), vptr.data_ptr(), nl, d_cows.data_ptr(),
                                          nc, N, Hkv, D, 16, dt, stream), "pa_copy_blocks_layers")
        ev[2].record()
        for li, (kp, vp) in enumerate(pools):
            check(L.pa_decode_step(out.data_ptr(), q[li].data_ptr(), kp.data_ptr(), vp.data_ptr(),
                                   k_new[li].data_ptr(), v_new[li].data_ptr(), d_slots.data_ptr(),
                                   d_tables.data_ptr(), d_lens.data_ptr(), B, Hq, Hkv, D, 16, N,
                                   MB, int(st_lens.max()), D ** -0.5, 0, dt, ws.data_ptr(),
                                   ws.numel(), stream), "pa_decode_step")
        ev[3].record()
        torch.cuda.synchronize()
        w1 = time.perf_counter()
        if t >= warmup:
            host_us.append((h1 - w0) * 1e6)
            cpp_us.append((c1 - c0) * 1e6)
            wall_us.append((w1 - w0) * 1e6)
            dev_us.append(ev[0].elapsed_time(ev[3]) * 1e3)
            copy_us.append(ev[1].elapsed_time(ev[2]) * 1e3)
            ncopies.append(nc)
    gc.enable()
    st = bm.stats()
    unshared = int(sum(-(-int(x) // 16) for x in st_lens))
    pairs = float(np.mean(ncopies))
    copy_bytes = pairs * nl * 2 * block_bytes * 2          # read + write, K and V, all layers
    copy_gbs = copy_bytes / (float(np.mean(copy_us)) * 1e-6) / 1e9 if pairs else 0.0
    res = {"metric": f"beam-search decode step over {nl} layers, µs/step (Llama-3-8B heads)",
           "value": round(float(np.mean(wall_us)), 2), "unit": "us/step", "n_gpus": 1,
           "steps": steps, "warmup": warmup, "higher_is_better": False, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": f"beam search: {P} prompts of {plen} tokens x {K} beams "
                                  f"(B={B}), Hq={Hq}, Hkv={Hkv}, D={D}, block 16, {nl} layers, "
                                  f"parents drawn with replacement each step",
                      "layers": nl},
           "host_bookkeeping_us_per_step": round(float(np.mean(host_us)), 2),
           "host_block_manager_us_per_step": round(float(np.mean(cpp_us)), 2),
           "wall_host_bm_device_us_p50": [round(float(np.median(x)), 2)
                                          for x in (wall_us, host_us, cpp_us, dev_us)],
           "device_us_per_step": round(float(np.mean(dev_us)), 2),
           "copy_pairs_per_step": round(pairs, 2),
           "copy_us_per_step": round(float(np.mean(copy_us)), 2),
           "blocks_used": int(st["used_blocks"]), "blocks_without_sharing": unshared,
           "shared_blocks": int(st["shared_blocks"]),
           "roofline": {"kernel": "copy_blocks_layers_kernel (pa_copy_blocks_layers; events "
                                  "around the launch)",
                        "bound": "hbm", "achieved": round(copy_gbs, 2), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(copy_gbs / HBM_PEAK_GBS, 4),
                        "traffic": None, "algorithmic_bytes": int(copy_bytes)}}
    print(json.dumps(res), flush=True)


def prefill_cpu_baseline(case, q, qs, budget_s):
    """The fp64 oracle (prefill_ref) on a bounded sample: query rows of the
    first sequence, 64 at a time, while the budget lasts; flops counted as in
    the GPU figure."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import bits_of, run_case
    from oracle.prefill import prefill_ref
    import dataclasses
    cores = len(os.sched_getaffinity(0))
    cpu_case = dataclasses.replace(case, k_tok=case.k_tok.cpu(), v_tok=case.v_tok.cpu(),
                                   q=case.q.cpu())
    ref = run_case(cpu_case, decode=False)
    qb = bits_of(q.cpu(), "bf16")
    L, n = int(case.lens[0]), int(qs[1] - qs[0])
    Hq, D = qb.shape[1], qb.shape[2]
    flops = 0
    rows = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        while time.perf_counter() - t0 < budget_s and rows < n:
            k = min(64, n - rows)
            # rows [rows, rows + k) of sequence 0's chunk: a chunk of k tokens ending
            # at position L - n + rows + k - 1
            Lk = L - n + rows + k
            prefill_ref(qb[rows:rows + k], ref["k_pool"], ref["v_pool"], ref["tables"][:1],
                        np.array([Lk]), np.array([0, k]), "bf16")
            flops += 4 * D * Hq * sum(Lk - k + i + 1 for i in range(k))
            rows += k
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{rows} query rows of sequence 0's chunk, {k if rows else 0} at a time"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the decode path has "
                                   "no multi-GPU sharding (see the design notes); run with "
                                   "--gpus 1"}))
        sys.exit(2)
    if args.prefill:
        prefill_bench(args)
        return
    if args.beam:
        beam_bench(args)
        return

    import numpy as np
    import torch

    import paged_kv_cache_212_amd as pk
    from paged_kv_cache_212_amd._lib import check, lib
    from paged_kv_cache_212_amd.ops import pa_dtype
    from workloads import make_case
    from workloads.configs import quantized, windowed

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.q_heads and args.workload != "llama3_8b_bf16":
        print(json.dumps({"error": "--q-heads applies to the llama3_8b_bf16 workload"}))
        sys.exit(2)
    if args.cow_literal and args.workload != "cow_parallel_bf16":
        print(json.dumps({"error": "--cow-literal applies to the cow_parallel_bf16 workload"}))
        sys.exit(2)
    kw = {"q_heads": args.q_heads} if args.q_heads else {}
    if args.cow_literal:
        kw["parked_forks"] = False
    case = make_case(args.workload, device=dev, **kw)
    if args.cow_literal:
        case.name = f"{case.name}_literal"
    if args.q_heads:
        case.name = f"{case.name}_hq{args.q_heads}"
    if args.shared_prefix:
        case.name = f"{case.name}_shared"
    quant = args.kv_cache is not None
    if quant:
        case = quantized(case, args.kv_cache)
    window = int(args.window)
    if window and quant:
        print(json.dumps({"error": "--window takes fp32/fp16/bf16 pools"}))
        sys.exit(2)
    if args.shared_prefix and (quant or window or args.mode != "step" or
                               args.partition_size not in (None, 0, -1)):
        print(json.dumps({"error": "--shared-prefix takes the fused step over fp16/bf16 pools, "
                                   "no window, the even split"}))
        sys.exit(2)
    if window:
        case = windowed(case, window, reuse=False)
        if args.partition_size is None:
            # a window keeps every range short: the library's even split
            case.partition_size = 0
    P = case.partition_size if args.partition_size is None else args.partition_size
    td = case.k_tok.dtype
    pool_td = {"fp8": torch.float8_e4m3fn, "i8": torch.int8}.get(args.kv_cache, td)
    print(f"[bench] {case.name}: B={case.num_seqs} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
          f"D={case.head_dim} {case.kv_dtype} sumL={int(case.lens.sum())} "
          f"blocks={case.num_blocks}", file=sys.stderr, flush=True)

    cache = pk.PagedKVCache(case.num_blocks, case.num_kv_heads, case.head_dim, td, dev,
                            free_order=case.free_order, fill=0,
                            cache_dtype=pool_td if quant else None, k_scale=case.k_scale,
                            v_scale=case.v_scale)
    cache.replay(case.script, case.rows, case.k_tok, case.v_tok)
    # host reservation for the step (C++ block manager), timed on its own on a
    # replica manager: slots + copy pairs + block-table export for the batch
    replica = pk.BlockManager(case.num_blocks, 16, case.free_order)
    for op in case.script:
        if op[0] == "add":
            replica.add_seq(op[1], op[2])
        elif op[0] == "extend":
            replica.extend(op[1], op[2])
        elif op[0] == "fork":
            replica.fork(op[1], op[2])
        elif op[0] == "release":
            replica.release_before(op[1], op[2])
        else:
            replica.free_seq(op[1])
    mb_plan = max(-(-int(x) // 16) for x in case.lens)
    batch_ids = np.ascontiguousarray(case.batch, dtype=np.int64)
    replica.step(batch_ids[:0], mb_plan)          # first-call set-up outside the timing
    plan_us = []
    for _ in range(20):                           # 20 consecutive steps; the median is reported
        t0 = time.perf_counter()
        tab = replica.step(batch_ids, mb_plan)[2]     # pa_bm_step: reserve + table export
        plan_us.append((time.perf_counter() - t0) * 1e6)
        mb_plan = max(mb_plan, tab.shape[1])
    host_plan_us = float(np.median(plan_us))
    plan = cache.plan_step(case.batch)
    nr = torch.as_tensor(case.new_rows(), device=dev)
    k_new = case.k_tok.index_select(0, nr).contiguous()
    v_new = case.v_tok.index_select(0, nr).contiguous()
    q = case.q.contiguous()
    cpu_case = None
    if args.cpu_seconds > 0:        # the oracle baseline reads the same stored bits
        import dataclasses
        cpu_case = dataclasses.replace(case, k_tok=case.k_tok.cpu(), v_tok=case.v_tok.cpu(),
                                       q=case.q.cpu())
    case.k_tok = case.v_tok = None
    layers = [(cache.k_pool, cache.v_pool)] + [(cache.k_pool.clone(), cache.v_pool.clone())
                                               for _ in range(args.layers - 1)]
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    B, Hq, D = q.shape
    Hkv, N = case.num_kv_heads, case.num_blocks
    MB = plan.tables.shape[1]
    ws = pk.ops.decode_workspace(B, Hq, Hkv, D, plan.max_context_len, P, pool_td, dev)
    P_used = pk.ops.decode_partition_size(B, Hq, Hkv, D, plan.max_context_len, P, pool_td)
    ncow = int(plan.cows.shape[0])
    shared = None
    if args.shared_prefix:
        # the host plan of the shared prefixes, timed on its own (it is made once
        # per step for all layers, from the tables the reservation exported)
        t0 = time.perf_counter()
        sh_pre, sh_rows, sh_start, sh_mg = pk.ops.shared_prefix_plan(plan.tables, plan.lens,
                                                                     args.shared_prefix)
        host_shared_plan_us = (time.perf_counter() - t0) * 1e6
        shared = cache.shared_plan(plan, args.shared_prefix)
        ws_sh = pk.ops.decode_shared_workspace(B, Hq, Hkv, D, plan.max_context_len, pool_td,
                                               dev)
        P_used = -1
    torch.cuda.synchronize()

    # Pre-bound C calls: the loop below only issues launches.
    L = lib()
    dt = pa_dtype(pool_td)
    stream = torch.cuda.current_stream().cuda_stream
    calls = []
    for kp, vp in layers:
        if window:
            # pa_decode_step_window: append + attention over the last W positions (+ merge)
            dec = (out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(), k_new.data_ptr(),
                   v_new.data_ptr(), plan.d_slots.data_ptr(), plan.d_tables.data_ptr(),
                   plan.d_lens.data_ptr(), B, Hq, Hkv, D, 16, N, MB, plan.max_context_len,
                   case.scale, window, P, dt, ws.data_ptr(), ws.numel(), stream)
            calls.append(((kp.data_ptr(), vp.data_ptr(), plan.d_cows.data_ptr(), ncow, N, Hkv,
                           D, 16, dt, stream), dec, None, None))
            continue
        if quant:
            # pa_decode_step_quant: quantizing append + attention (+ merge)
            dec = (out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(), k_new.data_ptr(),
                   v_new.data_ptr(), plan.d_slots.data_ptr(), plan.d_tables.data_ptr(),
                   plan.d_lens.data_ptr(), B, Hq, Hkv, D, 16, N, MB, plan.max_context_len,
                   case.scale, P, dt, case.k_scale, case.v_scale, ws.data_ptr(), ws.numel(),
                   stream)
            calls.append(((kp.data_ptr(), vp.data_ptr(), plan.d_cows.data_ptr(), ncow, N, Hkv,
                           D, 16, dt, stream), dec, None, None))
            continue
        if shared is not None:
            # pa_decode_step_shared: prefix pass + the rest on the even split + merge
            pre_d, rows_d, start_d, mg = shared
            dec = (out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(),
                   k_new.data_ptr(), v_new.data_ptr(), plan.d_slots.data_ptr(),
                   plan.d_tables.data_ptr(), plan.d_lens.data_ptr(), pre_d.data_ptr(),
                   rows_d.data_ptr() if rows_d.numel() else None, start_d.data_ptr(),
                   start_d.numel() - 1, rows_d.numel(), mg, B, Hq, Hkv, D, 16, N, MB,
                   plan.max_context_len, case.scale, dt, ws_sh.data_ptr(), ws_sh.numel(), stream)
            calls.append(((kp.data_ptr(), vp.data_ptr(), plan.d_cows.data_ptr(), ncow, N, Hkv,
                           D, 16, dt, stream), dec, None, None))
            continue
        # pa_decode_step: append of the step's tokens + attention (+ merge)
        dec = (out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(), k_new.data_ptr(),
               v_new.data_ptr(), plan.d_slots.data_ptr(), plan.d_tables.data_ptr(),
               plan.d_lens.data_ptr(), B, Hq, Hkv, D, 16, N, MB, plan.max_context_len,
               case.scale, P, dt, ws.data_ptr(), ws.numel(), stream)
        dec_sep = (out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(),
                   plan.d_tables.data_ptr(), plan.d_lens.data_ptr(), B, Hq, Hkv, D, 16, N, MB,
                   plan.max_context_len, case.scale, P, dt, ws.data_ptr(), ws.numel(), stream)
        app = (kp.data_ptr(), vp.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
               plan.d_slots.data_ptr(), B, N, Hkv, D, 16, dt, stream)
        calls.append((
            (kp.data_ptr(), vp.data_ptr(), plan.d_cows.data_ptr(), ncow, N, Hkv, D, 16, dt,
             stream),
            dec, app, dec_sep))
    f_copy, f_step = L.pa_copy_blocks, L.pa_decode_step
    f_step_part, f_step_merge = L.pa_decode_step_partial, L.pa_decode_step_merge
    f_app, f_part, f_merge = L.pa_cache_append, L.pa_decode_partial, L.pa_decode_merge
    f_time = L.pa_time_next_attention
    f_step_quant, f_step_window = L.pa_decode_step_quant, L.pa_decode_step_window
    f_step_shared = L.pa_decode_step_shared if shared is not None else None
    mode = ("quant" if quant else "window" if window else "shared" if shared is not None
            else args.mode)

    def step(i, ev=None, with_copy=True):
        c_copy, c_dec, c_app, c_dec_sep = calls[i % len(calls)]
        if ncow and with_copy:
            check(f_copy(*c_copy), "pa_copy_blocks")
        if mode in ("quant", "window", "shared"):
            if ev is not None:
                # shared: the events land on the even split's kernel (the
                # private rest), not on the prefix pass before it
                check(f_time(ev[0].cuda_event, ev[1].cuda_event), "pa_time_next_attention")
            if mode == "quant":
                check(f_step_quant(*c_dec), "pa_decode_step_quant")
            elif mode == "shared":
                check(f_step_shared(*c_dec), "pa_decode_step_shared")
            else:
                check(f_step_window(*c_dec), "pa_decode_step_window")
            return
        if args.mode == "step":
            if ev is not None:
                # the first kernel's own dispatch records the two events
                check(f_time(ev[0].cuda_event, ev[1].cuda_event), "pa_time_next_attention")
            check(f_step(*c_dec), "pa_decode_step")
            return
        if args.mode == "separate":
            check(f_app(*c_app), "pa_cache_append")
        if ev is not None:
            # the attention kernel's own dispatch records the two events
            check(f_time(ev[0].cuda_event, ev[1].cuda_event), "pa_time_next_attention")
        if args.mode == "separate":
            check(f_part(*c_dec_sep), "pa_decode_partial")     # the attention kernel
            check(f_merge(*c_dec_sep), "pa_decode_merge")
        else:
            check(f_step_part(*c_dec), "pa_decode_step_partial")   # attention (+ new tokens)
            check(f_step_merge(*c_dec), "pa_decode_step_merge")    # merge + new-token writes

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    def timed(with_events):
        """K steps bracketed by synchronisations and two events on the stream;
        with_events: each attention kernel's dispatch also records two events
        (they add a few microseconds per step)."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(args.steps)] if with_events else None
        if evs:
            for pair in evs:           # torch creates the HIP events on first record
                for e in pair:
                    e.record()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        start.record()
        for i in range(args.steps):
            step(i, evs[i] if evs else None)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps, (time.perf_counter() - w0) * 1e3, evs

    # the headline: nothing but the steps in the timed region
    ms_step, wall_ms, _ = timed(False)
    print(f"[bench] timed {args.steps} steps: {ms_step * 1e3:.2f} us/step", file=sys.stderr,
          flush=True)
    evs, ms_step_ev = None, None
    if not args.no_events:
        ms_step_ev, _, evs = timed(True)
        print(f"[bench] second pass, attention kernels timed: {ms_step_ev * 1e3:.2f} us/step",
              file=sys.stderr, flush=True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    decode_only_us = ms_step * 1e3
    if ncow:
        # the same loop without the copy-on-write copies: decode alone
        torch.cuda.synchronize()
        start.record()
        for i in range(args.steps):
            step(i, None, with_copy=False)
        end.record()
        torch.cuda.synchronize()
        decode_only_us = start.elapsed_time(end) / args.steps * 1e3

    kv_bytes = case.kv_bytes()
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    # unique K/V bytes: blocks shared by several sequences (copy-on-write
    # prefixes) are counted once, at their largest filled length
    fill = np.zeros(N, dtype=np.int64)
    for b_i, L_i in enumerate(plan.lens.tolist()):
        nb = -(-int(L_i) // 16)
        if nb:
            f = np.full(nb, 16, dtype=np.int64)
            f[-1] = int(L_i) - 16 * (nb - 1)
            np.maximum.at(fill, plan.tables[b_i, :nb], f)
    kv_unique = int(fill.sum()) * Hkv * 2 * D * case.elt_bytes
    stream_ctx = stream_read_context(torch, dev)
    variant = ", ".join(x for x in (
        f"{Hq} query heads" if args.q_heads else "",
        f"{case.kv_dtype} KV codes" if quant else "",
        f"sliding window {window}" if window else "",
        "literal reading (no copies)" if args.cow_literal else "",
        f"shared prefixes of >= {args.shared_prefix} blocks attended once per group"
        if shared is not None else "") if x)
    # paging waste: unused slots in the blocks the batch's tables hold
    bm_stats = cache.bm.stats()
    slack = int(bm_stats["slack_slots"])
    res = {"metric": metric_for(args.workload, variant), "value": round(value, 2),
           "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": case.dtype, "data": "synthetic",
           "config": {"workload": f"{case.name}: one decode step, B={B}, Hq={Hq}, Hkv={Hkv}, "
                                  f"D={D}, block 16, "
                                  + (f"{case.kv_dtype} KV codes (per-pool scales, widened "
                                     f"to bf16 on the matrix cores)" if quant else
                                     f"{case.dtype} KV") + ", fp32 out"
                                  + (f", sliding window of {window} positions (out-of-window "
                                     f"blocks released)" if window else ""),
                      "global_batch": B, "context_tokens": int(case.lens.sum()),
                      "max_context_len": plan.max_context_len, "partition_size": P_used,
                      "cow_copies": ncow, "layers_rotated": args.layers,
                      "parallelism": "single GPU"},
           "us_per_step": round(ms_step * 1e3, 3),
           "decode_only_us_per_step": round(decode_only_us, 3),
           "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
           "kv_bytes_per_step": kv_bytes,
           "kv_bytes_unique_per_step": kv_unique,
           "value_unique_gbs": round(kv_unique / (ms_step * 1e-3) / 1e9, 2),
           "stream_read_context": stream_ctx,
           "host_plan_us": round(host_plan_us, 1),
           "pool_blocks_used": int(bm_stats["used_blocks"]),
           "paging_slack_slots": slack,
           "paging_waste_pct": round(100.0 * slack / max(1, slack + int(bm_stats["tokens"])), 3),
           "paging_max_slack_per_seq": int(max(-(-int(x) // 16) * 16 - int(x)
                                               for x in case.lens)),
           "pool_blocks_without_window": int(sum(-(-int(x) // 16) for x in case.lens)),
           "wall_ms_timed_region": round(wall_ms, 3)}
    if shared is not None:
        ng = len(sh_start) - 1
        pre_tok = int(sum(int(sh_pre[int(sh_rows[sh_start[g]])]) for g in range(ng)))
        res["shared_prefix"] = {
            "groups": ng, "members": int(len(sh_rows)), "largest_group": int(sh_mg),
            "min_shared_blocks": args.shared_prefix,
            # K/V read by the prefix pass: each group's prefix once
            "prefix_kv_bytes": pre_tok * Hkv * 2 * D * case.elt_bytes,
            # K/V read by the even split: every sequence after its prefix
            "rest_kv_bytes": int((case.attended_lens().astype(np.int64) -
                                  sh_pre.astype(np.int64)).sum()) * Hkv * 2 * D * case.elt_bytes,
            "host_plan_us": round(host_shared_plan_us, 1)}
    if evs:
        kern_us = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
        part_ms = dec_ms = float(kern_us.mean()) * 1e-3
        res["attention_kernel_us_p10_p50_p90"] = [round(float(x), 3) for x in
                                                  np.percentile(kern_us, [10, 50, 90])]
        # start-to-start of consecutive attention kernels: one step each (with the
        # dispatch events' own cost)
        per = np.array([evs[i][0].elapsed_time(evs[i + 1][0])
                        for i in range(len(evs) - 1)]) * 1e3
        res["step_us_p10_p50_p90_with_kernel_events"] = [round(float(x), 3) for x in
                                                         np.percentile(per, [10, 50, 90])]
        res["us_per_step_with_kernel_events"] = round(ms_step_ev * 1e3, 3)
        # table entries walked: from the block holding the first attended position
        att = case.attended_lens().astype(np.int64)
        if shared is not None:
            # the even split's kernel attends each sequence after its shared prefix
            att = att - sh_pre.astype(np.int64)
        tables_bytes = int(sum(-(-int(x) // 16) - (int(x) - int(a)) // 16
                               for x, a in zip(case.lens, att))) * 4
        # K/V of every attended token, q, the table entries walked, the lengths and
        # the fp32 output; in the phased step the kernel also reads the new
        # tokens (k_new, v_new) and the slot indices
        kv_att = int(att.sum()) * Hkv * 2 * D * case.elt_bytes
        alg = kv_att + q.numel() * q.element_size() + tables_bytes + B * 4 + out.numel() * 4
        if mode in ("phased", "quant", "window", "step", "shared"):
            alg += 2 * k_new.numel() * k_new.element_size() + B * 8
        achieved = alg / (part_ms * 1e-3) / 1e9
        res["attention_kernel_us"] = round(dec_ms * 1e3, 3)
        if mode == "quant":
            kname = (f"attention kernel of pa_decode_step_quant ({case.kv_dtype} codes; new "
                     f"tokens encoded and fused in)")
        elif mode == "window":
            kname = (f"attention kernel of pa_decode_step_window (last {window} positions; new "
                     f"tokens fused in)")
        elif mode == "shared":
            kname = ("attention kernel of pa_decode_step_shared (each sequence after its shared "
                     "prefix, even split; new tokens fused in)")
        elif mode == "separate":
            kname = "attention partition kernel (pa_decode_partial)"
        elif args.mode == "phased":
            kname = "attention kernel of pa_decode_step_partial (new tokens fused in)"
        else:
            kname = "attention kernel of pa_decode_step (new tokens fused in)"
        res["roofline"] = {"kernel": kname,
                           "bound": "hbm", "achieved": round(achieved, 2),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": traffic_for(case.name),
                           "launch_us": round(part_ms * 1e3, 3),
                           "algorithmic_bytes": alg}
        res["attention_vs_stream_read"] = round(achieved / stream_ctx["gbs"], 4)
    if cpu_case is not None:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cpu_case, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
