#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

A step is one pass of the decode hot path over one synthetic batch: append
the batch's new token rows into their slots, then paged decode attention over
every sequence's blocks.  By default the step is one pa_decode_append call
(the decode kernel stores the new rows itself for 16-bit caches); with
--unfused it is pa_reshape_and_cache followed by pa_decode.  The default
workload is the largest single-GPU batch, the 70B-class decode layer: 32
sequences of 8,000 positions, 64 query / 8 KV heads, head_dim 128, fp16,
block size 16 (500 shuffled blocks per sequence).

Reported: KV GB/s (algorithmic K+V bytes of the batch per step time) and
sequence-heads per second; the attention kernel's roofline fraction against
the 8 TB/s HBM peak, its duration taken live by events the library records
around that kernel alone; and the CPU oracle on a bounded sample of the same
batch.

    python bench.py [--steps K] [--warmup W] [--config llama8b|llama70b|...]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "pa_decode KV GB/s (fraction of HBM peak) + seq·heads/s on 1 MI355X"
HBM_PEAK_GBS = 8000.0
# dense 16-bit MFMA (fp8 and fp4 KV are widened to 16 bits)
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 2500.0, "fp4": 2500.0}
CSRC = os.path.join(ROOT, "paged_kv_cache_342_amd", "csrc")
# sources of the kernels a pa_decode call runs; profiler traffic recorded for
# other sources is stale and is not reported
DECODE_SOURCES = ("pa_device.h", "decode_common.h", "decode_core.hip", "decode_mfma_kernel.h", "decode_mfma.hip",
                  "decode_cascade.hip", "decode_prefill.hip", "decode_valu.hip", "cache_ops.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(w, budget_s: float, row_scales: bool = False, window=None):
    """The fp64 oracle over whole sequences of the same batch, until the time budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import harness as OH
    from oracle import pa_oracle as O

    log("cpu baseline: building oracle pools")
    if row_scales:
        cd = w.cache_dtype
        kc, vc = O.new_pool(w.num_blocks, w.Hkv, w.bs, w.D, cd), O.new_pool(w.num_blocks, w.Hkv, w.bs, w.D, cd)
        ks = np.ones((w.num_blocks, w.Hkv, w.bs), np.float32)
        vs = ks.copy()
        for s in range(w.B):
            L = int(w.context_lens[s])
            if L:
                k, v = w.seq_kv(s)
                O.reshape_and_cache_scaled(k, v, kc, vc, ks, vs, O.slots_for(w.block_tables[s], 0, L, w.bs), w.bs,
                                           w.src_dtype, cd)
    else:
        kc, vc = OH.build_pools(w)
    q = w.query()
    done_seqs = 0
    kv = 0
    t_total = 0.0
    passes = 0
    while t_total < budget_s and passes < 50:
        for s in range(w.B):
            t0 = time.perf_counter()
            if row_scales:
                O.decode_scaled(q, kc, vc, ks, vs, w.block_tables, w.context_lens, w.scale, w.group, w.q_dtype,
                                seqs=[s], cache_dtype=cd)
            elif window is not None:
                O.decode_window(q, kc, vc, w.block_tables, w.context_lens, w.scale, w.group, window[0], window[1],
                                w.cache_dtype, w.q_dtype, w.k_scale, w.v_scale, seqs=[s])
            elif w.query_start is None:
                O.decode_one(q[s], kc, vc, w.block_tables[s], int(w.context_lens[s]), w.scale, w.group,
                             w.cache_dtype, w.q_dtype, w.k_scale, w.v_scale)
            else:
                O.decode_multi(q, kc, vc, w.block_tables, w.context_lens, w.query_start, w.scale, w.group,
                               w.cache_dtype, w.q_dtype, w.k_scale, w.v_scale, seqs=[s])
            t_total += time.perf_counter() - t0
            done_seqs += 1
            L = int(w.context_lens[s])
            n_att = L if window is None else min(L, window[0] + window[1])
            kv += n_att * w.Hkv * w.D * 2 * {"fp8": 8, "fp4": 4}.get(w.cache_dtype, 16) // 8
            if t_total >= budget_s:
                break
        passes += 1
    threads = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": kv / t_total / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done_seqs} whole sequences of the same batch ({kv} KV bytes) in {t_total:.1f} s of "
                  f"fp64 NumPy gather + attention; seq*heads/s = {done_seqs * w.Hq / t_total:.1f}; cpu: {cpu}",
    }


def decode_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_key(name: str, row_scales: bool) -> str:
    """The name a bench line's recorded traffic is kept under: the workload's
    name (as the bench builds it, with its --fp4 / --group suffix), plus
    '+row_scales' for the calls with a scale per row."""
    return name + ("+row_scales" if row_scales else "")


def recorded_traffic(workload: str):
    """HBM bytes per pa_decode call (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy
    of known size) from the committed rocprofv3 record, if it was taken on the
    current kernel sources; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get("workloads", {}).get(workload)
    if not r or rec.get("decode_source_sha256_16") != decode_source_hash():
        return None
    return r.get("hbm_bytes_per_call")


def block_manager_bench(w, steps: int = 200):
    """The batch's host bookkeeping through the library's block manager.

    The manager is brought to the workload's state (for shared prefixes, each
    prompt is stored once and forked into its samples, whose first appends
    copy the partially filled shared block), then each of `steps` decode steps
    appends one token to every sequence and builds the block tables and
    lengths a pa_decode call takes.  Host time per step through the Python
    binding, and the tail waste of the workload's own lengths."""
    import numpy as np

    import paged_kv_cache_342_amd as pa

    bs, B = w.bs, w.B
    lens = w.context_lens.astype(np.int64)
    bm = pa.BlockManager(w.num_blocks + B * ((steps + bs - 1) // bs + 1), bs)
    seqs = np.arange(B, dtype=np.int64)
    if w.name == "shared_prefix":
        samples, plen = w.meta["samples"], w.meta["shared_len"].astype(np.int64)
        for k in range(len(plen)):
            bm.add(-1 - k)
            bm.append(-1 - k, int(plen[k]))
            for j in range(samples):
                bm.fork(-1 - k, k * samples + j)
            bm.free(-1 - k)
        _, pairs = bm.append_batch(seqs, lens - np.repeat(plen, samples))
    else:
        for s in range(B):
            bm.add(s)
        _, pairs = bm.append_batch(seqs, lens)
    st = bm.stats()
    ones = np.ones(B, np.int32)
    width = int((lens.max() + steps + bs - 1) // bs)
    # one table matrix kept across steps, as a serving loop would: padded once,
    # then only block ids are written
    tables, clens = np.full((B, width), -1, np.int32), np.empty(B, np.int32)
    t0 = time.perf_counter()
    for _ in range(steps):
        bm.append_batch(seqs, ones)
        bm.tables(seqs, width, out=tables, lens_out=clens, pad=False)
    per_step = (time.perf_counter() - t0) / steps
    return {"host_us_per_step": round(per_step * 1e6, 2), "steps": steps,
            "ops": "append_batch(B seqs, 1 token each) + tables(B seqs) into a kept matrix",
            "tail_waste": round(st["tail_waste"], 5), "blocks_in_use": st["blocks_in_use"],
            "shared_blocks": st["shared_blocks"], "cow_pairs": int(len(pairs))}


def _identity_layout(w, batch, slots_new):
    """Renumber physical blocks so each sequence's blocks are consecutive and in
    logical order (block tables become ranges); returns the new token slots."""
    import numpy as np
    import torch

    nblk = (w.context_lens.astype(np.int64) + w.bs - 1) // w.bs
    order = [int(b) for s in range(w.B) for b in w.block_tables[s, :nblk[s]]]
    if len(set(order)) != len(order):
        raise SystemExit("--identity-tables needs a workload whose sequences share no blocks")
    rest = sorted(set(range(w.num_blocks)) - set(order))
    perm = np.empty(w.num_blocks, np.int64)
    perm[np.array(order + rest, np.int64)] = np.arange(w.num_blocks)
    pt = torch.from_numpy(perm).to(batch.kc.device)
    raw = (lambda t: t.view(torch.uint8)) if batch.kc.element_size() == 1 else (lambda t: t.view(torch.int16))
    for name in ("kc", "vc"):
        old = getattr(batch, name)
        new = torch.empty_like(raw(old))
        new[pt] = raw(old)
        setattr(batch, name, new.view(old.dtype))
    tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w.block_tables = tables
    batch.tables = torch.from_numpy(tables).to(batch.kc.device)
    b = slots_new // w.bs
    return pt[b] * w.bs + slots_new % w.bs


def hbm_ceilings(dev, mib=512, reps=5):
    """What plain kernels reach on this device, timed like the step: a torch
    device copy of `mib` MiB (read + written bytes counted), a torch sum over
    1 GiB (read bytes), and the library's read probe (pa_read_probe: the
    decode kernels' 16-byte nontemporal loads, each wave streaming its own
    4 KiB chunks) over 1 GiB, each after a read of another 1 GiB buffer evicts
    L2/MALL.  The median over `reps`, in GB/s."""
    import numpy as np
    import torch

    evict = torch.ones(1 << 27, dtype=torch.int64, device=dev)
    src = torch.ones(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    big = torch.ones(1 << 27, dtype=torch.int64, device=dev)

    def timed(fn):
        ts = []
        for i in range(reps + 1):
            evict.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    t_copy = timed(lambda: dst.copy_(src))
    t_read = timed(lambda: big.sum())
    import paged_kv_cache_342_amd as pa
    nbytes = big.numel() * 8
    sink = torch.empty(256, dtype=torch.int32, device=dev)
    t_probe = timed(lambda: pa.read_probe(big, 4096, sink))
    res = {"copy_gbs": round(2 * src.numel() / t_copy / 1e9, 1), "copy_bytes": 2 * src.numel(),
           "read_gbs": round(nbytes / t_read / 1e9, 1), "read_bytes": nbytes,
           "probe_read_gbs": round(nbytes / t_probe / 1e9, 1),
           "kernels": "torch copy_ and sum; pa_read_probe (4 KiB chunks, each wave streaming its own)"}
    del evict, src, dst, big, sink
    return res


def select_workload(config: str, group: int = 0, fp4: bool = False, block_size: int = 0):
    """The synthetic batch of a bench line: the named workload (the heavy-tailed
    one at another block size), or its lengths and shapes with `group` query
    heads per KV head, or with an FP4 cache."""
    import workloads as W

    if block_size:
        if config != "heavy_tail":
            raise SystemExit("--block-size applies to the heavy_tail workload (its block size is swept)")
        w = W.make(config, bs=block_size)
    else:
        w = W.make(config)
    if group:
        if w.query_start is not None or w.name == "shared_prefix":
            raise SystemExit("--group applies to the plain decode workloads")
        w = W.custom(f"{w.name}_g{group}", w.seed, w.context_lens, w.Hkv * group, w.Hkv, w.D, w.bs,
                     w.cache_dtype, w.q_dtype)
    if fp4:
        if w.query_start is not None or w.name == "shared_prefix":
            raise SystemExit("--fp4 applies to the plain decode workloads")
        w = W.custom(f"{w.name}_fp4", w.seed, w.context_lens, w.Hq, w.Hkv, w.D, w.bs, "fp4", w.q_dtype)
    return w


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama70b")
    ap.add_argument("--no-flush", action="store_true", help="do not evict L2/MALL between steps")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time (0 = skip)")
    ap.add_argument("--identity-tables", action="store_true",
                    help="ablation: move every sequence's blocks into consecutive physical blocks, in order "
                         "(same values, no scattered indirection)")
    ap.add_argument("--group", type=int, default=0,
                    help="decode workloads: the same lengths, KV heads and dtypes with this many query heads per KV "
                         "head (a fresh seeded layout and values; for kernel-choice measurements)")
    ap.add_argument("--row-scales", action="store_true",
                    help="FP8 workloads: one scale per (slot, kv head) row (pa_reshape_and_cache_scaled + "
                         "pa_decode_scaled) instead of one per tensor")
    ap.add_argument("--fp4", action="store_true",
                    help="decode workloads: the same lengths and shapes with an FP4 (E2M1) cache, a scale per row "
                         "(fresh seeded values; implies --row-scales)")
    ap.add_argument("--block-size", type=int, default=0, choices=[0, 8, 16, 32],
                    help="heavy_tail: the same lengths and values in blocks of 8, 16 (its default) or 32 positions")
    ap.add_argument("--cascade", action="store_true",
                    help="shared_prefix: pa_reshape_and_cache + pa_decode_shared_prefix, each prompt's shared prefix "
                         "read once for its samples (the roofline counts those unique bytes)")
    ap.add_argument("--window", default="",
                    help="SINK,WINDOW: attention sinks plus a sliding window (pa_reshape_and_cache + "
                         "pa_decode_window); the bytes counted are those of the attended positions")
    ap.add_argument("--unfused", action="store_true",
                    help="time the step as two calls, pa_reshape_and_cache then pa_decode")
    ap.add_argument("--no-graph", action="store_true", help="skip timing the step replayed from a HIP graph")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB a few times (outside the timed region), "
                         "to scale profiler byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this path is single-GPU by design)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_342_amd as pa
    import workloads as W
    from workloads.device import DeviceBatch

    dev = torch.device("cuda:0")
    w = select_workload(args.config, args.group, args.fp4, args.block_size)
    if args.fp4:
        args.row_scales = True
    log(f"workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} bs={w.bs} cache={w.cache_dtype} "
        f"sum(L)={int(w.context_lens.sum())}")
    multi = w.query_start is not None  # several queries per sequence: pa_decode_multi
    if multi and (args.unfused or args.identity_tables or args.row_scales):
        raise SystemExit("--unfused, --identity-tables and --row-scales apply to the decode workloads only")
    if args.row_scales and w.cache_dtype not in ("fp8", "fp4"):
        raise SystemExit("--row-scales applies to FP8 (and FP4) workloads")
    rs = args.row_scales
    win = None
    if args.cascade and w.name != "shared_prefix":
        raise SystemExit("--cascade applies to the shared_prefix workload")
    cascade = args.cascade
    if args.window:
        win = tuple(int(x) for x in args.window.split(","))
        if len(win) != 2 or win[0] < 0 or win[1] < 1:
            raise SystemExit("--window takes SINK,WINDOW with SINK >= 0 and WINDOW >= 1")
        if multi or rs:
            raise SystemExit("--window applies to the decode workloads with a scale per tensor")
    batch = DeviceBatch(w, device=dev, skip_last_append=not multi, row_scales=rs)
    if multi:  # the step re-appends the query tokens' own rows, then attends
        nqs = np.diff(w.query_start).astype(np.int64)
        last = W.WriteOp("append", np.arange(w.B, dtype=np.int64), w.context_lens.astype(np.int64) - nqs,
                         w.context_lens.astype(np.int64))
        k_new, v_new, slots_new = batch.rows_for(last)
        q_start = torch.from_numpy(np.ascontiguousarray(w.query_start)).to(dev)
    else:
        k_new, v_new, slots_new = batch.rows_for(w.ops[-1])
    if args.identity_tables:
        slots_new = _identity_layout(w, batch, slots_new)
    if not multi:
        k_last, v_last = batch.last_rows()  # the same rows, [B, Hkv, D] by sequence
    log("pools filled")
    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy: 3 x {args.calib_copy_mb} MiB read + written")
    out = torch.empty(tuple(batch.q.shape), dtype=batch.q.dtype, device=dev)
    ws_bytes = (pa.decode_multi_workspace_size(w.B, w.Hkv, w.group, w.D, w.bs, w.max_context_len, w.max_queries)
                if multi else pa.decode_workspace_size(w.B, w.Hkv, w.group, w.D, w.bs, w.max_context_len))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    # Cache eviction between steps: READ a 1 GiB buffer (larger than the 256 MB
    # MALL plus the L2s).  A write-based flush would leave dirty lines whose
    # write-back then competes with the decode's reads inside the timed region.
    flush = None if args.no_flush else torch.ones(1 << 27, dtype=torch.int64, device=dev)

    def evict():
        if flush is not None:
            flush.sum()

    def append():
        if rs:
            pa.reshape_and_cache_scaled(k_new, v_new, batch.kc, batch.vc, batch.kss, batch.vss, slots_new)
        else:
            pa.reshape_and_cache(k_new, v_new, batch.kc, batch.vc, slots_new, w.k_scale, w.v_scale)

    if cascade:
        samples, plen = w.meta["samples"], w.meta["shared_len"].astype(np.int64)
        group_start = torch.tensor(np.arange(len(plen) + 1) * samples, dtype=torch.int32, device=dev)
        prefix_lens = torch.tensor(plen, dtype=torch.int32, device=dev)
        cws = torch.empty(pa.decode_shared_prefix_workspace_size(w.B, len(plen), samples, w.Hkv, w.group, w.D, w.bs,
                                                                  w.max_context_len), dtype=torch.uint8, device=dev)

    def decode():
        if cascade:
            pa.decode_shared_prefix(batch.q, batch.kc, batch.vc, batch.tables, batch.lens, group_start, prefix_lens,
                                    samples, w.scale, max_context_len=w.max_context_len, out=out, workspace=cws)
        elif win:
            pa.decode_window(batch.q, batch.kc, batch.vc, batch.tables, batch.lens, w.scale, win[0], win[1],
                             max_context_len=w.max_context_len, k_scale=w.k_scale, v_scale=w.v_scale, out=out,
                             workspace=ws)
        elif rs:
            pa.decode_scaled(batch.q, batch.kc, batch.vc, batch.kss, batch.vss, batch.tables, batch.lens, w.scale,
                             max_context_len=w.max_context_len, out=out, workspace=ws)
        else:
            pa.decode(batch.q, batch.kc, batch.vc, batch.tables, batch.lens, w.scale,
                      max_context_len=w.max_context_len, k_scale=w.k_scale, v_scale=w.v_scale, out=out, workspace=ws)

    def decode_append():
        pa.decode_append(batch.q, batch.kc, batch.vc, k_last, v_last, batch.tables, batch.lens, w.scale,
                         max_context_len=w.max_context_len, k_scale=w.k_scale, v_scale=w.v_scale, out=out,
                         workspace=ws)

    def decode_multi():
        pa.decode_multi(batch.q, batch.kc, batch.vc, batch.tables, batch.lens, q_start, w.max_queries, w.scale,
                        max_context_len=w.max_context_len, k_scale=w.k_scale, v_scale=w.v_scale, out=out,
                        workspace=ws)

    two_calls = args.unfused or multi or rs or win is not None or cascade
    second = decode_multi if multi else decode

    def step():
        if two_calls:
            append()
            second()
        else:
            decode_append()

    for i in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    def timed_steps(kernel_events: bool):
        """K steps, each after the cache eviction, between events on torch's
        current stream (the stream every call launches on); with two calls a
        middle event separates the append from the attention call.  With
        kernel_events the library also records e[3] / e[4] at the start and
        end of the call's attention kernel itself (hipExtLaunchKernel's
        events), which adds ~15 us of event handling to each step."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            evict()  # outside the step's events
            ev[i][0].record()
            if two_calls:
                append()
                ev[i][1].record()
            if kernel_events:
                pa.time_next_attention_kernel(ev[i][3], ev[i][4])
            second() if two_calls else decode_append()
            ev[i][2].record()
        torch.cuda.synchronize()
        return ev, time.perf_counter() - t0

    # the headline: K clean steps; then the same K steps again, with the
    # attention kernel's own start/stop events for the roofline
    ev, wall = timed_steps(False)
    step_ms = [e[0].elapsed_time(e[2]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev] if two_calls else step_ms
    ms_step = float(np.mean(step_ms))
    ms_dec = float(np.mean(dec_ms))
    kev, _ = timed_steps(True)
    kern_ms = [e[3].elapsed_time(e[4]) for e in kev]
    ms_kern = float(np.mean(kern_ms))
    ms_step_kev = float(np.mean([e[0].elapsed_time(e[2]) for e in kev]))

    # the same step captured once in a HIP graph and replayed (the cache
    # eviction stays outside the graph and outside the events)
    graph_ms = None
    if not args.no_graph:
        try:
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step()
            torch.cuda.synchronize()
            gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
            for i in range(args.steps):
                evict()
                gev[i][0].record()
                g.replay()
                gev[i][1].record()
            torch.cuda.synchronize()
            graph_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in gev]))
            log(f"graph replay: {graph_ms * 1e3:.1f} us per step")
        except RuntimeError as e:  # the eager figures stand without it
            log(f"graph replay not timed: {e}")
    # positions each sequence attends to: all, or the sink's and the window's
    attended = (w.context_lens.astype(np.int64) if win is None else
                np.minimum(w.context_lens.astype(np.int64), win[0] + win[1]))
    bits = {"fp8": 8, "fp4": 4}.get(w.cache_dtype, 16)
    kv_bytes = int(attended.sum()) * w.Hkv * w.D * 2 * bits // 8
    if rs:  # each (position, kv head) row also carries a 4-byte K and V scale
        kv_bytes += int(w.context_lens.astype(np.int64).sum()) * w.Hkv * 4 * 2
    # the cascade reads each prompt's prefix once per KV head: those are the
    # bytes its kernels must move (the metric's value keeps every sequence's own)
    kern_bytes = kv_bytes
    if cascade:
        shared = int((plen * (samples - 1)).sum())
        kern_bytes = (int(attended.sum()) - shared) * w.Hkv * w.D * 2 * bits // 8
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = kern_bytes / (ms_kern * 1e-3) / 1e9
    # algorithmic flops: 4 * D per (query head, position seen) -- QK and PV
    seen = (attended if not multi else
            np.array([sum(int(L) - n + j + 1 for j in range(n)) for L, n in zip(w.context_lens, nqs)]))
    flops = 4 * w.D * w.Hq * int(seen.sum())
    tflops = flops / (ms_kern * 1e-3) / 1e12
    mfma_peak = MFMA_PEAK_TFLOPS[w.cache_dtype]
    mfma_bound = tflops / mfma_peak > achieved / HBM_PEAK_GBS
    log(f"step {ms_step * 1e3:.1f} us (median {np.median(step_ms) * 1e3:.1f}), decode {ms_dec * 1e3:.1f} us "
        f"(median {np.median(dec_ms) * 1e3:.1f}), attention kernel {ms_kern * 1e3:.1f} us "
        f"(median {np.median(kern_ms) * 1e3:.1f}), wall/step incl. flush {wall / args.steps * 1e3:.3f} ms")

    ceil = hbm_ceilings(dev)
    log(f"plain copy {ceil['copy_gbs']} GB/s (read + write), plain read {ceil['read_gbs']} GB/s, "
        f"read probe {ceil['probe_read_gbs']} GB/s")

    bm = block_manager_bench(w)
    log(f"block manager: {bm['host_us_per_step']} us per step on the host, tail waste {bm['tail_waste']:.4f}")

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(w, args.cpu_budget, rs, win)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f16": "f16", "bf16": "bf16", "fp8": "fp8e4m3", "fp4": "fp4e2m1"}[w.cache_dtype],
        "data": "synthetic",
        "config": {
            "workload": w.name, "decode_kernel": os.environ.get("PA_DECODE_VARIANT", "default"), "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
            "block_size": w.bs, "cache_dtype": w.cache_dtype, "q_dtype": w.q_dtype, "seed": w.seed,
            "sum_context_len": int(w.context_lens.sum()), "kv_bytes": kv_bytes, "parallelism": "single-gpu",
            **({"kernel_bytes_unique": kern_bytes} if cascade else {}),
            "l2_mall_flush_between_steps": flush is not None, "identity_tables": args.identity_tables,
            "row_scales": rs,
            **({"sink_tokens": win[0], "window_tokens": win[1], "sum_attended_positions": int(attended.sum())}
               if win else {}),
            "step": ("pa_reshape_and_cache + pa_decode_multi" if multi else
                     "pa_reshape_and_cache + pa_decode_window" if win else
                     "pa_reshape_and_cache + pa_decode_shared_prefix" if cascade else
                     "pa_reshape_and_cache_scaled + pa_decode_scaled" if rs else
                     "pa_reshape_and_cache + pa_decode" if args.unfused else "pa_decode_append"),
            **({"queries_per_seq": w.max_queries, "total_queries": int(w.query_start[-1])} if multi else {}),
        },
        "seq_heads_per_s": round(w.B * w.Hq / (ms_step * 1e-3), 1),
        "attention_tflops": round(tflops, 2),
        "hbm_fraction": round(value / HBM_PEAK_GBS, 4),
        "decode_us": round(ms_dec * 1e3, 2),
        "attention_kernel_us": round(ms_kern * 1e3, 2),
        "step_us_with_kernel_events": round(ms_step_kev * 1e3, 2),
        "graph_replay_us_per_step": None if graph_ms is None else round(graph_ms * 1e3, 2),
        "hbm_copy": {**ceil, "frac_of_copy": round(value / ceil["copy_gbs"], 4),
                     "frac_of_read": round(value / ceil["read_gbs"], 4),
                     "frac_of_probe_read": round(value / ceil["probe_read_gbs"], 4)},
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(tflops if mfma_bound else achieved, 2),
            "peak": mfma_peak if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(tflops / mfma_peak if mfma_bound else achieved / HBM_PEAK_GBS, 4),
            "traffic": None if args.identity_tables or args.unfused else
                       recorded_traffic(traffic_key(w.name, rs) + (f"+window{win[0]},{win[1]}" if win else "")
                                        + ("+cascade" if cascade else "")),
            "kernel": ("attention kernel of pa_decode_multi: MFMA kernel over (query, head) columns (long query "
                       "chunks: workgroups whose waves share K/V chunks through LDS)" if multi else
                       "attention kernel of pa_decode_scaled: MFMA kernel with row scales" if rs else
                       "attention kernels of pa_decode_shared_prefix, from the start of the prefix pass to the end "
                       "of the suffix pass (the prefix state merge between them included); achieved counts each "
                       "prompt's prefix once" if cascade else
                       "attention kernel of pa_decode_window: decode kernel over the sink and window chunks" if win
                       else
                       "attention kernel of pa_decode: decode kernel (balanced slices)" if args.unfused else
                       "attention kernel of pa_decode_append: decode kernel (balanced slices, append fused for "
                       "16-bit caches)"),
            "timing": "achieved = algorithmic bytes / mean duration of that kernel alone, from start/stop events "
                      "its launch records on the call's stream (hipExtLaunchKernel), over a second pass of the same "
                      "K timed steps; the headline step is timed in a first pass without them, since they add "
                      "~15 us of event handling per step",
        },
        "cpu_baseline": cpu,
        "block_manager": bm,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
