#!/usr/bin/env python3
"""Paged decode step on one MI355X: KV append, copy-on-write copy and
block-table GQA decode attention through libpkv.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--layers L]
    python bench.py --path multi [--config NAME] [--query-tokens n]
    python bench.py --path swap [--config NAME]
    python bench.py --path shared [--config NAME]

A step is one pass of the device hot path over one batch (by default the
llama3-8b-layer batch: 256 sequences of 512-8192 tokens, 32 query / 8 KV heads,
head_dim 128, bf16, block size 16): pkv_copy_blocks (when the batch has
copy-on-write pairs), then the append of one new token per sequence and the
decode attention (pkv_attention_decode_append; ``--unfused``: pkv_write, then
pkv_attention_decode), with the split-KV merge.
Inputs are resident in HBM before the timed region.  ``--layers`` pool pairs
with identical block tables are cycled, one per step, so that consecutive steps
read different memory (as a model's layers do) and no step is served from the
previous step's cached lines.  The timed steps replay each layer's step as a
HIP graph captured once (``--no-graph``: eager launches); the attention
kernel's own duration comes from an eager pass with HIP events around it.
Prints one JSON line.

``--path multi`` times pkv_attention_multi instead: n new query tokens per
sequence of the configuration (tokens to verify, or a prefill chunk), each
attending the history up to its own position.  ``--path swap`` times a
preemption round trip on the configuration's shape: the latest quarter of the
sequences leave the HBM pools for pinned host memory (pkv_swap_out) and come
back (pkv_swap_in); its roofline is the host link's.  ``--path shared`` times
pkv_attention_decode_shared on the shared-prefix configuration (by default):
each group's prefix is read once per block of rows, not once per sequence.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
# PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 encoding / 8 bits
PCIE_PEAK_GBPS = 32.0 * 16 * 128 / 130 / 8
METRIC = "paged decode attention KV-read GB/s (% of MI355X HBM peak); tokens/s"
# Sources of each kernel, under paged_attention_slot_amd/csrc/ (the build
# script's flags shape the code too).
KERNEL_SOURCES = {
    "attn_balanced_kernel": ("attn_decode.hip", "lse_merge.h", "pkv_device.h", "../build.py"),
    "attn_partition_kernel": ("attn_decode.hip", "lse_merge.h", "pkv_device.h", "../build.py"),
    "attn_multi_kernel": ("attn_multi.hip", "mfma_attend.h", "mfma_route.h", "lse_merge.h",
                          "pkv_device.h", "../build.py"),
    "attn_shared": ("attn_shared.hip", "mfma_attend.h", "pkv_device.h", "../build.py"),
    "attn_mfma_balanced_kernel": ("attn_decode.hip", "mfma_attend.h", "lse_merge.h",
                                  "pkv_device.h", "../build.py"),
    "swap_blocks_kernel": ("swap.hip", "../build.py"),
}


def cpu_baseline(wl, budget_s: float, kv_dtype: str | None = None) -> dict:
    """The CPU oracle (fp64 NumPy, as it stands) on a bounded sample of the same
    workload: its block manager and writes first (untimed), then copy + write of
    the step and attention sequence by sequence, cycling over the batch, until
    ``budget_s`` elapses.  ``kv_dtype`` "fp8_e4m3" / "int8": the oracle of the
    quantized caches (its attention dequantizes the pools, then attends)."""
    import numpy as np

    from oracle.attention import attention_decode
    from oracle.replay import OracleState, QuantOracleState

    st = (QuantOracleState(wl, kv_dtype, keep_values=False) if kv_dtype
          else OracleState(wl, keep_values=False))
    st.build_context()
    st.decode_tables()
    t0 = time.perf_counter()
    st.decode_device_part()
    done = []
    while time.perf_counter() - t0 <= budget_s:
        s = len(done) % wl.num_seqs
        if kv_dtype:
            st.attention(seqs=[s])
        else:
            attention_decode(wl.q, st.k_pool, st.v_pool, st.block_tables, st.seq_lens, wl.scale,
                             seqs=[s])
        done.append(s)
    el = time.perf_counter() - t0
    lens = st.seq_lens[done].astype(np.int64)
    e = 1 if kv_dtype else wl.elem_bytes
    kv = int(lens.sum()) * (2 * wl.num_kv_heads * wl.head_dim * e +
                            (8 * wl.num_kv_heads if kv_dtype == "int8" else 0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    return {"value": kv / el / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(done)} sequence attentions cycling over the {wl.num_seqs}-sequence "
                      f"batch ({int(lens.sum())} cached positions, {kv / 1e6:.1f} MB of K/V) "
                      f"plus the step's copy and write, in {el:.2f} s; fp64 NumPy, one process",
            "seconds": el, "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0))}


def kernel_source_sha256(kernel: str = "attn_balanced_kernel") -> str:
    """Hash of a kernel's sources (matches profile records)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "paged_attention_slot_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the counter record under profiles/ for this
    kernel and workload, if the kernel sources are unchanged since; else None."""
    import glob
    import re
    sha = kernel_source_sha256(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for m in re.finditer(r"<!-- pkv-traffic (\{.*?\}) -->", fh.read()):
                rec = json.loads(m.group(1))
                if rec["kernel"] == kernel and rec["workload"] == workload and \
                        rec["source_sha256"] == sha:
                    return (rec["fetch_kib"] * rec["fetch_scale"] +
                            rec["write_kib"] * rec["write_scale"]) * 1024.0
    return None


def stream_read_gbps(nbytes: int = 4 << 30, iters: int = 10, workgroups: int = 8192,
                     buffers: int = 1) -> float:
    """Achievable read rate on this device: libpkv's plain coalesced stream
    kernel over ``nbytes`` (median of ``iters`` runs, HIP events).  With
    ``buffers`` > 1 the runs cycle over that many buffers of ``nbytes``, as the
    measured steps cycle over layer pools, so no run finds its bytes in the
    last-level cache."""
    import numpy as np
    import torch

    from paged_attention_slot_amd import ops
    nbytes -= nbytes % 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(buffers)]
    sink = torch.zeros(workgroups, dtype=torch.int32, device="cuda")
    for buf in bufs:
        ops.stream_read(buf, sink, workgroups)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        ops.stream_read(bufs[i % buffers], sink, workgroups)
        b.record()
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    del bufs
    torch.cuda.empty_cache()
    return nbytes / t / 1e9


def stream_read_same_size_gbps(nbytes: int, buffers: int) -> dict:
    """The calibration stream at one launch's algorithmic bytes: the rate a
    plain coalesced read of that size reaches, launch ramp and drain
    included (best of three grid sizes)."""
    rates = {wg: stream_read_gbps(nbytes, iters=20, workgroups=wg, buffers=buffers)
             for wg in (2048, 4096, 8192)}
    best = max(rates, key=rates.get)
    return {"bytes": nbytes - nbytes % 16, "buffers": buffers, "gbps": rates[best],
            "workgroups": best}


def _common(args, wl, metric, value, unit, t_step, dtype, config, roofline, detail):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": t_step * 1e3, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "config": config, "roofline": roofline, "cpu_baseline": None, "detail": detail}


def _threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def _timed(fn, K, W, marks):
    """Run ``fn(i, rec)`` W times untimed, then K times with ``marks`` HIP
    events per step recorded by ``rec(j)``; returns (wall seconds per step,
    array [K, marks-1] of event intervals in seconds)."""
    import numpy as np
    import torch
    for i in range(W):
        fn(i, lambda j: None)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(marks)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        fn(i, lambda j, i=i: ev[i][j].record())
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / K
    iv = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(marks - 1)]
                   for i in range(K)]) * 1e-3
    return wall, iv


def bench_multi(args) -> int:
    """pkv_attention_multi over the configuration's batch, n query tokens per
    sequence at the end of each history."""
    import ctypes

    import numpy as np
    import torch

    from paged_attention_slot_amd import lib, ops
    from paged_attention_slot_amd.runtime import DecodeStep
    from workloads import config_workload, multi_queries

    n = int(args.query_tokens)
    quant = args.kv_dtype != "model"
    t0 = time.perf_counter()
    wl = config_workload(args.config)
    step = DecodeStep(wl, layers=args.layers, kv_dtype=args.kv_dtype if quant else None)
    for layer in range(args.layers):       # the decode token completes every history
        step.copy(layer)
        step.write(layer)
    N, Hq, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lens = wl.seq_lens.astype(np.int64)
    qh, offs = multi_queries(wl, n)            # at most L new tokens per sequence
    nq = np.diff(offs).astype(np.int64)
    total = int(offs[-1])
    gen_s = time.perf_counter() - t0
    dev = step.device
    if wl.dtype != "bf16":
        raise SystemExit("bench.py --path multi: the multi-token kernel takes bf16 caches")
    q = torch.from_numpy(qh.view(np.int16)).to(dev).view(torch.bfloat16)
    qo = torch.from_numpy(offs).to(dev)
    out = torch.empty_like(q)
    pt = int(args.partition_tokens or 0)
    need = lib().pkv_attention_multi_workspace_bytes(
        N, Hq, total, n, int(lens.max()), pt, ctypes.byref(ops.geom_of(step.k_cache)))
    ws = torch.empty(max(int(need), 16), dtype=torch.uint8, device=dev)
    e = 1 if quant else wl.elem_bytes
    # algorithmic bytes: every cached position's K and V read once (INT8: and
    # its two scales), q read, out written, table entries and lengths read
    kv_bytes = int(lens.sum()) * (2 * Hkv * D * e + (8 * Hkv if args.kv_dtype == "int8" else 0))
    e = wl.elem_bytes
    io_bytes = 2 * total * Hq * D * e + 4 * int(((lens + wl.block_size - 1)
                                                 // wl.block_size).sum()) + 8 * N
    alg_bytes = kv_bytes + io_bytes
    # flops: query j of a sequence of length L sits at position L - n + j and
    # attends its own position and all before it (q.k and p.v: 4*D per pair)
    pairs = int(sum(int(((L - k) + 1 + L) * k // 2) for L, k in zip(lens, nq)))
    flops = 4.0 * D * Hq * pairs
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    L_ = args.layers

    def run(i, rec):
        ks, vs = step._scales(i % L_)
        rec(0)
        ops.attention_multi(q, qo, step.k_caches[i % L_], step.v_caches[i % L_],
                            step.block_tables, step.seq_lens, wl.scale, n, out=out,
                            max_seq_len=step.max_seq_len, partition_tokens=pt, workspace=ws,
                            k_scale=step.k_scale, v_scale=step.v_scale, k_scales=ks,
                            v_scales=vs)
        rec(1)
    t_step, iv = _timed(run, args.steps, args.warmup, 2)
    t_k = float(np.mean(iv[:, 0]))
    mfma = flops / alg_bytes > ridge
    achieved = (flops / t_k / 1e12) if mfma else (alg_bytes / t_k / 1e9)
    peak = MFMA_BF16_PEAK_TFLOPS if mfma else HBM_PEAK_GBPS
    name = f"{wl.name}+multi{n}" + (f"+{args.kv_dtype}" if quant else "")
    roof = {"bound": "mfma" if mfma else "hbm", "kernel": "attn_multi_kernel",
            "achieved": achieved, "peak": peak, "unit": "TFLOP/s" if mfma else "GB/s",
            "frac": achieved / peak, "traffic": None,
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
            "algorithmic_bytes_per_launch": alg_bytes, "flops_per_launch": flops,
            "avg_launch_us": t_k * 1e6,
            "note": "event time covers the main kernel and the partition merge"}
    roof["traffic"] = recorded_traffic("attn_multi_kernel", name)
    config = {"workload": name, "num_seqs": N, "query_tokens_per_seq": n, "total_queries": total,
              "partition_tokens": pt or "automatic",
              "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": wl.block_size,
              "sum_seq_lens": int(lens.sum()), "max_seq_len": int(lens.max()),
              "layers_cycled": L_, "seed": wl.seed}
    detail = {"kv_bytes": kv_bytes, "hbm_gbps": alg_bytes / t_k / 1e9,
              "tflops": flops / t_k / 1e12, "queries_per_s": total / t_step,
              "input_generation_s": gen_s, "workspace_bytes": int(need)}
    res = _common(args, wl, "paged multi-token attention GB/s of K/V (new query tokens per "
                  "sequence over the cached history)", alg_bytes / t_step / 1e9, "GB/s", t_step,
                  args.kv_dtype if quant else wl.dtype, config, roof, detail)
    if not args.no_cpu_baseline and not quant:
        res["cpu_baseline"] = multi_cpu_baseline(wl, step, qh, offs, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


def multi_cpu_baseline(wl, step, qh, offs, budget_s):
    """The oracle's attention_multi, sequence by sequence over the batch until
    the budget is spent.  Each sequence's blocks are copied to host arrays
    first (untimed)."""
    import numpy as np
    import torch

    from oracle.attention import attention_multi
    from paged_attention_slot_amd.runtime import to_host_bits
    B = wl.block_size
    done, el = [], 0.0
    while el <= budget_s:
        s = len(done) % wl.num_seqs
        L = int(wl.seq_lens[s])
        nb = -(-L // B)
        ids = torch.from_numpy(step.block_tables_h[s, :nb].astype(np.int64)).to(step.device)
        kp = to_host_bits(step.k_cache.index_select(0, ids))
        vp = to_host_bits(step.v_cache.index_select(0, ids))
        table = np.arange(nb, dtype=np.int32)[None]
        q = qh[offs[s]:offs[s + 1]]
        t0 = time.perf_counter()
        attention_multi(q, np.asarray([0, q.shape[0]], np.int32), kp, vp, table,
                        np.asarray([L], np.int32), wl.scale)
        el += time.perf_counter() - t0
        done.append(s)
    lens = wl.seq_lens[done].astype(np.int64)
    kv = int(lens.sum()) * 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
    return {"value": kv / el / 1e9, "unit": "GB/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{len(done)} sequences' multi-token attention ({int(lens.sum())} cached "
                      f"positions, {kv / 1e6:.1f} MB of K/V) in {el:.2f} s of oracle time; "
                      f"fp64 NumPy, one process"}


def bench_shared(args) -> int:
    """pkv_attention_decode_shared over the configuration's decode step, with
    the plain decode kernel timed on the same pools beside it."""
    import numpy as np

    from paged_attention_slot_amd.runtime import DecodeStep
    from workloads import config_workload

    quant = args.kv_dtype != "model"
    t0 = time.perf_counter()
    wl = config_workload(args.config)
    gen_s = time.perf_counter() - t0
    if wl.dtype != "bf16":
        raise SystemExit("bench.py --path shared: the shared-prefix kernels take bf16 workloads")
    step = DecodeStep(wl, layers=args.layers, kv_dtype=args.kv_dtype if quant else None)
    for layer in range(args.layers):
        step.copy(layer)
        step.write(layer)
    gs, pl, mg, mp, ms = step.shared_groups()
    lens = wl.seq_lens.astype(np.int64)
    per_pos = (2 * wl.num_kv_heads * wl.head_dim * (1 if quant else wl.elem_bytes) +
               (8 * wl.num_kv_heads if args.kv_dtype == "int8" else 0))
    logical = int(lens.sum()) * per_pos
    # unique positions: distinct (block, offset) slots the batch attends
    B = wl.block_size
    slots = set()
    for s in range(wl.num_seqs):
        t = np.arange(int(lens[s]))
        slots.update((step.block_tables_h[s, t // B].astype(np.int64) * B + t % B).tolist())
    unique = len(slots) * per_pos
    # algorithmic bytes of this design: each group's prefix once per block of
    # member rows, each sequence's own positions once, q and out
    starts, plens = gs.cpu().numpy(), pl.cpu().numpy()
    G = wl.num_q_heads // wl.num_kv_heads
    per64 = 64 // G
    mpb = 16 * (1 if min(mg, per64) * G <= 16 else 2 if min(mg, per64) * G <= 32 else 4) // G
    pre_reads = own = 0
    for g in range(plens.size):
        n = int(starts[g + 1] - starts[g])
        P = int(plens[g]) if n >= 2 else 0
        pre_reads += -(-n // mpb) * P if P else 0
        own += int(np.sum(lens[starts[g]:starts[g + 1]] - np.minimum(P, lens[starts[g]:starts[g + 1]])))
    qo = 2 * wl.num_seqs * wl.num_q_heads * wl.head_dim * wl.elem_bytes
    alg = (pre_reads + own) * per_pos + qo
    L_ = args.layers

    def run(i, rec):
        rec(0)
        step.attention_shared(i % L_)
        rec(1)
    t_step, iv = _timed(run, args.steps, args.warmup, 2)
    t_sh = float(np.mean(iv[:, 0]))

    def run_plain(i, rec):
        rec(0)
        step.attention(i % L_)
        rec(1)
    _, ivp = _timed(run_plain, args.steps, args.warmup, 2)
    t_plain = float(np.mean(ivp[:, 0]))
    # The per-sequence attention bytes (every history position's K and V of
    # every sequence, q, out) as for the decode line: logical bytes, which
    # exceed what HBM serves when the prefix is read once for many sequences.
    alg_logical = logical + qo + 4 * int(((lens + B - 1) // B).sum()) + 4 * wl.num_seqs
    achieved = alg_logical / t_sh / 1e9
    roof = {"bound": "hbm", "kernel": "attn_shared", "achieved": achieved,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None,
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
            "algorithmic_bytes_per_launch": alg_logical, "avg_launch_us": t_sh * 1e6,
            "note": "attn_shared = attn_suffix_kernel + attn_prefix_kernel (which also "
                    "combines each member's pieces; event time and traffic cover both); "
                    "achieved counts logical bytes (each sequence's whole history), which "
                    "exceed the HBM peak because each group's prefix is read once per block "
                    "of member rows; detail.unique_gbps counts every distinct cached "
                    "position once"}
    sname = f"{wl.name}+shared" + (f"+{args.kv_dtype}" if quant else "")
    roof["traffic"] = recorded_traffic("attn_shared", sname)
    config = {"workload": sname, "num_seqs": wl.num_seqs,
              "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
              "head_dim": wl.head_dim, "block_size": B, "groups": int(plens.size),
              "max_group_size": int(mg), "max_prefix_len": int(mp), "max_suffix_len": int(ms),
              "sum_seq_lens": int(lens.sum()), "layers_cycled": L_, "seed": wl.seed}
    detail = {"logical_kv_bytes": logical, "unique_kv_bytes": unique,
              "design_bytes": alg, "design_gbps": alg / t_sh / 1e9,
              "logical_gbps": logical / t_sh / 1e9, "unique_gbps": unique / t_sh / 1e9,
              "shared_us": t_sh * 1e6, "plain_decode_us": t_plain * 1e6,
              "speedup_vs_plain_decode": t_plain / t_sh,
              "plain_decode_logical_gbps": logical / t_plain / 1e9,
              "input_generation_s": gen_s}
    res = _common(args, wl, "paged decode attention KV-read GB/s, logical (shared prefix read "
                  "once per group)", logical / t_step / 1e9, "GB/s", t_step,
                  args.kv_dtype if quant else wl.dtype, config, roof, detail)
    if not args.no_cpu_baseline and not quant:
        cb = cpu_baseline(wl, args.cpu_budget)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(res), flush=True)
    return 0


def bench_swap(args) -> int:
    """Preemption round trip on the configuration's shape: the paused
    sequences' blocks go to pinned host memory and come back."""
    import numpy as np
    import torch

    from paged_attention_slot_amd import ops
    from paged_attention_slot_amd.runtime import DecodeStep
    from workloads import preemption_config_workload

    t0 = time.perf_counter()
    wl = preemption_config_workload(args.config)
    gen_s = time.perf_counter() - t0
    step = DecodeStep(wl)
    (_, p_out), (_, p_in) = step.swap_events
    # One step moves the paused sequences from their current device blocks
    # (where swap-in put them) to their host blocks and back again.
    back = np.ascontiguousarray(p_in[:, ::-1])
    dev = step.device
    po = torch.from_numpy(back).to(dev)
    pi = torch.from_numpy(np.ascontiguousarray(p_in)).to(dev)
    P = int(po.shape[0])
    bb = wl.block_size * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
    launch_bytes = P * bb * 2                      # K and V blocks per launch
    kc, vc, host = step.k_cache, step.v_cache, step.host

    def run(i, rec):
        rec(0)
        ops.swap_out(po, kc, vc, host)
        rec(1)
        ops.swap_in(pi, host, kc, vc)
        rec(2)
    t_step, iv = _timed(run, args.steps, args.warmup, 3)
    t_out, t_in = float(np.mean(iv[:, 0])), float(np.mean(iv[:, 1]))
    # the link's practical rate: the runtime's copy of one contiguous buffer
    # of the same size each way
    dbuf = torch.empty(launch_bytes, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(launch_bytes, dtype=torch.uint8, pin_memory=True)

    def cal(i, rec):
        rec(0)
        hbuf.copy_(dbuf, non_blocking=True)
        rec(1)
        dbuf.copy_(hbuf, non_blocking=True)
        rec(2)
    _, ic = _timed(cal, 5, 1, 3)
    d2h, h2d = launch_bytes / np.mean(ic[:, 0]) / 1e9, launch_bytes / np.mean(ic[:, 1]) / 1e9
    achieved = launch_bytes / t_out / 1e9
    name = f"{wl.name}"
    roof = {"bound": "pcie", "kernel": "swap_blocks_kernel", "achieved": achieved,
            "peak": PCIE_PEAK_GBPS, "unit": "GB/s", "frac": achieved / PCIE_PEAK_GBPS,
            "traffic": recorded_traffic("swap_blocks_kernel", name),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
            "algorithmic_bytes_per_launch": launch_bytes, "avg_launch_us": t_out * 1e6,
            "note": "swap-out launch (device to host); peak = PCIe 5.0 x16, one direction; "
                    "traffic counts every moved byte once read and once written"}
    config = {"workload": name, "num_seqs": wl.num_seqs, "paused_seqs": len(wl.meta["swapped"]),
              "blocks_per_direction": P, "block_bytes_kv": 2 * bb,
              "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
              "block_size": wl.block_size, "num_blocks": wl.num_blocks,
              "host_blocks": wl.num_host_blocks, "seed": wl.seed}
    detail = {"swap_out_us": t_out * 1e6, "swap_in_us": t_in * 1e6,
              "swap_out_gbps": launch_bytes / t_out / 1e9,
              "swap_in_gbps": launch_bytes / t_in / 1e9,
              "contiguous_copy_d2h_gbps": float(d2h), "contiguous_copy_h2d_gbps": float(h2d),
              "swap_out_frac_of_contiguous_copy": float(launch_bytes / t_out / 1e9 / d2h),
              "swap_in_frac_of_contiguous_copy": float(launch_bytes / t_in / 1e9 / h2d),
              "input_generation_s": gen_s}
    res = _common(args, wl, "KV block swap GB/s over the host link (swap-out + swap-in of the "
                  "paused sequences)", 2 * launch_bytes / t_step / 1e9, "GB/s", t_step, wl.dtype,
                  config, roof, detail)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = swap_cpu_baseline(wl, step, back, p_in, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


def swap_cpu_baseline(wl, step, p_out, p_in, budget_s):
    """The oracle's swap_blocks over the same pair lists, out and back, on host
    copies of the pools, until the budget is spent."""
    import numpy as np

    from oracle.cache_ops import swap_blocks
    from paged_attention_slot_amd.runtime import to_host_bits
    kp, vp = to_host_bits(step.k_cache), to_host_bits(step.v_cache)
    hk = np.zeros((wl.num_host_blocks,) + kp.shape[1:], kp.dtype)
    hv = np.zeros_like(hk)
    rounds, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 <= budget_s:
        swap_blocks(p_out, kp, hk)
        swap_blocks(p_out, vp, hv)
        swap_blocks(p_in, hk, kp)
        swap_blocks(p_in, hv, vp)
        rounds += 1
    el = time.perf_counter() - t0
    nbytes = rounds * 2 * len(p_out) * kp[0].nbytes * 2
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rounds} out-and-back rounds of {len(p_out)} block pairs (K and V) "
                      f"between host arrays in {el:.2f} s; NumPy block copies, one thread"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--path", default="decode", choices=["decode", "multi", "swap", "shared"],
                    help="decode step (default), multi-token query attention, block swap, or "
                         "shared-prefix decode attention")
    ap.add_argument("--config", default=None,
                    help="workload (default: llama3-8b-layer, the largest configuration of "
                         "the decode step on one GPU; shared-prefix-cow for --path shared)")
    ap.add_argument("--query-tokens", type=int, default=4,
                    help="--path multi: new query tokens per sequence")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--partition-tokens", type=int, default=None)
    ap.add_argument("--kv-dtype", default="model", choices=["model", "fp8_e4m3", "int8"],
                    help="cache element type: the workload's (default) or one-byte codes")
    ap.add_argument("--no-graph", action="store_true",
                    help="decode path: time eager launches instead of replaying the step as a "
                         "HIP graph")
    ap.add_argument("--unfused", action="store_true",
                    help="decode path: append with the separate write kernel "
                         "(pkv_write, then pkv_attention_decode) instead of the fused "
                         "pkv_attention_decode_append")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run the stream-read calibration kernel (4 GiB) and print GB/s")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU; --gpus must be 1 (no multi-GPU path)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from paged_attention_slot_amd.runtime import DecodeStep
    from workloads import CONFIGS, config_workload, copy_bytes, write_bytes

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate:
        print(json.dumps({"stream_read_gbps": stream_read_gbps(), "bytes": 4 << 30}), flush=True)
        return 0
    if args.config is None:
        args.config = "shared-prefix-cow" if args.path == "shared" else "llama3-8b-layer"
    if args.path == "multi":
        return bench_multi(args)
    if args.path == "shared":
        return bench_shared(args)
    if args.path == "swap":
        return bench_swap(args)
    cfg = CONFIGS[args.config]
    t0 = time.perf_counter()
    wl = config_workload(args.config)
    gen_s = time.perf_counter() - t0
    quant = args.kv_dtype != "model"
    step = DecodeStep(wl, layers=args.layers, partition_tokens=args.partition_tokens,
                      kv_dtype=None if not quant else args.kv_dtype)
    L, K, W = args.layers, args.steps, args.warmup
    N = wl.num_seqs
    lens = wl.seq_lens.astype(np.int64)
    e = 1 if quant else wl.elem_bytes          # cache element bytes
    qe = wl.elem_bytes                         # query / output element bytes
    # K and V of every cached position; INT8 also reads its two fp32 scales
    per_pos = 2 * wl.num_kv_heads * wl.head_dim * e + (8 * wl.num_kv_heads
                                                        if args.kv_dtype == "int8" else 0)
    kv_bytes = int(lens.sum()) * per_pos
    q_bytes = N * wl.num_q_heads * wl.head_dim * qe
    workload_name = wl.name if not quant else f"{wl.name}+{args.kv_dtype}"
    table_bytes = 4 * int(((lens + wl.block_size - 1) // wl.block_size).sum()) + 4 * N
    # the step's append folded into the attention kernel (bf16/f32 pools):
    # it also reads the new-token rows and writes them to their slots
    fused = not quant and not args.unfused
    new_bytes = 2 * N * wl.num_kv_heads * wl.head_dim * e
    part_bytes = kv_bytes + q_bytes + table_bytes          # partition kernel, algorithmic
    folded = fused and step.append_folded                  # the kernel stores the new rows
    if folded:
        part_bytes += 2 * new_bytes + 4 * N
    attn_bytes = part_bytes + q_bytes                      # + the output rows
    n_cow = int(step.cow_pairs.shape[0])

    for i in range(W):
        step.step(i % L, fused=fused)
    torch.cuda.synchronize()

    # Kernel durations: eager launches with HIP events around each phase on
    # the launch stream.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        layer = i % L
        e0, e1, e2, e3 = ev[i]
        e0.record()
        step.copy(layer)
        if fused:
            e1.record()
            step.attention_append(layer, phases=1)
            e2.record()
            step.attention_append(layer, phases=2)
        else:
            step.write(layer)
            e1.record()
            step.attention(layer, phases=1)
            e2.record()
            step.attention(layer, phases=2)
        e3.record()
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t_start
    wall = eager_wall

    # Back to back, one event pair around K launches (layers cycled), so no
    # event sits between two kernels: the attention kernel alone (its average
    # launch duration: the roofline), then the attention with its merge (the
    # attention including the reduce).  When the append is not folded into
    # the attention kernel, its row-copy kernel is left out of both.
    def back_to_back(fn):
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        for i in range(L):
            fn(i)
        torch.cuda.synchronize()
        s0.record()
        for i in range(K):
            fn(i % L)
        s1.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) * 1e-3 / K

    if folded:
        t_part = back_to_back(lambda layer: step.attention_append(layer, phases=1))
        t_attn = back_to_back(lambda layer: step.attention_append(layer, phases=3))
    else:
        t_part = back_to_back(lambda layer: step.attention(layer, phases=1))
        t_attn = back_to_back(lambda layer: step.attention(layer, phases=3))
    graph_wall = None
    if not args.no_graph:
        # The step (copy -> append + attention -> merge, or copy -> write ->
        # attention -> merge) of each layer captured once as a HIP graph and
        # replayed: launches cost no host time.
        graphs = []
        for layer in range(L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step.step(layer, fused=fused)
            graphs.append(g)
        for i in range(W):
            graphs[i % L].replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(K):
            graphs[i % L].replay()
        torch.cuda.synchronize()
        graph_wall = time.perf_counter() - t_start
        wall = graph_wall

    cw = np.array([a.elapsed_time(b) for a, b, _, _ in ev]) * 1e-3
    part = np.array([b.elapsed_time(c) for _, b, c, _ in ev]) * 1e-3
    merge = np.array([c.elapsed_time(d) for _, _, c, d in ev]) * 1e-3
    dev_step = np.array([a.elapsed_time(d) for a, _, _, d in ev]) * 1e-3
    t_step = wall / K
    achieved = part_bytes / t_part / 1e9
    props = torch.cuda.get_device_properties(0)

    res = {
        "metric": METRIC,
        "value": kv_bytes / t_step / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.kv_dtype if quant else wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": workload_name,
            "kv_dtype": args.kv_dtype if quant else wl.dtype,
            "num_seqs": N,
            "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim,
            "block_size": wl.block_size,
            "seq_lens": (f"uniform[{cfg.len_range[0]},{cfg.len_range[1]}]" if cfg.len_range
                         else "fixed" if cfg.fixed_lens else "shared-prefix"),
            "sum_seq_lens": int(lens.sum()),
            "max_seq_len": int(lens.max()),
            "num_blocks": wl.num_blocks,
            "cow_pairs": n_cow,
            "split": step.split,
            "layers_cycled": L,
            "seed": wl.seed,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": {"balanced": "attn_balanced_kernel", "partitions": "attn_partition_kernel",
                       "matrix-balanced": "attn_mfma_balanced_kernel",
                       "matrix": "attn_multi_kernel"}[step.split["mode"]],
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None,
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
            "algorithmic_bytes_per_launch": part_bytes,
            "avg_launch_us": t_part * 1e6,
        },
        "cpu_baseline": None,
        "detail": {
            "kv_bytes_per_step": kv_bytes,
            "attention_gbps": attn_bytes / t_attn / 1e9,
            "attention_frac_of_peak": attn_bytes / t_attn / 1e9 / HBM_PEAK_GBPS,
            "attention_us": t_attn * 1e6,
            "timing": ("attention kernel and attention + merge: one event pair around "
                       f"{K} back-to-back launches each; per-phase figures: events around "
                       "each phase of eager steps"),
            "partition_us_median": float(np.median(part)) * 1e6,
            "partition_us_p10_p90": [float(np.percentile(part, 10)) * 1e6,
                                     float(np.percentile(part, 90)) * 1e6],
            "merge_us_mean": float(np.mean(merge)) * 1e6,
            "append": (("folded into the attention kernel" if step.append_folded else
                        "row-copy kernel, then the attention (pkv_attention_decode_append)")
                       if fused else "separate write kernel"),
            "kv_loads": ("cacheable (the batch shares blocks)" if step.kv_shared
                         else "non-temporal where one wave or query block covers a KV head's "
                              "group (each block read once)"),
            "copy_write_us_mean": float(np.mean(cw)) * 1e6,
            "device_step_us_mean": float(np.mean(dev_step)) * 1e6,
            "step_timing": "hip graph replay" if graph_wall is not None else "eager launches",
            "eager_ms_per_step": eager_wall / K * 1e3,
            "graph_ms_per_step": None if graph_wall is None else graph_wall / K * 1e3,
            "write_bytes": (write_bytes(N, wl.num_kv_heads, wl.head_dim, e) if not quant else
                            N * wl.num_kv_heads * wl.head_dim * 2 * (qe + e)),
            "copy_bytes": copy_bytes(n_cow, wl.block_size, wl.num_kv_heads, wl.head_dim, e),
            "decode_tokens_per_s": N / t_step,
            "attended_tokens_per_s": float(lens.sum()) / t_attn,
            "host_tables_us": step.host_tables_s * 1e6,
            "input_generation_s": gen_s,
            "device": {"name": props.name, "cus": props.multi_processor_count,
                       "gcn_arch": getattr(props, "gcnArchName", "")},
        },
    }
    res["roofline"]["traffic"] = recorded_traffic(res["roofline"]["kernel"], workload_name)
    achievable = stream_read_gbps()
    res["detail"]["stream_read_gbps"] = achievable
    res["detail"]["partition_frac_of_stream_read"] = achieved / achievable
    same = stream_read_same_size_gbps(part_bytes, max(L, 4))
    res["detail"]["stream_read_same_size"] = same
    res["detail"]["partition_frac_of_same_size_stream_read"] = achieved / same["gbps"]
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, args.cpu_budget, args.kv_dtype if quant else None)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        res["detail"]["cpu_baseline_extra"] = {k: cb[k] for k in ("seconds", "host_cpus",
                                                                  "affinity_cpus")}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
