#!/usr/bin/env python3
"""Paged decode step on one MI355X: KV append, copy-on-write copy and
block-table GQA decode attention through libpkv.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--layers L]

A step is one pass of the device hot path over one batch: pkv_copy_blocks
(when the batch has copy-on-write pairs), pkv_write of one new token per
sequence, then pkv_attention_decode (partition kernel, then the split-KV merge).
Inputs are resident in HBM before the timed region.  ``--layers`` pool pairs
with identical block tables are cycled, one per step, so that consecutive steps
read different memory (as a model's layers do) and no step is served from the
previous step's cached lines.  Prints one JSON line.
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
METRIC = "paged decode attention KV-read GB/s (% of MI355X HBM peak); tokens/s"


def cpu_baseline(wl, budget_s: float) -> dict:
    """The CPU oracle (fp64 NumPy, as it stands) on a bounded sample of the same
    workload: its block manager and writes first (untimed), then copy + write of
    the step and attention sequence by sequence, cycling over the batch, until
    ``budget_s`` elapses."""
    import numpy as np

    from oracle.attention import attention_decode
    from oracle.replay import OracleState

    st = OracleState(wl, keep_values=False)
    st.build_context()
    st.decode_tables()
    t0 = time.perf_counter()
    st.decode_device_part()
    done = []
    while time.perf_counter() - t0 <= budget_s:
        s = len(done) % wl.num_seqs
        attention_decode(wl.q, st.k_pool, st.v_pool, st.block_tables, st.seq_lens, wl.scale,
                         seqs=[s])
        done.append(s)
    el = time.perf_counter() - t0
    lens = st.seq_lens[done].astype(np.int64)
    kv = int(lens.sum()) * 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
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


def kernel_source_sha256() -> str:
    """Hash of the attention kernel's sources (matches profile records)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("paged_attention_slot_amd/csrc/attn_decode.hip",
              "paged_attention_slot_amd/csrc/pkv_device.h"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the counter record under profiles/ for this
    kernel and workload, if the kernel sources are unchanged since; else None."""
    import glob
    import re
    sha = kernel_source_sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for m in re.finditer(r"<!-- pkv-traffic (\{.*?\}) -->", fh.read()):
                rec = json.loads(m.group(1))
                if rec["kernel"] == kernel and rec["workload"] == workload and \
                        rec["source_sha256"] == sha:
                    return (rec["fetch_kib"] * rec["fetch_scale"] +
                            rec["write_kib"] * rec["write_scale"]) * 1024.0
    return None


def stream_read_gbps(nbytes: int = 4 << 30, iters: int = 10, workgroups: int = 8192) -> float:
    """Achievable read rate on this device: libpkv's plain coalesced stream
    kernel over ``nbytes`` (median of ``iters`` runs, HIP events)."""
    import numpy as np
    import torch

    from paged_attention_slot_amd import ops
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(workgroups, dtype=torch.int32, device="cuda")
    ops.stream_read(buf, sink, workgroups)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        ops.stream_read(buf, sink, workgroups)
        b.record()
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    del buf
    torch.cuda.empty_cache()
    return nbytes / t / 1e9


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3-0.6b-layer")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--partition-tokens", type=int, default=None)
    ap.add_argument("--kv-dtype", default="model", choices=["model", "fp8_e4m3", "int8"],
                    help="cache element type: the workload's (default) or one-byte codes")
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
    part_bytes = kv_bytes + q_bytes + table_bytes          # partition kernel, algorithmic
    attn_bytes = part_bytes + q_bytes                      # + the output rows
    n_cow = int(step.cow_pairs.shape[0])

    for i in range(W):
        step.step(i % L)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        layer = i % L
        e0, e1, e2, e3 = ev[i]
        e0.record()
        step.copy(layer)
        step.write(layer)
        e1.record()
        step.attention(layer, phases=1)
        e2.record()
        step.attention(layer, phases=2)
        e3.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    cw = np.array([a.elapsed_time(b) for a, b, _, _ in ev]) * 1e-3
    part = np.array([b.elapsed_time(c) for _, b, c, _ in ev]) * 1e-3
    merge = np.array([c.elapsed_time(d) for _, _, c, d in ev]) * 1e-3
    dev_step = np.array([a.elapsed_time(d) for a, _, _, d in ev]) * 1e-3
    t_step = wall / K
    t_attn = float(np.mean(part + merge))
    achieved = part_bytes / float(np.mean(part)) / 1e9
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
            "kernel": ("attn_balanced_kernel" if step.split["mode"] == "balanced"
                       else "attn_partition_kernel"),
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None,
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
            "algorithmic_bytes_per_launch": part_bytes,
            "avg_launch_us": float(np.mean(part)) * 1e6,
        },
        "cpu_baseline": None,
        "detail": {
            "kv_bytes_per_step": kv_bytes,
            "attention_gbps": attn_bytes / t_attn / 1e9,
            "attention_frac_of_peak": attn_bytes / t_attn / 1e9 / HBM_PEAK_GBPS,
            "partition_us_median": float(np.median(part)) * 1e6,
            "partition_us_p10_p90": [float(np.percentile(part, 10)) * 1e6,
                                     float(np.percentile(part, 90)) * 1e6],
            "merge_us_mean": float(np.mean(merge)) * 1e6,
            "copy_write_us_mean": float(np.mean(cw)) * 1e6,
            "device_step_us_mean": float(np.mean(dev_step)) * 1e6,
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
    if not args.no_cpu_baseline and not quant:
        cb = cpu_baseline(wl, args.cpu_budget)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        res["detail"]["cpu_baseline_extra"] = {k: cb[k] for k in ("seconds", "host_cpus",
                                                                  "affinity_cpus")}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
