"""Benchmark of one step of the paged attention path on one MI355X.

A step = kv_append of the batch's new tokens + one paged_attention call over
the batch (every row of the hot path), on seeded synthetic inputs already
resident in HBM.  Default workload: the Llama-3-8B-shaped decode layer (64
sequences, contexts U{128..4096}, 32 query / 8 KV heads, d 128, 16-token
blocks).  Several device copies of the batch are cycled so consecutive steps
do not re-read the same lines from the 256 MB last-level cache.

Prints ONE JSON line on stdout:
  value       KV-read GB/s of the whole step: algorithmic K+V bytes (every
              cached token of every sequence read once) / step time;
  roofline    the attention call (split-K decode + merge), timed with HIP
              events on its stream around every call of the timed region,
              against the 8 TB/s HBM peak; `traffic` comes from rocprofv3
              FETCH_SIZE/WRITE_SIZE counters stored under profiles/ (null if
              the kernels changed since);
  cpu_baseline the float64 CPU oracle on a bounded sample of the same batch.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config i]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode KV-read GB/s (% of HBM peak); prefill TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_tables_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def workload_desc(wl) -> str:
    ql = wl.query_lens
    return (f"{wl.name}: {wl.num_seqs} seqs ({int((ql == 1).sum())} decode, {int((ql > 1).sum())} prefill), "
            f"Hq {wl.num_q_heads}, Hkv {wl.num_kv_heads}, d {wl.head_dim}, block {wl.block_size}, "
            f"{wl.num_blocks} pool blocks")


def traffic_from_profile(cfg: int, kernel_key: str):
    """HBM bytes per attention call from committed rocprofv3 counters, if they match the sources."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(f"config{cfg}", {}).get(kernel_key)
    if not ent or ent.get("source_digest") != source_digest():
        return None
    return ent.get("hbm_bytes_per_call")


def cpu_baseline(wl, k2, v2, budget_s: float):
    """Time the float64 oracle (as it stands) on whole sequences of the batch until the budget is used."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cores = len(os.sched_getaffinity(0))
    bytes_done, t_used, seqs, passes = 0, 0.0, 0, 0
    qsl = wl.query_start_loc
    t0 = time.perf_counter()
    # whole sequences, in batch order, repeating the batch until ~budget seconds of oracle work
    while t_used < budget_s:
        for s in range(wl.num_seqs):
            rows = list(range(int(qsl[s]), int(qsl[s + 1])))
            if not rows:
                continue
            oracle.paged_attention(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                   wl.num_kv_heads, wl.scale, rows=rows)
            seqs += 1
            bytes_done += wl.kv_read_bytes([s])
            t_used = time.perf_counter() - t0
            if t_used >= budget_s:
                break
        passes += 1
    return {"value": round(bytes_done / t_used / 1e9, 4), "unit": "GB/s", "cores": int(min(threads, cores)),
            "kind": "oracle",
            "sample": f"{seqs} sequence passes over the {wl.num_seqs}-sequence batch (whole sequences, all heads, "
                      f"batch repeated {passes}x), "
                      f"{bytes_done / 1e6:.1f} MB of K/V in {t_used:.1f} s; float64 NumPy oracle; "
                      f"BLAS threads {threads}, host cores {cores}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload: 0..4 (1 = Llama-3-8B decode)")
    ap.add_argument("--copies", type=int, default=3, help="device copies of the batch cycled per step")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the step, run a plain device copy of MIB MiB --steps times "
                         "(reference kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the attention shards by "
              "KV heads or sequences with no collective; see DESIGN.md). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    import paged_kv_cache_tables_amd as pkv

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    pkv.load_library()

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(args.steps):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "steps": args.steps}), flush=True)
        return

    log(f"generating config {args.config} ...")
    wl = workloads.make_config(args.config)

    def up(a, dt):
        if dt == torch.bfloat16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    base = dict(q=up(wl.q, torch.bfloat16), k_new=up(wl.k_new, torch.bfloat16), v_new=up(wl.v_new, torch.bfloat16),
                slots=up(wl.slot_mapping, torch.int64), kc=up(wl.k_cache, torch.bfloat16),
                vc=up(wl.v_cache, torch.bfloat16), bt=up(wl.block_tables, torch.int32),
                sl=up(wl.seq_lens, torch.int32), qsl=up(wl.query_start_loc, torch.int32))
    copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(args.copies - 1)]
    ws_bytes = pkv.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                   wl.max_blocks_per_seq, wl.block_size)
    for c in copies:
        c["out"] = torch.empty_like(c["q"])
        c["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(c, ev=None):
        pkv.kv_append(c["k_new"], c["v_new"], c["slots"], c["kc"], c["vc"], stream=stream)
        if ev is not None:
            ev[0].record(stream)
        pkv.paged_attention(c["out"], c["q"], c["kc"], c["vc"], c["bt"], c["sl"], c["qsl"], wl.scale,
                            wl.max_query_len, workspace=c["ws"], stream=stream)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(copies[i % len(copies)])
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(copies[i % len(copies)], evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_per_step = elapsed * 1e3 / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    attn_avg_ms = float(np.mean(attn_ms))
    kv_bytes = wl.kv_read_bytes()
    uniq_bytes = wl.unique_kv_read_bytes()
    dec = wl.decode_seqs()
    pre = wl.prefill_seqs()
    flops = 4 * wl.head_dim * wl.num_q_heads * wl.causal_pairs(pre)
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = uniq_bytes / (attn_avg_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_desc(wl), "config_index": args.config, "seed": wl.meta["seed"],
                   "kv_bytes_per_step": kv_bytes, "unique_kv_bytes_per_step": uniq_bytes,
                   "decode_rows": int(len(dec)), "prefill_rows": int(wl.query_lens[pre].sum()) if len(pre) else 0,
                   "appended_tokens": wl.num_q_tokens, "device_copies_cycled": len(copies)},
        "decode_tokens_per_s": round(len(dec) / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "paged_attention call (split-K decode + LSE merge"
                     + (" + prefill" if len(pre) else "") + ")",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "avg_call_us": round(attn_avg_ms * 1e3, 3),
                     "algorithmic_bytes_per_call": uniq_bytes,
                     "traffic": traffic_from_profile(args.config, "paged_attention")},
    }
    if len(pre):
        result["prefill_tflops_if_alone"] = None   # the mixed call is reported as one unit
        result["prefill_flops_per_call"] = flops
    log(f"step {ms_per_step * 1e3:.1f} us, attention call {attn_avg_ms * 1e3:.1f} us, "
        f"{value:.0f} GB/s step, {achieved:.0f} GB/s attention")

    if not args.no_cpu:
        import oracle
        k2, v2 = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
        result["cpu_baseline"] = cpu_baseline(wl, k2, v2, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
