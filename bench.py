"""Benchmark of the paged attention path on one MI355X.

A step = the append of the batch's new tokens + attention over the batch (every
row of the hot path), on seeded synthetic inputs already resident in HBM: one
paged_attention_append call (the append fused into the attention call; with
--step separate, kv_append then paged_attention; the 8-bit cache always uses
its two calls).  Default workload (the headline): the 70B-class decode layer
at full single-GPU shape (256 sequences, contexts lognormal with median 1024
capped at 8192, 64 query / 8 KV heads, d 128, 16-token blocks).  Several
device copies of the batch are cycled so consecutive steps do not re-read the
same lines from the 256 MB last-level cache.

Prints ONE JSON line on stdout:
  value         KV-read GB/s of the whole step: algorithmic K+V bytes (every
                cached token of every sequence read once) / wall-clock step time;
  roofline      the attention call (fused append + split-K decode + merge, and
                prefill on the mixed batch), timed with one HIP event pair
                around the timed region on its stream, against the 8 TB/s HBM
                peak; `traffic` comes from rocprofv3 FETCH_SIZE/WRITE_SIZE
                counters stored under profiles/ (null if the kernels changed since);
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same batch,
                scaled to the whole batch (same unit as value), with the
                GPU/oracle time ratio;
  per_config    the same record for the other configurations: the tiny batch
                (GPU call time; oracle single-threaded and on all cores), the
                Llama-3-8B decode layer, the mixed batch with its shared prefix
                (mixed call, decode-only and prefill-only sub-batches: decode on
                unique and logical bytes, prefill in TFLOP/s of causal pairs
                against the 2.5 PFLOP/s bf16 peak) and the long-context batch;
                each with its roofline, 8-bit-pool call and CPU baseline;
  call_us, separate_calls, graph, append, allocator, measured_peaks:
                single-call spread, the two-call step, a HIP-graph replay,
                kv_append alone at T = 64, 4288, 65536, the host allocator, and
                a device copy / GEMM / the library's read and matrix-core probes.

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


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def cpu_baseline(wl, k2, v2, budget_s: float, f8=None, gpu_call_s=None, threads=None):
    """Time the float64 oracle (as it stands) on whole sequences of the batch, in a seeded random
    order, until ``budget_s`` seconds are used (at least one sequence), and scale to the whole
    batch by the oracle's work per sequence (query rows x keys).  ``value`` is in the unit of the
    GPU figure: K+V bytes of the whole batch (one per value with ``f8``: the 8-bit pools'
    oracle) / the estimated whole-batch oracle time.  ``threads``: BLAS thread limit (None =
    all).  With ``gpu_call_s`` the record carries the whole-batch time ratio oracle / GPU."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    qsl = wl.query_start_loc
    ql = np.diff(qsl).astype(np.int64)
    L = wl.seq_lens.astype(np.int64)
    seqs = [s for s in range(wl.num_seqs) if ql[s] > 0]
    work = {s: int(ql[s]) * int(L[s]) for s in seqs}
    total_work = sum(work.values())
    order = np.random.default_rng(12345).permutation(len(seqs))
    done_work, n_done, passes = 0, 0, 0
    ctx = threadpool_limits(limits=threads) if threads else threadpool_limits(limits=None)
    with ctx:
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        elapsed = 0.0
        while elapsed < budget_s or n_done == 0:
            for idx in order:
                s = seqs[int(idx)]
                rows = list(range(int(qsl[s]), int(qsl[s + 1])))
                if f8 is None:
                    oracle.paged_attention(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                           wl.num_kv_heads, wl.scale, rows=rows)
                else:
                    oracle.paged_attention_fp8(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.query_start_loc,
                                               wl.num_kv_heads, wl.scale, f8.k_scale, f8.v_scale, rows=rows)
                done_work += work[s]
                n_done += 1
                elapsed = time.perf_counter() - t0
                if elapsed >= budget_s:
                    break
            passes += 1
    est_batch_s = elapsed * total_work / done_work
    batch_bytes = wl.kv_read_bytes() // (1 if f8 is None else 2)
    rec = {"value": round(batch_bytes / est_batch_s / 1e9, 4), "unit": "GB/s",
           "cores": int(min(blas_threads, cores)), "kind": "oracle",
           "sample": f"{n_done} whole sequences of the {wl.num_seqs}-sequence batch in a seeded random order "
                     f"({done_work / total_work:.3f} of the batch's rows x keys) in {elapsed:.1f} s, scaled to the "
                     f"whole batch: {est_batch_s:.2f} s; float64 NumPy oracle"
                     + (" over the 8-bit pools" if f8 is not None else "")
                     + f"; BLAS threads {blas_threads}, host cores {cores}",
           "est_batch_s": round(est_batch_s, 4)}
    if gpu_call_s:
        rec["oracle_over_gpu_time"] = round(est_batch_s / gpu_call_s, 1)
    return rec


class Device:
    """Device-side copy of a workload (pools with this step's tokens not yet appended)."""

    def __init__(self, wl, dev, torch):
        import numpy as np
        self.wl, self.dev, self.torch = wl, dev, torch

        def up(a, dt):
            if dt == torch.bfloat16:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.up = up
        self.t = dict(q=up(wl.q, torch.bfloat16), k_new=up(wl.k_new, torch.bfloat16),
                      v_new=up(wl.v_new, torch.bfloat16), slots=up(wl.slot_mapping, torch.int64),
                      kc=up(wl.k_cache, torch.bfloat16), vc=up(wl.v_cache, torch.bfloat16),
                      bt=up(wl.block_tables, torch.int32), sl=up(wl.seq_lens, torch.int32),
                      qsl=up(wl.query_start_loc, torch.int32))

    def clone(self):
        c = object.__new__(Device)
        c.wl, c.dev, c.torch, c.up = self.wl, self.dev, self.torch, self.up
        c.t = {k: v.clone() for k, v in self.t.items()}
        return c

    def subset(self, seqs):
        """Query rows, tables and lengths of the listed sequences (pools shared, already appended)."""
        import numpy as np
        torch, wl = self.torch, self.wl
        seqs = np.asarray(seqs, dtype=np.int64)
        qsl = wl.query_start_loc
        rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs]) if len(seqs) else np.zeros(0, np.int64)
        ql = (qsl[seqs + 1] - qsl[seqs]).astype(np.int32)
        sub_qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        return dict(q=self.t["q"][torch.from_numpy(rows).to(self.dev)].contiguous(),
                    bt=self.up(wl.block_tables[seqs], torch.int32), sl=self.up(wl.seq_lens[seqs], torch.int32),
                    qsl=self.up(sub_qsl, torch.int32), num_seqs=len(seqs), max_query_len=int(ql.max()) if len(ql) else 0)


def time_calls(fn, n, warm, stream, torch):
    """HIP-event times (ms) of n calls of fn on `stream`, after `warm` untimed calls."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def region_ms(fn, n, warm, stream, torch):
    """Average ms of n back-to-back calls of fn, from one HIP event pair around all of them on
    `stream` (no event between calls: each costs the stream idle time of its own)."""
    for _ in range(warm):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def sub_attention_ms(pkv, d, sub, scale, stream, torch, n=100):
    """paged_attention over a sub-batch (its own output and workspace): (per-call times with an
    event pair around each call, average over n back-to-back calls)."""
    wl = d.wl
    out = torch.empty_like(sub["q"])
    ws = torch.empty(pkv.workspace_bytes(sub["num_seqs"], wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                         wl.max_blocks_per_seq, wl.block_size, max(1, sub["max_query_len"])),
                     dtype=torch.uint8, device=d.dev)
    call = pkv.paged_attention(out, sub["q"], d.t["kc"], d.t["vc"], sub["bt"], sub["sl"], sub["qsl"], scale,
                               sub["max_query_len"], workspace=ws, stream=stream, prepare=True)
    return time_calls(call, 30, 3, stream, torch), region_ms(call, n, 10, stream, torch)


def prefill_report(pkv, d, stream, torch):
    wl = d.wl
    pre = wl.prefill_seqs()
    flops = 4 * wl.head_dim * wl.num_q_heads * wl.causal_pairs(pre)
    ms, avg = sub_attention_ms(pkv, d, d.subset(pre), wl.scale, stream, torch)
    tf = flops / (avg * 1e-3) / 1e12
    return {"workload": f"prefill rows of {wl.name}: {len(pre)} chunks, {int(wl.query_lens[pre].sum())} rows, "
                        f"prefixes {sorted(int(wl.seq_lens[s] - wl.query_lens[s]) for s in pre)}",
            "flops_per_call": flops, "call_us_avg": round(avg * 1e3, 3),
            "call_us_median": round(pct(ms, 50) * 1e3, 3),
            "call_us_p10": round(pct(ms, 10) * 1e3, 3), "call_us_p90": round(pct(ms, 90) * 1e3, 3),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "timing": "HIP events around 100 back-to-back calls after 10 untimed ones, / 100 (call_us_avg)",
                         "note": "flops = 4 d Hq x causal (row, key) pairs; the call also launches the "
                                 "(empty) decode grid and the merge launch that carries the planner"}}


def long_prefix_report(pkv, dev, torch, stream):
    """One 512-row chunk over a 65536-token cached prefix with the mixed batch's heads (Hq 32,
    Hkv 8, d 128): 16 row tiles per KV head, too few for the device, so the planner cuts them
    along the keys.  Timed like the prefill rows of the mixed batch."""
    import workloads
    wl = workloads.custom("long-prefix-chunk", [(65536 + 512, 512)], 32, 8, 128, 16, seed=31)
    d = Device(wl, dev, torch)
    pkv.kv_append(d.t["k_new"], d.t["v_new"], d.t["slots"], d.t["kc"], d.t["vc"], stream=stream)
    torch.cuda.synchronize()
    rec = prefill_report(pkv, d, stream, torch)
    rec["roofline"]["note"] = ("flops = 4 d Hq x causal (row, key) pairs; 16 items per KV head cut into pieces "
                               "of consecutive key tiles, merged by the last piece of each item")
    del d
    torch.cuda.empty_cache()
    return rec


def append_report(pkv, dev, torch, stream):
    """kv_append alone into a scratch pool: T new tokens of 8 KV heads x d 128 to random distinct slots."""
    Hkv, D, bs = 8, 128, 16
    res = {}
    for T in (64, 4288, 65536):
        nb = (T + bs - 1) // bs + 16
        kc = torch.zeros(nb, bs, Hkv, D, dtype=torch.bfloat16, device=dev)
        vc = torch.zeros_like(kc)
        kn = torch.randn(T, Hkv, D, device=dev).to(torch.bfloat16)
        vn = torch.randn(T, Hkv, D, device=dev).to(torch.bfloat16)
        g = torch.Generator(device="cpu").manual_seed(T)
        slots = torch.randperm(nb * bs, generator=g)[:T].to(torch.int64).to(dev)

        call = pkv.kv_append(kn, vn, slots, kc, vc, stream=stream, prepare=True)
        ms = time_calls(call, 20, 3, stream, torch)
        avg = region_ms(call, 20, 3, stream, torch)
        moved = 2 * 2 * T * Hkv * D * 2     # K and V, read once and written once
        res[f"T{T}"] = {"us_avg": round(avg * 1e3, 3), "us_median_with_events": round(pct(ms, 50) * 1e3, 3),
                        "GBps": round(moved / (avg * 1e-3) / 1e9, 1)}
        del kc, vc, kn, vn, slots, call
    return res


def graph_report(pkv, c, wl, torch, n=30):
    """One step (the fused append + attention call) captured in a HIP graph and replayed: the
    per-step time without the Python and launch overhead of the eager call."""
    t = c.t

    def body():
        pkv.paged_attention_append(t["out"], t["q"], t["k_new"], t["v_new"], t["slots"], t["kc"], t["vc"],
                                   t["bt"], t["sl"], t["qsl"], wl.scale, wl.max_query_len, workspace=t["ws"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    ms = time_calls(g.replay, n, 3, cur, torch)
    avg = region_ms(g.replay, n, 3, cur, torch)
    torch.cuda.synchronize()
    del g
    return {"graph_step_us_avg": round(avg * 1e3, 3), "graph_step_us_median": round(pct(ms, 50) * 1e3, 3),
            "graph_step_us_p10": round(pct(ms, 10) * 1e3, 3), "replays": n}


def fp8_report(pkv, d, torch, stream, bf16_call_us, n=100, copies=3):
    """The same batch over 8-bit (E4M3) pools: kv_append_fp8 of the step's tokens, then
    paged_attention_fp8 timed like the bf16 call (copies cycled); GB/s of the code bytes."""
    import workloads
    wl = d.wl
    f8 = workloads.fp8_pools(wl)
    t = d.t
    pools = []
    for i in range(copies):
        kc = torch.from_numpy(f8.k_cache).to(d.dev)
        vc = torch.from_numpy(f8.v_cache).to(d.dev)
        pkv.kv_append_fp8(t["k_new"], t["v_new"], t["slots"], kc, vc, f8.k_scale, f8.v_scale, stream=stream)
        pools.append((kc, vc))
    out = torch.empty_like(t["q"])
    ws = torch.empty(pkv.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                         wl.max_blocks_per_seq, wl.block_size, wl.max_query_len),
                     dtype=torch.uint8, device=d.dev)
    it = [0]
    calls = [pkv.paged_attention_fp8(out, t["q"], kc, vc, t["bt"], t["sl"], t["qsl"], wl.scale, wl.max_query_len,
                                     f8.k_scale, f8.v_scale, workspace=ws, stream=stream, prepare=True)
             for kc, vc in pools]

    def call():
        calls[it[0] % copies]()
        it[0] += 1
    ms = time_calls(call, n, 3, stream, torch)
    med = region_ms(call, n, 3, stream, torch)
    code_bytes = wl.kv_read_bytes() // 2
    uniq = wl.unique_kv_read_bytes() // 2
    # the append of the step's new tokens alone
    kc, vc = pools[0]
    ams = time_calls(lambda: pkv.kv_append_fp8(t["k_new"], t["v_new"], t["slots"], kc, vc, f8.k_scale,
                                               f8.v_scale, stream=stream), 20, 3, stream, torch)
    res = {"workload": workload_desc(wl) + ", E4M3 pools (scales 2^-4, 2^-3)",
           "kv_code_bytes_per_call": code_bytes, "call_us_avg": round(med * 1e3, 3),
           "call_us_median": round(pct(ms, 50) * 1e3, 3), "call_us_p10": round(pct(ms, 10) * 1e3, 3),
           "GBps": round(uniq / (med * 1e-3) / 1e9, 1), "frac_of_hbm_peak": round(uniq / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "speedup_vs_bf16_call": round(bf16_call_us / (med * 1e3), 3),
           "append_fp8_us_median": round(pct(ams, 50) * 1e3, 3)}
    del pools, out, ws, calls
    torch.cuda.empty_cache()
    return res


def prefill_fp8_report(pkv, d, torch, stream):
    """The mixed batch's chunked-prefill rows over 8-bit pools, TFLOP/s of causal pairs."""
    import workloads
    wl = d.wl
    f8 = workloads.fp8_pools(wl)
    kc = torch.from_numpy(f8.k_cache).to(d.dev)
    vc = torch.from_numpy(f8.v_cache).to(d.dev)
    t = d.t
    pkv.kv_append_fp8(t["k_new"], t["v_new"], t["slots"], kc, vc, f8.k_scale, f8.v_scale, stream=stream)
    pre = wl.prefill_seqs()
    sub = d.subset(pre)
    out = torch.empty_like(sub["q"])
    ws = torch.empty(pkv.workspace_bytes(sub["num_seqs"], wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                         wl.max_blocks_per_seq, wl.block_size, sub["max_query_len"]),
                     dtype=torch.uint8, device=d.dev)

    call = pkv.paged_attention_fp8(out, sub["q"], kc, vc, sub["bt"], sub["sl"], sub["qsl"], wl.scale,
                                   sub["max_query_len"], f8.k_scale, f8.v_scale, workspace=ws, stream=stream,
                                   prepare=True)
    med = region_ms(call, 20, 3, stream, torch)
    flops = 4 * wl.head_dim * wl.num_q_heads * wl.causal_pairs(pre)
    tf = flops / (med * 1e-3) / 1e12
    del kc, vc, out, ws, call
    torch.cuda.empty_cache()
    return {"call_us_avg": round(med * 1e3, 3), "TFLOPs": round(tf, 1), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}


def allocator_report(pkv, n_rounds=5):
    """Host block allocator: allocate / free of the mixed batch's requests (200 prompts, half
    sharing a 1024-token prefix, 16-token blocks, a pool with 10% spare), us per call."""
    import numpy as np
    rng = np.random.default_rng(7)
    bs = 16
    shared = list(rng.integers(0, 32000, 1024))
    prompts = []
    for i in range(200):
        n = int(rng.integers(256, 4096))
        head = shared if i % 2 == 0 else []
        prompts.append(np.asarray(head + list(rng.integers(0, 32000, n)), dtype=np.int32))
    need = sum(-(-(len(p) + 64) // bs) for p in prompts)
    a = pkv.BlockAllocator(int(need * 1.1) + 1, bs)
    t_alloc, t_free, reused, n_ops = 0.0, 0.0, 0, 0
    for _ in range(n_rounds):
        ids = []
        t0 = time.perf_counter()
        for p in prompts:
            aid, blocks, pre = a.allocate(p, len(p) + 64)
            ids.append(aid)
            reused += pre
        t1 = time.perf_counter()
        for aid, p in zip(ids, prompts):
            a.free(aid, p)
        t2 = time.perf_counter()
        t_alloc += t1 - t0
        t_free += t2 - t1
        n_ops += len(prompts)
    return {"workload": "200 prompts of 256..4096 tokens (+64 to generate), half after a shared 1024-token "
                        "prefix, 16-token blocks, pool = blocks needed + 10%, 5 rounds of allocate all / free all",
            "allocate_us_per_call": round(t_alloc / n_ops * 1e6, 2), "free_us_per_call": round(t_free / n_ops * 1e6, 2),
            "cached_prefix_tokens_per_round": reused // n_rounds,
            "note": "host C++ through ctypes, token ids passed as int32 arrays"}


def measured_peaks(torch, dev, stream):
    x = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    x.fill_(1.0)
    y = torch.empty_like(x)
    ms = time_calls(lambda: y.copy_(x), 10, 2, stream, torch)
    copy_gbs = 2 * x.numel() * 4 / (pct(ms, 50) * 1e-3) / 1e9
    del x, y
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    ms = time_calls(lambda: torch.mm(a, b), 10, 3, stream, torch)
    tf = 2 * n ** 3 / (pct(ms, 50) * 1e-3) / 1e12
    del a, b
    # the library's own probes: a streaming read (the decode kernel's load) and a matrix-core loop
    # (the prefill kernel's instruction) on all compute units
    import paged_kv_cache_tables_amd as pkv
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    buf = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    read_call = pkv.peak_read(buf, sink, stream=stream, prepare=True)
    read_ms = region_ms(read_call, 5, 2, stream, torch)
    read_gbs = buf.numel() / (read_ms * 1e-3) / 1e9
    del read_call, buf
    iters = 10000
    flops = pkv.peak_mfma_bf16(iters, sink, stream=stream)
    mfma_ms = region_ms(lambda: pkv.peak_mfma_bf16(iters, sink, stream=stream), 5, 1, stream, torch)
    mfma_tf = flops / (mfma_ms * 1e-3) / 1e12
    return {"device_copy_GBps": round(copy_gbs, 1), "device_copy_note": "1 GiB copy, bytes read + written",
            "bf16_gemm_TFLOPs": round(tf, 1), "bf16_gemm_note": "torch.mm 8192^3 bf16 (hipBLASLt)",
            "stream_read_GBps": round(read_gbs, 1),
            "stream_read_note": "pkv_peak_read: 2 GiB read once with non-temporal 16-byte loads",
            "mfma_bf16_TFLOPs": round(mfma_tf, 1),
            "mfma_bf16_note": "pkv_peak_mfma_bf16: back-to-back 32x32x16 bf16 MFMAs, 2 waves per SIMD, no memory"}


def time_step(pkv, torch, stream, wl, copies, mode, steps, warmup, f8=None):
    """Time `steps` steps of the batch after `warmup` untimed ones, cycling the device copies.

    mode "fused": one paged_attention_append call per step; "separate": kv_append then
    paged_attention; "fp8": kv_append_fp8 then paged_attention_fp8.  Every call is checked
    and marshalled once per copy (PreparedCall), so the timed loop issues bare C calls and the
    host stays ahead of the device.  Returns the wall-clock step time, the attention call time
    (one HIP event pair around the timed region on the library's stream, / steps: with the
    fused step the region holds nothing but those calls; no event inside the region, since
    each one costs the stream ~5 us of idle time), and single-call times of a later pass."""
    for c in copies:
        t = c.t
        if mode == "fp8":
            c.append = pkv.kv_append_fp8(t["k_new"], t["v_new"], t["slots"], t["kc"], t["vc"], f8.k_scale,
                                         f8.v_scale, stream=stream, prepare=True)
            c.attend = pkv.paged_attention_fp8(t["out"], t["q"], t["kc"], t["vc"], t["bt"], t["sl"], t["qsl"],
                                               wl.scale, wl.max_query_len, f8.k_scale, f8.v_scale,
                                               workspace=t["ws"], stream=stream, prepare=True)
            c.fused = None
        else:
            c.append = pkv.kv_append(t["k_new"], t["v_new"], t["slots"], t["kc"], t["vc"], stream=stream,
                                     prepare=True)
            c.attend = pkv.paged_attention(t["out"], t["q"], t["kc"], t["vc"], t["bt"], t["sl"], t["qsl"],
                                           wl.scale, wl.max_query_len, workspace=t["ws"], stream=stream,
                                           prepare=True)
            c.fused = pkv.paged_attention_append(t["out"], t["q"], t["k_new"], t["v_new"], t["slots"], t["kc"],
                                                 t["vc"], t["bt"], t["sl"], t["qsl"], wl.scale, wl.max_query_len,
                                                 workspace=t["ws"], stream=stream, prepare=True)
    fused = mode == "fused"

    def run(n, evs=None):
        for i in range(n):
            c = copies[i % len(copies)]
            if fused:
                if evs is not None:
                    evs[i][0].record(stream)
                c.fused()
            else:
                c.append()
                if evs is not None:
                    evs[i][0].record(stream)
                c.attend()
            if evs is not None:
                evs[i][1].record(stream)

    run(warmup)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    run(steps)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_ms = ev0.elapsed_time(ev1) / steps
    n_spread = min(steps, 30)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_spread)]
    run(n_spread, evs)
    torch.cuda.synchronize()
    spread = [a.elapsed_time(b) for a, b in evs]
    hot = time_calls(lambda: (copies[0].fused if fused else copies[0].attend)(), 10, 2, stream, torch)
    return {"ms_per_step": elapsed * 1e3 / steps, "call_ms": call_ms, "spread_ms": spread, "hot_ms": hot}


def device_copies(wl, dev, torch, pkv, n_copies, f8=None):
    """n_copies device copies of the batch (bf16 pools, or the 8-bit pools of ``f8``), each with
    its own output and workspace."""
    base = Device(wl, dev, torch)
    if f8 is not None:
        base.t["kc"] = torch.from_numpy(f8.k_cache).to(dev)
        base.t["vc"] = torch.from_numpy(f8.v_cache).to(dev)
    copies = [base] + [base.clone() for _ in range(n_copies - 1)]
    ws_bytes = pkv.workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                   wl.max_blocks_per_seq, wl.block_size, wl.max_query_len)
    for c in copies:
        c.t["out"] = torch.empty_like(c.t["q"])
        c.t["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    return copies


def step_record(wl, cfg, st, mode, kv_bytes, uniq_bytes, traffic_key):
    """The step's throughput and the attention call's roofline (HBM) from a time_step result."""
    pre = wl.prefill_seqs()
    dec = wl.decode_seqs()
    achieved = uniq_bytes / (st["call_ms"] * 1e-3) / 1e9
    kernel = {"fused": "paged_attention_append call (append + ",
              "separate": "kv_append + paged_attention step (",
              "fp8": "kv_append_fp8 + paged_attention_fp8 step ("}[mode]
    kernel += "split-K decode + LSE merge" + (" + prefill" if len(pre) else "") + ")"
    return {
        "ms_per_step": round(st["ms_per_step"], 5),
        "step_GBps": round(kv_bytes / (st["ms_per_step"] * 1e-3) / 1e9, 2),
        "decode_tokens_per_s": round(len(dec) / (st["ms_per_step"] * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "timing": "HIP events around the timed region on the library's stream, / steps",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "avg_call_us": round(st["call_ms"] * 1e3, 3),
                     "algorithmic_bytes_per_call": uniq_bytes,
                     "algorithmic_bytes_note": "K+V bytes of every cached token of every sequence, each physical "
                                               "block of a shared prefix counted once"
                                               + ("; one byte per value (E4M3 codes)" if mode == "fp8" else ""),
                     "traffic": traffic_from_profile(cfg, traffic_key)},
        "call_us": {"median": round(pct(st["spread_ms"], 50) * 1e3, 3),
                    "p10": round(pct(st["spread_ms"], 10) * 1e3, 3),
                    "p90": round(pct(st["spread_ms"], 90) * 1e3, 3),
                    "hot_cache_median": round(pct(st["hot_ms"], 50) * 1e3, 3),
                    "note": "event pair around each " + ("call" if mode == "fused" else "attention call")
                            + " in a pass after the timed region"},
    }


def config_record(cfg, args, torch, pkv, dev, stream, headline=False):
    """Everything measured on one configuration: the timed step with its roofline, the mixed
    batch's sub-batches, the 8-bit pools' call, the two-call step and a graph replay (headline
    only), and the CPU oracle baseline."""
    import numpy as np
    import oracle
    import workloads
    log(f"config {cfg}: generating ...")
    wl = workloads.make_config(cfg)
    fp8 = headline and args.kv == "fp8"
    f8 = workloads.fp8_pools(wl) if fp8 else None
    mode = "fp8" if fp8 else args.step
    copies = device_copies(wl, dev, torch, pkv, args.copies, f8)
    base = copies[0]
    st = time_step(pkv, torch, stream, wl, copies, mode, args.steps, args.warmup, f8)
    div = 2 if fp8 else 1                        # one byte per value for E4M3 pools
    kv_bytes, uniq_bytes = wl.kv_read_bytes() // div, wl.unique_kv_read_bytes() // div
    dec, pre = wl.decode_seqs(), wl.prefill_seqs()
    rec = {"workload": workload_desc(wl), "config_index": cfg, "seed": wl.meta["seed"],
           "kv_bytes_per_step": kv_bytes, "unique_kv_bytes_per_step": uniq_bytes,
           "decode_rows": int(len(dec)), "prefill_rows": int(wl.query_lens[pre].sum()) if len(pre) else 0,
           "appended_tokens": wl.num_q_tokens, "device_copies_cycled": len(copies),
           "kv_cache": "e4m3, per-pool scales 2^-4 (K), 2^-3 (V)" if fp8 else "bf16",
           "steps": args.steps, "warmup": args.warmup,
           "step": {"fused": "paged_attention_append (kv_append fused into the attention call)",
                    "separate": "kv_append + paged_attention", "fp8": "kv_append_fp8 + paged_attention_fp8"}[mode]}
    rec.update(step_record(wl, cfg, st, mode, kv_bytes, uniq_bytes,
                           {"fused": "paged_attention_append", "separate": "paged_attention",
                            "fp8": "paged_attention_fp8"}[mode]))
    log(f"config {cfg}: step {st['ms_per_step'] * 1e3:.1f} us, call {st['call_ms'] * 1e3:.1f} us, "
        f"{rec['roofline']['frac']:.3f} of HBM peak")
    if cfg == 0:
        rec["roofline"]["note"] = "a few KiB of K/V: launch-bound, the fraction is not meaningful"
    if len(pre) and not fp8 and cfg != 0:
        # the mixed batch: decode-only and prefill-only sub-batches in calls of their own
        dms, dmed = sub_attention_ms(pkv, base, base.subset(dec), wl.scale, stream, torch)
        ub, lb = wl.unique_kv_read_bytes(dec), wl.kv_read_bytes(dec)
        rec["decode_only"] = {"call_us_avg": round(dmed * 1e3, 3), "call_us_median": round(pct(dms, 50) * 1e3, 3),
                              "unique_bytes": ub, "logical_bytes": lb,
                              "roofline": {"bound": "hbm", "achieved": round(ub / (dmed * 1e-3) / 1e9, 1),
                                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": round(ub / (dmed * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                           "note": "unique bytes (shared prefix blocks once)"},
                              "logical_GBps": round(lb / (dmed * 1e-3) / 1e9, 1)}
        rec["prefill_only"] = prefill_report(pkv, base, stream, torch)
        flops = rec["prefill_only"]["flops_per_call"]
        floor_s = max(uniq_bytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
        sum_s = uniq_bytes / (HBM_PEAK_GBS * 1e9) + flops / (BF16_PEAK_TFLOPS * 1e12)
        rec["roofline"]["mixed_floor_us"] = round(floor_s * 1e6, 2)
        rec["roofline"]["mixed_frac"] = round(floor_s / (st["call_ms"] * 1e-3), 4)
        rec["roofline"]["mixed_sum_floor_us"] = round(sum_s * 1e6, 2)
        rec["roofline"]["mixed_note"] = ("floor = max(unique bytes / 8 TB/s, causal-pair flops / 2.5 PFLOP/s); "
                                         "sum floor = the two added")
    if headline and mode == "fused" and not args.no_extras:
        sep = time_step(pkv, torch, stream, wl, copies, "separate", args.steps, 3)
        rec["separate_calls"] = {"step_us": round(sep["ms_per_step"] * 1e3, 3),
                                 "step_GBps": round(kv_bytes / (sep["ms_per_step"] * 1e-3) / 1e9, 2),
                                 "attention_call_us_median": round(pct(sep["spread_ms"], 50) * 1e3, 3)}
        rec["graph"] = graph_report(pkv, base, wl, torch)
    if not fp8 and not args.no_extras:
        log(f"config {cfg}: 8-bit pools ...")
        rec["fp8"] = fp8_report(pkv, base, torch, stream, rec["roofline"]["avg_call_us"])
        if len(pre) and cfg != 0:
            rec["prefill_only"]["fp8"] = prefill_fp8_report(pkv, base, torch, stream)
            log(f"config {cfg}: a chunk over a long prefix ...")
            rec["prefill_only"]["long_prefix_chunk"] = long_prefix_report(pkv, dev, torch, stream)
    del copies, base
    torch.cuda.empty_cache()
    if not args.no_cpu:
        log(f"config {cfg}: CPU oracle ...")
        gpu_s = st["call_ms"] * 1e-3
        if fp8:
            k2, v2 = oracle.kv_append_fp8(f8.k_cache, f8.v_cache, wl.k_new, wl.v_new, wl.slot_mapping,
                                          f8.k_scale, f8.v_scale)
        else:
            k2, v2 = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
        budget = args.cpu_budget if headline else args.cpu_budget_other
        rec["cpu_baseline"] = cpu_baseline(wl, k2, v2, budget, f8, gpu_call_s=gpu_s)
        if cfg == 0:
            rec["cpu_baseline_single_thread"] = cpu_baseline(wl, k2, v2, min(budget, 2.0), f8, gpu_call_s=gpu_s,
                                                             threads=1)
        del k2, v2
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=2, help="headline workload: 0..4 (2 = 70B-class decode)")
    ap.add_argument("--copies", type=int, default=3, help="device copies of the batch cycled per step")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time for the headline configuration's cpu_baseline")
    ap.add_argument("--cpu-budget-other", type=float, default=6.0,
                    help="seconds of oracle time for each other configuration's cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default="bf16",
                    help="cache element type of the headline step: bf16 (default) or 8-bit E4M3 codes with "
                         "per-pool scales (kv_append_fp8 + paged_attention_fp8; implies --no-extras)")
    ap.add_argument("--step", choices=["fused", "separate"], default="fused",
                    help="timed step: paged_attention_append, or kv_append then paged_attention (bf16 cache)")
    ap.add_argument("--no-extras", action="store_true",
                    help="the headline configuration only (no other configurations, sub-batches, 8-bit "
                         "pools, append sweep, allocator or peak measurements)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the step, run a plain device copy of MIB MiB --steps times "
                         "(reference kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--long-prefix-only", action="store_true",
                    help="instead of the step, time only the prefill call of one 512-row chunk over a "
                         "65536-token cached prefix (its items cut along the keys) and print its record")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the attention would "
              "shard by KV heads or by sequences, with no collective). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
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
    if args.kv == "fp8":
        args.no_extras = True
    stream = torch.cuda.current_stream(dev)
    if args.long_prefix_only:
        print(json.dumps({"long_prefix_chunk": long_prefix_report(pkv, dev, torch, stream)}), flush=True)
        return

    head = config_record(args.config, args, torch, pkv, dev, stream, headline=True)
    fp8 = args.kv == "fp8"
    result = {
        "metric": METRIC,
        "value": head["step_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (E4M3 K/V cache)" if fp8 else "bf16",
        "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "config_index", "seed", "kv_bytes_per_step",
                                        "unique_kv_bytes_per_step", "decode_rows", "prefill_rows",
                                        "appended_tokens", "device_copies_cycled", "kv_cache")},
        "decode_tokens_per_s": head["decode_tokens_per_s"],
        "step": head["step"],
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "call_us": head["call_us"],
    }
    for k in ("separate_calls", "graph", "fp8", "decode_only", "prefill_only"):
        if k in head:
            result[k] = head[k]
    if not args.no_extras:
        result["per_config"] = {}
        for cfg in (0, 1, 2, 3, 4):
            if cfg != args.config:
                result["per_config"][f"config{cfg}"] = config_record(cfg, args, torch, pkv, dev, stream)
        log("append, allocator, peaks ...")
        result["append"] = append_report(pkv, dev, torch, stream)
        result["allocator"] = allocator_report(pkv)
        result["measured_peaks"] = measured_peaks(torch, dev, stream)
        achieved = result["roofline"]["achieved"]
        result["measured_peaks"]["decode_frac_of_device_copy"] = round(
            achieved / result["measured_peaks"]["device_copy_GBps"], 4)
        result["measured_peaks"]["decode_frac_of_stream_read"] = round(
            achieved / result["measured_peaks"]["stream_read_GBps"], 4)
        c3 = result["per_config"].get("config3") or (head if args.config == 3 else None)
        if c3 is not None and "prefill_only" in c3:
            tf = c3["prefill_only"]["roofline"]["achieved"]
            result["measured_peaks"]["prefill_frac_of_bf16_gemm"] = round(
                tf / result["measured_peaks"]["bf16_gemm_TFLOPs"], 4)
            result["measured_peaks"]["prefill_frac_of_mfma_loop"] = round(
                tf / result["measured_peaks"]["mfma_bf16_TFLOPs"], 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
