"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the path over one synthetic batch with every input
already resident in HBM.  The headline workload is the 8B-class decode
batch (Hq 32 / Hkv 8 / head_dim 128, 64 requests with kv lengths uniform
in [512, 4096], a 512K-slot randomly permuted pool, page_size 1): a step is
``store_kv`` of the 64 new K/V rows and the split-KV paged decode, run as
one store + decode launch and the LSE merge.  The line also carries the
other workloads (``--configs``, all of them by default): the extend batch (8
chunked-prefill requests over prefixes up to 8K, 4 of them sharing one
2,048-slot prefix), the long-tail decode batch, the mixed batch at page_size
1 and 16, the embedding gather and the attention-layer prologue.

Prints ONE JSON line (rank 0, N = 1).  ``value`` = distinct K/V bytes the
decode must read / (wall time of the K timed steps / K).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
EXTRA_WARM_S = 0.5              # untimed warm-up per extra workload (seconds of its own steps)
METRIC = "paged decode KV GB/s + extend TFLOP/s on 1 MI355X, % of roofline"
# every library source and the public headers: a stored traffic figure is
# used only while none of them has changed since the counters were taken
CSRC_DIR = os.path.join(ROOT, "paged_kv_attention_30_amd", "csrc")
INCLUDE_DIR = os.path.join(ROOT, "include")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_c2_traffic.md")

WORKLOAD_TEXT = {
    "C1": "tiny paged GQA decode + store_kv: Hq 16 / Hkv 8 / D 128, batch 4, kv lens "
          "[17, 64, 100, 255], 1,024-slot randomly permuted pool, page_size 1, bf16 N(0,1), "
          "seed 1 (latency-bound: 1.8 MB of K/V)",
    "C2": "paged GQA decode + store_kv: Hq 32 / Hkv 8 / D 128, batch 64, kv lens U[512,4096], "
          "524,288-slot randomly permuted pool, page_size 1, bf16 N(0,1), seed 2",
    "C3": "causal chunked-prefill extend + store_kv: Hq 32 / Hkv 8 / D 128, batch 8, prefixes "
          "[2048 x4 shared, 0, 1024, 4096, 8192], extend lens U[512,2048], page_size 1, seed 3",
    "C4": "long-tail paged decode + store_kv: Hq 64 / Hkv 8 / D 128, batch 256, kv lens "
          "lognormal(median 2048, sigma 1) clipped to [1024, 32768], split-KV + LSE merge, seed 4",
    "C5a": "mixed batch, page_size 1: store_kv of 2,175 rows + decode of 127 requests "
           "(lens U[256,8192]) + extend (prefix 6144, extend 2048); 64 requests share a "
           "1,024-token prefix; Hq 32 / Hkv 8, seed 5",
    "C5b": "mixed batch as C5a at page_size 16 (16-slot pages, page permutation), seed 5",
    "PRO": "attention-layer prologue (q/k RMSNorm + RoPE + store_kv): a chunk of 8,192 tokens at "
           "positions 0..8191, Hq 32 / Hkv 8 / D 128 (Qwen3-8B-class), merged qkv bf16 N(0,1), "
           "norm weights N(0,1), RoPE base 1e6, slots a random permutation of a 524,288-slot pool, "
           "seed 42",
    "KVC": "host KV cache manager (page allocator + radix prefix cache, C++): 1,024 requests, "
           "each one of 32 Zipf(1.1)-popular 1,024-token system prompts + 128..256 own tokens, "
           "32..64 decode steps, page_size 16, 262,144-slot pool, 128 rows, seed 7",
    "GRAPH": "decode step (store_kv + paged decode) replayed from captured HIP graphs (padding "
             "node + one store + decode launch, or + the two calls) vs the eager one-launch "
             "planned call: Hq 32 / Hkv 8 / D 128, kv lens U[512,4096], 524,288-slot pool, "
             "batch 1 / 8 / 32 / 64 of a 64-bucket ladder [1,2,4,8,16,...,64], seed 43",
    "EMB": "embedding gather: 8,192 token ids uniform over a 151,936 x 4,096 bf16 table "
           "(Qwen3-8B-class vocabulary and hidden size, one tensor-parallel rank), ids int32, "
           "table N(0,1), seed 41",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sources() -> list:
    files = [os.path.join(CSRC_DIR, f) for f in os.listdir(CSRC_DIR)]
    files += [os.path.join(INCLUDE_DIR, f) for f in os.listdir(INCLUDE_DIR)]
    return sorted(f for f in files if f.endswith((".hip", ".hpp", ".cpp", ".h")))


def kernel_hash() -> str:
    """Hash of every library source file (names and contents)."""
    h = hashlib.sha256()
    for f in kernel_sources():
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def upload(inp):
    """Copy one synthetic batch to the GPU (bf16 tensors keep their bits)."""
    import torch

    def up(a):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            x = x.view(torch.int16).view(torch.bfloat16)
        return x.to("cuda")
    t = {"k": up(inp.k_pool), "v": up(inp.v_pool), "pt": up(inp.page_table),
         "out_loc": up(inp.out_loc), "k_new": up(inp.k_new), "v_new": up(inp.v_new)}
    if inp.num_decode:
        t.update(dq=up(inp.dec_q), d_rows=up(inp.dec_req_rows), d_lens=up(inp.dec_seq_lens),
                 d_max=int(inp.dec_seq_lens.max()))
    if inp.num_extend:
        t.update(eq=up(inp.ext_q), e_rows=up(inp.ext_req_rows), e_pre=up(inp.ext_prefix_lens),
                 e_ext=up(inp.ext_extend_lens), e_off=up(inp.ext_q_offsets),
                 e_max=int(inp.ext_extend_lens.max()),
                 e_kv=int((inp.ext_prefix_lens + inp.ext_extend_lens).max()))
    return t


class Run:
    """One workload on the GPU: uploads once, then enqueues steps."""

    def __init__(self, inp, split_tokens: int = 0, fuse_store: bool = True):
        import torch
        import paged_kv_attention_30_amd as msgl
        self.torch, self.msgl, self.inp = torch, msgl, inp
        self.t = upload(inp)
        self.split = split_tokens
        t = self.t
        self.dec_out = self.dec_lse = self.ws = None
        if inp.num_decode:
            B, hq = inp.num_decode, inp.num_q_heads
            self.dec_out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
            self.dec_lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
            need, self.split_used = msgl.paged_decode_workspace_size(
                B, hq, inp.num_kv_heads, t["d_max"], split_tokens)
            self.ws = msgl.alloc_workspace(need)
        if inp.num_extend:
            T = inp.ext_tokens
            self.ext_out = torch.empty((T, inp.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
            self.ext_lse = torch.empty((T, inp.num_q_heads), dtype=torch.float32, device="cuda")
            self.ext_ws = msgl.alloc_workspace(msgl.paged_extend_workspace_size(
                inp.num_extend, inp.num_q_heads, inp.num_kv_heads, t["e_max"], t["e_kv"]))

        # validated and marshalled once; each phase is then one library call.
        # A decode-only batch (one new row per request) stores and decodes in
        # one launch, as the attention layer's forward runs the two.
        self.fused = bool(fuse_store and inp.num_decode and not inp.num_extend
                          and inp.out_loc.shape[0] == inp.num_decode)
        self.p_store = msgl.plan_store_kv(t["k"], t["v"], t["k_new"], t["v_new"], t["out_loc"])
        if self.fused:
            self.p_dec = msgl.plan_store_kv_paged_decode(
                t["dq"], t["k"], t["v"], t["k_new"], t["v_new"], t["out_loc"], t["pt"],
                t["d_lens"], t["d_max"], inp.sm_scale, req_rows=t["d_rows"],
                page_size=inp.page_size, split_tokens=split_tokens, out=self.dec_out,
                lse=self.dec_lse, workspace=self.ws)
        elif inp.num_decode:
            self.p_dec = msgl.plan_paged_decode(
                t["dq"], t["k"], t["v"], t["pt"], t["d_lens"], t["d_max"], inp.sm_scale,
                req_rows=t["d_rows"], page_size=inp.page_size, split_tokens=split_tokens,
                out=self.dec_out, lse=self.dec_lse, workspace=self.ws)
        if inp.num_extend:
            self.p_ext = msgl.plan_paged_extend(
                t["eq"], t["k"], t["v"], t["pt"], t["e_pre"], t["e_ext"], t["e_off"], t["e_max"],
                t["e_kv"], inp.sm_scale, req_rows=t["e_rows"], page_size=inp.page_size,
                out=self.ext_out, lse=self.ext_lse, workspace=self.ext_ws)

    def store(self):
        self.p_store.run()

    def decode(self):
        self.p_dec.run()

    def extend(self):
        self.p_ext.run()

    def step(self):
        if not self.fused:
            self.store()
        if self.inp.num_decode:
            self.decode()
        if self.inp.num_extend:
            self.extend()

    def phases(self):
        ph = [] if self.fused else [("store", self.store)]
        if self.inp.num_decode:
            ph.append(("decode", self.decode))
        if self.inp.num_extend:
            ph.append(("extend", self.extend))
        return ph

    def capture(self):
        """Record each phase of a step as a HIP graph (as a serving loop replays its
        decode step), so the timed loop launches graphs and host-side argument
        marshalling never leaves the GPU idle between kernels."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graphs = {}
        for name, fn in self.phases():
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            self.graphs[name] = g
        torch.cuda.synchronize()


def timed_steps(run: Run, steps: int, warmup: int, graphs: bool = False,
                min_warm_s: float = 0.0):
    """Warm up, then time exactly ``steps`` whole steps, then each phase alone.

    Warm-up is ``warmup`` steps, continued (when ``min_warm_s`` > 0) until
    that many seconds of steps have run: after seconds of host-side input
    generation the GPU idles down, and a few steps do not bring its clock
    back (the extend read 12-14% slower after 3 warm-up steps than after 50).

    The steps are bracketed by two HIP events only (an event recorded between
    two kernels leaves the GPU idle for several microseconds, so none sits
    inside the timed steps).  Each phase's average duration then comes from
    ``steps`` back-to-back calls of that phase alone, bracketed the same way.
    Each phase is one planned library call (validated and marshalled when the
    run was set up), or with ``graphs`` the replay of its captured graph."""
    torch = run.torch
    if graphs:
        run.capture()
        calls = {name: g.replay for name, g in run.graphs.items()}
    else:
        calls = dict(run.phases())
    order = [c for c in ("store", "decode", "extend") if c in calls]

    def step():
        for c in order:
            calls[c]()

    w0 = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    while time.perf_counter() - w0 < min_warm_s:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    phase = {}
    for c in order:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            calls[c]()
        b.record()
        torch.cuda.synchronize()
        phase[c] = a.elapsed_time(b) / steps
    return dict(total_ms=total_ms, wall_s=wall, store_ms=[phase.get("store", 0.0)],
                dec_ms=[phase.get("decode", 0.0)], ext_ms=[phase.get("extend", 0.0)])


def step_distribution(run: Run, steps: int):
    """Median and p10 / p90 of single steps, each between its own pair of HIP
    events and followed by a synchronisation (so each includes the event and
    launch latency that the back-to-back figure leaves out)."""
    torch = run.torch
    calls = dict(run.phases())
    order = [c for c in ("store", "decode", "extend") if c in calls]
    ts = []
    for _ in range(steps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for c in order:
            calls[c]()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    p10, p50, p90 = np.percentile(ts, [10, 50, 90])
    return {"single_step_ms_p10": round(float(p10), 4), "single_step_ms_median": round(float(p50), 4),
            "single_step_ms_p90": round(float(p90), 4)}


def cold_decode_ms(run: Run, reps: int = 10):
    """Decode time with L2 and the 256 MB Infinity Cache flushed before each call.

    The flush reads a 1 GiB buffer (a read leaves the caches holding clean
    lines of it, so the decode pays no write-backs for the flush)."""
    torch = run.torch
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    out = []
    graphs = getattr(run, "graphs", None)
    call = graphs["decode"].replay if graphs else run.decode
    for _ in range(reps):
        torch.sum(scratch, dim=0, out=sink)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    del scratch
    return float(np.median(out))


def load_traffic(khash: str):
    """Measured HBM bytes per decode call from the committed counter summary.

    Returns None when there is no summary or it was taken on other kernel
    sources (its recorded hash differs from the current one).
    """
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", " ", "|")):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_hash") != khash:
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_description() -> str:
    """CPU model, logical CPUs visible / usable, and the BLAS numpy uses."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{d.get('internal_api')} ({d.get('num_threads')} "
                f"thread{'' if d.get('num_threads') == 1 else 's'})"
                for d in threadpool_info() if d.get("user_api") == "blas"]
        if libs:
            blas = ", ".join(libs)
    except ImportError:  # pragma: no cover
        pass
    return f"{model}, {os.cpu_count()} logical CPUs visible, {usable} usable; numpy BLAS {blas}"


# --- CPU baseline: the oracle on the host cores ------------------------------
# The oracle's page-table walk is a Python loop (it holds the interpreter lock),
# so "all cores" means a pool of forked worker processes, each with one BLAS
# thread; it runs before the GPU is initialised, so forking is safe.  The
# workload being timed sits in this module global when the pool forks, and
# the workers read it copy-on-write.
_CPU_JOB = {}


def _cpu_task(task):
    import oracle
    kind, a, b = task
    j = _CPU_JOB
    if kind == "decode":
        inp = j["inp"]
        sel = slice(a, b)
        oracle.paged_decode(inp.dec_q[sel], j["kp"], j["vp"], inp.page_table,
                            inp.dec_req_rows[sel], inp.dec_seq_lens[sel], inp.sm_scale,
                            inp.num_kv_heads)
    else:
        inp = j["inp"]
        oracle.paged_extend(inp.ext_q, j["kp"], j["vp"], inp.page_table, inp.ext_req_rows,
                            inp.ext_prefix_lens, inp.ext_extend_lens, inp.ext_q_offsets,
                            inp.sm_scale, inp.num_kv_heads, query_subset=j["rows"][a:b])
    return 0


def _time_tasks(tasks, workers: int, reps: int = 3) -> float:
    """Median wall time of ``reps`` passes over ``tasks`` after one warm-up
    pass: in this process (``workers`` = 1) or spread over a forked pool."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    times = []
    with threadpool_limits(limits=1):
        if workers == 1:
            for i in range(reps + 1):
                t0 = time.perf_counter()
                for t in tasks:
                    _cpu_task(t)
                if i:
                    times.append(time.perf_counter() - t0)
        else:
            with mp.get_context("fork").Pool(workers) as pool:
                for i in range(reps + 1):
                    t0 = time.perf_counter()
                    pool.map(_cpu_task, tasks, chunksize=1)
                    if i:
                        times.append(time.perf_counter() - t0)
    return float(np.median(times))


def cpu_baselines() -> dict:
    """The fp64 oracle timed on the host (rank 0, before the GPU is touched):
    on one core and on every usable core, median of 3 passes after 1 warm-up.

    Decode: the whole tiny batch, the whole headline batch and the first 32
    decode requests of the mixed batch (GB/s of distinct K/V read).  Extend:
    8 query rows spread over each request of the chunked-prefill batch
    (TFLOP/s of causal pairs).  Per-request (decode) or 4-row (extend) tasks;
    both modes run the same task list."""
    import oracle
    from workloads import make_config, metrics
    usable = len(os.sched_getaffinity(0))
    workers = max(1, min(usable, 16))
    host = host_description()
    res = {}

    def decode_case(name, nreq):
        inp = make_config(name)
        kp, vp = oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
        n = min(nreq, inp.num_decode)
        _CPU_JOB.clear()
        _CPU_JOB.update(inp=inp, kp=kp, vp=vp)
        kv = metrics.decode_kv_bytes(inp.page_table, inp.dec_req_rows[:n], inp.dec_seq_lens[:n],
                                     inp.num_kv_heads, 128)
        tasks = [("decode", i, i + 1) for i in range(n)]
        t1 = _time_tasks(tasks, 1)
        tn = _time_tasks(tasks, workers)
        _CPU_JOB.clear()
        return {"requests": n, "kv_mb": round(kv / 1e6, 2),
                "one_core_s": round(t1, 4), "one_core_GBps": round(kv / t1 / 1e9, 4),
                "all_cores_s": round(tn, 4), "all_cores_GBps": round(kv / tn / 1e9, 4),
                "requests_per_s_all_cores": round(n / tn, 2)}

    log("CPU baseline: decode C1 / C2 / C5a")
    res["C1"] = decode_case("C1", 4)
    res["C2"] = decode_case("C2", 64)
    res["C5a_decode"] = decode_case("C5a", 32)

    log("CPU baseline: extend C3")
    inp = make_config("C3")
    kp, vp = oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
    rows, pairs = [], 0
    for r in range(inp.num_extend):
        base, E, P = int(inp.ext_q_offsets[r]), int(inp.ext_extend_lens[r]), int(inp.ext_prefix_lens[r])
        for i in np.linspace(0, E - 1, 8).astype(int).tolist():
            rows.append(base + i)
            pairs += P + i + 1
    _CPU_JOB.clear()
    _CPU_JOB.update(inp=inp, kp=kp, vp=vp, rows=rows)
    tasks = [("extend", a, a + 4) for a in range(0, len(rows), 4)]
    flops = 4 * inp.num_q_heads * 128 * pairs
    t1 = _time_tasks(tasks, 1)
    tn = _time_tasks(tasks, workers)
    _CPU_JOB.clear()
    res["C3_extend"] = {"query_rows": len(rows), "causal_pairs": pairs, "flops": flops,
                        "one_core_s": round(t1, 4), "one_core_TFLOPs": round(flops / t1 / 1e12, 6),
                        "all_cores_s": round(tn, 4), "all_cores_TFLOPs": round(flops / tn / 1e12, 6),
                        "tokens_per_s_all_cores": round(len(rows) / tn, 1)}
    c2 = res["C2"]
    return {"value": c2["all_cores_GBps"], "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": (f"fp64 numpy oracle, whole 64-request headline decode batch "
                       f"({c2['kv_mb']} MB of distinct K/V), one process per request over "
                       f"{workers} worker processes with 1 BLAS thread each, median of 3 passes "
                       f"after 1 warm-up; per-workload one-core and all-core figures (decode "
                       f"C1, C2, C5a, extend C3) under 'workloads'"),
            "one_core": {"value": c2["one_core_GBps"], "unit": "GB/s", "cores": 1},
            "workloads": res, "host": host}


def embedding_run(steps: int, warmup: int):
    """Time back-to-back planned embedding gathers (HBM-bound row copy)."""
    import torch
    import paged_kv_attention_30_amd as msgl
    g = torch.Generator(device="cuda").manual_seed(41)
    V, H, n = 151936, 4096, 8192
    table = torch.randn((V, H), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    ids = torch.randint(0, V, (n,), generator=g, device="cuda", dtype=torch.int32)
    out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
    plan = msgl.plan_embedding_gather(table, ids, out=out)
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        plan.run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    alg = n * H * 2 * 2 + n * 4           # rows read + rows written + ids
    del table, out
    return {"workload": WORKLOAD_TEXT["EMB"], "gather_ms": round(ms, 4),
            "alg_bytes": alg, "GBps": round(alg / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(n / (ms * 1e-3), 1)}


def prologue_run(steps: int, warmup: int):
    """Time back-to-back fused prologues (q/k RMSNorm + RoPE + store; HBM-bound)."""
    import torch
    import paged_kv_attention_30_amd as msgl
    g = torch.Generator(device="cuda").manual_seed(42)
    T, Hq, Hkv, D, S = 8192, 32, 8, 128, 524288
    qkv = torch.randn((T, (Hq + 2 * Hkv) * D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.empty((S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    qw = torch.randn((D,), generator=g, device="cuda").to(torch.bfloat16)
    kw = torch.randn((D,), generator=g, device="cuda").to(torch.bfloat16)
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    loc = torch.randperm(S, generator=g, device="cuda")[:T].to(torch.int32)
    cache = msgl.rope_cos_sin_cache(32768, D, 1_000_000.0)
    q_out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    plan = msgl.plan_qk_norm_rope_store(qkv, k, v, pos, cache, loc, Hq, Hkv, qw, kw, 1e-6, q_out)
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        plan.run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    # qkv rows in; q out, k and v rows to the pool; positions, slots, table rows
    alg = T * (Hq + 2 * Hkv) * D * 2 + T * (Hq + 2 * Hkv) * D * 2 + T * 4 * 2 + T * D * 4
    del qkv, k, v, q_out
    return {"workload": WORKLOAD_TEXT["PRO"], "prologue_ms": round(ms, 4), "alg_bytes": alg,
            "GBps": round(alg / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1)}


def kvcache_run():
    """Host-only: a request trace through the C++ manager (via the binding, with
    the Python scheduling loop of workloads.kvtrace.drive) and, on a sample,
    through the oracle; plus per-call match / key-compare times."""
    import time
    from workloads.kvtrace import kv_trace, drive
    import oracle
    import paged_kv_attention_30_amd as msgl
    tr = kv_trace()
    kv = msgl.KVCache(tr.num_slots, tr.page_size, tr.max_rows, tr.max_len)
    t0 = time.perf_counter()
    st = drive(kv, tr)
    t_cpp = time.perf_counter() - t0
    sample = kv_trace(num_requests=128)
    ko = oracle.KVCacheOracle(sample.num_slots, sample.page_size, sample.max_rows, sample.max_len)
    t0 = time.perf_counter()
    drive(ko, sample)
    t_or = time.perf_counter() - t0
    # per call: match of a cached 1,280-token prompt (warm tree), key compare of
    # two equal 1,024-token runs
    ids = tr.prompts[0]
    kv.match(ids)
    ko2 = oracle.KVCacheOracle(tr.num_slots, tr.page_size, tr.max_rows, tr.max_len)
    drive(ko2, kv_trace(num_requests=8))
    ids8 = kv_trace(num_requests=8).prompts[0]
    reps = 2000
    t0 = time.perf_counter()
    for _ in range(reps):
        kv.match(ids8)
    m_cpp = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    for _ in range(200):
        ko2.match(ids8)
    m_or = (time.perf_counter() - t0) / 200
    a = np.arange(1024, dtype=np.int32)
    t0 = time.perf_counter()
    for _ in range(reps):
        msgl.compare_key(a, a)
    c_cpp = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    for _ in range(200):
        oracle.compare_key(a, a)
    c_or = (time.perf_counter() - t0) / 200
    kv.close()
    return {"workload": WORKLOAD_TEXT["KVC"], "requests": st["admitted"],
            "prefix_reuse": round(st["matched_tokens"] / st["prompt_tokens"], 4),
            "decode_tokens": st["decode_tokens"], "manager_calls": st["calls"],
            "trace_s": round(t_cpp, 4), "requests_per_s": round(st["admitted"] / t_cpp, 1),
            "calls_per_s": round(st["calls"] / t_cpp, 1),
            "match_us": round(m_cpp * 1e6, 2), "compare_key_1024_us": round(c_cpp * 1e6, 3),
            "note": "times include the Python scheduling loop and ctypes marshalling",
            "cpu_baseline": {"kind": "oracle", "cores": 1,
                             "requests_per_s": round(128 / t_or, 1),
                             "match_us": round(m_or * 1e6, 2),
                             "compare_key_1024_us": round(c_or * 1e6, 3),
                             "sample": "first 128 requests of the same trace"}}


def graph_run(steps: int, warmup: int):
    """Per-step time of store_kv + paged_decode at small batches: eager planned
    calls against the graph runner (padding launch + graph replay)."""
    import torch
    import paged_kv_attention_30_amd as msgl
    g = torch.Generator(device="cuda").manual_seed(43)
    S, HQ, HKV, D, MAXB, W = 524288, 32, 8, 128, 64, 4096
    k = torch.randn((S, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((S, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    perm = torch.randperm(S - 1, generator=g, device="cuda").to(torch.int32)
    table = torch.zeros((MAXB + 1, W), dtype=torch.int32, device="cuda")
    table[:MAXB] = perm[:MAXB * W].view(MAXB, W)
    table[MAXB, 0] = S - 1
    lens = torch.randint(512, 4097, (MAXB,), generator=g, device="cuda", dtype=torch.int32)
    rows = torch.arange(MAXB, dtype=torch.int32, device="cuda")
    loc = table[rows.long(), (lens - 1).long()].contiguous()
    q = torch.randn((MAXB, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn((MAXB, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((MAXB, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    # the rows are disjoint, so the one-launch store + decode is valid
    runner = msgl.DecodeGraph(k, v, table, HQ, MAXB, W, scale, MAXB, S - 1, fused_store=True)
    runner2 = msgl.DecodeGraph(k, v, table, HQ, MAXB, W, scale, MAXB, S - 1)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    res = {}
    for bs in (1, 8, 32, 64):
        pf = msgl.plan_store_kv_paged_decode(q[:bs], k, v, kn[:bs], vn[:bs], loc[:bs], table,
                                             lens[:bs], W, scale, req_rows=rows[:bs])
        eager = timed(pf.run)
        for r in (runner, runner2):
            r.q[:bs].copy_(q[:bs]); r.k_new[:bs].copy_(kn[:bs]); r.v_new[:bs].copy_(vn[:bs])
            r.seq_lens[:bs].copy_(lens[:bs]); r.req_rows[:bs].copy_(rows[:bs])
            r.out_loc[:bs].copy_(loc[:bs])
        graph = timed(lambda: runner.run(bs))
        graph2 = timed(lambda: runner2.run(bs))
        res[str(bs)] = {"bucket": runner.bucket(bs), "eager_fused_ms": round(eager, 4),
                        "graph_fused_ms": round(graph, 4), "graph_two_call_ms": round(graph2, 4)}
    runner.close()
    runner2.close()
    del k, v
    return {"workload": WORKLOAD_TEXT["GRAPH"], "per_batch": res}


def decode_kernel_label(inp, split_used: int) -> str:
    """Name of the decode kernel instance a call launches, by the library's own rule: kv
    heads per workgroup = largest of 8 / 4 / 2 / 1 dividing Hkv; balanced split (two waves
    per kv head when their LDS fits in 160 KiB) unless a fixed chunk size is used."""
    hkv, ratio = inp.num_kv_heads, inp.num_q_heads // inp.num_kv_heads
    kvb = next(k for k in (8, 4, 2, 1) if hkv % k == 0)
    if split_used > 0:
        return f"decode_fixed_kernel<{kvb}>"
    wave_lds = 32 * 128 + 64                     # V tile + hand-over slot, bf16 elements
    lds2 = (kvb * 2 * wave_lds + kvb * ratio * 128) * 2
    return f"decode_balanced_kernel<{kvb}, {2 if lds2 <= 160 * 1024 else 1}>"


def store_bytes_of(inp):
    """store_kv moves each new K and V row in and out once, plus its int64 index."""
    n_new = int(inp.out_loc.shape[0])
    return 4 * n_new * inp.num_kv_heads * 128 * 2 + 8 * n_new


def decode_figures(inp, res, steps, fused=False):
    """KV bytes, algorithmic bytes and mean duration of one decode call (with
    the store's bytes when the store runs in the same launch)."""
    from workloads import metrics
    kv = metrics.decode_kv_bytes(inp.page_table, inp.dec_req_rows, inp.dec_seq_lens,
                                 inp.num_kv_heads, 128)
    alg = metrics.decode_bytes(inp.page_table, inp.dec_req_rows, inp.dec_seq_lens,
                               inp.num_q_heads, inp.num_kv_heads, 128, page_size=inp.page_size)
    if fused:
        alg += store_bytes_of(inp)
    dec_ms = float(np.mean(res["dec_ms"]))
    return kv, alg, dec_ms


def extend_figures(inp, res):
    from workloads import metrics
    fl = metrics.extend_flops(inp.ext_prefix_lens, inp.ext_extend_lens, inp.num_q_heads, 128)
    ext_ms = float(np.mean(res["ext_ms"]))
    return fl, ext_ms


def summarize(name, inp, run, res, steps):
    d = {"workload": WORKLOAD_TEXT.get(name, name)}
    step_ms = res["total_ms"] / steps
    d["ms_per_step"] = round(step_ms, 4)
    if inp.num_decode and inp.num_extend:
        # the mixed batch's tokens per second over the whole step (decode requests
        # plus extend tokens, store included)
        d["step_tokens_per_s"] = round((inp.num_decode + inp.ext_tokens) / (step_ms * 1e-3), 1)
    n_new = int(inp.out_loc.shape[0])
    store_bytes = store_bytes_of(inp)
    d["store_rows"] = n_new
    if run.fused:
        d["store"] = "in the decode launch (msgl_store_kv_paged_decode)"
    else:
        d["store_ms"] = round(float(np.mean(res["store_ms"])), 4)
        d["store_GBps"] = (round(store_bytes / (d["store_ms"] * 1e-3) / 1e9, 1)
                           if d["store_ms"] > 0 else None)
        d["store_hbm_frac"] = (round(store_bytes / (d["store_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                               if d["store_ms"] > 0 else None)
    if inp.num_decode:
        kv, alg, dec_ms = decode_figures(inp, res, steps, run.fused)
        d["decode_ms"] = round(dec_ms, 4)
        d["decode_kv_gb"] = round(kv / 1e9, 4)
        d["decode_kv_GBps"] = round(kv / (dec_ms * 1e-3) / 1e9, 1)
        d["decode_alg_GBps"] = round(alg / (dec_ms * 1e-3) / 1e9, 1)
        d["decode_hbm_frac"] = round(alg / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        d["decode_tokens_per_s"] = round(inp.num_decode / (dec_ms * 1e-3), 1)
        d["decode_split_tokens"] = run.split_used
    if inp.num_extend:
        fl, ext_ms = extend_figures(inp, res)
        d["extend_ms"] = round(ext_ms, 4)
        d["extend_tflops"] = round(fl / (ext_ms * 1e-3) / 1e12, 2)
        d["extend_mfma_frac"] = round(fl / (ext_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        d["extend_tokens_per_s"] = round(inp.ext_tokens / (ext_ms * 1e-3), 1)
    return d


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--configs", default="C1,C3,C4,C5a,C5b,EMB,PRO",
                    help="extra workloads (comma list of C1,C3,C4,C5a,C5b,EMB,PRO; '' for none)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--separate-store", action="store_true",
                    help="decode-only batches: store_kv and the decode as two launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--graphs", action="store_true",
                    help="replay each phase from a captured HIP graph instead of planned calls")
    ap.add_argument("--only", default="",
                    help="run just this workload's steps (for profilers) and print its timing")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the attention "
              "shards by request or by kv head with no exchange between GPUs)",
              file=sys.stderr)
        return 2

    cpu = None
    if not args.no_cpu_baseline and not args.only:
        # before anything initialises the GPU: the pool forks this process
        cpu = cpu_baselines()

    import torch
    import paged_kv_attention_30_amd as msgl
    from workloads import make_config

    msgl.load()
    if args.only == "KVC":
        print(json.dumps({"only": "KVC", **kvcache_run()}))
        return 0
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.calibrate_copy} MiB three times")
    if args.only == "EMB":
        print(json.dumps({"only": "EMB", **embedding_run(args.steps, args.warmup)}))
        return 0
    if args.only == "PRO":
        print(json.dumps({"only": "PRO", **prologue_run(args.steps, args.warmup)}))
        return 0
    if args.only == "GRAPH":
        print(json.dumps({"only": "GRAPH", **graph_run(args.steps, args.warmup)}))
        return 0
    if args.only:
        inp_o = make_config(args.only)
        run_o = Run(inp_o, args.split_tokens, not args.separate_store)
        res_o = timed_steps(run_o, args.steps, args.warmup, args.graphs)
        print(json.dumps({"only": args.only, **summarize(args.only, inp_o, run_o, res_o, args.steps)}))
        return 0

    log("generating the headline decode batch")
    inp = make_config("C2")
    run = Run(inp, args.split_tokens, not args.separate_store)
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps")
    res = timed_steps(run, args.steps, args.warmup, args.graphs)
    head = summarize("C2", inp, run, res, args.steps)
    kv, alg, dec_ms = decode_figures(inp, res, args.steps, run.fused)
    step_s = res["total_ms"] * 1e-3 / args.steps
    value = kv / step_s / 1e9
    if not args.no_cold:
        head["decode_ms_cold_l2_mall_flushed"] = round(cold_decode_ms(run), 4)

    head.update(step_distribution(run, args.steps))

    khash = kernel_hash()
    traffic = load_traffic(khash)
    roofline = {"bound": "hbm", "achieved": round(alg / (dec_ms * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(alg / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": (f"{decode_kernel_label(inp, run.split_used)} (store_kv fused) + "
                           "merge_kernel (one msgl_store_kv_paged_decode call)" if run.fused else
                           f"{decode_kernel_label(inp, run.split_used)} + merge_kernel "
                           "(one msgl_paged_decode call)"),
                "alg_bytes_per_launch": alg, "avg_launch_ms": round(dec_ms, 4)}
    fused = run.fused
    del run
    torch.cuda.empty_cache()

    extras = {"C2": head}
    for name in [c for c in args.configs.split(",") if c]:
        log(f"workload {name}")
        if name in ("EMB", "PRO"):
            fn = embedding_run if name == "EMB" else prologue_run
            extras[name] = fn(max(10, args.steps // 2), 3)
            torch.cuda.empty_cache()
            continue
        inp_x = make_config(name)
        run_x = Run(inp_x, args.split_tokens, not args.separate_store)
        n_x = max(10, args.steps // 5)
        res_x = timed_steps(run_x, n_x, 3, args.graphs, min_warm_s=EXTRA_WARM_S)
        extras[name] = summarize(name, inp_x, run_x, res_x, n_x)
        del run_x
        torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["total_ms"] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT["C2"],
                   "step": ("store_kv(64 rows) + paged_decode (+LSE merge) in one "
                            "msgl_store_kv_paged_decode launch + the merge" if fused else
                            "store_kv(64 rows) + paged_decode (+LSE merge)"),
                   "split_tokens": head.get("decode_split_tokens"), "page_size": 1,
                   "launch": "hip_graph_replay" if args.graphs else "planned_calls"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
        "kernel_hash": khash,
        "peaks": {"hbm_GBps": HBM_PEAK_GBS, "mfma_bf16_dense_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                  "clock_GHz": 2.4, "source": "MI355X published figures (the bf16 figure is "
                  "dense, at the 2.4 GHz peak engine clock)"},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
