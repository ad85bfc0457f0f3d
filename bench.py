"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--all-configs]

One step = the whole hot path at the headline workload: bf16 causal attention,
B=1 H=16 Nq=Nk=16384 D=128, scale 1/sqrt(128): the fused forward (O, LSE) followed by
the backward (dQ, dK, dV from the saved LSE). Inputs are seeded synthetic N(0,1) values
rounded to bf16, resident in HBM before timing starts.

Prints ONE JSON line on stdout:
  value        useful TFLOP/s of the step: (fwd + bwd useful FLOPs) / step time, with
               useful FLOPs counted on visible (i, j) pairs only: fwd 2 (Dqk + Dv) A,
               bwd 2 (3 Dqk + 2 Dv) A per (b, h), A = N (N + 1) / 2 for causal
  roofline     for the kernel that takes the most time per step: its algorithmic FLOPs
               per launch / its average launch duration (HIP events on the launch stream
               over the timed region), against the bf16 dense MFMA peak; "traffic" is its
               HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
               summary, or null when the kernel sources changed since it was taken
  cpu_baseline the CPU fp64 oracle on one head of the same workload (fwd + bwd), scaled
               to TFLOP/s of useful work
--all-configs additionally prints per-workload timings of the other configurations to
stderr (not part of the JSON line), with the CPU oracle's time on each configuration
(sampled (b, h) pairs, extrapolated; skipped with --no-cpu-baseline). Forward and decode
rows are GPU time per call from HIP graph replay (`timing: "graph replay"`), which leaves
out the host-side cost of each call; the others are HIP events around single calls.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published

B, H, N, D = 1, 16, 16384, 128

PROFILE_HBM = os.path.join(ROOT, "profiles", "fwd_bwd_causal_b1h16n16384d128_hbm_counters.md")
PROFILE_NAMES = {"fwd_bf16": "fwd_bf16_kernel<128, 128, false, false, false>",
                 "bwd_dkdv": "bwd_dkdv_kernel<128, 128, false, false, false>",
                 "bwd_dq": "bwd_dq_kernel<128, 128, false, false, false>"}


def kernel_source_hash() -> str:
    """sha256 over the kernel sources and the build script (their code and flags)."""
    import hashlib
    pkg = os.path.join(ROOT, "block_sparse_attention_fmha_amd")
    csrc = os.path.join(pkg, "csrc")
    files = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h", ".cpp")))
    h = hashlib.sha256()
    for f in files + ["../build.py"]:
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE summary,
    or None when that summary was taken with different kernel sources (or is missing)."""
    try:
        text = open(PROFILE_HBM).read()
    except OSError:
        return None
    tag = "Kernel sources sha256: "
    if tag not in text or text.split(tag, 1)[1].split()[0].strip("`") != kernel_source_hash():
        return None
    name = PROFILE_NAMES.get(kernel)
    for row in text.splitlines():
        if name and row.startswith(f"| `{name}`"):
            return int(round(float(row.strip("|").split("|")[-1]) * 2**20))
    return None


def causal_pairs(n: int) -> int:
    return n * (n + 1) // 2


def useful_flops(b, h, a, dqk, dv):
    fwd = 2.0 * b * h * (dqk + dv) * a
    bwd = 2.0 * b * h * (3 * dqk + 2 * dv) * a
    return fwd, bwd


def kernel_flops(b, h, a, dqk, dv):
    """Algorithmic (useful) FLOPs each kernel of the step contributes."""
    return {
        "fwd_bf16": 2.0 * b * h * a * (dqk + dv),             # S = Q K^T, O = P V
        "bwd_dkdv": 2.0 * b * h * a * (2 * dqk + 2 * dv),     # S, dP, dV, dK
        "bwd_dq": 2.0 * b * h * a * dqk,                      # dQ (S, dP recomputed, not counted)
    }


def gpu_step_timing(steps: int, warmup: int):
    import torch
    import block_sparse_attention_fmha_amd as fa
    from block_sparse_attention_fmha_amd import synth

    dev = torch.device("cuda:0")
    q, k, v, do = synth.attention_inputs(synth.case_seed(2, 0), B, N, N, H, D, D, "bf16", with_dout=True)
    tq, tk, tv, tdo = (t.to_torch(dev) for t in (q, k, v, do))
    del q, k, v, do
    out = torch.empty_like(tq)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
    ws = torch.empty(fa.bwd_workspace_size(B, H, N), dtype=torch.uint8, device=dev)
    mask = fa.Mask("causal")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fmha_fwd(tq, tk, tv, mask=mask, out=out, lse=lse)
        fa.fmha_bwd(tq, tk, tv, out, lse, tdo, mask=mask, dq=dq, dk=dk, dv=dv, workspace=ws,
                    stage_events=None if ev is None else ev[1:5])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per = {"fwd_bf16": 0.0, "bwd_preprocess": 0.0, "bwd_dkdv": 0.0, "bwd_dq": 0.0}
    for e in evs:
        per["fwd_bf16"] += e[0].elapsed_time(e[1])
        per["bwd_preprocess"] += e[1].elapsed_time(e[2])
        per["bwd_dkdv"] += e[2].elapsed_time(e[3])
        per["bwd_dq"] += e[3].elapsed_time(e[4])
    per = {k: v / steps for k, v in per.items()}
    return total_ms / steps, per


def profile_other_rows(reps: int):
    """For rocprofv3 runs: `reps` launches each of the split-KV decode (B=8 H=32 Nq=1
    Nk=32768 D=128, 16 splits; partial + combine kernels), the same with 8 grouped K/V
    heads and with one (multi-query), the fp32 wide-head forward
    (B=4 H=8 N=512 D=1024) and the block-sparse causal forward (B=2 H=8 N=8192 D=128,
    128 x 128 tiles, relative bias) with its block-mask build."""
    import torch
    import block_sparse_attention_fmha_amd as fa
    dev = torch.device("cuda:0")
    q = torch.randn(8, 1, 32, 128, device=dev).bfloat16()
    k = torch.randn(8, 32768, 32, 128, device=dev).bfloat16()
    v = torch.randn(8, 32768, 32, 128, device=dev).bfloat16()
    for _ in range(reps):
        fa.fmha_fwd_splitkv(q, k, v, 16)
    torch.cuda.synchronize()
    del k, v
    k = torch.randn(8, 32768, 8, 128, device=dev).bfloat16()   # 8 K/V heads for the 32 query heads
    v = torch.randn(8, 32768, 8, 128, device=dev).bfloat16()
    for _ in range(reps):
        fa.fmha_fwd_splitkv(q, k, v, 16)
    torch.cuda.synchronize()
    del k, v
    k = torch.randn(8, 32768, 1, 128, device=dev).bfloat16()   # one K/V head (multi-query)
    v = torch.randn(8, 32768, 1, 128, device=dev).bfloat16()
    for _ in range(reps):
        fa.fmha_fwd_splitkv(q, k, v, 16)
    torch.cuda.synchronize()
    del q, k, v
    q, k, v = (torch.randn(4, 512, 8, 1024, device=dev) for _ in range(3))
    for _ in range(reps):
        fa.fmha_fwd(q, k, v)
    torch.cuda.synchronize()
    del q, k, v
    q, k, v = (torch.randn(2, 8192, 8, 128, device=dev).bfloat16() for _ in range(3))
    m = fa.Mask("causal")
    for _ in range(reps):
        bs = fa.build_block_mask(m, 2, 8192, 8192, 128, 128)
        fa.fmha_fwd(q, k, v, mask=m, bias_slope=-0.01, block_sparse=bs)
    torch.cuda.synchronize()


def host_info():
    """The host the CPU oracle runs on: CPU model, logical CPUs, the CPUs this process may
    use, the thread-count environment and the BLAS thread pools numpy's products use."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    env = {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS",
                                      "BLIS_NUM_THREADS") if k in os.environ}
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    except Exception:
        blas = []
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "affinity_cpus": affinity,
            "thread_env": env, "blas_pools": blas}


def oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        return max(i.get("num_threads", 1) for i in info) if info else 1
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline():
    """The CPU fp64 oracle, as it stands, on one head of the workload (fwd + bwd)."""
    import oracle
    from block_sparse_attention_fmha_amd import synth
    q, k, v, do = synth.attention_inputs(synth.case_seed(2, 0), B, N, N, H, D, D, "bf16", with_dout=True)
    t0 = time.perf_counter()
    oracle.backward_bh(q.values[0, :, 0], k.values[0, :, 0], v.values[0, :, 0], do.values[0, :, 0], 0, 0,
                       scale=1.0 / math.sqrt(D), mask=oracle.MaskSpec("causal"))
    dt = time.perf_counter() - t0
    f, b = useful_flops(1, 1, causal_pairs(N), D, D)
    return {"value": round((f + b) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(oracle_threads()),
            "kind": "oracle",
            "sample": f"head 0 of {H} (b=0), full N={N} causal fwd+bwd, {dt:.1f} s wall; "
                      f"the rate of that head is the whole workload's (every head costs the same)",
            "host": host_info()}


def oracle_config_timings(log):
    """The CPU oracle beside the other configurations: each timed on a stated sample of
    (batch, head) pairs and extrapolated linearly to the whole configuration (every pair of
    a configuration costs the same: the oracle materialises each (b, h) score matrix).
    About half a minute of CPU work in all. Returns the extrapolated seconds per
    configuration key ("1", "3", "4/4096", "4/8192", "5a", "5b")."""
    import numpy as np
    import oracle
    from block_sparse_attention_fmha_amd import synth

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    whole = {}

    def report(config, workload, secs, done, total, unit_desc, key=None):
        whole[key or config] = secs * total / done
        log(oracle=config, workload=workload, sample=f"{done} of {total} {unit_desc}",
            sample_s=round(secs, 3), extrapolated_s=round(secs * total / done, 2), threads=oracle_threads())

    # 1: fp32 forward B=1 H=1 N=128 D=64 causal (whole)
    q, k, v = synth.attention_inputs(synth.case_seed(1, 0), 1, 128, 128, 1, 64, 64, "fp32")
    secs = timed(lambda: oracle.forward(q.values, k.values, v.values, mask=oracle.MaskSpec("causal")))
    report("1", "fwd fp32 B=1 H=1 N=128 D=64 causal", secs, 1, 1, "(b, h)")
    # 3: block-sparse forward B=2 H=8 N=8192 D=128, relative bias, causal tiles (one head)
    n = 8192
    q, k, v = synth.attention_inputs(synth.case_seed(3, 0), 1, n, n, 1, 128, 128, "bf16")
    idx = np.arange(n)
    secs = timed(lambda: oracle.forward_bh(q.values[0, :, 0], k.values[0, :, 0], v.values[0, :, 0], idx, 0, 0,
                                           n, n, scale=1.0 / math.sqrt(128), bias_slope=-0.01,
                                           mask=oracle.MaskSpec("causal")))
    report("3", "block-sparse fwd bf16 B=2 H=8 N=8192 D=128 causal, bias -0.01", secs, 1, 16, "(b, h)")
    # 4: backward B=1 H=16, causal: N=4096 D=128 and the MLA shape N=8192 Dqk=192 Dv=128 (one
    # head each); N=16384 D=128 is the cpu_baseline line itself
    for n, dqk, dv in ((4096, 128, 128), (8192, 192, 128)):
        q, k, v, do = synth.attention_inputs(synth.case_seed(4, n), 1, n, n, 1, dqk, dv, "bf16", with_dout=True)
        secs = timed(lambda: oracle.backward_bh(q.values[0, :, 0], k.values[0, :, 0], v.values[0, :, 0],
                                                do.values[0, :, 0], 0, 0, scale=1.0 / math.sqrt(dqk),
                                                mask=oracle.MaskSpec("causal")))
        report("4", f"bwd bf16 B=1 H=16 N={n} Dqk={dqk} Dv={dv} causal", secs, 1, 16, "(b, h)", key=f"4/{n}")
    # 5a: split-KV decode B=8 H=32 Nq=1 Nk=32768 D=128, 16 splits + combine (8 (b, h) pairs)
    nk = 32768
    q, k, v = synth.attention_inputs(synth.case_seed(5, 0), 1, 1, nk, 8, 128, 128, "bf16")
    secs = timed(lambda: oracle.combine_partials(oracle.split_partials(q.values, k.values, v.values, 16, 64)))
    report("5a", "split-KV decode bf16 B=8 H=32 Nq=1 Nk=32768 D=128, 16 splits + combine", secs, 8, 256, "(b, h)")
    # 5b: fp32 wide head B=4 H=8 N=512 D=1024 (one (b, h))
    q, k, v = synth.attention_inputs(synth.case_seed(5, 1), 1, 512, 512, 1, 1024, 1024, "fp32")
    secs = timed(lambda: oracle.forward(q.values, k.values, v.values))
    report("5b", "fwd fp32 B=4 H=8 N=512 D=1024", secs, 1, 32, "(b, h)")
    return whole


def all_configs_report(oracle_too: bool = True):
    """Extra timings of the other workloads, to stderr (median, with min and 90th
    percentile, of events around single calls or of HIP graph replays), and the CPU
    oracle's time on each configuration (sampled; see oracle_config_timings)."""
    import numpy as np
    import torch
    import block_sparse_attention_fmha_amd as fa
    from block_sparse_attention_fmha_amd import synth  # document ids (data only)
    dev = torch.device("cuda:0")

    # spread of the last measurement (min and 90th percentile, ms), added to the next log line
    spread = {}

    def timeit(fn, reps=50, warm=10):
        """Median ms of `reps` calls, each between two events (after `warm` untimed calls)."""
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(); fn(); b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        spread.update(ms_min=round(float(np.min(ts)), 4), ms_p90=round(float(np.percentile(ts, 90)), 4))
        return float(np.median(ts))

    def gpu_time(fn, reps=20, warm=10, replays=15):
        """GPU time per call in ms: `reps` calls captured in one HIP graph, the median over
        `replays` replays (300 timed calls). Unlike events around single calls this excludes
        the host-side cost of a call (argument marshalling, launch), which is several
        microseconds and dominates kernels of a few tens of microseconds."""
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for _ in range(reps):
                    fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(); g.replay(); b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / reps)
        del g
        spread.update(ms_min=round(float(np.min(ts)), 4), ms_p90=round(float(np.percentile(ts, 90)), 4))
        return float(np.median(ts))

    def log(**kw):
        if "ms" in kw and spread:   # the spread of the timing `ms` reports (measured last)
            kw.update(spread)
            spread.clear()
        sys.stderr.write(json.dumps(kw) + "\n")
        sys.stderr.flush()

    ora = oracle_config_timings(log) if oracle_too else {}

    def vs_oracle(key, ms):
        """The configuration's CPU oracle time over this GPU time (both whole-configuration)."""
        return {"x_vs_oracle": round(ora[key] * 1e3 / ms)} if key in ora else {}

    # forward grid: N x D x mask x softcap (B=1 H=16)
    for n in (1024, 4096, 16384):
        for d in (64, 128):
            q, k, v = (torch.randn(1, n, 16, d, device=dev).bfloat16() for _ in range(3))
            for kind in ("none", "causal", "sliding_window"):
                for cap in (0.0, 30.0):
                    m = fa.Mask(kind, window=1024)
                    ms = gpu_time(lambda: fa.fmha_fwd(q, k, v, mask=m, softcap=cap))
                    if kind == "none":
                        a = n * n
                    elif kind == "causal":
                        a = causal_pairs(n)
                    else:
                        a = sum(min(i, 1024) + 1 for i in range(n))
                    f = 2.0 * 16 * 2 * d * a
                    log(workload="fwd_bf16", N=n, D=d, mask=kind, softcap=cap, ms=round(ms, 4),
                        tflops=round(f / ms / 1e9, 1), frac=round(f / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                        timing="graph replay")
    # key-split forward (grids short of the CUs), against the same call without the split
    for hh, nq, nk, d, kind in ((16, 256, 32768, 128, "none"), (16, 1024, 8192, 128, "none"),
                                (16, 1024, 8192, 64, "causal"), (2, 4096, 4096, 128, "causal"),
                                (16, 2048, 2048, 128, "causal")):
        q = torch.randn(1, nq, hh, d, device=dev).bfloat16()
        k, v = (torch.randn(1, nk, hh, d, device=dev).bfloat16() for _ in range(2))
        m = fa.Mask(kind)
        ms_off = gpu_time(lambda: fa.fmha_fwd(q, k, v, mask=m, key_split=False))
        ms = gpu_time(lambda: fa.fmha_fwd(q, k, v, mask=m))   # timed last: its spread is logged
        a = nq * nk if kind == "none" else sum(min(nk, i + 1 + nk - nq) for i in range(nq))
        f = 2.0 * hh * 2 * d * a
        log(workload="fwd_bf16_key_split", H=hh, Nq=nq, Nk=nk, D=d, mask=kind, ms=round(ms, 4),
            ms_unsplit=round(ms_off, 4), tflops=round(f / ms / 1e9, 1),
            frac=round(f / ms / 1e9 / PEAK_BF16_TFLOPS, 4), workspace_bytes=fa.fwd_workspace_size(q, k, v, mask=m),
            timing="graph replay")
    del q, k, v
    # split-KV decode
    q = torch.randn(8, 1, 32, 128, device=dev).bfloat16()
    k = torch.randn(8, 32768, 32, 128, device=dev).bfloat16()
    v = torch.randn(8, 32768, 32, 128, device=dev).bfloat16()
    for s in (1, 2, 4, 8, 16):
        ms = gpu_time(lambda: fa.fmha_fwd_splitkv(q, k, v, s))
        byts = 2 * k.numel() * 2
        log(workload="splitkv", splits=s, ms=round(ms, 4), GBs=round(byts / ms / 1e6, 1),
            frac=round(byts / ms / 1e6 / PEAK_HBM_GBS, 4), timing="graph replay",
            **(vs_oracle("5a", ms) if s == 16 else {}))
    del k, v
    # grouped-query and multi-query decode: H=32 query heads over 8 or 1 K/V heads; the
    # algorithmic bytes are the K/V of the K/V heads
    for hkv in (8, 1):
        k = torch.randn(8, 32768, hkv, 128, device=dev).bfloat16()
        v = torch.randn(8, 32768, hkv, 128, device=dev).bfloat16()
        for s in (4, 16, 64):
            ms = gpu_time(lambda: fa.fmha_fwd_splitkv(q, k, v, s))
            byts = 2 * k.numel() * 2
            log(workload="splitkv_grouped", H=32, Hkv=hkv, splits=s, ms=round(ms, 4),
                GBs=round(byts / ms / 1e6, 1), frac=round(byts / ms / 1e6 / PEAK_HBM_GBS, 4),
                timing="graph replay")
        del k, v
    # fp32 wide head
    q, k, v = (torch.randn(4, 512, 8, 1024, device=dev) for _ in range(3))
    ms = gpu_time(lambda: fa.fmha_fwd(q, k, v))
    f = 2.0 * 4 * 8 * 2048 * 512 * 512
    log(workload="fwd_fp32_d1024", ms=round(ms, 4), tflops=round(f / ms / 1e9, 2),
        frac=round(f / ms / 1e9 / PEAK_FP32_TFLOPS, 4), timing="graph replay", **vs_oracle("5b", ms))
    del q, k, v
    # fp32 parity workload (latency-bound: one 32-row workgroup)
    q, k, v = (torch.randn(1, 128, 1, 64, device=dev) for _ in range(3))
    m = fa.Mask("causal")
    ms = gpu_time(lambda: fa.fmha_fwd(q, k, v, mask=m))
    f = 2.0 * 2 * 64 * causal_pairs(128)
    log(workload="fwd_fp32_n128_d64_causal", ms=round(ms, 4), tflops=round(f / ms / 1e9, 4),
        frac=round(f / ms / 1e9 / PEAK_FP32_TFLOPS, 6), timing="graph replay", **vs_oracle("1", ms))
    # block-sparse forward: B=2 H=8 N=8192 D=128, 128 x 128 sparse tiles from the element
    # mask, relative bias -0.01 |i - j|; useful FLOPs on the visible pairs only
    n, bsz, hh = 8192, 2, 8
    q, k, v = (torch.randn(bsz, n, hh, 128, device=dev).bfloat16() for _ in range(3))
    docs = synth.document_ids(synth.case_seed(3, 2), bsz, n)
    dev_docs = torch.from_numpy(docs).to(dev)
    for kind, w_, p_ in (("causal", 0, 0), ("sliding_window", 2730, 0), ("block_diagonal", 0, 0),
                         ("prefix_lm", 0, 1024)):
        m = fa.Mask(kind, window=w_, prefix=p_, doc_q=dev_docs if kind == "block_diagonal" else None,
                    doc_k=dev_docs if kind == "block_diagonal" else None)
        ms_bm = timeit(lambda: fa.build_block_mask(m, bsz, n, n, 128, 128))
        bs = fa.build_block_mask(m, bsz, n, n, 128, 128)
        ms = timeit(lambda: fa.fmha_fwd(q, k, v, mask=m, bias_slope=-0.01, block_sparse=bs))
        a = visible_pairs(kind, n, w_, p_, docs)
        f = 2.0 * hh * 256 * a
        tiles = int(bs.partial_cnt.sum().item() + bs.full_cnt.sum().item())
        log(workload="fwd_bf16_block_sparse", N=n, B=bsz, H=hh, D=128, mask=kind, ms=round(ms, 4),
            tflops=round(f / ms / 1e9, 1), frac=round(f / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            visited_tiles=tiles, of_tiles=bsz * (n // 128) ** 2, build_block_mask_ms=round(ms_bm, 4),
            **(vs_oracle("3", ms) if kind == "causal" else {}))
        # the backward through the transposed lists (dQ, dK, dV), same mask and bias
        do = torch.randn_like(q)
        out, lse = fa.fmha_fwd(q, k, v, mask=m, bias_slope=-0.01, block_sparse=bs)
        dq, dk, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.bwd_workspace_size(bsz, hh, n), dtype=torch.uint8, device=dev)
        ms = timeit(lambda: fa.fmha_bwd(q, k, v, out, lse, do, mask=m, bias_slope=-0.01, block_sparse=bs,
                                        dq=dq, dk=dk, dv=dv_, workspace=ws))
        fb = 2.0 * hh * (3 * 128 + 2 * 128) * a
        log(workload="bwd_bf16_block_sparse", N=n, B=bsz, H=hh, D=128, mask=kind, ms=round(ms, 4),
            tflops=round(fb / ms / 1e9, 1), frac=round(fb / ms / 1e9 / PEAK_BF16_TFLOPS, 4))
        del do, out, lse, dq, dk, dv_, ws
    # the same documents as packed variable-length sequences (no mask inside a document,
    # same bias): the block-diagonal workload without lists
    lens = [int(c) for b in range(bsz) for c in np.bincount(docs[b])]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=dev)
    qp, kp, vp = (x.reshape(bsz * n, hh, 128) for x in (q, k, v))
    ms = timeit(lambda: fa.fmha_fwd_varlen(qp, kp, vp, cu, cu, max(lens), max(lens), bias_slope=-0.01))
    f = 2.0 * hh * 256 * visible_pairs("block_diagonal", n, 0, 0, docs)
    log(workload="fwd_bf16_varlen_documents", N=n, B=bsz, H=hh, D=128, sequences=len(lens), ms=round(ms, 4),
        tflops=round(f / ms / 1e9, 1), frac=round(f / ms / 1e9 / PEAK_BF16_TFLOPS, 4))
    out, lse = fa.fmha_fwd_varlen(qp, kp, vp, cu, cu, max(lens), max(lens), bias_slope=-0.01)
    dop = torch.randn_like(qp)
    ms = timeit(lambda: fa.fmha_bwd_varlen(qp, kp, vp, out, lse, dop, cu, cu, max(lens), max(lens), bias_slope=-0.01))
    fb = 2.0 * hh * (3 * 128 + 2 * 128) * visible_pairs("block_diagonal", n, 0, 0, docs)
    log(workload="bwd_bf16_varlen_documents", N=n, B=bsz, H=hh, D=128, sequences=len(lens), ms=round(ms, 4),
        tflops=round(fb / ms / 1e9, 1), frac=round(fb / ms / 1e9 / PEAK_BF16_TFLOPS, 4))
    del q, k, v, qp, kp, vp, out, lse, dop
    # backward workloads (causal, B=1 H=16), incl. the MLA-shaped head Dqk=192 Dv=128
    for n, dqk, dv in ((4096, 64, 64), (4096, 128, 128), (16384, 64, 64), (8192, 192, 128)):
        q = torch.randn(1, n, 16, dqk, device=dev).bfloat16()
        k = torch.randn(1, n, 16, dqk, device=dev).bfloat16()
        v = torch.randn(1, n, 16, dv, device=dev).bfloat16()
        do = torch.randn(1, n, 16, dv, device=dev).bfloat16()
        m = fa.Mask("causal")
        out, lse = fa.fmha_fwd(q, k, v, mask=m)
        dq, dk, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.bwd_workspace_size(1, 16, n), dtype=torch.uint8, device=dev)
        ms = timeit(lambda: fa.fmha_bwd(q, k, v, out, lse, do, mask=m, dq=dq, dk=dk, dv=dv_, workspace=ws))
        f = useful_flops(1, 16, causal_pairs(n), dqk, dv)[1]
        log(workload="bwd_bf16", N=n, Dqk=dqk, Dv=dv, mask="causal", ms=round(ms, 4),
            tflops=round(f / ms / 1e9, 1), frac=round(f / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            **(vs_oracle(f"4/{n}", ms) if (n, dqk) in ((4096, 128), (8192, 192)) else {}))
        del q, k, v, do, out, lse, dq, dk, dv_, ws


# ---------------------------------------------------------------------------------------
# rocprofv3 summaries (profiles/*.md) from the databases of the commands below, which
# `--summarize-profiles DIR` reads from DIR/{trace,fetch,write,sq1,sq2}/run_results.db
# (and DIR/bench_all.log, the `--all-configs` line of the same box, if present).

PROFILE_CMDS = {
    "trace": "timeout -k 10 240 rocprofv3 --kernel-trace --stats -d $OUT/trace -o run -- "
             "python3 $R/bench.py --profile --steps 5 --warmup 2",
    "fetch": "timeout -s KILL 180 rocprofv3 --pmc FETCH_SIZE -d $OUT/fetch -o run -- "
             "python3 $R/bench.py --profile --steps 2 --warmup 1",
    "write": "timeout -s KILL 180 rocprofv3 --pmc WRITE_SIZE -d $OUT/write -o run -- "
             "python3 $R/bench.py --profile --steps 2 --warmup 1",
    "sq1": "timeout -s KILL 180 rocprofv3 --pmc SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
           "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
           "GRBM_GUI_ACTIVE -d $OUT/sq1 -o run -- python3 $R/bench.py --profile --steps 1 --warmup 1",
    "sq2": "timeout -s KILL 180 rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F32 "
           "SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_INSTS_SALU SQ_LDS_DATA_FIFO_FULL GRBM_GUI_ACTIVE "
           "-d $OUT/sq2 -o run -- python3 $R/bench.py --profile --steps 1 --warmup 1",
}
PROFILE_PRE = "R=$PWD; OUT=<results directory>; cd /tmp; export TMPDIR=/tmp"
PROFILE_COPY = "__amd_rocclr_copyBuffer"
PROFILE_HEAD = ["fwd_bf16_kernel<128, 128, false, false, false>", "bwd_preprocess_kernel<128>",
                "bwd_dkdv_kernel<128, 128, false, false, false>", "bwd_dq_kernel<128, 128, false, false, false>"]
# (row label, kernel, which of its dispatches: (part, parts) of them in launch order)
PROFILE_OTHER = [
    ("split-KV partial, 32 K/V heads", "splitkv_partial_kernel<128>", (0, 1)),
    ("split-KV on the matrix cores, 8 K/V heads", "splitkv_mfma_kernel<128>", (0, 2)),
    ("split-KV on the matrix cores, 1 K/V head", "splitkv_mfma_kernel<128>", (1, 2)),
    ("split-KV combine (all three)", "splitkv_combine_kernel<128>", (0, 1)),
    ("fp32 wide-head forward", "fwd_f32_kernel<1024, 128>", (0, 1)),
    ("block-sparse forward", "fwd_bf16_kernel<128, 128, true, false, true>", (0, 1)),
    ("block-mask build, both orientations", "classify_kernel", (0, 1)),
]


def _short_kernel(name: str) -> str:
    import re
    n = re.sub(r"^void ", "", name)
    n = n.replace("fmha::(anonymous namespace)::", "")
    return re.sub(r"\([^<>]*\)$", "", n).strip()


def _dispatch_part(values_by_dispatch, part, parts, what):
    """The values of one contiguous part of a kernel's dispatches, in launch order."""
    keys = sorted(values_by_dispatch)
    if not keys or len(keys) % parts:
        raise SystemExit(f"profile summary: {what}: {len(keys)} dispatches, not a multiple of {parts}")
    n = len(keys) // parts
    return [values_by_dispatch[k] for k in keys[part * n:(part + 1) * n]]


def summarize_profiles(src: str, out_dir: str):
    import sqlite3
    need = {k: os.path.join(src, k, "run_results.db") for k in ("trace", "fetch", "write", "sq1", "sq2")}
    for k, f in need.items():
        if not os.path.exists(f):
            raise SystemExit(f"profile summary: missing {f} (the `{k}` pass)")

    con = sqlite3.connect(need["trace"])
    trace = {}
    for i, (name, start, end) in enumerate(con.execute("select name, start, end from kernels order by start")):
        trace.setdefault(_short_kernel(name), {})[i] = (end - start) / 1000.0
    total_us = sum(sum(v.values()) for v in trace.values())

    def counters(db):
        c = sqlite3.connect(db)
        d = {}
        for k, cn, v, disp in c.execute("select kernel_name, counter_name, value, dispatch_id from counters_collection"):
            row = d.setdefault(_short_kernel(k), {}).setdefault(cn, {})
            row[disp] = row.get(disp, 0.0) + v
        return d

    fetch, write, sq1, sq2 = (counters(need[k]) for k in ("fetch", "write", "sq1", "sq2"))

    def require(table, kernel, what):
        if kernel not in table:
            raise SystemExit(f"profile summary: kernel `{kernel}` has no {what} row (names seen: "
                             f"{', '.join(sorted(table))})")
        return table[kernel]

    def trace_stats(kernel, part=(0, 1)):
        v = _dispatch_part(require(trace, kernel, "kernel-trace"), *part, what=kernel)
        last = v[-5:]
        return len(v), sum(v) / len(v), sum(last) / len(last), sum(v)

    def counter(table, kernel, cname, part=(0, 1), what="counter"):
        row = require(table, kernel, what)
        if cname not in row:
            raise SystemExit(f"profile summary: `{kernel}` lacks {cname}")
        v = _dispatch_part(row[cname], *part, what=f"{kernel} {cname}")
        return sum(v) / len(v)

    fscale = 512 * 1024 / counter(fetch, PROFILE_COPY, "FETCH_SIZE", what="FETCH_SIZE")
    wscale = 512 * 1024 / counter(write, PROFILE_COPY, "WRITE_SIZE", what="WRITE_SIZE")
    src_hash = kernel_source_hash()
    hashline = (f"Kernel sources sha256: `{src_hash}` (the kernels these numbers were taken with; bench.py "
                f"reports the traffic only while the sources hash to this value).")
    note = ("`bench.py --profile` runs the warm-up and timed fwd+bwd steps of the causal bf16 B=1 H=16 "
            "Nq=Nk=16384 D=128 workload, then the same number of launches each of the split-KV decode "
            "(B=8 H=32 Nq=1 Nk=32768 D=128, 16 splits; with 32, then 8, then 1 K/V heads), the fp32 wide-head "
            "forward (B=4 H=8 N=512 D=1024) and the block-sparse causal forward (B=2 H=8 N=8192 D=128, "
            "128x128 tiles, relative bias) with its block-mask build, then one plain 512 MiB device copy.")
    calib = (f"Calibration: a plain device copy of 512 MiB (`{PROFILE_COPY}`, 512 MiB read + 512 MiB written) "
             f"reads FETCH_SIZE = {512 * 1024 / fscale:.0f} KiB and WRITE_SIZE = {512 * 1024 / wscale:.0f} KiB, "
             f"so the scale factors are **fetch x{fscale:.3f}, write x{wscale:.3f}**.")
    bench_note = ""
    bl_path = os.path.join(src, "bench_all.log")
    if os.path.exists(bl_path):
        lines = [ln for ln in open(bl_path).read().splitlines() if ln.startswith("{\"metric\"")]
        if lines:
            bl = json.loads(lines[-1])
            kk = bl["kernels"]
            bench_note = (f"Same box, same call, `python3 bench.py --all-configs` (HIP events on the launch stream, "
                          f"{bl['steps']} timed steps): fwd {kk['fwd_bf16']['ms'] * 1000:.0f} µs, dK/dV "
                          f"{kk['bwd_dkdv']['ms'] * 1000:.0f} µs, dQ {kk['bwd_dq']['ms'] * 1000:.0f} µs, preprocess "
                          f"{kk['bwd_preprocess']['ms'] * 1000:.0f} µs per launch; {bl['value']} TFLOP/s for the step.")

    TRH = ["| kernel | calls | avg µs (all) | avg µs (last 5) | total µs | % of traced GPU time |",
           "|---|---|---|---|---|---|"]
    HBH = ["| kernel | FETCH_SIZE KiB/dispatch (raw avg) | scaled read MiB | WRITE_SIZE KiB/dispatch | "
           "scaled write MiB | HBM MiB per launch |", "|---|---|---|---|---|---|"]
    SQH = ["| kernel | MFMA insts | VALU insts | VALU/MFMA | TRANS/MFMA | SALU/MFMA | LDS insts | MFMA busy | "
           "LDS bank-conflict cycles / LDS active |", "|---|---|---|---|---|---|---|---|---|"]

    def trace_row(label, kernel, part=(0, 1)):
        n, avg, last, tot = trace_stats(kernel, part)
        return f"| `{label}` | {n} | {avg:.1f} | {last:.1f} | {tot:.1f} | {100 * tot / total_us:.1f} |"

    def hbm(kernel, part=(0, 1)):
        f = counter(fetch, kernel, "FETCH_SIZE", part, "FETCH_SIZE")
        w = counter(write, kernel, "WRITE_SIZE", part, "WRITE_SIZE")
        return f, w, (f * fscale + w * wscale) / 1024

    def hbm_row(label, kernel, part=(0, 1)):
        f, w, t = hbm(kernel, part)
        return f"| `{label}` | {f:.0f} | {f * fscale / 1024:.1f} | {w:.0f} | {w * wscale / 1024:.1f} | {t:.1f} |"

    def sq_row(label, kernel, part=(0, 1), mfma_cycles=32):
        c = lambda t, n: counter(t, kernel, n, part, "SQ")
        mf, va = c(sq2, "SQ_INSTS_MFMA"), c(sq2, "SQ_INSTS_VALU")
        busy = c(sq1, "SQ_VALU_MFMA_BUSY_CYCLES") / (c(sq1, "GRBM_GUI_ACTIVE") / 8 * 1024)
        bank = c(sq1, "SQ_LDS_BANK_CONFLICT") / max(1.0, c(sq1, "SQ_LDS_IDX_ACTIVE"))
        r = lambda x: f"{x / mf:.2f}" if mf else "-"
        return (f"| `{label}` | {mf:.4g} | {va:.4g} | {r(va)} | {r(c(sq2, 'SQ_INSTS_VALU_TRANS_F32'))} | "
                f"{r(c(sq2, 'SQ_INSTS_SALU'))} | {c(sq2, 'SQ_INSTS_LDS'):.4g} | {busy:.3f} | {bank:.3f} |")

    os.makedirs(out_dir, exist_ok=True)
    cmd = lambda *ks: ["```", *(PROFILE_CMDS[k] for k in ks), "```"]
    head_t = [trace_row(k, k) for k in PROFILE_HEAD] + [trace_row(PROFILE_COPY, PROFILE_COPY)]
    with open(os.path.join(out_dir, "fwd_bwd_causal_b1h16n16384d128_trace.md"), "w") as fh:
        fh.write("\n".join([
            "# Kernel trace: causal bf16 fwd+bwd, B=1 H=16 Nq=Nk=16384 D=128", "",
            f"Command (on the MI355X box, from the repository root, `{PROFILE_PRE}`); summary written by "
            f"`python3 bench.py --summarize-profiles $OUT`:", "", *cmd("trace"), "",
            f"{note} {hashline}", "", bench_note, "", *TRH, *head_t, ""]))
    with open(os.path.join(out_dir, "fwd_bwd_causal_b1h16n16384d128_hbm_counters.md"), "w") as fh:
        fh.write("\n".join([
            "# HBM traffic counters: causal bf16 fwd+bwd, B=1 H=16 Nq=Nk=16384 D=128", "",
            f"Commands (same setup as the kernel trace, `{PROFILE_PRE}`; one counter per pass):", "",
            *cmd("fetch", "write"), "", hashline, "", calib, "", *HBH, *(hbm_row(k, k) for k in PROFILE_HEAD), ""]))
    with open(os.path.join(out_dir, "fwd_bwd_causal_b1h16n16384d128_sq_counters.md"), "w") as fh:
        fh.write("\n".join([
            "# SQ counters: causal bf16 fwd+bwd, B=1 H=16 Nq=Nk=16384 D=128", "",
            f"{hashline} Commands (on the MI355X box, from the repository root, `{PROFILE_PRE}`), one pass each:",
            "", *cmd("sq1", "sq2"), "",
            "Values are per dispatch (averaged). GRBM_GUI_ACTIVE is summed over the 8 XCDs (per-XCD busy cycles = "
            "value / 8). MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI_ACTIVE / 8 x 1024 SIMDs); one 32x32x16 bf16 "
            "MFMA counts 32 busy cycles. SQ_INSTS_VALU includes the MFMA instructions.", "",
            *SQH, *(sq_row(k, k) for k in PROFILE_HEAD), ""]))

    # other workloads: bandwidth / rate lines from the trace (average of the last 5 launches)
    lines = []
    for (label, kernel, part), hkv in zip(PROFILE_OTHER[:3], (32, 8, 1)):
        byts = 2 * 8 * 32768 * hkv * 128 * 2
        _, _, us, _ = trace_stats(kernel, part)
        gbs = byts / (us * 1e-6) / 1e9
        f, w, t = hbm(kernel, part)
        where = ("" if gbs <= PEAK_HBM_GBS else
                 " — above the HBM peak: part of the K/V was served from the 256 MB last-level cache, "
                 "since the same K/V is read on every launch")
        lines.append(f"- {label}: {byts / 2**20:.0f} MiB of K/V per launch in {us:.1f} µs = **{gbs:.0f} GB/s** "
                     f"({100 * gbs / PEAK_HBM_GBS:.1f}% of 8 TB/s){where}; HBM counters {t:.1f} MiB per launch.")
    _, _, us, _ = trace_stats("fwd_f32_kernel<1024, 128>")
    f32 = 2.0 * 4 * 8 * 2048 * 512 * 512
    lines.append(f"- fp32 wide head: {f32 / 1e9:.1f} GFLOP in {us:.1f} µs = **{f32 / us / 1e6:.1f} TFLOP/s** "
                 f"({100 * f32 / us / 1e6 / PEAK_FP32_TFLOPS:.1f}% of the {PEAK_FP32_TFLOPS} TFLOP/s fp32 MFMA peak).")
    other_t = [trace_row(l, k, p) for l, k, p in PROFILE_OTHER]
    other_h = [hbm_row(l, k, p) for l, k, p in PROFILE_OTHER]
    other_s = [sq_row(l, k, p) for l, k, p in PROFILE_OTHER]
    with open(os.path.join(out_dir, "splitkv_fp32wide_blocksparse_kernels.md"), "w") as fh:
        fh.write("\n".join([
            "# Kernel trace and counters: split-KV decode (all and grouped K/V heads), fp32 wide-head forward, "
            "block-sparse forward", "",
            "Workloads: split-KV decode bf16 B=8 H=32 Nq=1 Nk=32768 D=128, 16 splits (partial + combine) with 32 "
            "K/V heads, then with 8 K/V heads shared by groups of 4 query heads, then with one K/V head for all 32 "
            "(multi-query); the grouped launches run `splitkv_mfma_kernel<128>` and are split here by launch order "
            "(8-head launches first); fp32 forward B=4 H=8 N=512 D=1024, no mask; block-sparse bf16 forward B=2 H=8 "
            "N=8192 D=128, causal element mask on 128x128 sparse tiles, relative bias -0.01|i-j|, with "
            "`build_block_mask` (`classify_kernel`: forward and transposed lists in one launch).", "",
            f"Same runs as the fwd+bwd profiles (`{PROFILE_PRE}`), summarised by "
            f"`python3 bench.py --summarize-profiles $OUT`, which stops with an error when a kernel "
            f"listed here has no row:", "", *cmd("trace", "fetch", "write", "sq1", "sq2"), "",
            note, "", hashline, "", calib, "", "## Kernel trace", "", *TRH, *other_t, "", *lines, "",
            "## HBM traffic", "", *HBH, *other_h, "", "## SQ counters", "",
            "(MFMA busy as in the fwd+bwd SQ summary; the fp32 kernel's 32x32x2 MFMA counts 64 busy cycles, so its "
            "busy fraction is twice the instruction count's share.)", "", *SQH, *other_s, ""]))
    print(f"wrote 4 summaries to {out_dir}")


def visible_pairs(kind, n, window, prefix, docs):
    """Visible (i, j) pairs summed over the batch rows (Nq = Nk = n)."""
    import numpy as np
    rows = docs.shape[0]
    i = np.arange(n, dtype=np.int64)
    if kind == "causal":
        per = int((i + 1).sum())
    elif kind == "sliding_window":
        per = int((np.minimum(i, window) + 1).sum())
    elif kind == "prefix_lm":
        per = int(np.minimum(n, np.maximum(prefix, i + 1)).sum())
    elif kind == "block_diagonal":
        return int(sum((np.bincount(docs[b]).astype(np.int64) ** 2).sum() for b in range(rows)))
    else:
        per = n * n
    return per * rows


def main():
    ap = argparse.ArgumentParser(description="attention hot-path benchmark (one MI355X)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-configs", action="store_true")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="write profiles/*.md from the rocprofv3 databases under DIR (no GPU needed)")
    ap.add_argument("--profile", action="store_true",
                    help="for rocprofv3: run --steps hot-path steps, then one plain 512 MiB device copy "
                         "(counter calibration), and exit without the JSON line")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, os.path.join(ROOT, "profiles"))
        return
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU only: the library has no multi-GPU path "
                         "(heads or key ranges would be sharded across GPUs; not built). Use --gpus 1.\n")
        sys.exit(2)

    if args.profile:
        import torch
        step_ms, per = gpu_step_timing(args.steps, args.warmup)
        profile_other_rows(args.steps)
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)      # reads 512 MiB, writes 512 MiB
        torch.cuda.synchronize()
        sys.stderr.write(f"profile run: {args.steps} steps, {step_ms:.3f} ms/step; copy 512 MiB done\n")
        return

    step_ms, per = gpu_step_timing(args.steps, args.warmup)
    a = causal_pairs(N)
    f_fwd, f_bwd = useful_flops(B, H, a, D, D)
    value = (f_fwd + f_bwd) / (step_ms * 1e-3) / 1e12
    kf = kernel_flops(B, H, a, D, D)
    dominant = max((k for k in per if k in kf), key=lambda k: per[k])
    achieved = kf[dominant] / (per[dominant] * 1e-3) / 1e12
    kernels = {k: {"ms": round(ms, 4)} for k, ms in per.items()}
    for k in kf:
        t = kf[k] / (per[k] * 1e-3) / 1e12
        kernels[k].update(tflops=round(t, 1), frac=round(t / PEAK_BF16_TFLOPS, 4))
    fwd_tf = f_fwd / (per["fwd_bf16"] * 1e-3) / 1e12
    bwd_ms = per["bwd_preprocess"] + per["bwd_dkdv"] + per["bwd_dq"]
    bwd_tf = f_bwd / (bwd_ms * 1e-3) / 1e12
    line = {
        "metric": "fwd/bwd TFLOP/s (useful FLOPs) + % of bf16 MFMA peak, causal N=16K D=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal attention fwd+bwd, bf16, B=1 H=16 Nq=Nk=16384 D=128",
                   "batch": B, "heads": H, "seq_len": N, "head_dim": D, "mask": "causal"},
        "fwd": {"ms": round(per["fwd_bf16"], 4), "tflops": round(fwd_tf, 1),
                "frac_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_tf, 1),
                "frac_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4)},
        "frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dominant)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    if args.all_configs:
        all_configs_report(oracle_too=not args.no_cpu_baseline)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
