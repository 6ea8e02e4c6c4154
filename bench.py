#!/usr/bin/env python3
"""Benchmark of the masked-token readout on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload all|tiny|llada|dream|lc_low|lc_high|llada_b16|ffn|ffn_tiny]
                    [--score conf|margin|neg_entropy] [--tau T]

A step is one denoising readout (compaction, masked LM-head GEMM with the
streaming vocabulary reduction, merge, top-k commit) over one synthetic
batch, with all inputs resident in HBM before timing starts.

The default (``--workload all``) runs the five seeded workloads one after
the other and prints ONE JSON line whose headline is the long-context
high-mask step (L=131072, d=4096, V=126464, M=117965 masked rows, 5% planted
rows, k=1024), the largest single-GPU workload and the one whose LM-head
GEMM is MFMA-bound; the other four (tiny; LLaDA-like semi-AR loop;
Dream-like; long-context low-mask) are nested under ``configs``, each with
its own throughput, roofline, per-step latency, transient device memory and
CPU-oracle baseline.  ``--workload NAME`` runs one workload alone.

The LLaDA-like loop decodes the last 1024 positions in blocks of 32, k=2 per
step, 32 consecutive steps with the mask/token state carried on the device
and the hidden states re-drawn every step; after 32 steps the state is reset
from a pristine device copy (inside the timed region).  llada_b16 decodes 16
such sequences together in one batched step (one pass over W_lm).

Per workload: masked tokens/s, the GEMM kernel's roofline (HIP events around
its launch on the library's stream), the per-step latency (median and p95,
from a second pass), device memory (resident before the step, the step's
transient peak above it, against the fp32 logits of all L rows and of the M
candidate rows), plain-torch readouts that materialise the logits, and the
fp64 CPU oracle timed on a bounded sample.  ``--score`` and ``--tau`` time
another selection policy (ranking by top-2 margin or negative entropy, whose
statistics the GEMM then also accumulates; threshold commits with cap k).
``--workload ffn`` times the sequence-chunked SwiGLU FFN of one layer over
the 128k-context LLaDA-like sequence (chunks of 8192 rows) instead.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOADS = {"tiny": "tiny", "llada": "llada_like_semi_ar", "dream": "dream_like",
             "lc_low": "long_ctx_low_mask", "lc_high": "long_ctx_high_mask",
             "llada_b16": "llada_like_semi_ar_batch16"}
FFN_WORKLOADS = {"ffn": "ffn_long_ctx_low_mask", "ffn_tiny": "ffn_tiny"}
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
CSRC = os.path.join(ROOT, "masked_token_logits_amd", "csrc")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the harness needs for kernel timing."""

    def __init__(self):
        self.lib = C.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.lib.hipEventDestroy.argtypes = [C.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]

    def event(self) -> int:
        e = C.c_void_p()
        if self.lib.hipEventCreate(C.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = C.c_float()
        if self.lib.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e: int) -> None:
        self.lib.hipEventDestroy(C.c_void_p(e))


def cpu_share() -> tuple[int, int]:
    """(threads the CPU oracle leg uses, cores visible to this process).

    The oracle uses every visible core, but no more than the process's CPU
    share when the environment states one (OMP_NUM_THREADS): on a host whose
    cores are shared between GPUs the affinity mask can show far more cores
    than one GPU's share."""
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        visible = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    n = visible
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n), visible


KERNEL_HEADERS = ("readout_internal.h", "online_state.h", "few_rows.h", "persistent_sched.h")


def kernel_source_sha(kernel_src: str) -> str:
    """sha256 over a GEMM kernel's source and the headers its code comes from
    (KERNEL_HEADERS, in that order, after the source)."""
    h = hashlib.sha256()
    for f in (kernel_src,) + tuple(os.path.join(CSRC, x) for x in KERNEL_HEADERS):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_from_profile(workload: str, kernel_src: str):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>_hbm_counters.md), or None when there is
    none or the kernel's sources changed since the counters were taken."""
    stem = os.path.splitext(os.path.basename(kernel_src))[0]
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    sha, hbm_bytes = parse_counter_summary(open(path).read())
    if sha is None or hbm_bytes is None or sha != kernel_source_sha(kernel_src):
        return None
    return hbm_bytes


def parse_counter_summary(text: str):
    """(source sha256, HBM bytes per launch) from a counter summary's text;
    None for a field that is missing."""
    m_sha = re.search(r"source sha256[^:\n]*:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    return (m_sha.group(1) if m_sha else None), (float(m_b.group(1)) if m_b else None)


def cpu_model() -> str | None:
    """The host CPU's model name from /proc/cpuinfo, with its family, model
    and stepping numbers (a virtual machine may report only the vendor's
    product line as the name), or None."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if info:
                        break
                    continue
                key, val = (s.strip() for s in line.split(":", 1))
                info.setdefault(key, val)
    except OSError:
        return None
    name = info.get("model name")
    if name is None:
        return None
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return f"{name} ({', '.join(ids)})" if ids else name


def _oracle_threads(n: int):
    """Context manager pinning the BLAS pool to n threads (threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n, user_api="blas")
    except Exception:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline(cfg, W, hidden_steps, mask0, tok0, budget_s: float = 6.0):
    """The fp64 oracle as it stands, on a bounded sample of the workload,
    with BLAS pinned to this process's cores.  The one-off fp64 widening of
    W_lm is timed apart (setup_seconds) and not counted."""
    import numpy as np

    import oracle
    threads, visible = cpu_share()
    with _oracle_threads(threads):
        t_setup = time.perf_counter()
        W64 = oracle.widen_bf16(W)
        setup = time.perf_counter() - t_setup
        t0 = time.perf_counter()
        if cfg.steps > 1:
            rows = passes = 0
            while passes < 10 and (passes == 0 or time.perf_counter() - t0 < budget_s):
                mask, tok = mask0, tok0
                for t in range(cfg.steps):
                    lo, hi = cfg.win
                    r = oracle.readout_step(hidden_steps[t], W, mask, tok, cfg.k, lo, hi, cfg.block, W64=W64)
                    rows += r.M
                    mask, tok = r.mask, r.tokens
                passes += 1
            sample = f"{passes} x all {cfg.steps} steps of the semi-AR pass ({rows} masked rows, full V each)"
        elif cfg.L * cfg.V <= 8 * 1024 * 1024:
            r = oracle.readout_step(hidden_steps[0], W, mask0, tok0, cfg.k, W64=W64)
            rows = r.M
            sample = f"the whole step ({rows} masked rows)"
        else:
            # consecutive blocks of the step's masked rows until the budget is spent
            pos = np.flatnonzero(mask0)
            rows = 0
            while rows < len(pos) and (rows == 0 or time.perf_counter() - t0 < budget_s):
                oracle.readout_rows(hidden_steps[0], W, pos[rows:rows + 256], W64=W64)
                rows = min(rows + 256, len(pos))
            sample = (f"first {rows} of the step's {len(pos)} masked rows, full V each "
                      f"(rows/s scaled to masked tokens/s)")
        dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="masked tokens/s", cores=threads, kind="oracle", sample=sample,
                seconds=round(dt, 3), setup_seconds=round(setup, 3), visible_cores=visible, cpu=cpu_model())


def cpu_baseline_ffn(cfg, X, Wg, Wu, Wd, budget_s: float = 10.0):
    """The fp64 FFN oracle as it stands, on consecutive blocks of rows until
    about ``budget_s`` seconds have passed."""
    import oracle
    threads, visible = cpu_share()
    with _oracle_threads(threads):
        t0 = time.perf_counter()
        rows = 0
        while rows < cfg.L and (rows == 0 or time.perf_counter() - t0 < budget_s):
            n = min(512, cfg.L - rows)
            oracle.ffn_rows(X[rows:rows + n], Wg, Wu, Wd)
            rows += n
        dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"first {rows} rows of the sequence, blocks of 512 (fp64 gate/up/down GEMMs)",
                seconds=round(dt, 3), visible_cores=visible, cpu=cpu_model())


def bench_ffn(args, name: str) -> dict:
    """One FFN layer over the whole sequence per step."""
    import numpy as np
    import torch

    import masked_token_logits_amd as mtl
    import workloads as WL

    cfg = WL.FFN_WORKLOADS[name]
    t_gen = time.perf_counter()
    Wg, Wu, Wd = WL.ffn_weights(cfg)
    X = WL.ffn_input(cfg)
    log(f"[bench] generated {name} inputs in {time.perf_counter() - t_gen:.1f}s")
    dev = torch.device("cuda", 0)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    Xt, Wgt, Wut, Wdt = to(X), to(Wg), to(Wu), to(Wd)
    Yt = torch.empty_like(Xt)
    ffn = mtl.SwiGLUFFN(Wgt, Wut, Wdt, cfg.chunk)
    del Wgt, Wut
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_mem = int(torch.cuda.memory_allocated())
    for _ in range(args.warmup):
        ffn(Xt, Yt)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        ffn(Xt, Yt)
        b.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    peak = int(torch.cuda.max_memory_allocated())
    flops = 6.0 * cfg.L * cfg.d * cfg.F
    achieved = flops / (float(step_ms.mean()) * 1e-3) / 1e12
    rec = {
        "metric": "FFN tokens/sec (sequence-chunked SwiGLU FFN, one layer)",
        "value": round(cfg.L * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init FFN weights of the named shape, no checkpoint or dataset)",
        "config": {
            "workload": f"{cfg.name} (L={cfg.L}, d={cfg.d}, F={cfg.F}, chunk={cfg.chunk}; one layer per step)",
            "L": cfg.L, "d": cfg.d, "F": cfg.F, "chunk": cfg.chunk,
            "transient_bytes": int(ffn.workspace.numel()),
            "unchunked_gate_up_act_bf16_bytes": 3 * cfg.L * cfg.F * 2,
            "peak_mem_bytes": peak,
            "resident_before_step_bytes": base_mem,
            "parallelism": "single GPU",
        },
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "k_gemm_persistent<kEpiSwiGLU> + k_gemm_persistent<kEpiStore> (both GEMMs of a step)",
                     "kernel_avg_us": round(float(step_ms.mean()) * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline_ffn(cfg, X, Wg, Wu, Wd)
    else:
        rec["cpu_baseline"] = None
    return rec


def torch_logits_baseline(cfg, Ht, Wt, mask_dev, reps: int = 5, cap_bytes: float = 48e9):
    """Plain-torch readouts that materialise the logits, timed on the first
    denoising step's state for the memory and time comparison.  'full' runs
    the LM head over all L positions; 'mask_only' runs it over the window's
    candidate rows only, with no streaming.  Both then take the softmax,
    each row's maximum and top-k over the candidates.  The candidate list is
    built once, outside the timing.  A variant is not run when its logits
    would need more than `cap_bytes` (bf16 + fp32 logits + fp32
    probabilities) or hold 2^31 elements or more; its size is reported."""
    import torch
    lo, hi = cfg.win
    pos = torch.nonzero(mask_dev[lo:hi]).flatten() + lo
    if cfg.block and pos.numel():
        b0 = lo + ((int(pos[0]) - lo) // cfg.block) * cfg.block
        pos = pos[pos < b0 + cfg.block]
    M = int(pos.numel())
    n = min(cfg.k, M)
    H = Ht.view(torch.bfloat16)
    W = Wt.view(torch.bfloat16)

    def readout(rows):
        P = torch.softmax((rows @ W.t()).float(), dim=-1)
        return P.max(dim=-1)

    def full():
        conf, _ = readout(H)
        return torch.topk(conf[pos], n).indices

    def mask_only():
        conf, _ = readout(H[pos])
        return torch.topk(conf, n).indices

    res = {"rows": {"full": cfg.L, "mask_only": M}, "k": n, "reps": reps}
    for name, fn, rows in (("full", full, cfg.L), ("mask_only", mask_only, M)):
        need = rows * cfg.V * 10
        if M == 0 or need > cap_bytes or rows * cfg.V >= 2**31:
            res[name] = {"not_run": f"{rows} x {cfg.V} logits, ~{need / 1e9:.0f} GB" if M else "no candidates"}
            continue
        fn()  # warm-up (library handles, allocator)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        times.sort()
        res[name] = {"ms_per_step": round(times[len(times) // 2], 4),
                     "transient_bytes": int(torch.cuda.max_memory_allocated() - base)}
    torch.cuda.empty_cache()
    return res


def bench_readout(args, short: str) -> dict:
    """One readout workload: the timed steps, then the latency pass, the
    torch readouts and the CPU oracle.  Returns its record."""
    import numpy as np
    import torch

    import masked_token_logits_amd as mtl
    import workloads as WL

    cfg = WL.WORKLOADS[WORKLOADS[short]]
    dev = torch.device("cuda", 0)
    t_gen = time.perf_counter()
    W = WL.w_lm(cfg)
    Bq = cfg.batch
    if Bq > 1:
        states = [WL.initial_state(cfg, b) for b in range(Bq)]
        mask0 = np.stack([m for m, _ in states])
        tok0 = np.stack([t for _, t in states])
    else:
        mask0, tok0 = WL.initial_state(cfg)
    Wt = torch.from_numpy(W.view(np.int16)).to(dev)
    hidden_steps, Hts = [], []
    for t in range(cfg.steps):   # upload step by step; batched host copies are dropped
        h = WL.hidden_batch(cfg, W, t) if Bq > 1 else WL.hidden(cfg, W, t)[0]
        Hts.append(torch.from_numpy(h.view(np.int16)).to(dev))
        hidden_steps.append(None if Bq > 1 else h)
    log(f"[bench] {short}: generated inputs in {time.perf_counter() - t_gen:.1f}s")

    m_pristine = torch.from_numpy(mask0).to(dev)
    t_pristine = torch.from_numpy(tok0).to(dev)
    mt = m_pristine.clone()
    tt = t_pristine.clone()
    stream = torch.cuda.current_stream(dev)
    rd = mtl.MaskedReadout(Wt, cfg.L * Bq, cfg.k, stream=stream)
    if args.slices:
        rd.set_slices(args.slices)
    total = args.warmup + args.steps
    m_slots = torch.zeros((total, Bq), dtype=torch.int32, device=dev)
    lo, hi = cfg.win
    seqs = [(cfg.k, lo, hi)] * Bq
    hip = Hip()
    ev = [(hip.event(), hip.event()) for _ in range(args.steps)]
    # everything a step reads or writes is allocated now: the peak above this
    # is the step's own transient memory
    torch.cuda.synchronize()
    resident = int(torch.cuda.memory_allocated())
    torch.cuda.reset_peak_memory_stats()

    def one(i: int, timed_index: int | None) -> None:
        t = i % cfg.steps
        if t == 0:
            mt.copy_(m_pristine)
            tt.copy_(t_pristine)
        if timed_index is None:
            mtl.dllm_masked_readout_set_gemm_events(rd.handle, None, None)
        else:
            a, b = ev[timed_index]
            mtl.dllm_masked_readout_set_gemm_events(rd.handle, a, b)
        out = {"m_out": m_slots.data_ptr() + 4 * Bq * i}
        if Bq > 1:
            rd.step_batch(Hts[t], mt, tt, seqs, cfg.block, out=out, score=args.score, tau=args.tau)
        else:
            rd.step(Hts[t], mt, tt, cfg.k, lo, hi, cfg.block, out=out, score=args.score, tau=args.tau)

    for i in range(args.warmup):
        one(i, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        one(args.warmup + j, j)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] {short}: timed {args.steps} steps in {elapsed * 1e3:.2f} ms")

    # Per-step latency, in a separate pass after the timed region: events
    # around each step on the library's stream (torch's current stream), the
    # state resets left outside them.
    mtl.dllm_masked_readout_set_gemm_events(rd.handle, None, None)
    lat = []
    for j in range(args.steps):
        t = (total + j) % cfg.steps
        if t == 0:
            mt.copy_(m_pristine)
            tt.copy_(t_pristine)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        if Bq > 1:
            rd.step_batch(Hts[t], mt, tt, seqs, cfg.block, score=args.score, tau=args.tau)
        else:
            rd.step(Hts[t], mt, tt, cfg.k, lo, hi, cfg.block, score=args.score, tau=args.tau)
        b.record(stream)
        lat.append((a, b))
    torch.cuda.synchronize()
    lat_us = np.sort(np.array([a.elapsed_time(b) for a, b in lat]) * 1e3)
    peak = int(torch.cuda.max_memory_allocated())

    Ms = m_slots.cpu().numpy().astype(np.int64).sum(axis=1)   # candidate rows per step, all sequences
    timed_M = Ms[args.warmup:]
    masked_rows = int(timed_M.sum())
    gemm_ms = np.array([hip.elapsed_ms(a, b) for a, b in ev])
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)

    d, V = cfg.d, cfg.V
    ext = args.score != "conf"
    small = Bq * (min(cfg.block, hi - lo) if cfg.block else hi - lo) <= 32
    rec_bytes = 24 if ext else 16
    slices = (V + 127) // 128
    flops = 2.0 * timed_M * d * V
    if Bq > 1:
        # Batched steps range from HBM-bound (few rows: W_lm's stream) to
        # MFMA-bound (many rows).  The bound is the one that takes longer at
        # the published peaks over the timed steps; both figures are kept.
        bytes_per = V * d * 2 + timed_M * d * 2 + timed_M * 4   # W_lm once, the rows, the row outputs
        t_mfma = float(flops.sum()) / (BF16_PEAK_TFLOPS * 1e12)
        t_hbm = float(bytes_per.sum()) / (HBM_PEAK_GBS * 1e9)
        secs = gemm_ms.sum() * 1e-3
        if t_mfma >= t_hbm:
            achieved = float(flops.sum()) / secs / 1e12
            roof = dict(bound="mfma", achieved=round(achieved, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=round(achieved / BF16_PEAK_TFLOPS, 4))
        else:
            achieved = float(bytes_per.sum()) / secs / 1e9
            roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBS, 4))
        roof["mfma_tflops"] = round(float(flops.sum()) / secs / 1e12, 1)
        roof["hbm_gbs"] = round(float(bytes_per.sum()) / secs / 1e9, 1)
        roof["roofline_time_frac"] = round(max(t_mfma, t_hbm) / secs, 4)
    elif small:
        # HBM-bound: every launch streams all of W_lm once plus the gathered
        # rows, and writes one partial record per (row, vocabulary slice):
        # 16 B (max, argmax, sum), 24 B with the margin / entropy terms.
        bytes_per = V * d * 2 + timed_M * d * 2 + timed_M * slices * rec_bytes + timed_M * 4
        achieved = float(bytes_per.sum()) / (gemm_ms.sum() * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
        roof["mfma_tflops"] = round(float(flops.sum()) / (gemm_ms.sum() * 1e-3) / 1e12, 2)
    else:
        achieved = float(flops.sum()) / (gemm_ms.sum() * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / BF16_PEAK_TFLOPS, 4))
    src = os.path.join(CSRC, "gemm_online.hip" if small else "gemm_persistent.hip")
    roof["traffic"] = None if ext else traffic_from_profile(short, src)
    ext_s = "true" if ext else "false"
    if small:  # a single sequence's GEMM also finds the candidate rows (third parameter)
        roof["kernel"] = "k_gemm_online<SmallTile, %s, %s>" % (ext_s, "false" if Bq > 1 else "true")
    else:
        roof["kernel"] = "k_gemm_persistent<kEpiReadout, %s>" % ext_s
    roof["kernel_avg_us"] = round(float(gemm_ms.mean()) * 1e3, 2)
    roof["algorithmic_flops_per_step"] = float(flops.mean())

    M_max = int(timed_M.max())
    rec = {
        "metric": "masked tokens/sec per denoise step",
        "value": round(masked_rows / elapsed, 1),
        "unit": "masked tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init LM head of the named shape, no checkpoint or dataset)",
        "config": {
            "workload": f"{cfg.name} (L={cfg.L}, d={d}, V={V}, k={cfg.k}"
                        + (f", block={cfg.block}, {cfg.steps}-step semi-AR loop" if cfg.block else "")
                        + (f", {Bq} sequences per batched step" if Bq > 1 else "") + ")",
            "batch": Bq,
            "L": cfg.L, "d": d, "V": V, "k": cfg.k,
            "masked_rows_per_step_max": M_max,
            "masked_rows_timed": masked_rows,
            "parallelism": "single GPU",
            "policy": {"score": args.score, "threshold": args.tau},
        },
        "memory": {
            "resident_before_step_bytes": resident,
            "peak_bytes": peak,
            "step_transient_bytes": peak - resident,
            "workspace_bytes": int(rd.workspace.numel()),
            "full_logits_fp32_bytes": cfg.L * Bq * V * 4,
            "mask_only_logits_fp32_bytes": M_max * V * 4,
            "how": "torch.cuda.max_memory_allocated over the timed and latency passes, minus the memory "
                   "allocated before the first step (W_lm, hidden states, mask/tokens, workspace)",
        },
        "roofline": roof,
        "latency": {
            "median_us": round(float(np.percentile(lat_us, 50)), 2),
            "p95_us": round(float(np.percentile(lat_us, 95)), 2),
            "steps": int(lat_us.size),
            "how": "HIP events around each step on the library's stream, in a pass after the timed region",
        },
    }
    if Bq == 1 and not args.no_torch_baseline:
        log(f"[bench] {short}: timing plain-torch readouts that materialise the logits")
        mt.copy_(m_pristine)
        rec["torch_logits_baseline"] = torch_logits_baseline(cfg, Hts[0], Wt, mt)
        rec["torch_logits_baseline"]["streamed_transient_bytes"] = peak - resident
    rd.close()
    del Hts, Wt, mt, tt, m_pristine, t_pristine, m_slots, rd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log(f"[bench] {short}: timing the CPU oracle on a bounded sample")
        if Bq > 1:
            # the oracle steps each sequence on its own: time sequence 0's pass
            hs0 = [WL.hidden(cfg, W, t, seq=0)[0] for t in range(cfg.steps)]
            rec["cpu_baseline"] = cpu_baseline(cfg, W, hs0, mask0[0], tok0[0])
            rec["cpu_baseline"]["sample"] += " (sequence 0 of the batch; sequences are independent)"
        else:
            rec["cpu_baseline"] = cpu_baseline(cfg, W, hidden_steps, mask0, tok0)
    else:
        rec["cpu_baseline"] = None
    return rec


def gemm_ceiling(stages: int = 20000, reps: int = 5) -> dict:
    """The compute-bound GEMM's practical ceiling on this GPU: its main
    loop's instruction mix alone (dllm_probe_gemm_mix) on random bf16
    operands, one workgroup per compute unit; median of `reps` launches."""
    import torch

    import masked_token_logits_amd as mtl
    dev = torch.device("cuda", 0)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device=dev)
    g.manual_seed(0xD11A)
    n = mtl.dllm_probe_source_bytes() // 2
    src = torch.randn(n, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    sink = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {"grid": cus, "stages": stages, "reps": reps,
           "how": "one 256-thread workgroup per CU; mode 0 = 64 v_mfma_f32_32x32x16_bf16 per wave and stage on "
                  "fragments held in registers; mode 1 = the main loop's mix (64 MFMAs, 32 ds_read_b128, 16 "
                  "whole-line global_load_lds from an L2-resident region, one barrier per stage); operands are "
                  "N(0,1) bf16 values, whose bit toggling sets the sustained MFMA clock"}
    flops = float(cus) * 4 * stages * 64 * 32768.0
    for mode, key in ((0, "mfma_only"), (1, "main_loop_mix")):
        times = []
        for r in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            st = mtl.dllm_probe_gemm_mix(mode, src, stages if r else 100, sink, cus, clocks, stream)
            b.record(stream)
            if st != mtl.DLLM_OK:
                raise mtl.DllmError(st, "dllm_probe_gemm_mix")
            torch.cuda.synchronize()
            if r:
                times.append(a.elapsed_time(b))
        ms = sorted(times)[len(times) // 2]
        tf = flops / (ms * 1e-3) / 1e12
        out[key] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / BF16_PEAK_TFLOPS, 4), "ms": round(ms, 3)}
        cyc, ticks = (int(x) for x in clocks.cpu().tolist())
        khz = mtl.dllm_probe_wall_clock_khz()
        if ticks > 0 and khz > 0:
            ghz = cyc / (ticks / (khz * 1e3)) / 1e9
            out[key]["shader_clock_ghz"] = round(ghz, 3)
            # MFMA pipe busy fraction at that clock: 32 cycles per 32x32x16 MFMA
            out[key]["mfma_busy_at_clock"] = round(tf * 1e12 / (cus * 4 * 1024.0 * ghz * 1e9), 4)
    return out


# The five seeded workloads of the default run, in order; the last is the headline.
ALL_ORDER = ("tiny", "llada", "dream", "lc_low", "lc_high")
NESTED_DROP = ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "steps", "warmup")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["all"] + sorted(WORKLOADS) + sorted(FFN_WORKLOADS), default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-torch-baseline", action="store_true",
                    help="skip the plain-torch logits readouts (e.g. under a profiler)")
    ap.add_argument("--slices", type=int, default=0, help="force the GEMM's vocabulary slice count")
    ap.add_argument("--score", choices=["conf", "margin", "neg_entropy"], default="conf",
                    help="ranking score of the selection (default: confidence)")
    ap.add_argument("--tau", type=float, default=None,
                    help="threshold commits (score >= tau, at least 1, at most k) instead of top-k")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the compute-bound GEMM's instruction-mix ceiling (dllm_probe_gemm_mix)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (reference for HBM byte counters)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the readout would shard W_lm by vocabulary, or the rows by sequence).",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    import masked_token_logits_amd as mtl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        x = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}))
        return 0
    mtl.load()
    if args.ceiling:
        print(json.dumps({"gemm_ceiling": gemm_ceiling()}), flush=True)
        return 0
    if args.workload in FFN_WORKLOADS:
        rec = bench_ffn(args, FFN_WORKLOADS[args.workload])
    elif args.workload != "all":
        rec = bench_readout(args, args.workload)
    else:
        recs = {}
        for short in ALL_ORDER:
            recs[short] = bench_readout(args, short)
            r = recs[short]
            log(f"[bench] {short}: {r['value']:.1f} masked tok/s, {r['roofline']['bound']} frac "
                f"{r['roofline']['frac']}")
        rec = dict(recs[ALL_ORDER[-1]])
        rec["configs"] = {}
        for short in ALL_ORDER:
            nested = {k: v for k, v in recs[short].items() if k not in NESTED_DROP}
            rec["configs"][WORKLOADS[short]] = nested
        rec["config"] = dict(rec["config"])
        rec["config"]["headline"] = ("the largest single-GPU workload, MFMA-bound; the other four are nested "
                                     "under 'configs' with their own roofline, latency, memory and CPU baseline")
        log("[bench] measuring the GEMM's instruction-mix ceiling")
        ceil = gemm_ceiling()
        rec["roofline"] = dict(rec["roofline"])
        rec["roofline"]["gemm_ceiling"] = ceil
        rec["roofline"]["frac_of_ceiling"] = round(rec["roofline"]["achieved"] / ceil["main_loop_mix"]["tflops"], 4)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
