"""Benchmark: attention forward + backward throughput on one MI355X.

One step = attn_fwd + the two backward kernels as attn_bwd runs them
(attn_bwd_dq_delta, which also forms delta = rowsum(dO o O), then
attn_bwd_dkdv) over one batch of synthetic inputs already resident in HBM:
the long-context workload B=1, H=16, N=8192, d=128, causal (the headline
throughput configuration).  Throughput counts the algorithmic FLOPs
7 * B * H * N^2 * d (forward: S = QK^T and P-bar V; backward: the S recompute,
dP, dV, dK, dQ; each 2 N^2 d per head, halved by the causal mask).

Prints ONE JSON line on stdout.  Each stage is a single kernel launch, timed
with HIP events on the stream it runs on; the roofline object reports the
kernel with the largest average duration.  The CPU baseline times the float64
oracle (forward + backward) on (batch, head) slices of the same workload, as many
as fit in about 12 seconds.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense BF16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
HBM_PEAK_GBS = 8000.0
METRIC = "attention fwd+bwd TFLOP/s and % of bf16 MFMA peak; mean signed O error on tied rows"
CSRC = os.path.join(ROOT, "precision_flash_attention_attn_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def source_hash() -> str:
    """Hash of the device code (kernels and the headers they include): stored
    counter readings stay valid while it is unchanged; host-side argument
    checks do not enter it."""
    h = hashlib.sha256()
    for name in sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".h"))):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    ent = t.get("kernels", {}).get(kernel)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def cpu_baseline(inp, wl, budget_s=12.0):
    """The float64 oracle (forward + backward) on (batch, head) slices of the
    workload, one after another until about budget_s seconds have passed."""
    from oracle import attention64 as a64
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    nsl = wl.b * wl.h
    done = 0
    t0 = time.perf_counter()
    while done < nsl and (time.perf_counter() - t0) < budget_s:
        b, h = divmod(done, wl.h)
        a64.slice_reference(inp.q[b, h], inp.k[b, h], inp.v[b, h], inp.do_bf16[b, h], causal=True,
                            scale=wl.scale)
        done += 1
    dt = time.perf_counter() - t0
    flops = done * 7 * wl.n * wl.n * wl.d  # algorithmic FLOPs of the slices done (causal)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {nsl} (batch, head) slices, N={wl.n} d={wl.d}, causal, "
                      f"float64 numpy forward+backward, {dt:.1f} s",
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_emulator(inp, wl, mode, budget_s=4.0):
    """The oracle's step-by-step BF16 flash emulator (a correctness tool, not
    a baseline) on query rows of slice (0, 0): the tied rows first, then rows
    spread over the sequence, in chunks of 64 until about budget_s seconds."""
    import numpy as np
    from oracle import flash_emu as fe
    n = wl.n
    tied = np.array(sorted({t for (b, h, t, _) in inp.forced_rows if b == 0 and h == 0}), dtype=int)
    rest = np.setdiff1d(np.linspace(0, n - 1, 1024).astype(int), tied)
    order = np.concatenate([tied, rest])
    done = 0
    t0 = time.perf_counter()
    while done < len(order) and (time.perf_counter() - t0) < budget_s:
        pos = order[done:done + 64]
        fe.flash_forward(inp.q[0, 0][pos], inp.k[0, 0], inp.v[0, 0], mode=mode, causal=True,
                         scale=wl.scale, q_pos=pos)
        done += len(pos)
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "query rows/s", "kind": "emulator (correctness tool)",
            "mode": mode, "sample": f"{done} query rows of slice (0, 0), N={n} d={wl.d}, causal "
                                    f"({min(done, len(tied))} tied), {dt:.1f} s"}


def run_mode(torch, pfa, inp, wl, mode, steps, warmup, candidates=("fwd", "bwd_dkdv", "bwd_dq")):
    """Warm up, then one pass of `steps` steps with a timing event pair around
    every stage (the per-stage durations), then the timed region of `steps`
    steps.  A timing event recorded between two kernels leaves a gap of about
    10 us on the stream, so the timed region brackets only the longest of
    `candidates`, whose duration the roofline uses.  Returns (wall ms per
    step, per-stage ms, that stage, its ms in the timed region, tied rows)."""
    dev = "cuda:0"
    to = lambda x: torch.from_numpy(x).to(dev)
    q, k, v = (to(x).to(torch.bfloat16).contiguous() for x in (inp.q, inp.k, inp.v))
    io = torch.float32 if mode == "fp32_out" else torch.bfloat16
    do = (to(inp.do_f32) if mode == "fp32_out" else to(inp.do_bf16).to(torch.bfloat16)).contiguous()
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), device=dev, dtype=io)
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
    flags = torch.empty((B, H, N), device=dev, dtype=torch.int32)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(pfa.attn_bwd_workspace_bytes(B, H, N, d, mode), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    # the backward as attn_bwd runs it: dQ (which also forms delta and, for an
    # FP32 dO, its BF16 copy), then dK and dV
    stages = ("fwd", "bwd_dq", "bwd_dkdv")
    calls = {
        "fwd": lambda: pfa.attn_fwd(q, k, v, o, lse, flags, causal=True, mode=mode, stream=stream),
        "bwd_dq": lambda: pfa.attn_bwd_dq_delta(q, k, v, o, do, lse, dq, ws, causal=True, mode=mode,
                                                stream=stream),
        "bwd_dkdv": lambda: pfa.attn_bwd_dkdv(q, k, v, do, lse, dk, dv, ws, causal=True, mode=mode,
                                              stream=stream),
    }
    event = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        for s in stages:
            calls[s]()
    torch.cuda.synchronize()
    ev = {s: [(event(), event()) for _ in range(steps)] for s in stages}
    for i in range(steps):
        for s in stages:
            ev[s][i][0].record(stream)
            calls[s]()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    avg_ms = {s: sum(a.elapsed_time(b) for a, b in ev[s]) / steps for s in stages}
    dom = max(candidates, key=lambda s: avg_ms[s])
    evd = [(event(), event()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for s in stages:
            if s == dom:
                evd[i][0].record(stream)
            calls[s]()
            if s == dom:
                evd[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = sum(a.elapsed_time(b) for a, b in evd) / steps
    ties = int(flags.sum().item())
    return wall / steps * 1e3, avg_ms, dom, dom_ms, ties


def time_delta_sources(torch, pfa, inp, steps, warmup):
    """Average duration of the backward's stage 1 with delta from rowsum(dP o P)
    and from rowsum(dO o O_hp) (O recomputed in FP32), after a BF16 forward."""
    dev = "cuda:0"
    to = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous()
    q, k, v, do = to(inp.q), to(inp.k), to(inp.v), to(inp.do_bf16)
    B, H, N, d = q.shape
    o, lse, _ = pfa.forward(q, k, v, causal=True, mode="bf16_out", flags=False)
    ws = torch.empty(pfa.attn_bwd_workspace_bytes(B, H, N, d), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    res = {}
    for src in ("dp_p", "do_ohp"):
        call = lambda: pfa.attn_bwd_delta(q, k, v, o, do, lse, ws, causal=True, delta_src=src, stream=stream)
        for _ in range(warmup):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        res[src] = round(e0.elapsed_time(e1) / steps, 4)
    return res


def tail_sums(torch, q, k, v, eps=1e-3):
    """tau [B, H, N, d] in float64: for each query row of causal attention with
    scale 1/sqrt(d), the sum over keys more than eps below the row's maximum
    score of exp(S - rm) V (the keys within eps of the maximum are the tied ones)."""
    N, d = q.shape[-2], q.shape[-1]
    s = torch.matmul(q.double(), k.double().transpose(-1, -2).contiguous()) * (1.0 / d ** 0.5)
    s = s.masked_fill(torch.ones(N, N, dtype=torch.bool, device=q.device).triu(1), float("-inf"))
    rm = s.amax(dim=-1, keepdim=True)
    w = torch.exp(s - rm).masked_fill(s >= rm - eps, 0.0)
    return torch.matmul(w, v.double())


def exact_attention(torch, q, k, v, chunk=2048):
    """Plain causal attention with scale 1/sqrt(d) in float64 on the GPU (torch
    operations, slices in chunks): the reference the signed errors are
    measured against."""
    B, H, N, d = q.shape
    out = torch.empty((B, H, N, d), dtype=torch.float64, device=q.device)
    mask = torch.ones(N, N, dtype=torch.bool, device=q.device).triu(1)
    qf, kf, vf = (t.reshape(B * H, N, d) for t in (q, k, v))
    of = out.view(B * H, N, d)
    for c0 in range(0, B * H, chunk):
        c1 = min(B * H, c0 + chunk)
        s = torch.matmul(qf[c0:c1].double(), kf[c0:c1].double().transpose(-1, -2).contiguous()) * (1.0 / d ** 0.5)
        s = s.masked_fill(mask, float("-inf"))
        of[c0:c1] = torch.matmul(torch.softmax(s, dim=-1), vf[c0:c1].double())
    return out


def ratio_interval(torch, plain, tie, groups, n_boot=2000, seed=1):
    """|mean plain| / |mean tie| with a 95% percentile bootstrap interval that
    resamples whole repetitions (groups), the same ones in both modes."""
    import numpy as np
    plain, tie, groups = (t.cpu().numpy() for t in (plain, tie, groups))
    _, g = np.unique(groups, return_inverse=True)
    ng = int(g.max()) + 1
    sp = np.bincount(g, weights=plain, minlength=ng)
    st_ = np.bincount(g, weights=tie, minlength=ng)
    rng = np.random.Generator(np.random.PCG64(seed))
    boots = []
    for b0 in range(0, n_boot, 100):
        idx = rng.integers(0, ng, size=(min(100, n_boot - b0), ng))
        boots.append(np.abs(sp[idx].sum(axis=1)) / np.abs(st_[idx].sum(axis=1)))
    lo, hi = np.quantile(np.concatenate(boots), [0.025, 0.975])
    return {"ratio": float(abs(sp.sum()) / abs(st_.sum())), "lo": float(lo), "hi": float(hi),
            "repetitions": ng}


def tail_oriented_stats(torch, pfa, x, to, eps=1e-3):
    """The signed O error on tied rows oriented by the tail, with V ~ N(0,1):
    per element s = -sign(tau) (O_mode - O_exact), O_exact the float64
    attention, tau the part of the row's unnormalised product that does not
    come from keys within eps of the row maximum, sum over the other keys of
    exp(S - rm) V (float64).  Plain BF16 rounds the sum of the tied V values
    (P-bar = 1) against the small remainder, so its s is negative; every step
    is odd in V, so for symmetric V the raw mean is zero in expectation and
    only this orientation shows the bias.  Unit: the row (mean of s over its
    features with tau != 0); mean, standard error across rows, and the plain /
    tie-aware ratio with a bootstrap interval over repetitions."""
    q, k, v = to(x.q), to(x.k), to(x.v)
    ref = exact_attention(torch, q, k, v)
    B, H, N, d = q.shape
    sign = torch.sign(tail_sums(torch, q, k, v, eps))
    _, _, fl = pfa.forward(q, k, v, causal=True, mode="bf16_out")
    cnt = (sign != 0).double().sum(dim=-1)
    rows = fl.bool() & (cnt > 0)
    res = {"shape": f"B{B} H{H} N{N} d{d}", "v": "N(0,1)", "reference": "float64 attention",
           "tied_rows": int(fl.sum().item()), "rows_with_tail": int(rows.sum().item())}
    per = {}
    for mode in ("bf16_out", "tie_aware_softmax", "fp32_out"):
        o, _, _ = pfa.forward(q, k, v, causal=True, mode=mode, flags=False)
        e = -sign * (o.double() - ref)
        per_row = (e.sum(dim=-1) / cnt.clamp(min=1))[rows]
        per[mode] = per_row
        n = per_row.numel()
        res[mode] = {"mean": float(per_row.mean().item()),
                     "se": float(per_row.std().item() / n ** 0.5) if n > 1 else None}
    groups = torch.nonzero(rows)[:, 0]          # the repetition (batch index) of each row
    res["reduction"] = ratio_interval(torch, per["bf16_out"], per["tie_aware_softmax"], groups)
    return res


def signed_error_stats(torch, pfa, inp, wl, reps=16384):
    """Mean signed O error on tied rows (rows whose tie flag is set), per mode,
    against the float64 attention of the same inputs: the tail-oriented
    statistic on the single-head tied-rows workload (B1 H1 N128 d64, 25% of
    rows with 2-4 tied maxima and Q x8) pooled over `reps` seeded
    repetitions with N(0,1) V (tail_oriented_stats); and the raw mean with
    V - 2 -- the pages' mostly negative V, where plain BF16 is biased negative
    and the tie-aware softmax removes most of it -- on the same pooled
    workload and on the benchmarked workload itself (there the tied keys carry
    a small share of each row's weight)."""
    from synth.inputs import generate_reps, workload
    dev = "cuda:0"
    to = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous()
    tied = generate_reps(workload(1), reps)
    out = {f"tied_rows_workload_x{reps}_tail_oriented": tail_oriented_stats(torch, pfa, tied, to)}
    for name, x, shape in ((f"tied_rows_workload_x{reps}_v_minus_2", tied, f"B{reps} H1 N128 d64"),
                           ("benchmarked_workload_v_minus_2", inp, f"B{wl.b} H{wl.h} N{wl.n} d{wl.d}")):
        q, k, v = to(x.q), to(x.k), to(x.v - 2.0)
        ref = exact_attention(torch, q, k, v)
        _, _, fl = pfa.forward(q, k, v, causal=True, mode="bf16_out")
        rows = fl.bool()
        res = {"shape": shape, "tied_rows": int(rows.sum().item()), "reference": "float64 attention"}
        for mode in ("bf16_out", "tie_aware_softmax", "fp32_out"):
            o, _, _ = pfa.forward(q, k, v, causal=True, mode=mode, flags=False)
            err = (o.double() - ref)[rows]
            res[mode] = {"mean_signed": float(err.mean().item()), "mean_abs": float(err.abs().mean().item())}
        res["reduction"] = abs(res["bf16_out"]["mean_signed"]) / max(abs(res["tie_aware_softmax"]["mean_signed"]), 1e-30)
        out[name] = res
    torch.cuda.synchronize()
    return out


def signed_error_rows(torch, pfa, inp, mode, eps=1e-3):
    """Mean signed O error of `mode` on the rows its tie flags mark, against the
    float64 attention of the same inputs: raw, and oriented by the tail as in
    tail_oriented_stats (reference and tail sums one (batch, head) slice at a
    time).  The row is the unit; returns mean and standard error of each, and
    the row count."""
    dev = "cuda:0"
    to = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous()
    q, k, v = to(inp.q), to(inp.k), to(inp.v)
    B, H, N, d = q.shape
    o, _, fl = pfa.forward(q, k, v, causal=True, mode=mode)
    raw, tail = [], []
    for b in range(B):
        for h in range(H):
            rows = fl[b, h].bool()
            if not bool(rows.any()):
                continue
            sl = lambda t: t[b:b + 1, h:h + 1]
            ref = exact_attention(torch, sl(q), sl(k), sl(v))[0, 0]
            sign = torch.sign(tail_sums(torch, q[b, h], k[b, h], v[b, h], eps))[rows]
            e = (o[b, h].double() - ref)[rows]
            raw.append(e.mean(dim=-1))
            cnt = (sign != 0).double().sum(dim=-1)
            keep = cnt > 0
            tail.append(((-sign * e).sum(dim=-1) / cnt.clamp(min=1))[keep])
    out = {"tied_rows": int(fl.sum().item()), "reference": "float64 attention"}
    for name, xs in (("raw", raw), ("tail", tail)):
        x = torch.cat(xs) if xs else torch.zeros(0, dtype=torch.float64, device=dev)
        n = x.numel()
        out[name] = {"mean": float(x.mean().item()) if n else None,
                     "se": float(x.std().item() / n ** 0.5) if n > 1 else None}
    return out


def report(torch, pfa, steps, warmup):
    """One JSON line per workload and mode (the five synthetic workloads, each
    in the modes it lists): wall time of a fwd+bwd step (the three kernels,
    inputs resident), TFLOP/s against the algorithmic count, tie rows, the
    signed O error on tied rows (BF16 modes; the FP32-output forward is the
    reference), and the float64 oracle's time on the host for the whole
    workload, extrapolated from the slices it finishes in a few seconds."""
    from synth.inputs import generate, workload
    for wid in (1, 2, 3, 4, 5):
        wl = workload(wid)
        inp = generate(wl)
        flops = wl.flops()
        lines = []
        for mode in wl.modes:
            ms, phases, *_ , ties = run_mode(torch, pfa, inp, wl, mode, steps, warmup)
            line = {"workload": wid, "name": wl.name, "shape": [wl.b, wl.h, wl.n, wl.d], "mode": mode,
                    "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                    "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                    "phases_ms": {k_: round(v_, 4) for k_, v_ in phases.items()}, "tie_rows": ties}
            line["signed_error"] = signed_error_rows(torch, pfa, inp, mode)
            lines.append(line)
        # the CPU leg after the GPU timings: seconds of an idle GPU lower its clocks
        cpu = cpu_baseline(inp, wl, budget_s=4.0)
        for line in lines:
            line.update(cpu_float64_s=round(flops / (cpu["value"] * 1e12), 3), cpu_sample=cpu["sample"],
                        cpu_cores=cpu["cores"])
            print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mode", default="bf16_out", choices=("bf16_out", "fp32_out", "tie_aware_softmax"))
    ap.add_argument("--workload", type=int, default=4, help="synthetic workload id (4 = long context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tie", action="store_true", help="skip the tie-aware mode timing")
    ap.add_argument("--no-delta-sources", action="store_true",
                    help="skip the timing of the alternative delta sources")
    ap.add_argument("--no-fp32", action="store_true", help="skip the fp32_out mode timing")
    ap.add_argument("--no-signed-error", action="store_true",
                    help="skip the signed O error statistics on tied rows")
    ap.add_argument("--report", action="store_true",
                    help="instead of the benchmark line, one JSON line per workload (1-5) and mode: "
                         "fwd+bwd time, TFLOP/s, tie rows, signed O error on tied rows, CPU float64 time")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (for scaling the "
                         "HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the (batch, head) slices would shard across GPUs with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return

    import precision_flash_attention_attn_amd as pfa
    from synth.inputs import generate, workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    pfa.lib()  # fail loudly if the HIP library is missing
    if args.report:
        report(torch, pfa, args.steps, args.warmup)
        return
    wl = workload(args.workload)
    inp = generate(wl)
    flops = wl.flops()
    # forward: two products (S = QK^T, P-bar V) of 2 N^2 d each per head, halved by the mask
    unit = wl.b * wl.h * wl.n * wl.n * wl.d // (2 if wl.causal else 1)  # N^2 d per head, masked
    fwd_flops = 4 * unit   # S = QK^T and P-bar V
    bwd_flops = flops - fwd_flops
    # algorithmic work of each kernel: dK/dV kernel = S recompute, dP, dV, dK (8 unit);
    # dQ kernel = dQ alone (2 unit) -- it recomputes S and dP, which count once, above
    kern_flops = {"fwd": fwd_flops, "bwd_dkdv": 8 * unit, "bwd_dq": 2 * unit}

    ms, phases, dom, dom_ms, ties = run_mode(torch, pfa, inp, wl, args.mode, args.steps, args.warmup,
                                             tuple(kern_flops))
    value = flops / (ms * 1e-3) / 1e12

    kname = {"fwd": "fwd_kernel", "bwd_dkdv": "bwd_dkdv_kernel", "bwd_dq": "bwd_dq_kernel"}
    achieved = kern_flops[dom] / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(kname[dom]), "kernel": kname[dom],
                "avg_launch_ms": round(dom_ms, 4),
                "algorithmic_flops_per_launch": kern_flops[dom]}

    extra = {"phases_ms": {s: round(t, 4) for s, t in phases.items()},
             "tie_rows": ties,
             "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
             "fwd_tflops": round(fwd_flops / (phases["fwd"] * 1e-3) / 1e12, 2),
             "bwd_tflops": round(bwd_flops / (sum(phases[s] for s in phases if s != "fwd") * 1e-3) / 1e12, 2)}
    if not args.no_tie and args.mode != "tie_aware_softmax":
        ms_t, ph_t, *_ = run_mode(torch, pfa, inp, wl, "tie_aware_softmax", args.steps, args.warmup)
        extra["tie_aware_softmax"] = {"value": round(flops / (ms_t * 1e-3) / 1e12, 2),
                                      "ms_per_step": round(ms_t, 4),
                                      "phases_ms": {s: round(t, 4) for s, t in ph_t.items()}}
    if not args.no_fp32 and args.mode != "fp32_out":
        # the cost of the FP32-output remedy on the same workload: FP32 O and dO,
        # the hi + lo P-bar operands (a second P-bar V product in the forward)
        ms_f, ph_f, *_ = run_mode(torch, pfa, inp, wl, "fp32_out", args.steps, args.warmup)
        extra["fp32_out"] = {"value": round(flops / (ms_f * 1e-3) / 1e12, 2),
                             "ms_per_step": round(ms_f, 4),
                             "phases_ms": {s: round(t, 4) for s, t in ph_f.items()}}

    if not args.no_delta_sources:
        # algorithmic work: S = QK^T and dP = dO V^T (dp_p), S and P V (do_ohp): 4 unit each
        ds = time_delta_sources(torch, pfa, inp, args.steps, args.warmup)
        extra["delta_sources"] = {src: {"ms": t, "tflops": round(4 * unit / (t * 1e-3) / 1e12, 2)}
                                  for src, t in ds.items()}

    if not args.no_signed_error:
        extra["signed_error_tied_rows"] = signed_error_stats(torch, pfa, inp, wl)

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": f"{wl.name}: B{wl.b} H{wl.h} N{wl.n} d{wl.d} causal, "
                                  f"mode {args.mode}, {wl.note}",
                      "batch": wl.b, "heads": wl.h, "seq_len": wl.n, "head_dim": wl.d,
                      "causal": wl.causal, "mode": args.mode, "parallelism": "single GPU"},
           "roofline": roofline}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, wl)
        out["cpu_emulator"] = cpu_emulator(inp, wl, args.mode)
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
