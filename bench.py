#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one forward and one backward pass (the dQ pass, which also forms
the per-row statistics, then the dK/dV pass: the kernels of fa_bwd) of bf16
causal attention at B=2, H=32, N=8192, d=128 on synthetic inputs already
resident in device memory.  Prints one JSON line.

  value      whole-step throughput in TFLOP/s (forward 4*B*H*N^2*d/2 plus
             backward 2.5x that, divided by the measured step time)
  roofline   the kernel with the largest share of the step time: its
             algorithmic FLOP per launch over its mean launch time (HIP events
             on the launch stream), against the dense bf16 MFMA peak
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload
             (whole heads, forward + backward), as a reference only

Options: --gpus N (only 1 is supported), --steps K, --warmup W,
--no-cpu-baseline, --workload NAME (any backward-capable workload; a
decoding workload such as decode_16x32x1x16384x128 instead times the split-KV
forward and reports GB/s against the HBM peak),
--calib-copy-mb M (launch one plain device copy of M MiB before timing, for
hardware-counter calibration), --all (also time every other workload and
print one extra JSON line per workload; not part of the driver contract).
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6        # MI355X dense bf16 MFMA (256 CU x 4096 x 2.4 GHz)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
METRIC = "attention fwd/bwd TFLOP/s (bf16, N=8192 d=128 causal) + % MFMA peak"
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


KERNEL_SOURCES = {
    "fwd_bf16_kernel": ["fa_fwd_bf16.hip"],
    "bwd_dkdv_kernel": ["fa_bwd_bf16.hip"],
    "bwd_dkdv256_kernel": ["fa_bwd_bf16.hip"],
    "bwd_dq_kernel": ["fa_bwd_bf16.hip"],
    "splitkv_bf16_kernel": ["fa_fwd_bf16.hip"],
    "splitkv_vec_kernel": ["fa_fwd_bf16.hip"],
    "bwd_blocksparse": ["fa_bwd_bf16.hip"],
}


def _code_only(text):
    """C++ source without comments and blank lines (so that editing a
    comment does not mark the counters of an unchanged kernel as stale)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln.strip())


def kernel_source_hash(kernel):
    """Hash of the code a kernel is built from (its file + shared headers,
    comments and blank lines removed)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_io_aware_amd", "csrc")
    files = KERNEL_SOURCES[kernel] + ["fa_device.h", "fa_internal.h"]
    for f in files:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _stored(kernel, workload, key):
    """A value `key: number` from the committed counter summary of a kernel
    on a workload, or None when there is none or the kernel sources changed
    since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(key + r":\s*([0-9.eE+]+)", text)
    m_h = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    if not m_b or not m_h or m_h.group(1) != kernel_source_hash(kernel):
        return None
    return float(m_b.group(1))


def stored_traffic(kernel, workload):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)."""
    return _stored(kernel, workload, "traffic_bytes_per_launch")


def stored_clock_ghz(kernel, workload):
    """The engine clock while the kernel ran: GRBM_GUI_ACTIVE cycles per XCD
    over the kernel's duration, from the same counter summary."""
    return _stored(kernel, workload, "gpu_clock_ghz")


def calib_copy(mb):
    """One plain device copy of `mb` MiB (read and written once), the
    reference for scaling the HBM byte counters."""
    import torch
    src = torch.ones(mb * (1 << 20) // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def time_workload(name, steps, warmup, calib_mb=0):
    import torch

    from exact_io_aware_amd import fa, workloads

    w = workloads.workload(name)
    B, H, N, d, causal = w["B"], w["H"], w["N"], w["d"], w["causal"][-1]
    dev = torch.device("cuda:0")
    x = workloads.workload_inputs(name, with_do=True, device=dev)
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    if w["dtype"] != "bf16":
        raise SystemExit(f"{name}: the step bench times bf16 workloads "
                         "(--all covers the fp32 ones)")
    scale = w["scale"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(q.shape, **f32) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    if calib_mb:
        calib_copy(calib_mb)

    mask = workloads.workload_mask(w)
    mask_t = torch.from_numpy(mask).to(dev) if mask is not None else None
    has_bwd = "bwd" in w["passes"]
    # The step's calls, each timed: dense backward workloads call the two
    # backward passes one by one, in fa_bwd's order (the dQ pass with the row
    # statistics, then the dK/dV pass); the block-sparse workload its forward
    # and its whole backward; forward-only workloads every causal mode they
    # list.
    if mask_t is not None:
        calls = [("fwd", lambda: fa.fa_fwd_blocksparse(
                     q, k, v, mask_t, scale=scale, causal=causal, out=o, lse=lse)),
                 ("bwd", lambda: fa.fa_bwd_blocksparse(
                     q, k, v, o, do, lse, mask_t, scale=scale, causal=causal,
                     workspace=ws, dq=dq, dk=dk, dv=dv))]
    elif has_bwd:
        calls = [("fwd", lambda: fa.fa_fwd(q, k, v, scale=scale, causal=causal,
                                           out=o, lse=lse)),
                 ("bwd_dq", lambda: fa.fa_bwd_dq_stats(q, k, v, o, do, lse, ws,
                                                       dq, scale=scale,
                                                       causal=causal)),
                 ("bwd_dkdv", lambda: fa.fa_bwd_dkdv(q, k, v, do, ws, dk, dv,
                                                     scale=scale, causal=causal))]
    else:
        calls = [("fwd" if c else "fwd_noncausal",
                  (lambda c=c: fa.fa_fwd(q, k, v, scale=scale, causal=c, out=o,
                                         lse=lse)))
                 for c in w["causal"]]
    names = tuple(n for n, _ in calls)
    ev = {n: [] for n in names}

    def rec():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step(record):
        marks = [rec()] if record else None
        for _, call in calls:
            call()
            if record:
                marks.append(rec())
        if record:
            for i, n in enumerate(names):
                ev[n].append((marks[i], marks[i + 1]))

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = rec()
    wall0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    t1 = rec()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / steps
    kern_ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / steps
               for n in names}
    if mask is not None:
        ff = 4.0 * d * 128 * 128 * float(mask.sum()) * B * H
    else:
        ff = fwd_flops(B, H, N, d, causal)
    alg = {"fwd": ff, "fwd_noncausal": fwd_flops(B, H, N, d, False),
           "bwd": 2.5 * ff, "bwd_dkdv": 0.8 * 2.5 * ff,
           "bwd_dq": 0.2 * 2.5 * ff}
    alg = {n: alg[n] for n in names}
    return dict(w=w, B=B, H=H, N=N, d=d, causal=causal, ms_step=ms_step,
                wall=wall, kern_ms=kern_ms, fwd_flops=ff,
                bwd_flops=2.5 * ff if has_bwd else 0.0, alg=alg,
                step_flops=sum(alg.values()), sparse=mask is not None)


def time_passes(name, steps, warmup, oracle_check=False):
    """Per-workload timing of every pass the workload lists (used by --all):
    the forward, and for workloads with a backward the whole fa_bwd (or
    fa_bwd_blocksparse) call, inputs O and LSE from the forward (untimed).
    With oracle_check each line also carries the parity and the oracle's
    throughput on a sample of whole heads (parity_and_baseline)."""
    import torch

    from exact_io_aware_amd import fa, workloads

    w = workloads.workload(name)
    dev = torch.device("cuda:0")
    x = workloads.workload_inputs(name, with_do="bwd" in w["passes"],
                                  device=dev)
    mask = workloads.workload_mask(w)
    mask_t = torch.from_numpy(mask).to(dev) if mask is not None else None
    out = []

    def median_ms(run):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            times.append((a, b))
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in times)[len(times) // 2]

    p_drop = w.get("p_drop", 0.0)
    for causal in w["causal"]:
        def fwd():
            if mask_t is not None:
                return fa.fa_fwd_blocksparse(x["q"], x["k"], x["v"], mask_t,
                                             scale=w["scale"], causal=causal)
            if p_drop:
                return fa.fa_fwd_dropout(x["q"], x["k"], x["v"], p_drop,
                                         w["drop_seed"], scale=w["scale"],
                                         causal=causal)
            return fa.fa_fwd(x["q"], x["k"], x["v"], scale=w["scale"],
                             causal=causal)
        if mask is not None:
            flops = 4.0 * w["d"] * 128 * 128 * float(mask.sum()) * w["B"] * w["H"]
        else:
            flops = fwd_flops(w["B"], w["H"], w["N"], w["d"], causal)
        peak = PEAK_F32_TFLOPS if w["dtype"] == "f32" else PEAK_BF16_TFLOPS
        passes = [("fwd", fwd, flops)]
        if "bwd" in w["passes"]:
            o, lse = fwd()
            ws = torch.empty(fa.fa_bwd_workspace_bytes(w["B"], w["H"], w["N"],
                                                       w["d"]),
                             dtype=torch.uint8, device=dev)
            grads = [torch.empty(x["q"].shape, dtype=torch.float32, device=dev)
                     for _ in range(3)]

            def bwd():
                kw = dict(scale=w["scale"], causal=causal, workspace=ws,
                          dq=grads[0], dk=grads[1], dv=grads[2])
                if mask_t is not None:
                    fa.fa_bwd_blocksparse(x["q"], x["k"], x["v"], o, x["do"],
                                          lse, mask_t, **kw)
                elif p_drop:
                    fa.fa_bwd_dropout(x["q"], x["k"], x["v"], o, x["do"], lse,
                                      p_drop, w["drop_seed"], **kw)
                else:
                    fa.fa_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, **kw)
            passes.append(("bwd", bwd, 2.5 * flops))
        for pname, run, fl in passes:
            ms = median_ms(run)
            tf = fl / (ms * 1e-3) / 1e12
            res = dict(workload=name, causal=causal, **{"pass": pname},
                       ms_median=ms, tflops=tf, frac_peak=tf / peak)
            if p_drop:
                res["p_drop"] = p_drop
            if oracle_check:
                got = run()
                torch.cuda.synchronize()
                if pname == "bwd":
                    got = grads
                res.update(parity_and_baseline(w, x, causal, mask, pname, got,
                                               fl))
            out.append(res)
    return out


def parity_and_baseline(w, x, causal, mask, pname, got, flops):
    """The fp64 oracle on a bounded sample of whole heads of a workload:
    parity of the GPU outputs on those heads (max-abs and relative RMS over
    the sampled heads, against the bars: fp32 max-abs 1e-5; bf16 max-abs
    2e-2 (x 256/(256-t) with dropout) and rel-RMS 5e-3), and the oracle's
    own throughput on them (the same algorithmic FLOP per head as the GPU
    line; it materialises the full N^2 even where causal)."""
    import numpy as np

    import oracle

    B, H = w["B"], w["H"]
    heads = [(0, 0)] if (B, H) == (1, 1) else [(0, 0), (B - 1, H - 1)]
    if w["N"] >= 16384:
        heads = heads[:1]
    f64 = lambda t: t.detach().double().cpu().numpy()  # noqa: E731
    names = ("O", "LSE") if pname == "fwd" else ("dQ", "dK", "dV")
    errs = {n: [0.0, 0.0, 0.0] for n in names}  # max-abs, sum sq diff, sum sq ref
    t_cpu = 0.0
    p_drop = w.get("p_drop", 0.0)
    t_drop = oracle.dropout_threshold(p_drop) if p_drop else 0
    for b, h in heads:
        q, k, v = (f64(x[n][b, h]) for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        if pname == "fwd":
            if p_drop:
                ref = oracle.attention_fwd_dropout_head(
                    q, k, v, w["scale"], causal, t_drop, w["drop_seed"],
                    b * H + h)
            else:
                ref = oracle.attention_fwd_head(q, k, v, w["scale"], causal,
                                                mask, 128, 128)
        else:
            do = f64(x["do"][b, h])
            if p_drop:
                ref = oracle.attention_bwd_dropout_head(
                    q, k, v, do, w["scale"], causal, t_drop, w["drop_seed"],
                    b * H + h)
            else:
                ref = oracle.attention_bwd_head(q, k, v, do, w["scale"],
                                                causal, mask, 128, 128)
        t_cpu += time.perf_counter() - t0
        for n, g, r in zip(names, got, ref):
            g = f64(g[b, h])
            ok = ~np.isneginf(r)
            d_ = g[ok] - r[ok]
            e = errs[n]
            e[0] = max(e[0], float(np.max(np.abs(d_))) if d_.size else 0.0)
            e[1] += float(np.sum(d_ * d_))
            e[2] += float(np.sum(r[ok] * r[ok]))
    fp32 = w["dtype"] == "f32"
    bar_abs = 1e-5 if fp32 else 2e-2 * 256.0 / (256 - t_drop)
    parity, passed = {}, True
    for n, (mx, sd, sr) in errs.items():
        rel = (sd / sr) ** 0.5 if sr > 0 else 0.0
        ok = mx <= bar_abs and (fp32 or rel <= 5e-3)
        passed &= ok
        parity[n] = {"max_abs": mx, "rel_rms": rel}
    head_flops = flops / (B * H) * len(heads)
    return {
        "parity": dict(parity, heads=[list(hh) for hh in heads],
                       max_abs_bar=bar_abs, rel_rms_bar=None if fp32 else 5e-3,
                       passed=passed),
        "cpu_baseline": {
            "value": head_flops / t_cpu / 1e12, "unit": "TFLOP/s",
            "cores": int(_blas_threads()), "kind": "oracle",
            "sample": (f"{len(heads)} whole head(s) {heads}, fp64 NumPy, "
                       f"full N^2 materialised, {t_cpu:.2f} s")},
    }


def decode_bytes(w, Nq=None):
    """Algorithmic HBM bytes of one decoding call: Q, K, V read once, O and
    LSE written once (bf16 tensors, fp32 LSE)."""
    Nq = w["Nq"] if Nq is None else Nq
    return w["B"] * w["H"] * (2 * 2 * Nq * w["d"] + 2 * 2 * w["Nk"] * w["d"]
                              + 4 * Nq)


def time_decode(name, steps, warmup, keep=None, oracle_check=False):
    """Timing of the split-KV forward on a decoding workload (used by --all):
    the whole fa_fwd_splitkv call (chunk pass + merge), median over steps.
    The work is a matrix-vector product per head, bound by HBM bandwidth, so
    the figure is algorithmic bytes (Q, K, V read once; O and LSE written
    once) over the median time, against the 8 TB/s HBM peak."""
    import torch

    from exact_io_aware_amd import fa, workloads

    w = workloads.workload(name)
    B, H, Nq, Nk, d = w["B"], w["H"], w["Nq"], w["Nk"], w["d"]
    dev = torch.device("cuda:0")
    x = workloads.make_decode_inputs(B, H, Nq, Nk, d, w["seed"], w["sigma"],
                                     device=dev)
    if keep is not None:
        keep.update(x)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, 0),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    out = []
    for causal in w["causal"]:
        def run():
            fa.fa_fwd_splitkv(x["q"], x["k"], x["v"], scale=w["scale"],
                              causal=causal, workspace=ws, out=o, lse=lse)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            times.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in times)[len(times) // 2]
        nbytes = decode_bytes(w)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res = dict(workload=name, causal=causal, **{"pass": "decode"},
                   ms_median=ms, gbytes_per_s=gbs,
                   frac_hbm_peak=gbs / PEAK_HBM_GBS,
                   chunks=fa.fa_fwd_splitkv_chunks(B, H, Nq, Nk, d, 0))
        if oracle_check:
            res.update(decode_parity(w, x, causal, o, lse))
        out.append(res)
    return out


def decode_parity(w, x, causal, o, lse, heads=((0, 0), (-1, -1))):
    """The decoding oracle on two whole heads: parity (bf16 bars) and its
    throughput in GB/s of the same algorithmic bytes."""
    import numpy as np

    import oracle

    f64 = lambda t: t.detach().double().cpu().numpy()  # noqa: E731
    errs = {"O": [0.0, 0.0, 0.0], "LSE": [0.0, 0.0, 0.0]}
    t_cpu = 0.0
    for b, h in heads:
        q, k, v = (f64(x[n][b, h]) for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        ref = oracle.attention_decode_head(q, k, v, w["scale"], causal)
        t_cpu += time.perf_counter() - t0
        for n, g, r in zip(("O", "LSE"), (o, lse), ref):
            d_ = f64(g[b, h]) - r
            e = errs[n]
            e[0] = max(e[0], float(np.max(np.abs(d_))))
            e[1] += float(np.sum(d_ * d_))
            e[2] += float(np.sum(r * r))
    parity, passed = {}, True
    for n, (mx, sd, sr) in errs.items():
        rel = (sd / sr) ** 0.5 if sr > 0 else 0.0
        passed &= mx <= 2e-2 and rel <= 5e-3
        parity[n] = {"max_abs": mx, "rel_rms": rel}
    per_head = decode_bytes(w) / (w["B"] * w["H"])
    return {"parity": dict(parity, heads=[list(hh) for hh in heads],
                           max_abs_bar=2e-2, rel_rms_bar=5e-3, passed=passed),
            "cpu_baseline": {"value": per_head * len(heads) / t_cpu / 1e9,
                             "unit": "GB/s", "cores": int(_blas_threads()),
                             "kind": "oracle",
                             "sample": f"{len(heads)} whole heads, fp64 NumPy, {t_cpu:.3f} s"}}


def cpu_baseline(name, budget_s=12.0, max_heads=8):
    """The fp64 oracle (forward + backward of whole heads) on host cores."""
    import numpy as np

    import oracle
    from exact_io_aware_amd import workloads

    threads = _blas_threads()
    w = workloads.workload(name)
    x = workloads.workload_inputs(name, with_do=True)
    causal = w["causal"][-1]
    mask = workloads.workload_mask(w)
    has_bwd = "bwd" in w["passes"]
    heads, t_total = 0, 0.0
    for b in range(w["B"]):
        for hh in range(w["H"]):
            q, k, v, do = (x[n][b, hh].double().numpy() for n in
                           ("q", "k", "v", "do"))
            t0 = time.perf_counter()
            oracle.attention_fwd_head(q, k, v, w["scale"], causal, mask)
            if has_bwd:
                oracle.attention_bwd_head(q, k, v, do, w["scale"], causal,
                                          mask)
            t_total += time.perf_counter() - t0
            heads += 1
            if t_total >= budget_s or heads >= max_heads:
                break
        if t_total >= budget_s or heads >= max_heads:
            break
    if mask is not None:
        head_fwd = 4.0 * w["d"] * 128 * 128 * float(mask.sum())
    else:
        head_fwd = fwd_flops(1, 1, w["N"], w["d"], causal)
    flops = (3.5 if has_bwd else 1.0) * head_fwd * heads
    what = "forward + backward" if has_bwd else "forward"
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": (f"{heads} whole heads (b,h) of {name}, {what}, fp64 "
                       f"NumPy materialising S and P (full N^2 even where "
                       f"causal or masked), {t_total:.1f} s")}


def cpu_baseline_decode(name, x, budget_s=12.0, max_heads=512):
    """The fp64 oracle's decoding attention on whole heads, on host cores
    (inputs `x` as drawn for the GPU timing; each head is copied to the host
    before its clock starts)."""
    import oracle
    from exact_io_aware_amd import workloads

    threads = _blas_threads()
    w = workloads.workload(name)
    heads, t_total = 0, 0.0
    for b in range(w["B"]):
        for hh in range(w["H"]):
            q, k, v = (x[n][b, hh].cpu().double().numpy()
                       for n in ("q", "k", "v"))
            t0 = time.perf_counter()
            oracle.attention_decode_head(q, k, v, w["scale"], True)
            t_total += time.perf_counter() - t0
            heads += 1
            if t_total >= budget_s or heads >= max_heads:
                break
        if t_total >= budget_s or heads >= max_heads:
            break
    per_head = decode_bytes(w) / (w["B"] * w["H"])
    return {"value": per_head * heads / t_total / 1e9, "unit": "GB/s",
            "cores": int(threads), "kind": "oracle",
            "sample": (f"{heads} whole heads (b,h) of {name}, fp64 NumPy "
                       f"decoding attention, {t_total:.2f} s")}


def decode_line(args):
    """The JSON line of a decoding workload (--workload decode_...)."""
    from exact_io_aware_amd import workloads
    w = workloads.workload(args.workload)
    x = {}
    r = time_decode(args.workload, args.steps, args.warmup, keep=x)[-1]
    # One query row runs the vector chunk pass, several the matrix-core one.
    kname = "splitkv_vec_kernel" if w["Nq"] == 1 else "splitkv_bf16_kernel"
    line = {
        "metric": "split-KV decoding attention GB/s (bf16, HBM-bound)",
        "value": round(r["gbytes_per_s"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_median"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": w["B"], "H": w["H"],
                   "Nq": w["Nq"], "Nk": w["Nk"], "d": w["d"],
                   "causal": True, "chunks": r["chunks"],
                   "seed": w["seed"], "sigma": w["sigma"]},
        "roofline": {
            "kernel": kname + " + splitkv_merge_kernel",
            "bound": "hbm",
            "achieved": round(r["gbytes_per_s"], 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(r["frac_hbm_peak"], 4),
            "traffic": stored_traffic(kname, args.workload),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline_decode(args.workload, x)
    print(json.dumps(line), flush=True)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return len(os.sched_getaffinity(0))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="causal_2x32x8192x128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0)
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--print-hash", action="store_true",
                    help="print the source hash of each timed kernel and exit")
    args = ap.parse_args()
    if args.print_hash:
        for k in KERNEL_SOURCES:
            print(k, kernel_source_hash(k))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this "
              "build has no multi-GPU path; the attention kernels shard by "
              "(batch, head) with no exchange, so each GPU would run this same "
              "single-GPU step on its share.", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from exact_io_aware_amd import fa
    fa.library()

    from exact_io_aware_amd import workloads as _wl
    if args.workload in _wl.DECODE_WORKLOADS:
        if args.calib_copy_mb:
            calib_copy(args.calib_copy_mb)
        decode_line(args)
        return
    if _wl.workload(args.workload).get("p_drop"):
        print(f"{args.workload} is a dropout workload: bench.py --all times it "
              "(fa_fwd_dropout, fa_bwd_dropout); the per-kernel step here "
              "times the dropout-free passes.", file=sys.stderr)
        sys.exit(2)
    r = time_workload(args.workload, args.steps, args.warmup,
                      args.calib_copy_mb)
    B, H, N, d = r["B"], r["H"], r["N"], r["d"]
    step_flops = r["step_flops"]
    value = step_flops / (r["ms_step"] * 1e-3) / 1e12
    km = r["kern_ms"]
    fwd_tf = r["fwd_flops"] / (km["fwd"] * 1e-3) / 1e12
    bwd_ms = sum(km[n] for n in km if n.startswith("bwd"))
    bwd_tf = r["bwd_flops"] / (bwd_ms * 1e-3) / 1e12 if bwd_ms else 0.0
    # The dominant kernel: the timed call with the most time (the block-sparse
    # backward's three kernels are timed as one call, fa_bwd_blocksparse,
    # reported as "bwd_blocksparse").
    dom = max(km, key=lambda n: km[n])
    achieved = r["alg"][dom] / (km[dom] * 1e-3) / 1e12
    # (At d = 128 without mask or dropout the dK/dV pass is the 256-key
    # kernel.)
    kname = {"fwd": "fwd_bf16_kernel", "fwd_noncausal": "fwd_bf16_kernel",
             "bwd_dkdv": "bwd_dkdv256_kernel" if d == 128 else "bwd_dkdv_kernel",
             "bwd_dq": "bwd_dq_kernel", "bwd": "bwd_blocksparse"}[dom]
    step_name = "fwd+bwd" if r["bwd_flops"] else "+".join(km)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "N": N, "d": d,
                   "causal": bool(r["causal"]), "step": step_name,
                   "block_sparse": r["sparse"],
                   "seed": r["w"]["seed"], "sigma": r["w"]["sigma"]},
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "fwd_frac_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        "bwd_frac_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
        "step_frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": {n: round(t, 4) for n, t in km.items()},
        "roofline": {
            "kernel": kname,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": stored_traffic(kname, args.workload),
        },
        "cpu_baseline": None,
    }
    # The same kernel against the dense bf16 peak at the clock the GPU ran
    # it at (256 CUs x 4096 flop/clk x f), f from the kernel's committed
    # counters (GRBM_GUI_ACTIVE per XCD over the kernel time).
    f_ghz = stored_clock_ghz(kname, args.workload)
    if f_ghz:
        peak_f = 256 * 4096 * f_ghz * 1e9 / 1e12
        line["roofline"]["clock_ghz"] = f_ghz
        line["roofline"]["clock_source"] = (
            f"GRBM_GUI_ACTIVE / kernel time, profiles/{kname}_{args.workload}_pmc.md")
        line["roofline"]["peak_at_clock"] = round(peak_f, 1)
        line["roofline"]["frac_measured_clock"] = round(achieved / peak_f, 4)
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(args.workload)
    if args.all:
        from exact_io_aware_amd import workloads
        for name in workloads.WORKLOADS:
            for res in time_passes(name, max(args.steps, 20), 3,
                                   oracle_check=not args.no_cpu_baseline):
                print(json.dumps(res), flush=True)
        for name in workloads.CONTEXT_WORKLOADS:
            for res in time_passes(name, max(args.steps, 20), 3,
                                   oracle_check=not args.no_cpu_baseline):
                print(json.dumps(res), flush=True)
        for name in workloads.DECODE_WORKLOADS:
            for res in time_decode(name, max(args.steps, 20), 3,
                                   oracle_check=not args.no_cpu_baseline):
                print(json.dumps(res), flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
