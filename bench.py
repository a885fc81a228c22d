#!/usr/bin/env python3
"""Benchmark of the MI355X log-mel front end (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one whole pass of the transform over one batch: for the default
workload, lm_from_pcm on 64 clips x 480000 int16 samples (30 s at 16 kHz),
n_fft 400, hop 160, 128 Slaney mels, float32 out -- the main kernel plus the
per-clip clamp fix-up.  Inputs are generated on the host, copied to HBM once
and stay resident; several input/output buffer sets are cycled so that every
step reads its input from HBM rather than from the 256 MB last-level cache.
The GPU raises its clocks over the first ~30 ms of sustained work (``--ramp``
prints that curve).  Before the warm-up steps of each workload, 500 ms of
fp32 matrix products (``--clock-ramp-ms``, ``--clock-ramp-kind``; unrelated
to the transform) bring it there, so that short runs with few warm-up steps
are timed at the sustained clocks too (plain copies, the other kind, leave
the compute clock where it was); the default warm-up (1000 steps) and the
200 timed steps follow unchanged.

Prints ONE JSON line: frames/s for the batch, the main kernel's achieved HBM
bandwidth against MI355X's 8 TB/s (event-timed on the stream it runs on),
and the fp64 oracle timed on this host's cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
FP32_VALU_PEAK_TFLOPS = 157.3     # published fp32 vector peak
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """Hash of every library source: counter figures taken on other sources are stale."""
    csrc = os.path.join(ROOT, "stft_log_mel_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".cpp", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def main_kernel_name(w, fft_variant: str = "auto") -> str:
    """The kernel lm_from_* launches for this workload (the library's own dispatch rule)."""
    if w.entry == "stft":
        return "stft_logmel_kernel"
    if w.n_fft == 400 and w.hop % 2 == 0 and fft_variant in ("auto", "split_mfma"):
        return "pcm400_kernel"
    if w.n_fft >= 8192:
        return "pcm_big_kernel"
    return "pcm_logmel_kernel"


def counter_traffic(workload: str):
    """HBM bytes per launch of the main kernel from committed rocprofv3 counter
    runs, if they were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def flops_per_frame(w) -> float:
    """Nominal arithmetic per frame (real FFT 2.5 N log2 N, window, power,
    packed mel FMAs): used for the FFT-rate context figure only."""
    import math
    if w.entry == "stft":
        return 3.0 * w.NF + 2.0 * 2 * w.NF
    N = w.n_fft
    return 2.5 * N * math.log2(N) + N + 3.0 * (N // 2 + 1) + 2.0 * 2 * (N // 2 + 1)


def sweep_one(w, steps: int, warmup: int):
    """One line of the n_fft sweep: step time, essential-byte rate and the
    main kernel's dispatch-stamped duration."""
    import numpy as np  # noqa: F401
    import torch

    import lm_synth
    import stft_log_mel_amd as lm

    dev = torch.device("cuda:0")
    x = torch.from_numpy(lm_synth.make_inputs(w)).to(dev)
    nbuf = max(1, min(8, -(-1_000_000_000 // w.essential_bytes()) + 1))
    ins = [x.clone() for _ in range(nbuf)]
    outs = [torch.empty(w.out_shape, dtype=torch.float32, device=dev) for _ in range(nbuf)]
    plan = lm.Plan(w.n_fft, w.hop, w.n_mels).set_mel(w.sample_rate, w.f_min, w.f_max)
    for i in range(warmup):
        plan.from_pcm(ins[i % nbuf], out=outs[i % nbuf])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(steps):
        plan.from_pcm(ins[i % nbuf], out=outs[i % nbuf])
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    plan.profile(True)
    for i in range(steps):
        plan.from_pcm(ins[i % nbuf], out=outs[i % nbuf])
    torch.cuda.synchronize()
    plan.profile(False)
    prof = plan.profile_read()
    main_ms = prof["main"]["ms"] / max(1, prof["main"]["count"])
    eb = w.essential_bytes()
    frames = w.B * w.n_frames
    print(json.dumps({"workload": w.name, "n_fft": w.n_fft, "hop": w.hop, "n_mels": w.n_mels, "B": w.B,
                      "T": w.T, "ms_per_step": round(ms, 5), "frames_per_s": round(frames / (ms / 1e3), 1),
                      "essential_bytes": eb, "essential_gbs_step": round(eb / (ms / 1e3) / 1e9, 1),
                      "kernel": main_kernel_name(w), "kernel_ms": round(main_ms, 5),
                      "kernel_gbs": round(eb / (main_ms / 1e3) / 1e9, 1),
                      "kernel_frac_of_8tbs": round(eb / (main_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                      "fft_tflops": round(frames * flops_per_frame(w) / (main_ms / 1e3) / 1e12, 2)}), flush=True)


def dft_gemm_probe(w, steps: int, warmup: int):
    """The dense alternative to the fused FFT at n_fft = 400: the windowed
    frames of the batch (192064 x 400, fp32) times the real DFT matrix
    (400 x 402: cos and -sin columns for bins 0..200, window folded in), one
    torch.matmul on the vendor BLAS in fp32.  Times the GEMM alone -- a lower
    bound for that design, which would still need the power, the mel
    projection and the log tail -- next to the library's whole fused step on
    the same batch."""
    import numpy as np
    import torch

    import stft_log_mel_amd as lm

    torch.backends.cuda.matmul.allow_tf32 = False
    dev = torch.device("cuda:0")
    x = torch.from_numpy(lm_synth_inputs(w)).to(dev)
    N, hop = w.n_fft, w.hop
    xf = torch.nn.functional.pad(x.float()[:, None, :], (N // 2, N // 2), mode="reflect")[:, 0, :]
    frames = xf.unfold(-1, N, hop).reshape(-1, N).contiguous()          # (B F, N)
    n = np.arange(N)[:, None].astype(np.float64)
    k = np.arange(N // 2 + 1)[None, :].astype(np.float64)
    win = 0.5 - 0.5 * np.cos(2 * np.pi * np.arange(N) / N)
    ang = 2 * np.pi * n * k / N
    D = np.concatenate([np.cos(ang), -np.sin(ang)], axis=1) * win[:, None]   # (N, 2 (N/2 + 1))
    Dm = torch.from_numpy(D.astype(np.float32)).to(dev)
    y = torch.empty(frames.shape[0], Dm.shape[1], dtype=torch.float32, device=dev)
    for _ in range(warmup):
        torch.matmul(frames, Dm, out=y)
    torch.cuda.synchronize()
    # sanity: the GEMM is the windowed one-sided DFT (against torch.fft.rfft on a few frames)
    ref = torch.fft.rfft(frames[:64] * torch.from_numpy(win.astype(np.float32)).to(dev), dim=-1)
    got = torch.complex(y[:64, :N // 2 + 1], y[:64, N // 2 + 1:])
    rel = (torch.abs(got - ref).max() / torch.abs(ref).max()).item()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        torch.matmul(frames, Dm, out=y)
    ev1.record(stream)
    torch.cuda.synchronize()
    gemm_ms = ev0.elapsed_time(ev1) / steps
    flop = 2.0 * frames.shape[0] * N * Dm.shape[1]
    # the library's fused step on the same batch
    plan = lm.Plan(N, hop, w.n_mels).set_mel(w.sample_rate, w.f_min, w.f_max)
    out = torch.empty(w.out_shape, dtype=torch.float32, device=dev)
    for _ in range(warmup):
        plan.from_pcm(x, out=out)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        plan.from_pcm(x, out=out)
    ev1.record(stream)
    torch.cuda.synchronize()
    fused_ms = ev0.elapsed_time(ev1) / steps
    print(json.dumps({"probe": "dft_as_fp32_gemm", "workload": w.name, "M": frames.shape[0], "K": N,
                      "N": Dm.shape[1], "gemm_ms": round(gemm_ms, 4), "gemm_tflops": round(flop / gemm_ms / 1e9, 1),
                      "fp32_matrix_peak_tflops": 157.3, "gemm_rel_err_vs_rfft": rel,
                      "fused_step_ms": round(fused_ms, 4), "gemm_over_fused_step": round(gemm_ms / fused_ms, 2)}),
          flush=True)


def lm_synth_inputs(w):
    import lm_synth
    return lm_synth.make_inputs(w)


PER_CONFIG = ("stft_b1", "pcm_f32_b8", "stft_b256", "pcm_f32_nfft16384")


def first_stage_dtype(w, fft_variant: str) -> str:
    """The arithmetic the workload's transform runs in."""
    if w.entry == "pcm" and main_kernel_name(w, fft_variant) == "pcm400_kernel":
        if fft_variant == "split_mfma":
            return "f32 (n_fft 400 16-point and 25-point stages: two-part fp16 operands, fp32 accumulate)"
        return "f32 (n_fft 400 first stage: two-part fp16 operands, fp32 accumulate)"
    return "f32"


class Run:
    """One workload resident on the GPU: inputs (several buffer sets, so that
    every step reads cold input), outputs, plan, and a step that runs the
    whole path once."""

    def __init__(self, w, dev, fft_variant="auto", single_pass=False, log=True):
        import torch

        import lm_synth
        import stft_log_mel_amd as lm

        self.w = w
        if log:
            print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
        t0 = time.time()
        if w.entry == "stft":
            self.host_in, self.host_filters = lm_synth.make_inputs(w)
        else:
            self.host_in, self.host_filters = lm_synth.make_inputs(w), None
        if log:
            print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        self.nbuf = max(1, min(8, -(-1_000_000_000 // w.essential_bytes()) + 1))   # cycle >= ~1 GB of buffers
        self.ins = [torch.from_numpy(self.host_in).to(dev) for _ in range(self.nbuf)]
        out_dt = torch.float16 if w.out_dtype == "f16" else torch.float32
        # outputs are filled once here (allocation-time initialisation), so the
        # first step that writes a buffer set does not also pay for the GPU's
        # first touch of its pages; the inputs were written by their copies
        self.outs = [torch.zeros(w.out_shape, dtype=out_dt, device=dev) for _ in range(self.nbuf)]
        if w.entry == "stft":
            self.filt = torch.from_numpy(self.host_filters).to(dev)
            self.plan = lm.Plan(400, 160, w.NM)
        else:
            self.plan = lm.Plan(w.n_fft, w.hop, w.n_mels, w.center, w.pad_mode, w.power, w.out_dtype)
            self.plan.set_mel(w.sample_rate, w.f_min, w.f_max)
            self.plan.set_fft_variant(fft_variant)
            self.plan.set_single_pass(single_pass)
        self.stream = torch.cuda.current_stream(dev)

    def step(self, i):
        if self.w.entry == "stft":
            self.plan.from_stft(self.ins[i % self.nbuf], self.filt, out=self.outs[i % self.nbuf])
        else:
            self.plan.from_pcm(self.ins[i % self.nbuf], out=self.outs[i % self.nbuf])

    def time(self, steps, warmup):
        """Mean ms per step over `steps` back-to-back steps (events only
        around the whole run), then per-step times from a second run with an
        event between steps, then the same steps with every launch stamped
        by its own dispatch (per-kernel means)."""
        import torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_wall = time.perf_counter()
        ev0.record(self.stream)
        for i in range(steps):
            self.step(i)
        ev1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        ms = ev0.elapsed_time(ev1) / steps
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(self.stream)
        for i in range(steps):
            self.step(i)
            evs[i + 1].record(self.stream)
        torch.cuda.synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
        pct = lambda q: per[min(len(per) - 1, int(round(q * (len(per) - 1))))]   # noqa: E731
        self.plan.profile(True)
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        self.plan.profile(False)
        prof = self.plan.profile_read()
        kern = {k: prof[k]["ms"] / max(1, prof[k]["count"]) for k in ("main", "fixup", "pack")}
        return {"ms_per_step": ms, "wall_s": wall, "p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9),
                "kernel_ms": kern}

    def last_output(self, steps):
        return self.outs[(steps - 1) % self.nbuf]

    def oracle_clip(self, b):
        import oracle
        w = self.w
        if w.entry == "stft":
            return oracle.from_stft(self.host_in[b:b + 1], self.host_filters)[0]
        W = oracle.mel_filterbank(w.sample_rate, w.n_fft, w.n_mels, w.f_min, w.f_max)
        return oracle.from_pcm(self.host_in[b:b + 1], w.n_fft, w.hop, W, center=w.center,
                               pad_mode=w.pad_mode, power=w.power)[0]


def ramp_one(w, dev, chunks=30, chunk_ms=3.0):
    """Step time in consecutive chunks of about chunk_ms of work, starting
    from an idle GPU (half a second of sleep first): one line per workload."""
    import torch
    r = Run(w, dev, log=False)
    r.step(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(r.stream)
    r.step(1)
    e1.record(r.stream)
    torch.cuda.synchronize()
    per = max(1, int(chunk_ms / max(e0.elapsed_time(e1), 1e-3)))
    time.sleep(0.5)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(chunks + 1)]
    ev[0].record(r.stream)
    for c in range(chunks):
        for i in range(per):
            r.step(i)
        ev[c + 1].record(r.stream)
    torch.cuda.synchronize()
    t, pts = 0.0, []
    for c in range(chunks):
        ms = ev[c].elapsed_time(ev[c + 1])
        t += ms
        pts.append([round(t, 2), round(ms / per * 1e3, 2)])
    print(json.dumps({"ramp": w.name, "steps_per_chunk": per, "elapsed_ms_and_us_per_step": pts}), flush=True)
    del r


def roofline_of(w, kernel_ms, fft_variant="auto"):
    """The main kernel against its bounding roofline: HBM bytes for every
    workload except the n_fft 16384 one, whose bound is the FFT arithmetic
    (nominal flops against the fp32 vector peak)."""
    frames = w.B * w.n_frames
    if w.entry == "pcm" and w.n_fft >= 8192:
        tf = frames * flops_per_frame(w) / (kernel_ms / 1e3) / 1e12
        return {"bound": "alu", "achieved": round(tf, 2), "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / FP32_VALU_PEAK_TFLOPS, 4),
                "frac_of_unpacked_fp32": round(tf / (FP32_VALU_PEAK_TFLOPS / 2), 4),
                "algorithmic_flops_per_launch": round(frames * flops_per_frame(w)),
                # HBM bytes per launch from the counters, for context (this
                # kernel's bound is its arithmetic)
                "traffic": counter_traffic(w.name), "algorithmic_bytes_per_launch": w.essential_bytes(),
                "kernel": main_kernel_name(w, fft_variant), "kernel_ms": round(kernel_ms, 5)}
    gbs = w.essential_bytes() / (kernel_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": counter_traffic(w.name),
            "algorithmic_bytes_per_launch": w.essential_bytes(),
            "kernel": main_kernel_name(w, fft_variant), "kernel_ms": round(kernel_ms, 5)}


def clock_ramp(dev, ms: float, kind: str = "copy") -> dict:
    """Bring the GPU to its sustained clocks before anything is timed, with
    work unrelated to the transform (none of its data, and the caches end up
    holding other data) until `ms` of device time have passed: plain 256 MB
    device-to-device copies ("copy") or fp32 4096 x 4096 matrix products
    ("gemm").  The warm-up steps and the timed steps follow unchanged."""
    import torch
    if ms <= 0:
        return {"ms": 0.0, "ops": 0, "kind": kind}
    if kind == "gemm":
        a = torch.randn(4096, 4096, device=dev)
        b = torch.randn(4096, 4096, device=dev)
        op = lambda: torch.mm(a, b)   # noqa: E731
    else:
        a = torch.empty(1 << 26, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        op = lambda: b.copy_(a)   # noqa: E731
    n, spent = 0, 0.0
    while spent < ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(8):
            op()
        e1.record()
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
        n += 8
    del a, b
    return {"ms": round(spent, 1), "ops": n, "kind": kind}


def floored_share(w, got):
    """How much of an output the per-clip floor decided: the share of values
    at the clip's floor (the largest output minus 2, i.e. log10 at hi - 8)
    and, where the main kernel's statistics regions are known (n_fft 400:
    16 frames x 4 bands; n_fft >= 8192: one frame x all bands), the share of
    regions holding such a value -- the regions the clamp fix-up rewrites
    (its gate, on region minima with a small slack, may take a few more)."""
    import numpy as np
    tol = 2e-3 if w.out_dtype == "f16" else 1e-6
    g = got.astype(np.float32)
    hi = g.reshape(g.shape[0], -1).max(axis=1)
    at = g <= (hi - 2.0 + tol)[:, None, None]
    res = {"values_at_floor": round(float(at.mean()), 7)}
    if w.entry == "pcm" and (w.n_fft == 400 or w.n_fft >= 8192):
        fr, bd = (16, 4) if w.n_fft == 400 else (1, at.shape[1])
        B, NM, F = at.shape
        nf, nb = -(-F // fr), -(-NM // bd)
        pad = np.zeros((B, nb * bd, nf * fr), dtype=bool)
        pad[:, :NM, :F] = at
        reg = pad.reshape(B, nb, bd, nf, fr).any(axis=(2, 4))
        res["regions"] = int(reg.size)
        res["region_shape"] = f"{fr} frames x {bd} bands"
        res["regions_holding_floored_values"] = round(float(reg.mean()), 7)
    return res


def torch_eager(run, steps, got, last):
    """Context only: the same chain composed from PyTorch's own GPU
    operators (torch.stft, squared magnitude, matmul, log10, amax, clamp)
    on the same GPU and the same resident inputs, with the library plan's
    filterbank; timed with events like the library's steps.  Returns its
    ms per step and its largest difference from `got`, the library's output
    of step `last`."""
    import numpy as np
    import torch
    w, dev = run.w, run.ins[0].device
    if w.entry == "pcm":
        fb = torch.from_numpy(run.plan.get_filters()).to(dev)               # (n_mels, n_fft/2 + 1)
        win = torch.hann_window(w.n_fft, periodic=True, dtype=torch.float32, device=dev)
        scale = 1.0 / 32768.0 if w.in_dtype == "i16" else 1.0

        def chain(i):
            x = run.ins[i % run.nbuf].to(torch.float32) * scale
            S = torch.stft(x, w.n_fft, hop_length=w.hop, window=win, center=w.center, pad_mode=w.pad_mode,
                           return_complex=True)
            P = (S.real.square() + S.imag.square()).contiguous()            # (B, NF, F)
            L = torch.log10(torch.clamp(torch.matmul(fb, P), min=1e-10))    # (B, n_mels, F)
            hi = L.amax(dim=(1, 2), keepdim=True)
            return (torch.maximum(L, hi - 8.0) + 4.0) / 4.0
    else:
        fb = run.filt.t().contiguous()                                      # (NF, NM)

        def chain(i):
            S = run.ins[i % run.nbuf]
            P = (S.real.square() + S.imag.square()).contiguous()            # (B, F, NF)
            L = torch.log10(torch.clamp(torch.matmul(P, fb), min=1e-10))    # (B, F, NM)
            hi = L.amax(dim=(1, 2), keepdim=True)
            return (torch.maximum(L, hi - 8.0) + 4.0) / 4.0
    n = max(1, min(steps, 50))
    for i in range(3):
        o = chain(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        o = chain(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    o = chain(last).cpu().numpy()   # the input buffer set that step read
    diff = float(np.abs(o.astype(np.float64) - got.astype(np.float64)).max())
    del o
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 5), "steps": n, "max_abs_diff_vs_library": diff,
            "what": "torch.stft + squared magnitude + torch.matmul with the plan's filterbank + log10 / amax / "
                    "clamp, PyTorch's own GPU operators (fp32), same GPU and resident inputs; context only"}


def per_config_entry(name, steps, warmup, dev, check_clips, ramp_ms, ramp_kind):
    """Time one of the other workloads and check a few of its clips."""
    import numpy as np
    import torch

    import lm_synth
    w = lm_synth.WORKLOADS[name]
    r = Run(w, dev, log=False)
    torch.cuda.synchronize()
    clock_ramp(dev, ramp_ms, ramp_kind)
    t = r.time(steps, warmup)
    got = r.last_output(steps).float().cpu().numpy()
    eager = torch_eager(r, steps, got, steps - 1)
    errs = [float(np.abs(got[b].astype(np.float64) - r.oracle_clip(b)).max()) for b in range(min(w.B, check_clips))]
    frames = w.B * w.n_frames
    entry = {
        "workload": w.name, "entry": f"lm_from_{w.entry}", "shape_in": list(r.host_in.shape),
        "shape_out": list(w.out_shape), "out": w.out_dtype, "dtype": first_stage_dtype(w, "auto"),
        "ms_per_step": round(t["ms_per_step"], 5),
        "ms_per_step_p10_p50_p90": [round(t["p10"], 5), round(t["p50"], 5), round(t["p90"], 5)],
        "frames_per_s": round(frames / (t["ms_per_step"] / 1e3), 1),
        "main_kernel_us": round(t["kernel_ms"]["main"] * 1e3, 2),
        "fixup_us": round(t["kernel_ms"]["fixup"] * 1e3, 2), "pack_us": round(t["kernel_ms"]["pack"] * 1e3, 2),
        "hbm_gbs_step": round(w.essential_bytes() / (t["ms_per_step"] / 1e3) / 1e9, 1),
        "roofline": roofline_of(w, t["kernel_ms"]["main"]),
        "parity": {"clips_checked": len(errs), "max_abs_err": max(errs),
                   "tol": 2e-3 if w.out_dtype == "f16" else 1e-4},
        "floor": floored_share(w, got),
        "torch_eager": {**eager, "library_speedup": round(eager["ms_per_step"] / t["ms_per_step"], 2)},
    }
    del r
    return entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU raises its clocks over the first ~30 ms of sustained work (see
    # --ramp): the default warm-up covers that, so the timed steps measure the
    # sustained rate
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="pcm_i16_b64")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-per-config", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-torch", action="store_true",
                    help="skip the PyTorch-operator composition of the same chain (context only)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--fft-variant", default="auto", choices=["auto", "split_mfma", "folded", "paired"],
                    help="n_fft = 400 transform (comparison only; auto is the library's choice)")
    ap.add_argument("--single-pass", action="store_true",
                    help="use the one-launch (cooperative) form of the per-clip floor where it applies")
    ap.add_argument("--sweep", action="store_true",
                    help="time every n_fft of the sweep workloads (one JSON line each, no CPU leg)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (5 times), to scale HBM counters")
    ap.add_argument("--clock-ramp-kind", default="gemm", choices=["copy", "gemm"])
    ap.add_argument("--clock-ramp-ms", type=float, default=500.0,
                    help="device time of unrelated work before each workload's warm-up steps, so that "
                         "short runs (few warm-up steps) are timed at the sustained clocks; 0 turns it off")
    ap.add_argument("--ramp", action="store_true",
                    help="print the step time of every workload in consecutive chunks from an idle GPU "
                         "(how long the clocks take to settle), then exit")
    ap.add_argument("--dft-gemm", action="store_true",
                    help="FFT-variant comparison: time the n_fft = 400 transform of the default workload "
                         "as one dense fp32 GEMM on the vendor BLAS (torch.matmul), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (clips shard across "
              "GPUs with no communication; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 28                                   # 2^28 floats = 1 GiB read + 1 GiB written
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_copy": 4 * n, "bytes_written_per_copy": 4 * n,
                                               "copies": 5}}), flush=True)
        return

    import lm_synth

    if args.dft_gemm:
        dft_gemm_probe(lm_synth.WORKLOADS["pcm_i16_b64"], args.steps, args.warmup)
        return

    if args.ramp:
        for name in ("pcm_i16_b64",) + PER_CONFIG:
            ramp_one(lm_synth.WORKLOADS[name], torch.device("cuda:0"))
        return

    if args.sweep:
        for n in lm_synth.SWEEP_SIZES:
            sweep_one(lm_synth.WORKLOADS[f"sweep_nfft{n}"], args.steps, args.warmup)
        return

    w = lm_synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    run = Run(w, dev, args.fft_variant, args.single_pass)
    torch.cuda.synchronize()
    ramp = clock_ramp(dev, args.clock_ramp_ms, args.clock_ramp_kind)
    t = run.time(args.steps, args.warmup)
    ms_per_step = t["ms_per_step"]
    main_ms, fix_ms, pack_ms = t["kernel_ms"]["main"], t["kernel_ms"]["fixup"], t["kernel_ms"]["pack"]
    per_step_bytes = w.essential_bytes()
    frames = w.B * w.n_frames
    value = frames / (ms_per_step / 1e3)
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step (wall {t['wall_s']:.3f}s), "
          f"main kernel {main_ms:.4f} ms, fixup {fix_ms:.4f} ms, pack {pack_ms:.4f} ms", file=sys.stderr, flush=True)
    got = run.last_output(args.steps).float().cpu().numpy()
    eager = None
    if not args.no_torch:
        eager = torch_eager(run, args.steps, got, args.steps - 1)
        print(f"[bench] PyTorch operators, same chain: {eager['ms_per_step']:.4f} ms/step", file=sys.stderr,
              flush=True)

    # the same batch through the all-fp32 folded transform (n_fft = 400 only):
    # the error the two-part fp16 first stage adds is read against it below
    got_fp32 = None
    if w.entry == "pcm" and main_kernel_name(w, args.fft_variant) == "pcm400_kernel" and not args.no_cpu:
        plan32 = __import__("stft_log_mel_amd").Plan(w.n_fft, w.hop, w.n_mels, w.center, w.pad_mode, w.power,
                                                      w.out_dtype)
        plan32.set_mel(w.sample_rate, w.f_min, w.f_max).set_fft_variant("folded")
        got_fp32 = plan32.from_pcm(run.ins[0]).float().cpu().numpy()
        del plan32

    # context: this GPU's streaming-copy rate (2 GiB read + 2 GiB written)
    cbuf = torch.empty(1 << 29, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(cbuf)
    cdst.copy_(cbuf)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(run.stream)
    for _ in range(5):
        cdst.copy_(cbuf)
    ev1.record(run.stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * cbuf.numel() * 4 / (ev0.elapsed_time(ev1) / 1e3) / 1e9
    del cbuf, cdst

    per_config = None
    if not args.no_per_config and args.workload == "pcm_i16_b64":
        per_config = {}
        for name in PER_CONFIG:
            print(f"[bench] per-config {name}", file=sys.stderr, flush=True)
            per_config[name] = per_config_entry(name, args.steps, args.warmup, dev,
                                                check_clips=1 if name != "stft_b256" else 2,
                                                ramp_ms=args.clock_ramp_ms, ramp_kind=args.clock_ramp_kind)
            torch.cuda.empty_cache()

    # the fp64 oracle on this host's cores, clips in order, cycling through the
    # batch again until about cpu_seconds have passed; each clip's first pass is
    # also a parity check of the timed output (and of the all-fp32 path's)
    parity = cpu = parity32 = None
    if not args.no_cpu:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        t_cpu = time.perf_counter()
        done = 0
        errs, errs32 = [], []
        sq_err = sq_ref = 0.0
        while True:
            ref = run.oracle_clip(done % w.B)
            if done < w.B:
                d = got[done].astype(np.float64) - ref
                errs.append(float(np.abs(d).max()))
                sq_err += float((d * d).sum())
                sq_ref += float((ref * ref).sum())
                if got_fp32 is not None:
                    errs32.append(float(np.abs(got_fp32[done].astype(np.float64) - ref).max()))
            done += 1
            if time.perf_counter() - t_cpu >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t_cpu
        cpu = {"value": round(done * w.n_frames / dt, 1), "unit": "frames/s",
               "cores": len(os.sched_getaffinity(0)), "blas_threads": int(blas_threads), "kind": "oracle",
               "sample": f"{done} clips ({done * w.n_frames} frames) of the same workload, taken in order "
                         f"and cycling through its {w.B} clips, fp64 numpy oracle, {dt:.1f}s"}
        parity = {"clips_checked": len(errs), "max_abs_err": max(errs),
                  "rel_frobenius": (sq_err / sq_ref) ** 0.5 if sq_ref > 0 else 0.0,
                  "tol": 2e-3 if w.out_dtype == "f16" else 1e-4}
        if errs32:
            parity32 = {"clips_checked": len(errs32), "max_abs_err": max(errs32),
                        "path": "folded 200-point transform, all fp32 (lm_plan_set_fft_variant LM_FFT_FOLDED)",
                        "tol": 1e-4}
        print(f"[bench] oracle: {done} clips in {dt:.1f}s, max |err| {max(errs):.2e}", file=sys.stderr,
              flush=True)

    fpf = flops_per_frame(w)
    line = {
        "metric": "log-mel frames/sec (B=64x30 s, n_fft=400, 128 mels) + HBM GB/s % of peak",
        "value": round(value, 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp": {"device_ms": ramp["ms"], "what": f"{ramp['ops']} {ramp['kind']} operations unrelated to the "
                       "transform before the warm-up steps of each workload (clocks to their sustained level)"},
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_p10_p50_p90": [round(t["p10"], 5), round(t["p50"], 5), round(t["p90"], 5)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": first_stage_dtype(w, args.fft_variant),
        "data": "synthetic (seeded speech-like int16 PCM)" if w.entry == "pcm" else "synthetic (seeded STFT)",
        "config": {
            "workload": w.name, "entry": f"lm_from_{w.entry}", "B": w.B,
            **({"T": w.T, "sample_rate": w.sample_rate, "n_fft": w.n_fft, "hop": w.hop, "n_mels": w.n_mels,
                "center": w.center, "pad_mode": w.pad_mode, "power": w.power, "in": w.in_dtype,
                "mel": "slaney/slaney-norm", "f_min": w.f_min, "f_max": w.f_max,
                "fft_variant": args.fft_variant, "single_pass": bool(args.single_pass)}
               if w.entry == "pcm" else {"F": w.F, "NF": w.NF, "NM": w.NM, "in": "complex64",
                                         "filters": "linear triangles (fp32)"}),
            "out": w.out_dtype, "frames_per_step": frames, "essential_bytes_per_step": per_step_bytes,
            "buffer_sets": run.nbuf,
        },
        "hbm_gbs_step": round(per_step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "hbm_frac_step": round(per_step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roofline_of(w, main_ms, args.fft_variant),
        "alu_context": {
            "nominal_flop_per_frame": round(fpf, 1),
            "tflops": round(frames * fpf / (main_ms / 1e3) / 1e12, 2),
            "fp32_vector_peak_tflops": FP32_VALU_PEAK_TFLOPS,
            "fp32_vector_unpacked_peak_tflops": FP32_VALU_PEAK_TFLOPS / 2,
        },
        "copy_context": {"copy_gbs": round(copy_gbs, 1),
                         "main_kernel_frac_of_copy": round(per_step_bytes / (main_ms / 1e3) / 1e9 / copy_gbs, 4),
                         "note": "torch copy_ of 2 GiB device to device, read + write bytes per second"},
        "fixup_ms": round(fix_ms, 5),
        "floor": floored_share(w, got),
        "torch_eager": ({**eager, "library_speedup": round(eager["ms_per_step"] / ms_per_step, 2)}
                        if eager else None),
        "pack_ms": round(pack_ms, 5),
        "cpu_baseline": cpu,
        "parity": parity,
        "parity_fp32_path": parity32,
        "per_config": per_config,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
