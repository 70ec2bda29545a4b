"""Benchmark of the batched causal long convolution on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 3] [--no-cpu-baseline]

One step = one call of the library's hot path over one batch of synthetic input (for the
default workload, sc_causal_conv_bf16 at B=8, C=1024, L=4096: load v and g, pad-to-2L FFT,
spectral product, inverse FFT, truncation, direct head, store r -- a single kernel).
After the timed region, the gradient call of the same workload (dv, dg from dr, v, g) is
timed the same way and reported in the `bwd` object (skip with --no-bwd); the exactly
causal real-valued call on the same inputs in the `fixed` object and at the long-context
shape (B=1, C=1536, L=65536) in `fixed_long` (skip both with --no-fixed); the pages' own
pipeline (torch.fft rfft, product, irfft; context only, not a target) in `pages_approach`
(skip with --no-pages-approach); the calls for a filter shared by the batch on the same
shape in the `shared` object (skip with --no-shared); the token-major (B, L, C) call on the
same inputs in the `token_major` object (skip with --no-blc); and the gate-stream calls (g
from the gate pre-activation on MFMA, alone and as the mixing step's prologue) in the
`gate` object (skip with --no-gate).
Inputs are resident in HBM before the timed region.  Several copies of the buffers are
rotated so that the 256 MB last-level cache cannot hold a step's working set.  Before the W
warmup steps, untimed launches of the same step run for --prewarm-ms (default 200 ms; the
`prewarm` object says how many): from idle the chip's clock ramps for about 30 ms, and W = 5
steps alone would put the timed steps on that ramp.  Every other timed call gets the same
pre-warm before its own timing.

Prints ONE JSON line.  `value` is causal-conv outputs (B*C*L) per second.  The
`roofline` object refers to the dominant kernel, timed with HIP events recorded on the
stream the kernel runs on; `cpu_baseline` is the float64 CPU oracle timed on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, AMD published (packed dual-fp32 FMA)
# What code built without packed fp32 (as this library is) can issue: 256 CUs x 4 SIMDs x
# 16 lanes x 2 flops per FMA x 2.4 GHz.  Add-heavy code (FFT butterflies) stays below it.
FP32_FMA_PEAK_UNPACKED_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
CACHE_BYTES = 256 << 20          # MI355X last-level (Infinity) cache


PREWARM_MS = 200.0   # set from --prewarm-ms


def prewarm(torch, fn) -> int:
    """Untimed calls of fn back to back for PREWARM_MS of wall time: from idle the chip's
    clock ramps for about 30 ms under load (the Medium call measured 0.191 ms at first,
    0.154 ms steady from about its 200th launch on), so a measurement that starts cold times
    the ramp.  Returns the number of calls."""
    calls = 0
    if PREWARM_MS <= 0:
        return 0
    t_end = time.perf_counter() + PREWARM_MS * 1e-3
    while time.perf_counter() < t_end:
        for i in range(16):
            fn(i)
        torch.cuda.synchronize()
        calls += 16
    return calls


def time_rounds(torch, stream, fn, n: int, rounds: int = 5, warm: bool = True):
    """Mean milliseconds per call of fn(i), i < n, launched back to back on `stream`, with
    HIP events recorded on that stream only at the boundaries of `rounds` equal rounds (an
    event between every two launches would add its own gap to each), after prewarm() unless
    warm is False.  Returns (mean over all calls, [mean per call of each round])."""
    if warm:
        prewarm(torch, fn)
    rounds = max(1, min(rounds, n))
    bounds = [round(r * n / rounds) for r in range(rounds + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(rounds + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for r in range(rounds):
        for i in range(bounds[r], bounds[r + 1]):
            fn(i)
        evs[r + 1].record(stream)
    torch.cuda.synchronize()
    per_round = [evs[r].elapsed_time(evs[r + 1]) / (bounds[r + 1] - bounds[r])
                 for r in range(rounds)]
    return evs[0].elapsed_time(evs[rounds]) / n, per_round


def launch_stats(torch, stream, fn, n: int, offset: int = 0) -> dict:
    """Per-launch durations of n calls fn(offset + i): an event pair on `stream` around each
    launch, all launches queued back to back before one synchronisation.  Returns the median,
    p10 and p90 in milliseconds."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(offset + i)
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    return {"n": n, "median": round(float(np.median(ms)), 5),
            "p10": round(float(np.percentile(ms, 10)), 5),
            "p90": round(float(np.percentile(ms, 90)), 5),
            "method": "an event pair on the launch stream around each launch, launches queued "
                      "back to back"}


def algorithmic_flops_per_output(L: int) -> float:
    """Real flops per output of the pad-2L FFT method with real-pair packing, the pruned
    first forward stage and the half-length real inverse: (12.75 log2 L + 28)."""
    return 12.75 * np.log2(L) + 28.0


def kernel_source_hash() -> str:
    """Hash of the kernel sources and of the build script (its per-file compiler options
    change the code a counter record describes)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "fft_causal_long_amd", "csrc", "*"))) + \
            [os.path.join(ROOT, "fft_causal_long_amd", "build.py")]:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 30   # the --calib-copy transfer: 2^28 float32 read and written


def kernel_matches(name: str, storage: str, L: int, rev: bool = False) -> bool:
    """Is this profiled kernel part of the timed hot path of the workload (the forward call,
    or with rev the gradient call)?  Exact template, so launches of the leakage probe, of
    other shapes or of the other direction do not count."""
    M = max(64, 1 << (L - 1).bit_length())
    flag = "true" if rev else "false"
    if storage == "i32":
        if L > 4096:
            # the four-step NTT modulo prime A: columns and inverse columns (per direction),
            # rows (shared by both directions)
            m1 = M // 4096
            return ("ntt4_rows<sc::ntt::PrimeA>" in name
                    or ("ntt4_columns_fwd<%d, %s, sc::ntt::PrimeA, false>" % (m1, flag)) in name
                    or ("ntt4_columns_inv<%d, %s>" % (m1, flag)) in name)
        return ("ntt_conv_kernel<%d, %s>" % (M, flag)) in name
    if L > 4096:
        return "fs_rows<" in name or (("fs_columns" in name or "head_kernel" in name)
                                      and (", %s>" % flag) in name)
    io = "bf16_io" if storage == "bf16" else "f32_io"
    if M == 4096:
        # the default form (the last template argument selects the matrix-core first pass)
        return ("fused4k_kernel<sc::%s, %s, false>" % (io, flag)) in name
    if M in (1024, 2048):
        return ("fused_dit_kernel<%d, sc::%s, %s>" % (M, io, flag)) in name
    return ("fused_conv_kernel<%d, sc::%s, %s>" % (M, io, flag)) in name


def four_step_calls(w, markers: int, where: str) -> float:
    """Calls of the four-step path in a counter run, from its count of marker dispatches:
    the call is several kernels (columns, rows, columns per part of the channels, then for
    the float kinds the head); one head kernel per float call, and the exact kind's
    inverse-column kernel once per part of channels (half a chunk when the call runs its
    chunks as halves on two streams: at least two channels per chunk and more than half a
    chunk of channels)."""
    if not markers:
        raise RuntimeError("%s: no dispatch to count four-step calls" % where)
    if w.storage != "i32":
        return float(markers)
    import fft_causal_long_amd as sc
    M = 1 << (w.L - 1).bit_length()
    chunk = sc.sc_workspace_bytes(sc.KIND_NTT_I32, w.B, w.C, w.L) // (24 * M)
    part = chunk // 2 if chunk >= 2 and w.channels > chunk // 2 else chunk
    return markers / -(-w.channels // part)


def four_step_marker(w) -> str:
    return "head_kernel" if w.storage != "i32" else "ntt4_columns_inv"


def record_traffic(w, fetch_dir: str, write_dir: str) -> dict:
    """Turn two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch, both run
    with --calib-copy) into HBM bytes per launch of the hot path.  Each counter is scaled
    by (known copy bytes) / (what it reads for the 1 GiB copy)."""
    import csv

    def per_dispatch(d, counter):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        hot, copy, calls = {}, [], set()
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            val = float(r["Counter_Value"])
            if "copyBuffer" in r["Kernel_Name"]:
                copy.append(val)
            elif kernel_matches(r["Kernel_Name"], w.storage, w.L):
                hot[r["Dispatch_Id"]] = hot.get(r["Dispatch_Id"], 0.0) + val
                if four_step_marker(w) in r["Kernel_Name"]:
                    calls.add(r["Dispatch_Id"])
        if not hot or len(copy) != 1:
            raise RuntimeError("%s: expected hot-path dispatches and one calibration copy" % d)
        scale = COPY_BYTES / (copy[0] * 1024.0)
        if w.L > 4096:
            return float(sum(hot.values())) / four_step_calls(w, len(calls), d) * 1024.0 * scale, \
                scale
        return float(np.mean(list(hot.values()))) * 1024.0 * scale, scale

    fetch, fs = per_dispatch(fetch_dir, "FETCH_SIZE")
    write, ws = per_dispatch(write_dir, "WRITE_SIZE")
    rec = {"workload": w.name, "source_hash": kernel_source_hash(),
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
           "bytes_per_launch": round(fetch + write), "fetch_scale": fs, "write_scale": ws,
           "algorithmic_bytes_per_launch": 3 * w.outputs * (2 if w.storage == "bf16" else 4)}
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % w.name)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def record_valu(w, sq_dir: str) -> dict:
    """From a rocprofv3 counter run with SQ_INSTS_VALU (summed over the chip, per dispatch),
    the VALU instructions one launch of the hot kernel issues; for the four-step path (several
    kernels per call), the instructions of one whole call."""
    import csv
    per, calls = {}, set()
    for r in csv.DictReader(open(os.path.join(sq_dir, "run_counter_collection.csv"))):
        if r["Counter_Name"] == "SQ_INSTS_VALU" and kernel_matches(r["Kernel_Name"], w.storage, w.L):
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
            if four_step_marker(w) in r["Kernel_Name"]:
                calls.add(r["Dispatch_Id"])
    if not per:
        raise RuntimeError("%s: no SQ_INSTS_VALU rows for the hot kernel" % sq_dir)
    if w.L > 4096:
        valu = float(sum(per.values())) / four_step_calls(w, len(calls), sq_dir)
    else:
        valu = float(np.mean(list(per.values())))
    rec = {"workload": w.name, "source_hash": kernel_source_hash(),
           "valu_instructions_per_launch": round(valu), "dispatches": len(per)}
    path = os.path.join(ROOT, "profiles", "valu_%s.json" % w.name)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def alu_issue(workload: str, kernel_ms: float):
    """The VALU issue floor of the hot kernel: its VALU instructions per launch (committed
    counter run on the current sources, else None) x 4 cycles per wave instruction over the
    1024 SIMDs at the nominal 2.4 GHz, against the live kernel time."""
    path = os.path.join(ROOT, "profiles", "valu_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    floor_us = rec["valu_instructions_per_launch"] * 4 / 1024 / 2.4e9 * 1e6
    return {"valu_instructions_per_launch": rec["valu_instructions_per_launch"],
            "issue_floor_us_at_2.4GHz": round(floor_us, 1), "kernel_us": round(kernel_ms * 1e3, 1),
            "frac": round(floor_us / (kernel_ms * 1e3), 4),
            "source": "profiles/valu_%s.json (rocprofv3 SQ_INSTS_VALU)" % workload}


FIXED_FRAC = 24   # fraction bits of both encodings in the exact real-valued measurements


def leakage_probe(sc, torch, dev, channels: int = 16) -> dict:
    """Future-token leakage max_{t<s} |r'_t - r_t| of the float path (fp32, L = 4096,
    Medium-shaped inputs), of the exact real-valued path on the same inputs, and of the
    exact integer path (L = 4096, integer inputs): v_s is changed at 8 seeded positions s,
    the original and the perturbed rows run in one launch."""
    from workloads import WORKLOADS, bf16_bits_to_f32, make_inputs, perturbation_positions

    def probe(v, g, pos, change, conv=None):
        conv = conv or sc.causal_conv
        rows = [v] + [change(v.copy(), s) for s in pos]
        vv = np.concatenate(rows, axis=0)
        gg = np.concatenate([g] * len(rows), axis=0)
        out = conv(torch.from_numpy(vv).to(dev), torch.from_numpy(gg).to(dev))
        r = out.cpu().numpy().astype(np.float64)
        leak = 0.0
        for i, s in enumerate(pos):
            if s > 0:
                leak = max(leak, float(np.abs(r[i + 1, :, :s] - r[0, :, :s]).max()))
        return leak, float(np.sqrt(np.mean(r[0] ** 2)))

    w3 = WORKLOADS[3]
    v, g = make_inputs(w3, B=1, C=channels)
    v, g = bf16_bits_to_f32(v), bf16_bits_to_f32(g)
    pos = perturbation_positions(w3.cid, w3.L)

    def bump(a, s):
        a[:, :, s] += 1.0
        return a
    f_leak, f_rms = probe(v, g, pos, bump)
    x_leak, _ = probe(v, g, pos, bump,
                      lambda a, b: sc.causal_conv_fixed(a, b, FIXED_FRAC, FIXED_FRAC))

    w5 = WORKLOADS[5]
    vi, gi = make_inputs(w5, B=1, C=channels)
    posi = perturbation_positions(w5.cid, w5.L)

    def swap(a, s):
        a[:, :, s] = np.where(a[:, :, s] >= 0, a[:, :, s] - 100, a[:, :, s] + 100)
        return a
    n_leak, _ = probe(vi, gi, posi, swap)
    return {"fp32_max_abs": f_leak, "fp32_rel_to_rms": f_leak / f_rms, "ntt_max_abs": n_leak,
            "fixed_max_abs": x_leak, "positions": len(pos), "channels": channels, "L": w3.L}


def copy_reference(torch, dev) -> dict:
    """The achievable HBM rate of a plain read-2 / write-1 stream on this machine: torch's
    elementwise c = a + b on 256 MiB float32 tensors (3 x 256 MiB per call, past the
    last-level cache with two rotating sets), best of five rounds of 10 calls."""
    n = 1 << 26
    sets = [[torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0) for _ in range(3)]
            for _ in range(2)]
    stream = torch.cuda.current_stream(dev)

    def call(i):
        a, b, c = sets[i % 2]
        torch.add(a, b, out=c)

    for i in range(10):
        call(i)
    best = min(time_rounds(torch, stream, call, 10, rounds=1, warm=False)[0] for _ in range(5))
    gbps = 3 * n * 4 / (best * 1e-3) / 1e9
    del sets
    return {"what": "torch.add(a, b, out=c), float32, 256 MiB each (read 2, write 1)",
            "ms_per_call": round(best, 5), "achieved_GBps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def fused_mfma_measure(sc, torch, stream, step, bufs, w, steps: int) -> dict:
    """The same call with SC_PATH_FUSED_MFMA (the first pass of both branch transforms as bf16
    matrix products), timed in three rounds alternating with rounds of the default call on
    the same buffers, so that both see the same clock."""
    import ctypes
    fn = sc.lib().sc_causal_conv_ex
    opt = sc.sc_options(sc.PATH_FUSED_MFMA, -1)
    sptr = stream.cuda_stream
    nsets = len(bufs)

    def call(i):
        a, b, c = bufs[i % nsets]
        st = fn(sc.KIND_BF16, a.data_ptr(), b.data_ptr(), c.data_ptr(), w.B, w.C, w.L,
                ctypes.byref(opt), None, 0, sptr)
        if st != 0:
            raise RuntimeError("sc_causal_conv_ex (fused mfma) failed: %s" % sc.sc_status_string(st))

    prewarm(torch, call)
    mf, base = [], []
    for _ in range(3):
        mf.append(time_rounds(torch, stream, call, steps, rounds=1, warm=False)[0])
        base.append(time_rounds(torch, stream, step, steps, rounds=1, warm=False)[0])
    return {"entry": "sc_causal_conv_ex, path SC_PATH_FUSED_MFMA",
            "what": "first radix-16 pass of both branch transforms as bf16 matrix products "
                    "(v_mfma_f32_32x32x16_bf16, three-part bf16 DFT matrix); not the default",
            "ms_per_call": round(min(mf), 5), "fused_ms": round(min(base), 5),
            "ratio_to_fused": round(min(mf) / min(base), 4),
            "rounds_ms": {"mfma": [round(x, 5) for x in mf], "fused": [round(x, 5) for x in base]},
            "method": "best of three rounds of K calls each, alternating with the default call"}


def pages_approach(torch, w, dev, steps: int, kernel_ms: float) -> dict:
    """For context only, not a target: the pages' own pipeline on this hardware -- standard
    FFT operators ("Caracal", background), here torch.fft on ROCm: rfft of v and g
    zero-padded to 2L, the spectral product, irfft, the first L values -- in float32 on the
    workload's inputs widened to float32 (torch has no bfloat16 FFT)."""
    from workloads import bf16_bits_to_f32, make_inputs
    v, g = make_inputs(w)
    if w.storage == "bf16":
        v, g = bf16_bits_to_f32(v), bf16_bits_to_f32(g)
    tv, tg = torch.from_numpy(v).to(dev), torch.from_numpy(g).to(dev)
    n = 2 * w.L
    stream = torch.cuda.current_stream(dev)

    def call(i):
        spec = torch.fft.rfft(tv, n=n) * torch.fft.rfft(tg, n=n)
        return torch.fft.irfft(spec, n=n)[..., :w.L]

    for _ in range(2):
        call(0)
    ms, _ = time_rounds(torch, stream, call, steps)
    return {"what": "torch.fft rfft(v, 2L) * rfft(g, 2L) -> irfft -> first L, float32; the "
                    "pages' approach on this hardware, context only",
            "ms_per_call": round(ms, 5), "value": round(w.outputs / (ms * 1e-3), 1),
            "unit": "outputs/s", "this_library_speedup": round(ms / kernel_ms, 2)}


def fixed_measure(sc, torch, w, dev, steps: int, warmup: int) -> dict:
    """Time the exactly causal real-valued call (sc_causal_conv_fixed_f32, fraction bits
    FIXED_FRAC for v and g) on the workload's inputs widened to float32: up to L = 4096 one
    kernel with no scratch, beyond that the four-step split per prime with a caller
    workspace (sc_causal_conv_fixed_f32_ws).  Algorithmic bytes per output: read v, g and
    write r as float32 (12)."""
    from workloads import bf16_bits_to_f32, make_inputs
    v, g = make_inputs(w)
    if w.storage == "bf16":
        v, g = bf16_bits_to_f32(v), bf16_bits_to_f32(g)
    if not sc.sc_fixed_range_ok(float(np.abs(v).max()), float(np.abs(g).max()), FIXED_FRAC,
                                FIXED_FRAC, w.L):
        raise RuntimeError("fixed-point range check failed for %s" % w.name)
    tv, tg = torch.from_numpy(v).to(dev), torch.from_numpy(g).to(dev)
    out = torch.empty_like(tv)
    need = sc.sc_workspace_bytes(sc.KIND_FIXED_F32, w.B, w.C, w.L)
    if (need != 0) != (w.L > 4096):
        raise RuntimeError("unexpected scratch size %d for %s" % (need, w.name))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    fn = sc.lib().sc_causal_conv_fixed_f32_ws
    entry = "sc_causal_conv_fixed_f32_ws" if need else "sc_causal_conv_fixed_f32"

    def call():
        st = fn(tv.data_ptr(), tg.data_ptr(), out.data_ptr(), w.B, w.C, w.L, FIXED_FRAC,
                FIXED_FRAC, ws.data_ptr() if need else None, need, stream.cuda_stream)
        if st != 0:
            raise RuntimeError("%s failed: %s" % (entry, sc.sc_status_string(st)))

    for _ in range(warmup):
        call()
    ms, _ = time_rounds(torch, stream, lambda i: call(), steps)
    gbps = 12 * w.outputs / (ms * 1e-3) / 1e9
    return {"workload": w.name, "entry": entry, "frac_bits": [FIXED_FRAC, FIXED_FRAC],
            "ms_per_call": round(ms, 5), "value": round(w.outputs / (ms * 1e-3), 1),
            "unit": "outputs/s", "hbm": {"algorithmic_bytes_per_call": 12 * w.outputs,
                                         "achieved_GBps": round(gbps, 1),
                                         "frac": round(gbps / HBM_PEAK_GBPS, 4)},
            "scratch_bytes": need}


def oracle_sample_rate(w, v, g, nthreads: int, budget_s: float, start: int = 8):
    """The direct-sum oracle of the workload (float64, or int64 for integer storage) on
    growing channel samples until one takes >= budget_s/2: (channels, seconds)."""
    import oracle
    nch = v.size // w.L
    vv = v.reshape(nch, w.L)
    gg = g.reshape(nch, w.L)
    n = min(start, nch)
    while True:
        t0 = time.perf_counter()
        if w.storage == "i32":
            oracle.causal_conv_i64(vv[:n], gg[:n], nthreads=nthreads)
        else:
            oracle.causal_conv_f64(vv[:n], gg[:n], nthreads=nthreads, with_scale=False)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 2 or n >= nch:
            return n, dt
        n = min(nch, max(2 * n, int(n * (budget_s / 2) / max(dt, 1e-3))))


def cpu_baseline(w, v, g, budget_s: float = 10.0):
    """Time the float64 oracle on growing channel samples until one takes >= budget_s/2,
    on all the host's threads and on one thread."""
    import oracle
    nthreads = oracle.default_threads()
    nch = w.B * w.C
    n, dt = oracle_sample_rate(w, v, g, nthreads, budget_s)
    n1, dt1 = oracle_sample_rate(w, v, g, 1, budget_s / 2, start=1)
    return {
        "value": n * w.L / dt,
        "unit": "outputs/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": "%d of %d channels (L=%d), float64 direct O(L^2) sum on the stored inputs, "
                  "%.2f s wall" % (n, nch, w.L, dt),
        "value_1_thread": n1 * w.L / dt1,
        "sample_1_thread": "%d of %d channels, %.2f s wall on one thread" % (n1, nch, dt1),
    }


def oracle_rate(run, total: int, per_unit: int, what: str, budget_s: float = 3.0) -> dict:
    """Time run(n) (an oracle function on the first n units of a workload) on growing n until
    one call takes >= budget_s / 2; report per_unit * n / time."""
    import oracle
    n = 1
    while True:
        t0 = time.perf_counter()
        run(n)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 2 or n >= total:
            break
        n = min(total, max(2 * n, int(n * (budget_s / 2) / max(dt, 1e-3))))
    return {"value": round(per_unit * n / dt, 1), "cores": oracle.default_threads(),
            "kind": "oracle", "sample": "%d of %d %s, %.2f s wall" % (n, total, what, dt)}


def next_rows_oracles(w, rec: dict) -> None:
    """The oracle of each measured NEXT-row call, timed on a bounded sample of the same
    workload (host cores), beside the GPU figure: gradients, exact real-valued call,
    shared filter (apply and gradients), gate."""
    import oracle
    from workloads import (bf16_bits_to_f32, make_gate_inputs, make_grad, make_inputs,
                           make_shared_filter)
    v, g = make_inputs(w)
    L = w.L
    if "bwd" in rec:
        dr = make_grad(w)
        d2, v2, g2 = dr.reshape(-1, L), v.reshape(-1, L), g.reshape(-1, L)
        f = oracle.causal_conv_bwd_i64 if w.storage == "i32" else \
            (lambda a, b, c: oracle.causal_conv_bwd_f64(a, b, c, with_scale=False))
        rec["bwd"]["cpu_oracle"] = dict(
            oracle_rate(lambda n: f(d2[:n], v2[:n], g2[:n]), d2.shape[0], L, "channels"),
            unit="positions/s")
    if "fixed" in rec:
        vf, gf = v.reshape(-1, L), g.reshape(-1, L)
        if w.storage == "bf16":
            vf, gf = bf16_bits_to_f32(vf), bf16_bits_to_f32(gf)
        rec["fixed"]["cpu_oracle"] = dict(
            oracle_rate(lambda n: oracle.causal_conv_fixed_f32(vf[:n], gf[:n], FIXED_FRAC,
                                                               FIXED_FRAC),
                        vf.shape[0], L, "channels", budget_s=2.0), unit="outputs/s")
    if "shared" in rec:
        k = make_shared_filter(w)
        dr = make_grad(w)

        def apply_(n):
            kb = np.ascontiguousarray(np.broadcast_to(oracle.as_f64(k[:n])[None], (w.B, n, L)))
            oracle.causal_conv_f64(v[:, :n], kb, with_scale=False)
        rec["shared"]["cpu_oracle"] = dict(oracle_rate(apply_, w.C, w.B * L, "channels (all rows)"),
                                           unit="outputs/s")
        rec["shared"]["bwd"]["cpu_oracle"] = dict(
            oracle_rate(lambda n: oracle.shared_conv_bwd_f64(dr[:, :n], v[:, :n], k[:n]), w.C,
                        w.B * L, "channels (all rows)"), unit="positions/s")
    if "gate" in rec:
        _, s_, W = make_gate_inputs(w, B=1)
        rec["gate"]["cpu_oracle"] = dict(
            oracle_rate(lambda n: oracle.gate_f64(s_[:, :64 * n], W[:64 * n]), w.C // 64, 64 * L,
                        "64-channel groups of one batch row"), unit="outputs/s")
    if "token_major" in rec:
        rec["token_major"]["cpu_oracle"] = "the channel-major oracle (cpu_baseline): the same sums"


def bwd_measure(sc, torch, w, dev, steps: int, warmup: int) -> dict:
    """Time the gradient call (dv and dg for one upstream gradient dr) on the same workload:
    inputs dr, v, g resident, buffers rotated like the forward, HIP events around each call
    on the launch stream.  Algorithmic work per position: read dr, v, g and write dv, dg
    (5 elements); two reversed causal convolutions, 2 x (12.75 log2 L + 28) flops."""
    from workloads import make_grad, make_inputs
    kind = {"f32": ("sc_causal_conv_bwd_f32", 4), "bf16": ("sc_causal_conv_bwd_bf16", 2),
            "i32": ("sc_causal_conv_bwd_ntt_i32", 4)}[w.storage]
    fn, esz = getattr(sc.lib(), kind[0]), kind[1]
    v, g = make_inputs(w)
    dr = make_grad(w)
    tdtype = {"f32": torch.float32, "bf16": torch.int16, "i32": torch.int32}[w.storage]
    host = [torch.from_numpy(x.view(np.int16) if w.storage == "bf16" else x) for x in (dr, v, g)]
    set_bytes = 5 * w.outputs * esz
    nsets = max(1, -(-2 * CACHE_BYTES // set_bytes))
    bufs = [[x.to(dev) for x in host] + [torch.empty(w.outputs, dtype=tdtype, device=dev)
                                         for _ in range(2)] for _ in range(nsets)]
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def call(i):
        b = bufs[i % nsets]
        st = fn(*[t.data_ptr() for t in b], w.B, w.C, w.L, sptr)
        if st != 0:
            raise RuntimeError("%s failed: %s" % (kind[0], sc.sc_status_string(st)))

    for i in range(warmup):
        call(i)
    ms, _ = time_rounds(torch, stream, call, steps)
    alg_bytes = 5 * w.outputs * esz
    gbps = alg_bytes / (ms * 1e-3) / 1e9
    rec = {"entry": kind[0], "ms_per_call": round(ms, 5),
           "value": round(w.outputs / (ms * 1e-3), 1), "unit": "positions/s",
           "buffer_sets": nsets,
           "hbm": {"algorithmic_bytes_per_call": alg_bytes, "achieved_GBps": round(gbps, 1),
                   "frac": round(gbps / HBM_PEAK_GBPS, 4)}}
    if w.storage != "i32":
        tf = 2 * algorithmic_flops_per_output(w.L) * w.outputs / (ms * 1e-3) / 1e12
        rec["alu"] = {"achieved_TFLOPs": round(tf, 2), "peak": FP32_FMA_PEAK_UNPACKED_TFLOPS,
                      "frac": round(tf / FP32_FMA_PEAK_UNPACKED_TFLOPS, 4),
                      "frac_of_published_157.3": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4)}
    del bufs
    return rec


def shared_measure(sc, torch, w, dev, steps: int, warmup: int) -> dict:
    """Time the filter-shared-by-the-batch calls on the workload's shape: the apply call
    sc_causal_conv_spec_* (v and the filter spectrum resident, buffers rotated like the
    forward), the spectrum call sc_filter_spectrum_*, and the gradient call
    sc_causal_conv_spec_bwd_* (dv and dk).  Algorithmic bytes per output: read v, write r
    (2 elements; the spectrum is per channel, not per output); for the gradients read dr and
    v, write dv (3 elements; dk is per channel)."""
    from workloads import make_grad, make_inputs, make_shared_filter
    bf = w.storage == "bf16"
    esz = 2 if bf else 4
    kname = "bf16" if bf else "f32"
    v, _ = make_inputs(w)
    k = make_shared_filter(w)
    to = (lambda a: torch.from_numpy(a.view(np.int16)).to(dev)) if bf else \
        (lambda a: torch.from_numpy(a).to(dev))
    set_bytes = 2 * w.outputs * esz
    nsets = max(1, -(-2 * CACHE_BYTES // set_bytes))
    bufs = [(to(v), torch.empty(w.outputs, dtype=torch.int16 if bf else torch.float32,
                                device=dev)) for _ in range(nsets)]
    tk = to(k)
    spec = torch.empty(sc.sc_filter_spectrum_bytes(w.C, w.L), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    fspec = getattr(sc.lib(), "sc_filter_spectrum_" + kname)
    fapply = getattr(sc.lib(), "sc_causal_conv_spec_" + kname)

    def mk_spec(i):
        st = fspec(tk.data_ptr(), spec.data_ptr(), w.C, w.L, sptr)
        if st != 0:
            raise RuntimeError("sc_filter_spectrum failed: %s" % sc.sc_status_string(st))

    def apply(i):
        a, o = bufs[i % nsets]
        st = fapply(a.data_ptr(), spec.data_ptr(), o.data_ptr(), w.B, w.C, w.L, sptr)
        if st != 0:
            raise RuntimeError("sc_causal_conv_spec failed: %s" % sc.sc_status_string(st))

    def timed(fn, n):
        for i in range(warmup):
            fn(i)
        return time_rounds(torch, stream, fn, n)[0]

    t_spec = timed(mk_spec, 5)
    t_apply = timed(apply, steps)
    gbps = 2 * w.outputs * esz / (t_apply * 1e-3) / 1e9
    tf = 2.0 / 3.0 * algorithmic_flops_per_output(w.L) * w.outputs / (t_apply * 1e-3) / 1e12
    del bufs

    dr = make_grad(w)
    et = torch.int16 if bf else torch.float32
    gsets = max(1, -(-2 * CACHE_BYTES // (3 * w.outputs * esz)))
    gbufs = [(to(dr), to(v), torch.empty(w.outputs, dtype=et, device=dev))
             for _ in range(gsets)]
    dk = torch.empty(w.C * w.L, dtype=et, device=dev)
    fbwd = getattr(sc.lib(), "sc_causal_conv_spec_bwd_" + kname)

    def bwd(i):
        d, a, o = gbufs[i % gsets]
        st = fbwd(d.data_ptr(), a.data_ptr(), spec.data_ptr(), o.data_ptr(), dk.data_ptr(),
                  w.B, w.C, w.L, sptr)
        if st != 0:
            raise RuntimeError("sc_causal_conv_spec_bwd failed: %s" % sc.sc_status_string(st))

    t_bwd = timed(bwd, steps)
    del gbufs
    gb_bwd = 3 * w.outputs * esz / (t_bwd * 1e-3) / 1e9
    return {"entry": "sc_causal_conv_spec_" + kname, "filter": "one per channel, shared by "
            "the %d batch rows (decaying random filters)" % w.B,
            "ms_per_call": round(t_apply, 5), "value": round(w.outputs / (t_apply * 1e-3), 1),
            "unit": "outputs/s", "spectrum_ms": round(t_spec, 5),
            "hbm": {"algorithmic_bytes_per_call": 2 * w.outputs * esz,
                    "achieved_GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)},
            "alu": {"achieved_TFLOPs": round(tf, 2), "peak": FP32_FMA_PEAK_UNPACKED_TFLOPS,
                    "frac": round(tf / FP32_FMA_PEAK_UNPACKED_TFLOPS, 4),
                    "frac_of_published_157.3": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4),
                    "flops_per_output": "2/3 of the per-row-gate method's"},
            "bwd": {"entry": "sc_causal_conv_spec_bwd_" + kname, "ms_per_call": round(t_bwd, 5),
                    "value": round(w.outputs / (t_bwd * 1e-3), 1), "unit": "outputs/s",
                    "algorithmic_bytes_per_call": 3 * w.outputs * esz,
                    "achieved_GBps": round(gb_bwd, 1),
                    "kernels": "apply (reversed) for dv, then the batch-summing dk kernel"}}


def blc_measure(sc, torch, w, dev, steps: int, warmup: int, conv_ms: float) -> dict:
    """Time the token-major call sc_causal_conv_blc_ex on the workload's inputs in (B, L, C)
    with a caller workspace (no allocation in the timed region), and beside it the same
    result made by torch transposes around the channel-major call (what a caller would do
    without it).  Algorithmic bytes as the channel-major call."""
    import ctypes
    from workloads import make_inputs
    v, g = make_inputs(w)
    kind = {"f32": sc.KIND_F32, "bf16": sc.KIND_BF16, "i32": sc.KIND_NTT_I32}[w.storage]
    et = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[w.storage]
    esz = {"f32": 4, "bf16": 2, "i32": 4}[w.storage]

    def tm(a):
        t = torch.from_numpy(np.ascontiguousarray(np.swapaxes(a, 1, 2)))
        if w.storage == "bf16":
            t = t.view(torch.int16)
        return t.to(dev).view(et)
    set_bytes = 3 * w.outputs * esz
    nsets = max(1, -(-2 * CACHE_BYTES // set_bytes))
    bufs = [(tm(v), tm(g), torch.empty((w.B, w.L, w.C), dtype=et, device=dev))
            for _ in range(nsets)]
    nbytes = sc.sc_blc_workspace_bytes(kind, w.B, w.L, w.C)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    fblc = sc.lib().sc_causal_conv_blc_ex

    def call(i):
        a, b, o = bufs[i % nsets]
        st = fblc(kind, a.data_ptr(), b.data_ptr(), o.data_ptr(), w.B, w.L, w.C, None,
                  ws.data_ptr(), nbytes, sptr)
        if st != 0:
            raise RuntimeError("sc_causal_conv_blc_ex failed: %s" % sc.sc_status_string(st))

    def torch_route(i):
        a, b, o = bufs[i % nsets]
        r = sc.causal_conv(a.transpose(1, 2).contiguous(), b.transpose(1, 2).contiguous())
        o.copy_(r.transpose(1, 2))

    for i in range(warmup):
        call(i)
    t_blc = time_rounds(torch, stream, call, steps)[0]
    for i in range(warmup):
        torch_route(i)
    t_torch = time_rounds(torch, stream, torch_route, max(3, steps // 2))[0]
    del bufs, ws
    gb = 3 * w.outputs * esz / (t_blc * 1e-3) / 1e9
    return {"entry": "sc_causal_conv_blc_ex", "layout": "(B, L, C)",
            "hbm": {"algorithmic_bytes_per_call": 3 * w.outputs * esz,
                    "achieved_GBps": round(gb, 1), "frac": round(gb / HBM_PEAK_GBPS, 4)},
            "ms_per_call": round(t_blc, 5), "value": round(w.outputs / (t_blc * 1e-3), 1),
            "unit": "outputs/s", "workspace_bytes": nbytes,
            "channel_major_ms": round(conv_ms, 5),
            "overhead_vs_channel_major": round(t_blc / conv_ms, 3),
            "torch_transposes_ms": round(t_torch, 5),
            "torch_transposes_note": "x.transpose(1, 2).contiguous() of v and g, the "
                                     "channel-major call, and a copy back to (B, L, C)"}


def gate_measure(sc, torch, w, dev, steps: int, warmup: int, conv_ms: float) -> dict:
    """Time the gate calls on the workload's shape: sc_gate_* (s -> g, channel-major), the
    mixing step with the gate as prologue sc_gate_conv_ex (channel-major) and
    sc_gate_conv_blc_ex (token-major), each with a caller workspace.  The gate kernel reads s
    and writes g (2 elements per output) and does 2 * 64 * 3 flops per output on MFMA."""
    import ctypes
    from workloads import make_gate_inputs
    bf = w.storage == "bf16"
    kind = sc.KIND_BF16 if bf else sc.KIND_F32
    et = torch.bfloat16 if bf else torch.float32
    esz = 2 if bf else 4
    v, s, W = make_gate_inputs(w)

    def dev_t(a, tm=False):
        if tm:
            a = np.ascontiguousarray(np.swapaxes(a, 1, 2))
        t = torch.from_numpy(a.view(np.int16) if bf else a)
        return t.to(dev).view(et)
    nsets = max(1, -(-2 * CACHE_BYTES // (3 * w.outputs * esz)))
    cm = [(dev_t(v), dev_t(s), torch.empty(w.outputs, dtype=et, device=dev)) for _ in range(nsets)]
    Wd = dev_t(W)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    lib = sc.lib()
    fgate = lib.sc_gate_bf16 if bf else lib.sc_gate_f32
    ws_cm = sc.sc_gate_conv_workspace_bytes(kind, w.B, w.C, w.L)
    ws_tm = sc.sc_gate_conv_blc_workspace_bytes(kind, w.B, w.L, w.C)
    ws = torch.empty(max(ws_cm, ws_tm, 256), dtype=torch.uint8, device=dev)

    def check(st, what):
        if st != 0:
            raise RuntimeError("%s failed: %s" % (what, sc.sc_status_string(st)))

    def gate_only(i):
        _, a, o = cm[i % nsets]
        check(fgate(a.data_ptr(), Wd.data_ptr(), o.data_ptr(), w.B, w.C, w.L, sptr), "sc_gate")

    def gate_conv(i):
        a, b, o = cm[i % nsets]
        check(lib.sc_gate_conv_ex(kind, a.data_ptr(), b.data_ptr(), Wd.data_ptr(), o.data_ptr(),
                                  w.B, w.C, w.L, None, ws.data_ptr(), ws_cm, sptr),
              "sc_gate_conv_ex")

    def timed(fn, n):
        for i in range(warmup):
            fn(i)
        return time_rounds(torch, stream, fn, n)[0]

    t_gate = timed(gate_only, steps)
    t_gc = timed(gate_conv, steps)
    del cm
    tm = [(dev_t(v, True), dev_t(s, True), torch.empty(w.outputs, dtype=et, device=dev))
          for _ in range(nsets)]

    def gate_conv_tm(i):
        a, b, o = tm[i % nsets]
        check(lib.sc_gate_conv_blc_ex(kind, a.data_ptr(), b.data_ptr(), Wd.data_ptr(),
                                      o.data_ptr(), w.B, w.L, w.C, None, ws.data_ptr(), ws_tm,
                                      sptr), "sc_gate_conv_blc_ex")
    t_gtm = timed(gate_conv_tm, steps)
    del tm, ws
    gb = 2 * w.outputs * esz / (t_gate * 1e-3) / 1e9
    tf = 2 * 64 * 3 * w.outputs / (t_gate * 1e-3) / 1e12
    peak_tf = 2500.0 if bf else 157.3
    return {"entries": ["sc_gate_" + ("bf16" if bf else "f32"), "sc_gate_conv_ex",
                        "sc_gate_conv_blc_ex"],
            "gate_ms": round(t_gate, 5),
            "gate_hbm": {"algorithmic_bytes_per_call": 2 * w.outputs * esz,
                         "achieved_GBps": round(gb, 1), "frac": round(gb / HBM_PEAK_GBPS, 4)},
            "gate_mfma": {"flops_per_output": 2 * 64 * 3, "achieved_TFLOPs": round(tf, 2),
                          "peak_TFLOPs": peak_tf, "frac": round(tf / peak_tf, 4)},
            "gate_conv_ms": round(t_gc, 5), "gate_conv_blc_ms": round(t_gtm, 5),
            "conv_ms": round(conv_ms, 5),
            "gate_conv_value": round(w.outputs / (t_gc * 1e-3), 1),
            "gate_conv_blc_value": round(w.outputs / (t_gtm * 1e-3), 1), "unit": "outputs/s"}


def other_measure(sc, torch, w, dev, steps: int, warmup: int, oracle_too: bool = True) -> dict:
    """The plain call on another workload of the set (same timing method as the headline:
    launches back to back on the launch stream, buffer sets rotated through HBM)."""
    from workloads import make_inputs
    fn_name, esz = {"i32": ("sc_causal_conv_ntt_i32", 4), "bf16": ("sc_causal_conv_bf16", 2),
                    "f32": ("sc_causal_conv_f32", 4)}[w.storage]
    fn = getattr(sc.lib(), fn_name)
    v, g = make_inputs(w)
    tdtype = {"f32": torch.float32, "bf16": torch.int16, "i32": torch.int32}[w.storage]
    hv = torch.from_numpy(v.view(np.int16) if w.storage == "bf16" else v)
    hg = torch.from_numpy(g.view(np.int16) if w.storage == "bf16" else g)
    nsets = max(1, min(3, -(-2 * CACHE_BYTES // (3 * w.outputs * esz))))
    bufs = [(hv.to(dev), hg.to(dev), torch.empty(w.outputs, dtype=tdtype, device=dev))
            for _ in range(nsets)]
    nbytes = sc.sc_workspace_bytes(sc.KIND_F32 if w.storage == "f32" else
                                   sc.KIND_BF16 if w.storage == "bf16" else sc.KIND_NTT_I32,
                                   w.B, w.C, w.L)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    fn_ws = getattr(sc.lib(), fn_name + "_ws")

    def step(i):
        a, b, c = bufs[i % nsets]
        st = fn_ws(a.data_ptr(), b.data_ptr(), c.data_ptr(), w.B, w.C, w.L,
                   ws.data_ptr() if nbytes else None, nbytes, sptr)
        if st != 0:
            raise RuntimeError("%s_ws failed: %s" % (fn_name, sc.sc_status_string(st)))

    for i in range(warmup):
        step(i)
    ms, _ = time_rounds(torch, stream, step, steps)
    stats = launch_stats(torch, stream, step, 50)
    alg_bytes = w.outputs * 3 * esz
    rec = {"workload": w.name, "entry": fn_name + "_ws", "ms_per_call": round(ms, 5),
           "value": round(w.outputs / (ms * 1e-3), 1), "unit": "outputs/s",
           "call_ms": stats,
           "hbm": {"algorithmic_bytes_per_call": alg_bytes,
                   "achieved_GBps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
                   "frac": round(alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}}
    # HBM bytes per call from the committed counter record (null when there is none for the
    # current kernel sources) and the VALU issue floor where a counter record exists
    traffic = measured_traffic(w.name)
    rec["hbm"]["traffic_bytes_per_call"] = traffic
    if traffic:
        rec["hbm"]["traffic_GBps"] = round(traffic / (ms * 1e-3) / 1e9, 1)
        rec["hbm"]["traffic_frac"] = round(traffic / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    issue = alu_issue(w.name, ms)
    if issue:
        rec["alu_issue"] = issue
    if w.storage != "i32":
        tf = algorithmic_flops_per_output(w.L) * w.outputs / (ms * 1e-3) / 1e12
        rec["alu"] = {"achieved_TFLOPs": round(tf, 2), "peak": FP32_FMA_PEAK_UNPACKED_TFLOPS,
                      "frac": round(tf / FP32_FMA_PEAK_UNPACKED_TFLOPS, 4),
                      "frac_of_published_157.3": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4)}
    del bufs, ws
    torch.cuda.empty_cache()
    if oracle_too:
        import oracle
        nt = oracle.default_threads()
        if w.L > 4096:
            # channels are independent: 64 seeded channels, the rate extrapolated to all
            rng = np.random.default_rng(np.random.SeedSequence([w.cid, 64]))
            pick = np.sort(rng.choice(w.B * w.C, size=min(64, w.B * w.C), replace=False))
            vs, gs = v.reshape(-1, w.L)[pick], g.reshape(-1, w.L)[pick]
            t0 = time.perf_counter()
            if w.storage == "i32":
                oracle.causal_conv_i64(vs, gs, nthreads=nt)
            else:
                oracle.causal_conv_f64(vs, gs, nthreads=nt, with_scale=False)
            dt = time.perf_counter() - t0
            rec["cpu_oracle"] = {"value": round(len(pick) * w.L / dt, 1), "unit": "outputs/s",
                                 "cores": nt, "kind": "oracle", "extrapolated": True,
                                 "sample": "%d seeded of %d channels, %.2f s wall; the rate "
                                           "applies to the whole workload since channels are "
                                           "independent" % (len(pick), w.B * w.C, dt)}
        else:
            n, dt = oracle_sample_rate(w, v, g, nt, 3.0)
            rec["cpu_oracle"] = {"value": round(n * w.L / dt, 1), "unit": "outputs/s",
                                 "cores": nt, "kind": "oracle",
                                 "sample": "%d of %d channels, %.2f s wall" % (n, w.B * w.C, dt)}
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prewarm-ms", type=float, default=200.0,
                    help="wall time of untimed hot-path launches before the warmup steps, so "
                         "that the timed steps see the clock the chip holds under load (0: off)")
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pages-approach", action="store_true",
                    help="skip the context timing of the torch.fft pipeline")
    ap.add_argument("--no-leakage", action="store_true",
                    help="skip the leakage probe (keeps profiler runs to the timed kernel)")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the timing of the gradient call (keeps profiler runs to the "
                         "forward kernel)")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the timing of the filter-shared-by-the-batch calls")
    ap.add_argument("--no-blc", action="store_true",
                    help="skip the timing of the token-major (B, L, C) call")
    ap.add_argument("--no-gate", action="store_true",
                    help="skip the timing of the gate-stream calls")
    ap.add_argument("--no-fixed", action="store_true",
                    help="skip the timing of the exactly causal real-valued call")
    ap.add_argument("--no-mfma", action="store_true",
                    help="skip timing the SC_PATH_FUSED_MFMA form of the bf16 call")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the plain call on the other workloads (Small, exact, long)")
    ap.add_argument("--no-stats", action="store_true",
                    help="skip the 50 individually timed launches after the timed steps")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain device copy of known size (profiler calibration)")
    ap.add_argument("--record-valu", metavar="SQ_DIR",
                    help="write profiles/valu_<workload>.json from a rocprofv3 --pmc run of "
                         "this script that collected SQ_INSTS_VALU")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "runs (FETCH_SIZE, WRITE_SIZE) of this script with --calib-copy")
    args = ap.parse_args(argv)

    if args.record_valu:
        from workloads import WORKLOADS
        print(json.dumps(record_valu(WORKLOADS[args.workload], args.record_valu)))
        return 0
    if args.record_traffic:
        from workloads import WORKLOADS
        print(json.dumps(record_traffic(WORKLOADS[args.workload], *args.record_traffic)))
        return 0

    global PREWARM_MS
    PREWARM_MS = args.prewarm_ms
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(channels shard across GPUs with no communication; run one process per GPU)",
              file=sys.stderr)
        return 2

    import torch
    import fft_causal_long_amd as sc
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if w.storage == "i32":
        fn_name, esz = "sc_causal_conv_ntt_i32", 4
    elif w.storage == "bf16":
        fn_name, esz = "sc_causal_conv_bf16", 2
    else:
        fn_name, esz = "sc_causal_conv_f32", 4
    fn = getattr(sc.lib(), fn_name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    v, g = make_inputs(w)
    tdtype = {"f32": torch.float32, "bf16": torch.int16, "i32": torch.int32}[w.storage]
    hv = torch.from_numpy(v.view(np.int16) if w.storage == "bf16" else v)
    hg = torch.from_numpy(g.view(np.int16) if w.storage == "bf16" else g)
    set_bytes = 3 * w.outputs * esz
    nsets = max(1, -(-2 * CACHE_BYTES // set_bytes))
    bufs = []
    for _ in range(nsets):
        bufs.append((hv.to(dev), hg.to(dev), torch.empty(w.outputs, dtype=tdtype, device=dev)))
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def step(i):
        a, b, c = bufs[i % nsets]
        st = fn(a.data_ptr(), b.data_ptr(), c.data_ptr(), w.B, w.C, w.L, sptr)
        if st != 0:
            raise RuntimeError("%s failed: %s" % (fn_name, sc.sc_status_string(st)))

    # untimed launches of the same step for --prewarm-ms (see prewarm()), then the W warmup
    # steps, then the K timed steps
    warm = {"ms": PREWARM_MS, "launches": prewarm(torch, step)}
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the K steps back to back on the launch stream, HIP events at 5 round boundaries (and
    # synchronisation on both sides); one step is one kernel launch, so the mean launch
    # duration is the region's time per step
    ms_per_step, round_ms = time_rounds(torch, stream, step, args.steps, warm=False)
    total_ms = ms_per_step * args.steps
    kernel_ms = ms_per_step
    # per-launch statistics over 50 more launches (outside the K timed steps)
    stats = None if args.no_stats else launch_stats(torch, stream, step, 50, args.steps)

    mfma = None
    if not args.no_mfma and w.storage == "bf16" and 2048 < w.L <= 4096:
        mfma = fused_mfma_measure(sc, torch, stream, step, bufs, w, args.steps)

    if args.calib_copy:
        # 1 GiB device-to-device copy: a known-size reference for the profiler's byte counters
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    outputs = w.outputs
    value = outputs * args.steps / (total_ms * 1e-3)
    alg_bytes = outputs * 3 * esz
    hbm_gbps = alg_bytes / (kernel_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)
    if w.storage == "i32":
        roof = {"bound": "hbm", "achieved": round(hbm_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(hbm_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
    else:
        # the kernel is bound by its vector-ALU instruction stream, not by HBM: its roofline
        # is the fp32 FMA peak that code compiled without packed fp32 can reach; the HBM
        # fraction the metric names is carried beside it (and in `hbm`)
        flops = algorithmic_flops_per_output(w.L) * outputs
        tf = flops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(tf, 2),
                "peak": round(FP32_FMA_PEAK_UNPACKED_TFLOPS, 2),
                "unit": "TFLOP/s", "frac": round(tf / FP32_FMA_PEAK_UNPACKED_TFLOPS, 4),
                "traffic": traffic,
                "peak_basis": "256 CU x 4 SIMD x 16 lanes x 2 flops (FMA) x 2.4 GHz, packed fp32 "
                              "off; AMD's published 157.3 TFLOP/s needs packed dual-fp32 FMAs",
                "frac_of_published_157.3": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4),
                "hbm_frac": round(hbm_gbps / HBM_PEAK_GBPS, 4)}
    rec = {
        "metric": "causal-conv outputs/sec (B\u00b7C\u00b7L) at L=%d + %% HBM roofline; NTT leakage=0" % w.L,
        "value": round(value, 1),
        "unit": "outputs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.storage != "i32" else "int32-mod-p",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "C": w.C, "L": w.L, "storage": w.storage,
                   "entry": fn_name, "buffer_sets": nsets},
        "roofline": roof,
        "alu_issue": alu_issue(w.name, kernel_ms),
        "hbm": {"algorithmic_bytes_per_launch": alg_bytes, "achieved_GBps": round(hbm_gbps, 1),
                "peak_GBps": HBM_PEAK_GBPS, "frac": round(hbm_gbps / HBM_PEAK_GBPS, 4)},
        "kernel_ms": {"mean": round(kernel_ms, 5), "rounds": [round(x, 5) for x in round_ms],
                      "method": "launches back to back, HIP events on the launch stream at "
                                "round boundaries"},
        "launch_ms": stats,
        "prewarm": warm,
    }
    if mfma is not None:
        rec["fused_mfma"] = mfma
    if not args.no_others:
        ref = copy_reference(torch, dev)
        rec["hbm"]["copy_reference"] = ref
        rec["hbm"]["frac_of_copy"] = round(hbm_gbps / ref["achieved_GBps"], 4)
    if not args.no_bwd:
        del bufs
        rec["bwd"] = bwd_measure(sc, torch, w, dev, max(5, args.steps // 2), args.warmup)
    if not args.no_shared and w.storage != "i32" and w.L <= 4096:
        rec["shared"] = shared_measure(sc, torch, w, dev, max(5, args.steps // 2), args.warmup)
    if not args.no_blc:
        rec["token_major"] = blc_measure(sc, torch, w, dev, max(5, args.steps // 2), args.warmup,
                                         kernel_ms)
    if not args.no_gate and w.storage != "i32" and w.C % 64 == 0:
        rec["gate"] = gate_measure(sc, torch, w, dev, max(5, args.steps // 2), args.warmup,
                                   kernel_ms)
    if not args.no_fixed and w.storage != "i32":
        rec["fixed"] = fixed_measure(sc, torch, w, dev, max(5, args.steps // 5), 2)
    if not args.no_pages_approach and w.storage != "i32":
        rec["pages_approach"] = pages_approach(torch, w, dev, max(5, args.steps // 5), kernel_ms)
    if not args.no_fixed and not args.no_others and args.workload == 3:
        # the exact real-valued call at the long-context shape (four-step split per prime)
        rec["fixed_long"] = fixed_measure(sc, torch, WORKLOADS[4], dev, 5, 2)
    if not args.no_others and args.workload == 3:
        # Tiny, Small, the Medium shape in fp32, exact, long (four-step), long exact
        rec["other_workloads"] = [other_measure(sc, torch, WORKLOADS[c], dev, 20, 3,
                                                not args.no_cpu_baseline)
                                  for c in (1, 2, 6, 5, 4, 7)]
    if not args.no_leakage:
        rec["leakage"] = leakage_probe(sc, torch, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, v, g)
        next_rows_oracles(w, rec)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
