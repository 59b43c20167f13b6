#!/usr/bin/env python3
"""Throughput of the fused attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
the forward (attn_fwd: O and lse) and the backward (attn_bwd's two launches:
dQ, which also forms D = rowsum(dO * O), then dK/dV) on the causal B=4 H=16
N=4096 d=128 bf16 workload.  Inputs are generated on the host from a fixed seed, copied to the
GPU, and resident in HBM before the timed region starts.

With `--workload` naming another attention shape (attn_inputs.WORKLOADS or
HEADDIM_WORKLOADS, e.g. b4_h16_n4096_d96_causal) a step is the same pass on
that shape; in fp32, where no backward is built, the forward alone.

With `--workload` naming a key/value-cache shape (attn_inputs.KV_WORKLOADS,
e.g. decode_b8_h32_nq1_nk8192_d128) a step is instead one attn_fwd_kv call
(per-chunk partial kernel + merge kernel) and `value` is the K/V bytes read
per second, the quantity that bounds decode; the chunked-prefill training
shape (prefill_b2_h16_nq512_nk4096_d128_fwdbwd) times attn_fwd_kv plus
attn_bwd_kv, in TFLOP/s over the visible query-key pairs.  With a
row-softmax shape (attn_inputs.SOFTMAX_WORKLOADS, softmax_m65536_n4096_bf16)
a step is one attn_softmax_rows call and `value` is the bytes it must move
(one read and one write of every element) per second.  With the FP8 shapes
(attn_inputs.MX_WORKLOADS) a step is one attn_fwd_mx (`..._mxfp8`) or
attn_fwd_fp8 (`..._fp8`) call.

Prints ONE JSON line.  `value` is fwd+bwd TFLOP/s by the formula
4*B*H*N^2*d (halved for causal) for the forward plus 2.5x that for the
backward, over the K timed steps.  `roofline` describes the kernel with the
largest share of the step time, timed live with HIP events recorded on the
stream the kernels run on.  `cpu_baseline` times the fp64 CPU oracle on a
bounded sample of the same workload (whole heads, forward + backward).
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (packed FMAs; 78.6 without them)
KERNELS = ("fwd", "bwd_dq", "bwd_dkdv")  # one step, in launch order
BWD_PHASES = (3, 1)  # attn_bwd_phase numbers of the backward kernels above
COUNTED_KERNELS = KERNELS + ("bwd_preprocess", "softmax_rows",)  # kernels the HBM byte counters cover
CSRC = os.path.join(ROOT, "tiled_online_softmax_attn_amd", "csrc")
KERNEL_SOURCES = {"fwd": "attn_fwd.hip", "bwd_preprocess": "attn_bwd.hip",
                  "bwd_dkdv": "attn_bwd_dkdv.hip", "bwd_dq": "attn_bwd.hip",
                  "softmax_rows": "softmax_rows.hip"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
PROBE_LIB = os.path.join(ROOT, "tiled_online_softmax_attn_amd", "libattn_probe.so")


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(kernel: str) -> str:
    """Digest of what a kernel's machine code is built from: its source, the
    shared device header and the compiler flags of that source."""
    from tiled_online_softmax_attn_amd import build as hip_build
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[kernel], "device_common.h"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    flags = hip_build.FLAGS + hip_build.source_flags(KERNEL_SOURCES[kernel])
    h.update(" ".join(f for f in flags if not f.startswith("-I")).encode())  # paths vary
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        e = t[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if e.get("source_digest") != source_digest(kernel):
        return None
    return e["fetch_bytes"] + e["write_bytes"]


def algorithmic(w, kernel: str):
    """(amount, unit, bound) per launch: FLOPs for the MFMA kernels, bytes for
    the memory-bound preprocess.  A block product over the unmasked causal
    half costs 2*B*H*N^2*d/2 FLOPs (half the forward's count).  Each backward
    kernel is credited with the products it actually runs: dK/dV runs four
    (S, dP, dV, dK), dQ runs three (S, dP, dQ).  The step value uses the
    formula count (2.5x the forward for the whole backward), so the extra
    recompute lowers `value` but not these per-kernel rates."""
    import torch
    BHN = w.B * w.H * w.N
    if kernel == "fwd":
        # the fp32 forward runs on plain fp32 FMAs (VALU), not the matrix unit
        return w.fwd_flops(), "flop", "alu" if w.dtype == torch.float32 else "mfma"
    if kernel == "bwd_dkdv":
        return w.fwd_flops() * 4 / 2, "flop", "mfma"
    if kernel == "bwd_dq":
        return w.fwd_flops() * 3 / 2, "flop", "mfma"
    # preprocess: read O, dO (bf16); write D (fp32)
    return BHN * w.d * 2 * 2 + BHN * 4, "byte", "hbm"


def measure_peaks(full: bool = False) -> dict:
    """Measured ceilings (libattn_probe.so, include/attn_probe.h): the dense
    bf16 MFMA rate with nothing else in the loop and with one or two groups
    of the softmax's per-score VALU work (FMA, exponential, add) per MFMA,
    the shader clock under that load, the v_exp_f32 rate, and a plain HBM
    copy.  Each probe is timed with HIP events on the stream it runs on;
    the best of `reps` launches is kept (the ceiling, not the average)."""
    import ctypes

    import torch
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built")
    L = ctypes.CDLL(PROBE_LIB)
    vp, i = ctypes.c_void_p, ctypes.c_int
    L.attn_probe_mfma.argtypes = [vp, vp, i, i, i, vp]
    L.attn_probe_exp.argtypes = [vp, vp, i, i, vp]
    L.attn_probe_copy.argtypes = [vp, vp, ctypes.c_longlong, vp]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    blocks = 1024  # 4 workgroups of 4 waves per CU: 4 waves per SIMD
    out = torch.empty(blocks * 256, device=dev)
    clk = torch.zeros(blocks * 2, device=dev, dtype=torch.int64)
    reps = 7 if full else 3

    def timed(launch):
        best = None
        for _ in range(reps + 1):  # the first launch warms up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = launch()
            e1.record(stream)
            if rc != 0:
                raise RuntimeError(f"probe launch failed: {rc}")
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None or ms < best else best
        return best

    def clock_ghz():
        c = clk.view(blocks, 2).double().cpu()
        ok = c[:, 1] > 0
        ghz = (c[ok, 0] / (c[ok, 1] / 1e8) / 1e9).sort().values
        return round(float(ghz[len(ghz) // 2]), 3)

    res = {"probe_blocks": blocks}
    iters = 20000 if full else 6000
    for groups in (0, 1, 2):
        ms = timed(lambda: L.attn_probe_mfma(out.data_ptr(), clk.data_ptr(), blocks, iters, groups, sh))
        flops = blocks * 4 * iters * 4 * 32768.0
        key = "mfma_bf16" if groups == 0 else f"mfma_bf16_softmax{groups}"
        res[f"{key}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
        res[f"{key}_clock_ghz"] = clock_ghz()
    eiters = 8000 if full else 3000
    ms = timed(lambda: L.attn_probe_exp(out.data_ptr(), clk.data_ptr(), blocks, eiters, sh))
    exps = blocks * 256 * eiters * 8.0
    ghz = clock_ghz()
    res["exp_per_s"] = float(f"{exps / (ms * 1e-3):.4g}")
    res["exp_clock_ghz"] = ghz
    # wave64 v_exp_f32 instructions per SIMD per cycle -> cycles per instruction
    res["exp_cycles_per_wave_instr"] = round(ghz * 1e9 / (exps / (ms * 1e-3) / 64 / 1024), 2)
    nbytes = (1 << 30) if full else (512 << 20)
    src = torch.ones(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    ms = timed(lambda: L.attn_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, sh))
    res["hbm_copy_gbs"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    res["hbm_copy_bytes"] = 2 * nbytes
    del src, dst
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, do, budget_s: float, backward: bool = True):
    import numpy as np

    import oracle
    lib = oracle.load()
    scale = float(np.float32(w.scale))
    f64 = lambda t: t.to("cpu").double().numpy()
    heads, t0 = 0, time.perf_counter()
    per_head = (w.fwd_flops() + (w.bwd_flops() if backward else 0.0)) / (w.B * w.H)
    for b in range(w.B):
        for h in range(w.H):
            qh, kh, vh, dh = f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h])
            oracle.attn_fwd(qh, kh, vh, w.causal, scale, lib=lib)
            if backward:
                oracle.attn_bwd(qh, kh, vh, dh, w.causal, scale, lib=lib)
            heads += 1
            eprint(f"[cpu_baseline] oracle head {heads}: {time.perf_counter() - t0:.1f} s")
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            continue
        break
    el = time.perf_counter() - t0
    return {"value": per_head * heads / el / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(lib), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{heads} of {w.B * w.H} heads of {w.name} (fp64 forward"
                      f"{' + backward' if backward else ''} per head, S and P materialised), "
                      f"{el:.1f} s"}


def cpu_baseline_single_thread(budget_s: float) -> dict:
    """The oracle's forward on one host thread, for the two small workloads
    (fp32 B1 H1 N256 d64 and bf16 B1 H8 N1024 d64), whole heads for at most
    budget_s seconds each: GFLOP/s by the same formula as the GPU."""
    import numpy as np

    import oracle
    from attn_inputs import WORKLOADS, workload_inputs
    lib = oracle.load()
    prev = oracle.num_threads(lib)
    oracle.set_num_threads(1, lib=lib)
    out = {}
    try:
        for name in ("single_head_f32", "h8_n1024_d64"):
            w = WORKLOADS[name]
            q, k, v = workload_inputs(w, with_dout=False)
            scale = float(np.float32(w.scale))
            f64 = lambda t: t.to("cpu").double().numpy()
            heads, t0 = 0, time.perf_counter()
            for h in range(w.B * w.H):
                b, hh = divmod(h, w.H)
                oracle.attn_fwd(f64(q[b, hh]), f64(k[b, hh]), f64(v[b, hh]), w.causal, scale,
                                lib=lib)
                heads += 1
                if time.perf_counter() - t0 >= budget_s:
                    break
            el = time.perf_counter() - t0
            out[name] = {"gflops": round(w.fwd_flops() / (w.B * w.H) * heads / el / 1e9, 3),
                         "heads": heads, "seconds": round(el, 3)}
    finally:
        oracle.set_num_threads(prev, lib=lib)
    return out


def kernel_key(name: str):
    """Map a device kernel name to the bench's kernel keys (None if foreign)."""
    if "attn_fwd_bf16_kernel" in name:
        return "fwd"
    if "bwd_preprocess_kernel" in name:
        return "bwd_preprocess"
    if "bwd_dkdv_kernel" in name:
        return "bwd_dkdv"
    if "bwd_dq_kernel" in name:
        return "bwd_dq"
    if "softmax_rows" in name:
        return "softmax_rows"
    if "MulFunctor" in name:  # the --copy-mib reference kernel (x * 1)
        return "copy"
    return None


def pmc_summary(dirs, copy_mib: float, workload: str) -> int:
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE passes (counter_collection.csv
    files under `dirs`) into profiles/traffic.json.  The plain copy kernel
    that `--copy-mib` runs (reads and writes copy_mib MiB) calibrates each
    counter: bytes = counter_KiB * 1024 * (known / measured on the copy)."""
    import csv
    import glob
    sums = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = kernel_key(r["Kernel_Name"])
                    if key is None:
                        continue
                    ent = sums.setdefault((key, r["Counter_Name"]), [])
                    ent.append(float(r["Counter_Value"]))
    avg = {k: sum(v) / len(v) for k, v in sums.items()}
    known_kib = copy_mib * 1024.0
    fetch_cal = known_kib / avg[("copy", "FETCH_SIZE")]
    write_cal = known_kib / avg[("copy", "WRITE_SIZE")]
    try:  # other workloads' entries are kept
        with open(TRAFFIC_FILE) as fh:
            out = json.load(fh)
    except (OSError, ValueError):
        out = {}
    per = {"calibration": {"copy_mib": copy_mib,
                           "copy_fetch_kib": avg[("copy", "FETCH_SIZE")],
                           "copy_write_kib": avg[("copy", "WRITE_SIZE")],
                           "fetch_factor": fetch_cal, "write_factor": write_cal}}
    for kn in COUNTED_KERNELS:
        if (kn, "FETCH_SIZE") not in avg or (kn, "WRITE_SIZE") not in avg:
            continue
        per[kn] = {"fetch_bytes": avg[(kn, "FETCH_SIZE")] * 1024 * fetch_cal,
                   "write_bytes": avg[(kn, "WRITE_SIZE")] * 1024 * write_cal,
                   "fetch_kib_raw": avg[(kn, "FETCH_SIZE")],
                   "write_kib_raw": avg[(kn, "WRITE_SIZE")],
                   "source_digest": source_digest(kn)}
    out[workload] = per
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def cpu_baseline_kv(w, q, k, v, budget_s: float):
    """The oracle's Nq x Nk forward on whole heads for about budget_s seconds;
    rate in K/V bytes per second, like the GPU value."""
    import numpy as np

    import oracle
    lib = oracle.load()
    scale = float(np.float32(w.scale))
    f64 = lambda t: t.to("cpu").double().numpy()
    heads, t0 = 0, time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            oracle.attn_fwd_rect(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), w.causal, scale, lib=lib)
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            continue
        break
    el = time.perf_counter() - t0
    eprint(f"[cpu_baseline] oracle: {heads} heads in {el:.1f} s")
    return {"value": w.kv_bytes() / (w.B * w.H) * heads / el / 1e9, "unit": "GB/s",
            "cores": oracle.num_threads(lib), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads of {w.name} (fp64 forward per head), "
                      f"{el:.1f} s"}


def bench_kv_fwdbwd(args, w):
    """One step = attn_fwd_kv + attn_bwd_kv (the training step of a chunked
    prefill: Nq queries at the end of an Nk-token sequence); TFLOP/s by the
    formula: 4 d times the visible (query, key) pairs for the forward, 2.5
    times that for the backward."""
    import torch

    import tiled_online_softmax_attn_amd as T
    from attn_inputs import kv_workload_inputs

    T.lib()
    dev = torch.device("cuda:0")
    eprint(f"[bench] generating inputs for {w.name}")
    q, k, v, do = kv_workload_inputs(w)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.Nq), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws_f = torch.empty(T.attn_fwd_kv_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, 0, w.dtype),
                       device=dev, dtype=torch.uint8)
    ws_b = torch.empty(T.attn_bwd_kv_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype),
                       device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        T.attn_fwd_kv(qd, kd, vd, o, lse, w.causal, w.scale, 0, ws_f, stream)
        if ev:
            ev[1].record(stream)
        T.attn_bwd_kv(qd, kd, vd, o, dod, lse, dq, dk, dv, ws_b, w.causal, w.scale, stream)
        if ev:
            ev[2].record(stream)

    eprint(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    eprint(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    f_fwd = w.flops()
    f_bwd = 2.5 * f_fwd
    value = (f_fwd + f_bwd) * args.steps / wall / 1e12
    bwd_rate = f_bwd / (bwd_ms * 1e-3) / 1e12
    fwd_rate = f_fwd / (fwd_ms * 1e-3) / 1e12
    dom = "bwd_kv" if bwd_ms >= fwd_ms else "fwd_kv"
    ach = bwd_rate if dom == "bwd_kv" else fwd_rate
    roofline = {"kernel": dom + " (one call)", "bound": "mfma", "achieved": round(ach, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": None}
    out = {
        "metric": f"chunked-prefill training step TFLOP/s (attn_fwd_kv + attn_bwd_kv), {w.name}",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q, K, V, dO)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "step": "attn_fwd_kv + attn_bwd_kv"},
        "fwd_ms": round(fwd_ms, 5), "bwd_ms": round(bwd_ms, 5), "fwd_tflops": round(fwd_rate, 2),
        "bwd_tflops": round(bwd_rate, 2), "roofline": roofline, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_kv(args, w):
    """One step = attn_fwd_kv over the whole cache workload."""
    import torch

    import tiled_online_softmax_attn_amd as T
    from attn_inputs import kv_workload_inputs

    T.lib()
    dev = torch.device("cuda:0")
    eprint(f"[bench] generating inputs for {w.name}")
    q, k, v = kv_workload_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.Nq), device=dev, dtype=torch.float32)
    ws = torch.empty(T.attn_fwd_kv_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, 0, w.dtype),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def step():
        T.attn_fwd_kv(qd, kd, vd, o, lse, w.causal, w.scale, 0, ws, stream)

    eprint(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    eprint(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    value = w.kv_bytes() * args.steps / wall / 1e9
    # bytes of one call: K and V once, Q read and O, lse written; the fp32
    # per-chunk partials are extra traffic of the split, not counted
    elem = torch.finfo(w.dtype).bits // 8
    algo = w.kv_bytes() + w.B * w.H * w.Nq * (2 * w.d * elem + 4)
    achieved = algo / (call_ms * 1e-3) / 1e9
    roofline = {"kernel": "fwd_kv (chunk partials + merge, one call)", "bound": "hbm",
                "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    cpu = None if args.no_cpu_baseline else cpu_baseline_kv(w, q, k, v,
                                                             args.cpu_baseline_seconds)
    out = {
        "metric": f"attention over a key/value cache, K/V bytes read per second, {w.name}",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q, K, V)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "step": "attn_fwd_kv"},
        "tflops": round(w.flops() / (call_ms * 1e-3) / 1e12, 2),
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_all(budget_s: float) -> int:
    """The oracle on a bounded sample (whole heads, about budget_s seconds) of
    each attention workload: forward, plus the backward where the workload
    has one; one JSON line each."""
    from attn_inputs import HEADDIM_WORKLOADS, WORKLOADS, workload_inputs
    for w in [*WORKLOADS.values(), *HEADDIM_WORKLOADS.values()]:
        eprint(f"[cpu_baseline] {w.name}")
        q, k, v, do = workload_inputs(w, with_dout=True)
        res = cpu_baseline(w, q, k, v, do, budget_s, backward=w.backward)
        print(json.dumps({"workload": w.name, **res}), flush=True)
    return 0


def copy_reference(copy_mib: float) -> None:
    """One plain device copy of copy_mib MiB (x * 1), the known-size kernel
    that calibrates the HBM byte counters."""
    if copy_mib <= 0:
        return
    import torch
    n = int(copy_mib * 1024 * 1024 // 4)
    src = torch.ones(n, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)  # reads and writes copy_mib MiB
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline_softmax(w, x, budget_s: float):
    """The oracle's row softmax, row by row, for about budget_s seconds; rate
    in bytes (one read + one write of each element) per second."""
    import oracle
    lib = oracle.load()
    rows, t0 = 0, time.perf_counter()
    while rows < w.M and time.perf_counter() - t0 < budget_s:
        oracle.softmax_row(x[rows].double().numpy(), lib=lib)
        rows += 1
    el = time.perf_counter() - t0
    eprint(f"[cpu_baseline] oracle: {rows} rows in {el:.1f} s")
    return {"value": w.hbm_bytes() / w.M * rows / el / 1e9, "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{rows} of {w.M} rows of {w.name} (fp64 safe softmax per row), "
                      f"{el:.1f} s"}


def bench_softmax(args, w):
    """One step = attn_softmax_rows over the whole M x N matrix."""
    import torch

    import tiled_online_softmax_attn_amd as T
    from attn_inputs import softmax_workload_inputs

    T.lib()
    dev = torch.device("cuda:0")
    eprint(f"[bench] generating inputs for {w.name}")
    x = softmax_workload_inputs(w)
    xd = x.to(dev)
    y = torch.empty_like(xd)
    stream = torch.cuda.current_stream()

    def step():
        T.attn_softmax_rows(xd, y, stream)

    copy_reference(args.copy_mib)

    eprint(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    eprint(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    value = w.hbm_bytes() * args.steps / wall / 1e9
    achieved = w.hbm_bytes() / (call_ms * 1e-3) / 1e9
    tr = measured_traffic("softmax_rows", w.name)
    roofline = {"kernel": "softmax_rows", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": None if tr is None else round(tr), "algorithmic_bytes": w.hbm_bytes(),
                "avg_launch_us": round(call_ms * 1e3, 2)}
    cpu = None if args.no_cpu_baseline else cpu_baseline_softmax(w, x, args.cpu_baseline_seconds)
    out = {
        "metric": f"fused row softmax, HBM bytes (one read + one write) per second, {w.name}",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": f"synthetic (seeded N(0,1) {'bf16' if w.dtype == torch.bfloat16 else 'fp32'} scores)",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "step": "attn_softmax_rows"},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_mx(args, w):
    """One step = attn_fwd_mx (Q, K in MXFP8, V bf16) over the whole workload,
    or, for the *_fp8 workload, attn_fwd_fp8 (Q, K, V in MXFP8, P in E4M3)."""
    import torch

    import tiled_online_softmax_attn_amd as T
    from attn_inputs import make_fp8_v, make_mx_inputs

    T.lib()
    fp8v = w.name.endswith("_fp8")
    dev = torch.device("cuda:0")
    eprint(f"[bench] generating inputs for {w.name}")
    q8, qs, k8, ks, v = make_mx_inputs(w.B, w.H, w.N, w.d, w.seed)
    q8d, qsd, k8d, ksd, vd = (t.to(dev) for t in (q8, qs, k8, ks, v))
    if fp8v:
        vt8, vts = make_fp8_v(w.B, w.H, w.N, w.d, w.seed + 1)
        vt8d, vtsd = vt8.to(dev), vts.to(dev)
    o = torch.empty_like(vd)
    lse = torch.empty((w.B, w.H, w.N), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()

    def step():
        if fp8v:
            T.attn_fwd_fp8(q8d, qsd, k8d, ksd, vt8d, vtsd, o, lse, w.causal, w.scale, stream)
        else:
            T.attn_fwd_mx(q8d, qsd, k8d, ksd, vd, o, lse, w.causal, w.scale, stream)

    eprint(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    eprint(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    flops = w.fwd_flops()
    value = flops * args.steps / wall / 1e12
    achieved = flops / (call_ms * 1e-3) / 1e12
    if fp8v:
        # both products on the FP8 matrix rate
        peak = PEAK_FP8_TFLOPS
        note = "S and P V on FP8 MFMA (5.0 PFLOP/s)"
    else:
        # half the FLOPs (S = Q K^T) on the FP8 matrix rate, half (P V) on bf16
        peak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
        note = "S on FP8 MFMA (5.0 PFLOP/s), P V on bf16 (2.5 PFLOP/s), half the FLOPs each"
    roofline = {"kernel": "fwd_fp8" if fp8v else "fwd_mx", "bound": "mfma",
                "achieved": round(achieved, 1), "peak": round(peak, 1), "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None, "peak_note": note,
                "avg_launch_us": round(call_ms * 1e3, 2),
                "vs_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        lib = oracle.load()
        import numpy as np
        heads, t0c = 0, time.perf_counter()
        for b in range(w.B):
            for h in range(w.H):
                qh = oracle.mx_decode(q8[b, h], qs[b, h], lib=lib)
                kh = oracle.mx_decode(k8[b, h], ks[b, h], lib=lib)
                if fp8v:
                    vh = oracle.mx_decode(vt8[b, h], vts[b, h], lib=lib)[:, :w.N].T.copy()
                else:
                    vh = v[b, h].double().numpy()
                oracle.attn_fwd(qh, kh, vh, w.causal,
                                float(np.float32(w.scale)), lib=lib)
                heads += 1
                if time.perf_counter() - t0c >= args.cpu_baseline_seconds:
                    break
            else:
                continue
            break
        el = time.perf_counter() - t0c
        cpu = {"value": flops / (w.B * w.H) * heads / el / 1e12, "unit": "TFLOP/s",
               "cores": oracle.num_threads(lib), "kind": "oracle",
               "sample": f"{heads} of {w.B * w.H} heads of {w.name} (decode + fp64 forward "
                         f"per head), {el:.1f} s"}
    out = {
        "metric": (f"fused attention fwd TFLOP/s, Q, K and V in MXFP8, P in E4M3, {w.name}"
                   if fp8v else f"fused attention fwd TFLOP/s, Q and K in MXFP8, {w.name}"),
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8-e4m3 (Q, K, V, P; E8M0 block scales) / bf16 (O)" if fp8v
                  else "fp8-e4m3 (Q, K; E8M0 block scales) / bf16 (V, P, O)"),
        "data": ("synthetic (seeded N(0,1) cast to E4M3, random E8M0 scales 2^-2..2^2; V^T " + ("E4M3 with scales per 32 keys)" if fp8v else "bf16 V)")),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "step": "attn_fwd_mx"},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-all", action="store_true",
                    help="time the oracle on a bounded sample of every attention workload "
                         "(host only, no GPU) and print one JSON line per workload")
    ap.add_argument("--copy-mib", type=float, default=0.0,
                    help="run one plain device copy of this many MiB before timing "
                         "(reference kernel for the HBM byte counters)")
    ap.add_argument("--peak", action="store_true",
                    help="measure the chip's ceilings (MFMA rate alone and with the softmax's "
                         "VALU work, shader clock, v_exp_f32 rate, HBM copy) and print them")
    ap.add_argument("--no-peak", action="store_true",
                    help="leave the measured ceilings out of the report line")
    ap.add_argument("--pmc-summary", nargs="+", default=None, metavar="DIR",
                    help="summarise rocprofv3 FETCH_SIZE/WRITE_SIZE passes into "
                         "profiles/traffic.json and exit (needs --copy-mib of the profiled run)")
    args = ap.parse_args()

    if args.pmc_summary:
        from attn_inputs import HEADLINE
        sys.exit(pmc_summary(args.pmc_summary, args.copy_mib, args.workload or HEADLINE))

    if args.cpu_baseline_all:
        sys.exit(cpu_baseline_all(args.cpu_baseline_seconds))

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        eprint("bench.py: the library runs on exactly one GPU; multi-GPU runs are not "
               "supported (heads would shard across GPUs with no exchange).")
        sys.exit(2)

    import torch

    import tiled_online_softmax_attn_amd as T
    from attn_inputs import (HEADDIM_WORKLOADS, HEADLINE, KV_WORKLOADS, MX_WORKLOADS,
                             SOFTMAX_WORKLOADS, WORKLOADS, workload_inputs)

    if not torch.cuda.is_available():
        eprint("bench.py needs a GPU")
        sys.exit(1)
    if args.peak:
        eprint("[bench] measuring the chip's ceilings")
        print(json.dumps({"peak_measured": measure_peaks(full=True),
                          "peak_nominal": {"mfma_bf16_tflops": PEAK_BF16_TFLOPS,
                                           "hbm_gbs": PEAK_HBM_GBS}}), flush=True)
        return
    if args.workload in KV_WORKLOADS:
        wk = KV_WORKLOADS[args.workload]
        (bench_kv_fwdbwd if wk.backward else bench_kv)(args, wk)
        return
    if args.workload in SOFTMAX_WORKLOADS:
        bench_softmax(args, SOFTMAX_WORKLOADS[args.workload])
        return
    if args.workload in MX_WORKLOADS:
        bench_mx(args, MX_WORKLOADS[args.workload])
        return
    w = {**WORKLOADS, **HEADDIM_WORKLOADS}[args.workload or HEADLINE]
    # the backward is built for bf16; in fp32 a step is the forward alone
    backward = w.dtype == torch.bfloat16
    run_kernels = KERNELS if backward else KERNELS[:1]
    T.lib()
    dev = torch.device("cuda:0")
    eprint(f"[bench] generating inputs for {w.name}")
    q, k, v, do = workload_inputs(w, with_dout=True)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    B, H, N, d = w.B, w.H, w.N, w.d
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = torch.empty(max(1, T.attn_bwd_workspace_bytes(B, H, N, d, w.dtype)), device=dev,
                     dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        T.attn_fwd(qd, kd, vd, o, lse, w.causal, w.scale, stream)
        if events is not None:
            events[1].record(stream)
        if not backward:
            return
        for i, ph in enumerate(BWD_PHASES):
            T.attn_bwd_phase(ph, qd, kd, vd, o, dod, lse, dq, dk, dv, ws, w.causal, w.scale,
                             stream)
            if events is not None:
                events[2 + i].record(stream)

    copy_reference(args.copy_mib)

    eprint(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(run_kernels) + 1)]
           for _ in range(args.steps)]
    eprint(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_kernel_ms = {kn: 0.0 for kn in run_kernels}
    samples = {kn: [] for kn in run_kernels}
    for e in evs:
        for i, kn in enumerate(run_kernels):
            t = e[i].elapsed_time(e[i + 1])
            per_kernel_ms[kn] += t
            samples[kn].append(t)
    event_total_ms = evs[0][0].elapsed_time(evs[-1][-1])
    ms_per_step = wall * 1e3 / args.steps
    flops_step = w.fwd_flops() + (w.bwd_flops() if backward else 0.0)
    value = flops_step * args.steps / wall / 1e12

    kernels = {}
    for kn in run_kernels:
        avg_ms = per_kernel_ms[kn] / args.steps
        amount, unit, bound = algorithmic(w, kn)
        if unit == "flop":
            achieved, u = amount / (avg_ms * 1e-3) / 1e12, "TFLOP/s"
            peak = PEAK_F32_VALU_TFLOPS if bound == "alu" else PEAK_BF16_TFLOPS
        else:
            achieved, peak, u = amount / (avg_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
        srt = sorted(samples[kn])
        kernels[kn] = {"avg_ms": round(avg_ms, 5), "median_ms": round(srt[len(srt) // 2], 5),
                       "min_ms": round(srt[0], 5), "bound": bound, "achieved": round(achieved, 2),
                       "peak": peak, "unit": u, "frac": round(achieved / peak, 4),
                       "traffic": measured_traffic(kn, w.name)}
        if kn == "bwd_dq":
            # of dQ's three block products only dQ = dS K is the method's
            # work (S and dP are recomputed): its rate counted that way
            algo = w.fwd_flops() / 2 / (avg_ms * 1e-3) / 1e12
            kernels[kn]["achieved_algorithmic"] = round(algo, 2)
            kernels[kn]["frac_algorithmic"] = round(algo / PEAK_BF16_TFLOPS, 4)
    dominant = max(run_kernels, key=lambda kn: per_kernel_ms[kn])
    dk_ = kernels[dominant]
    roofline = {"kernel": dominant, "bound": dk_["bound"], "achieved": dk_["achieved"],
                "peak": dk_["peak"], "unit": dk_["unit"], "frac": dk_["frac"],
                "traffic": dk_["traffic"]}

    peaks = None
    if not args.no_peak:
        eprint("[bench] measuring the chip's ceilings (after the timed region)")
        peaks = measure_peaks(full=False)
        if roofline["unit"] == "TFLOP/s":
            roofline["peak_measured"] = peaks["mfma_bf16_tflops"]
            roofline["frac_of_measured"] = round(roofline["achieved"] / peaks["mfma_bf16_tflops"], 4)
        else:
            roofline["peak_measured"] = peaks["hbm_copy_gbs"]
            roofline["frac_of_measured"] = round(roofline["achieved"] / peaks["hbm_copy_gbs"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        eprint("[bench] timing the oracle on the host")
        cpu = cpu_baseline(w, q, k, v, do, args.cpu_baseline_seconds, backward)
        if w.name == HEADLINE:
            cpu["single_thread_small_workloads"] = cpu_baseline_single_thread(3.0)

    fwd_ms = kernels["fwd"]["avg_ms"]
    bwd_ms = sum(kernels[kn]["avg_ms"] for kn in run_kernels[1:])
    if w.name == HEADLINE:
        metric = "fused attention fwd/bwd TFLOP/s + % bf16 MFMA peak, causal B4 H16 N4096 d128"
    else:
        metric = f"fused attention {'fwd/bwd' if backward else 'fwd'} TFLOP/s, {w.name}"
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == torch.float32 else "bf16",
        "data": (f"synthetic (seeded N(0,1) {'fp32' if w.dtype == torch.float32 else 'bf16'} "
                 f"Q, K, V{', dO' if backward else ''})"),
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "step": "forward + backward" if backward else "forward"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(w.fwd_flops() / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(w.bwd_flops() / (bwd_ms * 1e-3) / 1e12, 2) if backward else None,
        "event_ms_per_step": round(event_total_ms / args.steps, 4),
        "roofline": roofline,
        "kernels": kernels,
        "peak_measured": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
