"""Throughput of the KDA chunked forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

A step is one kda_chunk_fwd call over the whole workload (gate, in-chunk
tiles, UT/WY solve, inter-chunk scan, outputs and statistics), inputs already
resident in HBM.  Prints ONE JSON line on stdout; diagnostics go to stderr.

The default workload is B=1, H=16, T=65536, dk=dv=128, bf16, g_min=-5,
chunk 16, S0 = 0 (synthetic inputs, seeded).  `roofline` uses the algorithmic
bytes of one launch (q, k, v, w, beta read, o written: 1282 B per token-head at
d = 128 in bf16, plus the fp32 final state) over the average duration of the
call's kernels (on the automatic path at this shape, the corrected plan: the
segment pass, the chaining of the segment maps and the correction pass, back
to back on one stream), timed with HIP events that
the library records on the launch stream before the first kernel and after the
last.
`cpu_baseline` times the fp64 oracle on the host on a bounded sample of the
same workload (all heads, the first tokens of the sequence).

Defaults: 40 untimed warm-up calls, then 50 timed ones.  The GPU needs about
35 ms of back-to-back calls before their duration settles (after start-up the
first call takes about 1.3 ms, calls 4-8 0.72-0.81 ms, the settled ones about
0.61-0.63 ms, as the clock settles to the load), so the warm-up spans that ramp
and the timed calls do not.  `--heads H` runs the workload with H heads and
`--seg-steps N` fixes the matrix-core plan's segment length (N steps of 32
tokens): together they hold each workgroup's work fixed while the number of
busy compute units changes.

Other modes print a line of the same form for other entry points:
`--mode decode` one recurrent decode call over a serving batch (kda_decode,
HBM roofline over the state read and written), `--mode bwd` one backward call
(kda_chunk_bwd, fp32 vector-ALU roofline over the state-sized contractions).
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

METRIC = "KDA chunk-fwd tokens/s (H16,d128,T64K,bf16) + % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
# fp32 vector peak: 256 CUs x 2.4 GHz x 128 fp32 FMA lanes per CU per clock x 2 flops
FP32_VALU_PEAK_TFLOPS = 157.3
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["chunked_gated_delta_amd/csrc/kda_mfma.hip", "chunked_gated_delta_amd/csrc/kda_fused.hip",
                  "chunked_gated_delta_amd/csrc/kda_mfma_util.h", "chunked_gated_delta_amd/csrc/kda_common.hip",
                  "chunked_gated_delta_amd/csrc/kda_host.cpp", "chunked_gated_delta_amd/csrc/kda_internal.h"]


def code_text(src: str) -> str:
    """C++/HIP source without its comments and with whitespace runs collapsed: what the compiler
    sees, so that an edit of a comment leaves the hash of the kernels alone."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash(read=None) -> str:
    """Hash of the code (comments aside) of the kernel sources the committed counters describe."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def kernel_short_name(name):
    """Short name of a library kernel (or of the calibration copy) in a rocprofv3 record."""
    for key, short in (("fused_kernel<true", "fused_out"), ("fused_kernel<false", "fused_state"),
                       ("fused_corr_kernel", "corr_pass"), ("correct_kernel", "correct"),
                       ("seg_combine_kernel", "seg_combine"), ("vec_", "vector")):
        if key in name:
            return short
    if "copyBuffer" in name or "elementwise_kernel<16" in name:
        return "copy"
    return None


def _pmc_per_kernel(csv_path, counter):
    """{kernel short name: value of `counter` in the last dispatch, summed over its instances}."""
    import csv
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        short = kernel_short_name(r["Kernel_Name"])
        if short:
            per[short][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {k: v[max(v)] for k, v in per.items()}


def summarize_pmc(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out_json, workload):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what they read for a 1 GiB copy, and store
    the HBM bytes per forward call (every kernel of the call) together with the kernel source hash."""
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = float(1 << 30)
    f_scale = copy_bytes / (1024.0 * _pmc_per_kernel(copy_fetch_csv, "FETCH_SIZE")["copy"])
    w_scale = copy_bytes / (1024.0 * _pmc_per_kernel(copy_write_csv, "WRITE_SIZE")["copy"])
    kernels = {}
    for k in sorted((set(fetch) | set(write)) - {"copy"}):
        kernels[k] = {"fetch_bytes": fetch.get(k, 0.0) * 1024 * f_scale, "write_bytes": write.get(k, 0.0) * 1024 * w_scale}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in kernels.values())
    out = {"workload": workload, "source_hash": source_hash(), "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": kernels, "bytes_per_call": total}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def measured_traffic(workload):
    """HBM bytes per call from the committed counter summary, if it matches the current kernels."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != source_hash() or d.get("workload") != workload:
        return None
    return d["bytes_per_call"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl) -> int:
    esz = 2 if wl.dtype == "bf16" else 4
    per_token_head = (3 * wl.dk + 2 * wl.dv) * esz + esz       # q, k, w, v in; o out; beta in
    state = wl.B * wl.H * wl.dk * wl.dv * 4                      # S_final out
    if wl.s0_sd is not None:
        state *= 2                                               # S0 in
    return wl.token_heads * per_token_head + state


def mfma_flops(wl) -> float:
    """Matrix-core work of the chunk-16 form per launch (2 flops per multiply-add):
    per chunk, Q K^T-style tiles (2 x C*C*dk), W and U~ (C*C*dk + C*C*dv),
    and the state products W S, Q S, K^T U (3 x C*dk*dv), plus P U (C*C*dv)."""
    C = 16
    per_chunk = 2 * (2 * C * C * wl.dk + C * C * wl.dk + C * C * wl.dv + 3 * C * wl.dk * wl.dv + C * C * wl.dv)
    return per_chunk * wl.B * wl.H * math.ceil(wl.T / C)


def cpu_baseline(inp, wl, target_s: float = 15.0):
    import numpy as np
    from chunked_gated_delta_amd import inputs as gen
    from oracle import oracle as orc
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(cores, 16, wl.B * wl.H))
    # sample: every (b, h), the first Ts tokens; Ts sized from a short calibration run
    cal_T = min(wl.T, 512)
    f = {k: (None if inp[k] is None else inp[k][:, :, :cal_T].float().cpu().numpy().astype(np.float64))
         for k in ("q", "k", "v", "w", "beta")}
    S0 = None if inp["S0"] is None else inp["S0"].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], S0, wl.g_min, nthreads=threads)
    cal = time.perf_counter() - t0
    Ts = int(min(wl.T, max(cal_T, cal_T * target_s / max(cal, 1e-3))))
    Ts = max(16, (Ts // 16) * 16)
    f = {k: inp[k][:, :, :Ts].float().cpu().numpy().astype(np.float64) for k in ("q", "k", "v", "w", "beta")}

    def run():
        t0 = time.perf_counter()
        orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], S0, wl.g_min, nthreads=threads)
        return time.perf_counter() - t0

    # where the whole sequence takes less than the target, the sample is run again back to back
    dt, reps = run(), 1
    while dt < target_s and reps < 100:
        dt += run()
        reps += 1
    return {
        "value": wl.B * Ts * reps / dt,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"all {wl.B * wl.H} (b,h) recurrences over the first {Ts} of {wl.T} tokens, {reps} runs "
                  f"(fp64 token-by-token, {threads} threads, {dt:.1f} s wall)",
    }


def sampled_heads(wl):
    """(b, h) pairs checked against the oracle at full size: every head of a small workload, else the
    first and the last."""
    if wl.B * wl.H <= 2:
        return [(b, h) for b in range(wl.B) for h in range(wl.H)]
    return [(0, 0), (wl.B - 1, wl.H - 1)]


def _tok_f64(x, heads, lo, hi):
    """Tokens [lo, hi) of the sampled heads of a [B,H,T,...] tensor, stacked as a batch of one-head
    sequences, in fp64."""
    import numpy as np
    return np.stack([x[b, h, lo:hi].float().cpu().numpy() for b, h in heads])[:, None].astype(np.float64)


def _state_f64(S, heads):
    """The sampled heads of a [B,H,dk,dv] state (None stays None), in fp64."""
    import numpy as np
    if S is None:
        return None
    return np.stack([S[b, h].float().cpu().numpy() for b, h in heads])[:, None].astype(np.float64)


def accuracy(inp, wl, o, S, threads):
    """err(o), err(S_final) = max |x - ref| / max |ref| on the sampled heads, against the fp64 oracle."""
    import numpy as np
    from oracle import oracle as orc
    heads = sampled_heads(wl)
    T = wl.T
    f = {n: _tok_f64(inp[n], heads, 0, T) for n in ("q", "k", "v", "w", "beta")}
    S0 = _state_f64(inp["S0"], heads)
    t0 = time.perf_counter()
    o_ref, S_ref = orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], S0, wl.g_min,
                                     nthreads=min(threads, len(heads)))
    dt = time.perf_counter() - t0
    og = np.stack([o[b, h].float().cpu().numpy() for b, h in heads])[:, None]
    Sg = np.stack([S[b, h].cpu().numpy() for b, h in heads])[:, None]
    err = lambda x, r: float(np.max(np.abs(x - r)) / np.max(np.abs(r)))
    return {"heads": [list(x) for x in heads], "err_o": err(og, o_ref), "err_S": err(Sg, S_ref),
            "oracle_s": round(dt, 1)}


def state_drift(inp, wl, threads, checkpoints):
    """S at each checkpoint T_i from chained GPU calls (the state of one call is the S0 of the next),
    against the fp64 oracle chained the same way (exact in fp64), on the sampled heads:
    [(T_i, err(S(T_i)), max |S_ref(T_i)|)]."""
    import numpy as np
    import torch
    from chunked_gated_delta_amd import chunk_fwd
    from oracle import oracle as orc
    heads = sampled_heads(wl)
    out, S_gpu, S_ref, lo = [], inp["S0"], _state_f64(inp["S0"], heads), 0
    for hi in checkpoints:
        sl = {n: inp[n][:, :, lo:hi].contiguous() for n in ("q", "k", "v", "w", "beta")}
        _, S_gpu, _ = chunk_fwd(sl["q"], sl["k"], sl["v"], sl["w"], sl["beta"], S_gpu, g_min=wl.g_min)
        torch.cuda.synchronize()
        f = {n: _tok_f64(inp[n], heads, lo, hi) for n in ("q", "k", "v", "w", "beta")}
        _, S_ref = orc.kda_reference(f["q"], f["k"], f["v"], f["w"], f["beta"], S_ref, wl.g_min,
                                     nthreads=min(threads, len(heads)))
        Sg = np.stack([S_gpu[b, h].cpu().numpy() for b, h in heads])[:, None]
        out.append([hi, float(np.max(np.abs(Sg - S_ref)) / np.max(np.abs(S_ref))), float(np.max(np.abs(S_ref)))])
        log(f"[bench] drift T={hi}: err(S)={out[-1][1]:.3e} max|S_ref|={out[-1][2]:.3e}")
        lo = hi
    return out


def decode_bytes(wl) -> int:
    """HBM bytes one decode call must move: the fp32 state read and written, plus the token's inputs
    and output (q, k, w, v, beta in, o out)."""
    esz = 2 if wl.dtype == "bf16" else 4
    state = wl.B * wl.H * wl.dk * wl.dv * 4 * 2
    return state + wl.token_heads * ((3 * wl.dk + 2 * wl.dv) * esz + esz)


def bench_decode(args, torch, gen):
    """Recurrent decode: one kda_decode call per step over a serving batch, states resident."""
    from chunked_gated_delta_amd import decode
    wl = gen.WORKLOADS["decode_b512" if args.workload == "headline" else args.workload]
    log(f"[bench] decode workload {wl}")
    t = gen.make_torch(wl, seed=args.seed, device="cuda")
    S = t["S0"].clone()
    o = torch.empty_like(t["v"])
    q, k, v, w, beta = (t[n] for n in ("q", "k", "v", "w", "beta"))
    for _ in range(args.warmup):
        decode(q, k, v, w, beta, S, g_min=wl.g_min, out=o)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        decode(q, k, v, w, beta, S, g_min=wl.g_min, out=o)
        evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = [a.elapsed_time(b) for a, b in evs]
    kern_avg = sum(kern) / len(kern)
    nbytes = decode_bytes(wl)
    achieved = nbytes / (kern_avg * 1e-3) / 1e9
    log(f"[bench] decode kernel ms: avg {kern_avg:.5f} min {min(kern):.5f} max {max(kern):.5f}; wall/step "
        f"{1e3 * wall / args.steps:.5f} ms")
    line = {
        "metric": "KDA recurrent decode tokens/s (B512 H16 d128, bf16 in, fp32 state)",
        "value": round(wl.B * wl.T / (wall / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "dk": wl.dk, "dv": wl.dv,
                   "g_min": wl.g_min if math.isfinite(wl.g_min) else "-inf", "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": nbytes,
                     "kernel_ms": round(kern_avg, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bwd_flops(wl) -> float:
    """Arithmetic of the chunk-form backward per launch (2 flops per multiply-add), counting only the
    state-sized contractions, per 16-token chunk and C*dk*dv each: the state chain recomputed
    (E = V - Kbar S and S' = e^Gam S + Ktil^T U: 2), dU's Ktil dS', dQbar = dO S^T,
    dKbar = dR S^T, dKtil = U dS'^T (4) and dS = Qbar^T dO - Kbar^T dR (2): 8 C dk dv multiply-adds.
    The C x C blocks (X, P, T, dA, dP) add under 10% at d = 128 and are left out."""
    C = 16
    return 2.0 * 8 * C * wl.dk * wl.dv * wl.B * wl.H * math.ceil(wl.T / C)


def bwd_bytes(wl) -> int:
    """HBM bytes a backward call must move: q, k, w, v, beta and dO in (input dtype), dq, dk, dw,
    dv and dbeta out (fp32), and the state-sized S0, dS_final in and dS0 out."""
    esz = 2 if wl.dtype == "bf16" else 4
    per_token_head = (3 * wl.dk + 2 * wl.dv + 1) * esz + (3 * wl.dk + wl.dv + 1) * 4
    state = wl.B * wl.H * wl.dk * wl.dv * 4 * (3 if wl.s0_sd is not None else 2)
    return wl.token_heads * per_token_head + state


def cpu_baseline_bwd(inp, dO, dSf, wl, target_s: float = 15.0):
    import numpy as np
    from oracle import oracle as orc
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(cores, 16, wl.B * wl.H))

    def run(Ts):
        f = {k: inp[k][:, :, :Ts].float().cpu().numpy().astype(np.float64) for k in ("q", "k", "v", "w", "beta")}
        S0 = None if inp["S0"] is None else inp["S0"].cpu().numpy().astype(np.float64)
        d = dO[:, :, :Ts].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        orc.kda_backward(f["q"], f["k"], f["v"], f["w"], f["beta"], S0, wl.g_min, d,
                         dSf.cpu().numpy().astype(np.float64), nthreads=threads)
        return time.perf_counter() - t0

    # the oracle keeps every state of a head (T * dk * dv * 8 bytes per thread), so the sample is the
    # first Ts <= 1024 tokens of every head, run `reps` times back to back for a stable timing
    Ts = max(16, (min(wl.T, 1024) // 16) * 16)
    cal = run(Ts)
    reps = int(max(1, min(200, target_s / max(cal, 1e-3))))
    dt = sum(run(Ts) for _ in range(reps))
    return {
        "value": wl.B * Ts * reps / dt,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"all {wl.B * wl.H} (b,h) adjoint recurrences over the first {Ts} of {wl.T} tokens, "
                  f"{reps} runs (fp64, states kept per token, {threads} threads, {dt:.1f} s wall)",
    }


def bench_bwd(args, torch, gen):
    """Backward of the chunked forward: one kda_chunk_bwd call per step on the headline shape."""
    from chunked_gated_delta_amd import chunk_bwd
    wl = gen.WORKLOADS[args.workload]
    log(f"[bench] backward workload {wl}")
    inp = gen.make_torch(wl, seed=args.seed, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(args.seed + 1)
    dO = torch.randn((wl.B, wl.H, wl.T, wl.dv), generator=g, device="cuda").to(gen.torch_dtype(wl.dtype))
    dSf = torch.randn((wl.B, wl.H, wl.dk, wl.dv), generator=g, device="cuda")
    q, k, v, w, beta, S0 = (inp[n] for n in ("q", "k", "v", "w", "beta", "S0"))
    ws = torch.empty(gen_bwd_ws(wl), dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        chunk_bwd(q, k, v, w, beta, dO, S0=S0, dS_final=dSf, g_min=wl.g_min, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        chunk_bwd(q, k, v, w, beta, dO, S0=S0, dS_final=dSf, g_min=wl.g_min, workspace=ws, stream=stream,
                  events=evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = [a.elapsed_time(b) for a, b in evs]
    kern_avg = sum(kern) / len(kern)
    log(f"[bench] backward call ms: avg {kern_avg:.4f} min {min(kern):.4f} max {max(kern):.4f}; wall/step "
        f"{1e3 * wall / args.steps:.4f} ms")
    flops = bwd_flops(wl)
    tflops = flops / (kern_avg * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle backward on the host ...")
        cpu = cpu_baseline_bwd(inp, dO, dSf, wl)
        log(f"[bench] cpu_baseline {cpu}")
    line = {
        "metric": "KDA chunked backward tokens/s (B1 H16 T65536 d128, bf16 in, fp32 gradients)",
        "value": round(wl.B * wl.T / (wall / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "dk": wl.dk, "dv": wl.dv,
                   "chunk": 16, "g_min": wl.g_min if math.isfinite(wl.g_min) else "-inf",
                   "inputs": wl.dtype, "parallelism": "single-gpu"},
        "roofline": {"bound": "alu", "achieved": round(tflops, 3), "peak": FP32_VALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / FP32_VALU_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": flops, "kernel_ms": round(kern_avg, 5),
                     "hbm_gbs": round(bwd_bytes(wl) / (kern_avg * 1e-3) / 1e9, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def gen_bwd_ws(wl) -> int:
    from chunked_gated_delta_amd import _lib
    from chunked_gated_delta_amd.api import make_shape
    code = _lib.DTYPE_BF16 if wl.dtype == "bf16" else _lib.DTYPE_F32
    return max(1, _lib.bwd_workspace_bytes(make_shape(wl.B, wl.H, wl.T, wl.dk, wl.dv, code), 16))


def phase_stamps(args):
    """--phase-stamps BLOCK: the workload's forward (automatic plan) through libkda_stamps.so, in which
    lane 0 of every wavefront of the segment pass's workgroup BLOCK records the shader clock
    (s_memtime) at six phase boundaries of each of the segment's first 48 intervals, into the end of
    the workspace.  After `--warmup` calls one more call is stamped, and the median over intervals
    6-46 of each phase's length (in shader-clock cycles) is printed per wavefront.  State wavefronts
    0-7: chain (the state step of step s), tile+V (a causal tile of step s+1, the V copy, and on
    wavefronts 6-7 of a corrected segment their transition slices), bar1 (wait at the first barrier),
    store (output rows and V staging), solve (the diagonal solve, wavefronts 6-7), bar2 (the rest up to
    the next interval: on wavefronts 4-5 of a corrected segment their transition slices, then the
    wait).  E wavefronts 8-15: E1, load (issue of the next step's inputs), trans (the transition
    slices of the chunk-0 group in a corrected segment), bar1, E2, bar2."""
    os.environ["KDA_LIB_PATH"] = os.path.join(ROOT, "chunked_gated_delta_amd", "libkda_stamps.so")
    os.environ["KDA_STAMP_BLOCK"] = str(args.phase_stamps)
    import statistics
    import torch
    from chunked_gated_delta_amd import chunk_fwd, workspace_bytes
    from chunked_gated_delta_amd import inputs as gen
    wl = gen.WORKLOADS[args.workload]
    if args.heads:
        wl = wl.with_(H=args.heads)
    t = gen.make_torch(wl, seed=args.seed, device="cuda")
    ws_n = workspace_bytes(wl.B, wl.H, wl.T, wl.dk, wl.dv, gen.torch_dtype(wl.dtype))
    ksteps, kk, nwaves = 48, 6, 16
    stamp_bytes = nwaves * ksteps * kk * 8
    if ws_n < stamp_bytes:
        sys.exit("--phase-stamps needs the matrix-core path (bf16, dk = dv = 128)")
    ws = torch.zeros(ws_n, dtype=torch.uint8, device="cuda")
    names = ("q", "k", "v", "w", "beta")
    for _ in range(max(1, args.warmup)):
        chunk_fwd(*(t[n] for n in names), t["S0"], g_min=wl.g_min, workspace=ws, seg_steps=args.seg_steps)
    torch.cuda.synchronize()
    ws[ws_n - stamp_bytes:].zero_()
    chunk_fwd(*(t[n] for n in names), t["S0"], g_min=wl.g_min, workspace=ws, seg_steps=args.seg_steps)
    torch.cuda.synchronize()
    pr = ws[ws_n - stamp_bytes:].view(torch.int64).cpu().tolist()
    print(f"phase stamps: workload {wl.name} (B{wl.B} H{wl.H} T{wl.T}), segment-pass workgroup {args.phase_stamps}, "
          f"median shader-clock cycles per 32-token step over intervals 6-46", flush=True)
    for w in range(nwaves):
        rows = []
        for it in range(6, ksteps - 1):
            a = pr[(w * ksteps + it) * kk:(w * ksteps + it + 1) * kk]
            nxt = pr[(w * ksteps + it + 1) * kk]
            if a[0] == 0 or a[3] == 0 or nxt == 0:
                continue
            rows.append([a[1] - a[0], a[2] - a[1], a[3] - a[2], a[4] - a[3], a[5] - a[4], nxt - a[5], nxt - a[0]])
        if not rows:
            continue
        med = [int(statistics.median(c)) for c in zip(*rows)]
        lab = (["chain", "tile+V", "bar1", "store", "solve", "bar2", "step"] if w < 8
               else ["E1", "load", "trans", "bar1", "E2", "bar2", "step"])
        print(f"wave {w:2d}: " + "  ".join(f"{l}={m}" for l, m in zip(lab, med)), flush=True)


def phase_stamps_bwd(args):
    """--mode bwd --phase-stamps BLOCK: the backward through libkda_stamps.so, in which lane 0 of every
    wavefront of the chain kernel's workgroup BLOCK (blocks below B*H*dv/16 run the forward chain, the
    rest the reverse one) records the shader clock at four points of each of the first 48 chunks.
    After `--warmup` calls one more call is stamped, and the median over chunks 6-46 of each phase's
    length (shader-clock cycles) is printed per wavefront.  Compute wavefronts (0-3 at dk = 128): work1
    (the state store, the chunk's partial product and its LDS write), barrier, work2 (summing the
    partials, the next chunk's operands, the update).  Loader wavefronts: landed (the wait until the
    next chunk's copies have landed), barrier, issue (issuing the copies of a chunk kDepth ahead)."""
    os.environ["KDA_LIB_PATH"] = os.path.join(ROOT, "chunked_gated_delta_amd", "libkda_stamps.so")
    os.environ["KDA_STAMP_BLOCK"] = str(args.phase_stamps)
    os.environ["KDA_STAMP_KERNEL"] = "grad" if args.stamp_grad else "chain"
    import statistics
    import torch
    from chunked_gated_delta_amd import chunk_bwd
    from chunked_gated_delta_amd import inputs as gen
    wl = gen.WORKLOADS[args.workload]
    if args.heads:
        wl = wl.with_(H=args.heads)
    inp = gen.make_torch(wl, seed=args.seed, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(args.seed + 1)
    dO = torch.randn((wl.B, wl.H, wl.T, wl.dv), generator=g, device="cuda").to(gen.torch_dtype(wl.dtype))
    dSf = torch.randn((wl.B, wl.H, wl.dk, wl.dv), generator=g, device="cuda")
    q, k, v, w, beta, S0 = (inp[n] for n in ("q", "k", "v", "w", "beta", "S0"))
    ws_n = gen_bwd_ws(wl)
    ksteps, kk, nwaves = 48, 6, 16
    stamp_bytes = nwaves * ksteps * kk * 8
    ws = torch.zeros(ws_n, dtype=torch.uint8, device="cuda")
    for _ in range(max(1, args.warmup)):
        chunk_bwd(q, k, v, w, beta, dO, S0=S0, dS_final=dSf, g_min=wl.g_min, workspace=ws)
    torch.cuda.synchronize()
    ws[ws_n - stamp_bytes:].zero_()
    chunk_bwd(q, k, v, w, beta, dO, S0=S0, dS_final=dSf, g_min=wl.g_min, workspace=ws)
    torch.cuda.synchronize()
    pr = ws[ws_n - stamp_bytes:].view(torch.int64).cpu().tolist()
    if args.stamp_grad:
        grad_stamps(wl, args.phase_stamps, pr, ksteps, kk)
        return
    nchain = wl.B * wl.H * (wl.dv // 16)
    nw = wl.dk // 32
    kind = "forward" if args.phase_stamps < nchain else "reverse"
    print(f"phase stamps: backward of {wl.name} (B{wl.B} H{wl.H} T{wl.T}), chain workgroup {args.phase_stamps} "
          f"({kind} chain), median shader-clock cycles per 16-token chunk over chunks 6-46", flush=True)
    for wv in range(nwaves):
        rows = []
        for n in range(6, ksteps - 1):
            a = pr[(wv * ksteps + n) * kk:(wv * ksteps + n) * kk + 4]
            nxt = pr[(wv * ksteps + n + 1) * kk]
            if 0 in a or nxt == 0:
                continue
            rows.append([a[1] - a[0], a[2] - a[1], a[3] - a[2], nxt - a[3], nxt - a[0]])
        if not rows:
            continue
        med = [int(statistics.median(c)) for c in zip(*rows)]
        lab = ["work1", "barrier", "work2", "rest", "chunk"] if wv < nw else ["landed", "barrier", "issue", "rest", "chunk"]
        print(f"wave {wv:2d}: " + "  ".join(f"{l}={m}" for l, m in zip(lab, med)), flush=True)


def grad_stamps(wl, block, pr, ksteps, kk):
    """Per wavefront of the gradient kernel's workgroup `block` (one per 16-token chunk): the setup
    (loads: issuing the chunk's w, v and dO loads; setup: the chunk's G, X, P and T, split into the
    loads of q, k, w and beta with the gates written to LDS, the barrier, the prefix, X and P, the
    sums of their partials and the solve for T; operands: the
    first products' A operands; wait: until the first S and dS' tiles have landed), the median over
    the value tiles of each tile phase (partial: the tile's K = dk partial products; bar1; single: E,
    U, dU, dR and dv on one wavefront each; bar2; products: the K = 16 products, dT, dP and dbeta;
    wait: until the next tile pair has landed, with the barrier), then the epilogue (dA: dT and dP
    out of the accumulators, T^T dT, dA and dbeta; pairs: the pair terms of X and P; scalings: the
    K = 16 products through the scalings of Qbar, Kbar and Ktil; outputs: dg, dw, dq and dk)."""
    import statistics
    nc = (wl.T + 15) // 16

    def at(wv, n, k):
        return pr[(wv * ksteps + n) * kk + k]

    print(f"phase stamps: backward of {wl.name} (B{wl.B} H{wl.H} T{wl.T}), gradient workgroup {block} "
          f"(head {block // nc}, chunk {block % nc}), shader-clock cycles", flush=True)
    ntile = wl.dv // 16
    lab = ["partial", "bar1", "single", "bar2", "products", "wait", "tile"]
    for wv in range(8):
        s = [at(wv, 8, k) for k in range(5)]
        if 0 in s:
            continue
        rows = []
        for t in range(ntile):
            a = [at(wv, t, k) for k in range(6)]
            nxt = at(wv, t + 1, 0) if t + 1 < ntile else at(wv, 9, 0)
            if 0 in a or nxt == 0:
                continue
            rows.append([a[1] - a[0], a[2] - a[1], a[3] - a[2], a[4] - a[3], a[5] - a[4], nxt - a[5], nxt - a[0]])
        med = [int(statistics.median(c)) for c in zip(*rows)] if rows else []
        e = [at(wv, 9, k) for k in range(5)]
        ep = (f"dA={e[1] - e[0]} pairs={e[2] - e[1]} scalings={e[3] - e[2]} outputs={e[4] - e[3]} "
              f"total={e[4] - s[0]}") if 0 not in e else "-"
        c = [at(wv, 10, k) for k in range(5)]
        sub = (f" (inputs={c[0] - s[1]} bar={c[1] - c[0]} prefix={c[2] - c[1]} XP={c[3] - c[2]} sums={c[4] - c[3]} "
               f"T={s[2] - c[4]})") if 0 not in c else ""
        print(f"wave {wv}: loads={s[1] - s[0]} setup={s[2] - s[1]}{sub} operands={s[3] - s[2]} wait={s[4] - s[3]} | "
              f"tiles (median of {len(rows)}): " + " ".join(f"{n}={m}" for n, m in zip(lab, med)) +
              f" | epilogue: {ep}", flush=True)


def oracle_threads(wl) -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(cores, 16, wl.B * wl.H))


def time_forward(torch, inp, wl, g_min, steps, warmup, kw):
    """`warmup` untimed calls, then `steps` timed ones; returns (average kernel ms over the call's
    kernels from HIP events on the launch stream, per-call kernel ms, wall seconds of the timed calls,
    statistics, o, S_final)."""
    from chunked_gated_delta_amd import HipEvent, chunk_fwd, decode_stats
    q, k, v, w, beta, S0 = (inp[n] for n in ("q", "k", "v", "w", "beta", "S0"))
    o = torch.empty_like(v)
    S = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    st = None
    for _ in range(warmup):
        _, _, st = chunk_fwd(q, k, v, w, beta, S0, out=o, S_final=S, g_min=g_min, **kw)
    torch.cuda.synchronize()
    if st is not None:
        log(f"[bench] warmup stats {decode_stats(st)}")
    evs = [(HipEvent(), HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        _, _, st = chunk_fwd(q, k, v, w, beta, S0, out=o, S_final=S, g_min=g_min, events=evs[i], **kw)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [b.elapsed_ms(e) for b, e in evs]
    return sum(kern_ms) / len(kern_ms), kern_ms, wall, decode_stats(st), o, S


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--path", default="auto", choices=["auto", "vector", "fused", "corr"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-accuracy", action="store_true",
                    help="skip the check of the sampled heads against the fp64 oracle (and, for the "
                         "million workload, the state drift curve)")
    ap.add_argument("--force-fallback", action="store_true",
                    help="every chunk takes a flagged chunk's handling (midpoint tiles or per-pair factors)")
    ap.add_argument("--force-pairwise", action="store_true", help="every chunk takes the per-pair factors")
    ap.add_argument("--stamp-grad", action="store_true",
                    help="with --mode bwd --phase-stamps BLOCK: stamp the gradient kernel's workgroup BLOCK "
                         "instead of the chain kernel's")
    ap.add_argument("--heads", type=int, default=0,
                    help="run the workload with this many heads instead of its own (0: the workload's)")
    ap.add_argument("--seg-steps", type=int, default=0,
                    help="matrix-core paths: fix the segment length in 32-token steps (0: the automatic plan)")
    ap.add_argument("--phase-stamps", type=int, default=None, metavar="BLOCK",
                    help="load libkda_stamps.so and print the median cycles of each phase of the segment pass's "
                         "32-token step, per wavefront, in workgroup BLOCK (head times segments plus segment: 0 is segment 0 of head 0)")
    ap.add_argument("--mode", default="forward", choices=["forward", "decode", "bwd"],
                    help="forward: the chunked forward (the headline); decode: one recurrent decode "
                         "step of a serving batch (workload decode_b512 unless --workload is given); "
                         "bwd: the backward of the chunked forward on the same workload")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain device copy of known size (for scaling HBM counters)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 counter CSVs into profiles/traffic_<workload>.json")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, os.path.join(PROFILES, f"traffic_{args.workload}.json"), args.workload)
        return

    if args.phase_stamps is not None:
        (phase_stamps_bwd if args.mode == "bwd" else phase_stamps)(args)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calib:
        n = 1 << 30
        x = torch.ones(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        log(f"copy_calib: copied {n} bytes x3")
        return

    from chunked_gated_delta_amd import inputs as gen

    if args.mode == "decode":
        bench_decode(args, torch, gen)
        return
    if args.mode == "bwd":
        bench_bwd(args, torch, gen)
        return

    wl = gen.WORKLOADS[args.workload]
    if args.heads:
        wl = wl.with_(H=args.heads)
    log(f"[bench] workload {wl}")
    inp = gen.make_torch(wl, seed=args.seed, device="cuda")
    torch.cuda.synchronize()
    kw = dict(path=args.path, force_fallback=2 if args.force_pairwise else int(args.force_fallback),
              seg_steps=args.seg_steps)
    kern_avg, kern_ms, wall, stats, o, S = time_forward(torch, inp, wl, wl.g_min, args.steps, args.warmup, kw)
    log(f"[bench] kernel ms: avg {kern_avg:.4f} min {min(kern_ms):.4f} max {max(kern_ms):.4f}; wall/step "
        f"{1e3 * wall / args.steps:.4f} ms; stats {stats}")
    extra = {}
    if not math.isfinite(wl.g_min):
        # the same inputs with the bounded gate: the cost of the flagged chunks' per-position blocks
        b_avg, _, b_wall, b_stats, _, _ = time_forward(torch, inp, wl, -5.0, args.steps, args.warmup, kw)
        extra["unbounded"] = {
            "flagged_frac": stats["n_flagged"] / max(1, stats["n_chunks"]),
            "bounded_kernel_ms": round(b_avg, 5), "bounded_value": round(wl.B * wl.T / (b_wall / args.steps), 1),
            "bounded_flagged": b_stats["n_flagged"],
            "throughput_loss": round(1.0 - (b_wall / wall), 4),
            "kernel_time_ratio": round(kern_avg / b_avg, 4)}
        log(f"[bench] bounded gate on the same w: {extra['unbounded']}")
    threads = oracle_threads(wl)
    if not args.no_accuracy:
        extra["accuracy"] = accuracy(inp, wl, o, S, threads)
        log(f"[bench] accuracy {extra['accuracy']}")
    if wl.name == "million" and not args.no_accuracy:
        extra["drift"] = state_drift(inp, wl, threads, [1 << 16, 1 << 18, 1 << 20])
    del o, S

    ms_per_step = 1e3 * wall / args.steps
    tokens = wl.B * wl.T
    value = tokens / (wall / args.steps)
    abytes = algorithmic_bytes(wl)
    achieved = abytes / (kern_avg * 1e-3) / 1e9
    # the stored counters describe the workload's own shape and plan
    traffic = measured_traffic(wl.name) if args.path != "vector" and not (args.heads or args.seg_steps) else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None if traffic is None else round(traffic),
                "bytes_per_launch": abytes, "kernel_ms": round(kern_avg, 5),
                "mfma_tflops": round(mfma_flops(wl) / (kern_avg * 1e-3) / 1e12, 2)}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host ...")
        cpu = cpu_baseline(inp, wl)
        log(f"[bench] cpu_baseline {cpu}")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "dk": wl.dk, "dv": wl.dv,
                   "chunk": wl.chunk, "g_min": wl.g_min if math.isfinite(wl.g_min) else "-inf",
                   "path": args.path, "seg_steps": args.seg_steps or "auto", "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stats": stats,
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
