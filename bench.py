#!/usr/bin/env python3
"""Benchmark of the chunkwise causal linear attention forward pass on one MI355X.

One step = one fla_linattn_fwd call (every stage of the path: load + feature map, decay
factors, intra-chunk, chunk state, inter-chunk scan, output combine) over one batch of
synthetic inputs already resident in HBM.  Default workload: the GLA-gated attention at
B=8, H=16, T=16384, dk=dv=128, bf16, chunk 64.

Prints ONE JSON line: tokens/s (B*T per second), with the roofline of the fused kernel
(algorithmic bytes per launch / average launch time from HIP events on the launch
stream) and the fp64 CPU oracle timed on a bounded sample of the same workload.

--mode bwd times the chunkwise backward instead (one step = one fla_linattn_bwd call:
dq, dk, dv, the decay gradient and the initial state's gradient, for upstream gradients
on the output and the final state), with the same roofline and oracle legs.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# the kernels' sources: counters taken on another version of them do not apply
KERNEL_SOURCES = [os.path.join(ROOT, "chunkwise_causal_linear_amd", "csrc", f)
                  for f in ("chunk_fwd.hpp", "chunk_inst.hip", "dispatch.hpp", "seg_state.hpp",
                            "exact_fwd.hpp", "gdn_fwd.hpp", "gdn_inst.hip", "proj.hpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per step that the FETCH_SIZE / WRITE_SIZE counters read for a workload (the
    committed counter summary), or None when there is none or the kernels' sources have
    changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            tc = json.load(f)
    except (OSError, ValueError):
        return None
    rec = tc.get("workloads", {}).get(name)
    if rec and tc.get("kernel_source_hash") == kernel_source_hash():
        return rec.get("hbm_bytes_per_step")
    return None


def algorithmic(w) -> tuple[float, float]:
    """Bytes the method must move and MFMA FLOPs it must do for one forward pass.
    Bytes: q, k, v, out once; the gate or per-token decay (fp32) once; gamma; the start
    state if given and the end state.  FLOPs per token-head: 2 * [(C+1)/2 * (dk+dv) + 2 * dk * dv] (causal half
    of the intra-chunk products, plus the state read-out and update)."""
    s = 2 if w.dtype == "bf16" else 4
    th = w.B * w.H * w.T
    ncol = w.dv + (1 if w.normalize else 0)
    b = th * (2 * w.dk + 2 * w.dv) * s
    if w.decay == "gate":
        b += th * w.dk * 4
    elif w.decay == "token":
        b += th * 4
    elif w.decay == "gamma":
        b += w.H * 4
    state = w.B * w.H * w.dk * ncol * 4
    b += state * (2 if w.init_sigma > 0 else 1)
    f = th * 2.0 * ((w.chunk + 1) / 2.0 * (w.dk + w.dv) + 2.0 * w.dk * w.dv)
    return float(b), f


def algorithmic_bwd(w) -> tuple[float, float]:
    """Bytes and MFMA FLOPs of one backward pass.  Bytes: q, k, v, dout read once; dq, dk, dv
    written once; the gate / per-token decay read once and its gradient written once
    (gamma: read only); dfinal read, the start state read if given, dinit written.
    FLOPs per token-head (three chunk scans, causal halves of the C x C products):
    2 * [(C+1)/2 * (3 dv + 3 dk) + 6 dk dv]."""
    s = 2 if w.dtype == "bf16" else 4
    th = w.B * w.H * w.T
    b = th * (4 * w.dk + 3 * w.dv) * s   # q, k, dq, dk (dk wide); v, dout, dv (dv wide)
    if w.decay == "gate":
        b += 2 * th * w.dk * 4
    elif w.decay == "token":
        b += 2 * th * 4
    elif w.decay == "gamma":
        b += w.H * 4
    state = w.B * w.H * w.dk * w.dv * 4
    b += state * (3 if w.init_sigma > 0 else 2)
    f = th * 2.0 * ((w.chunk + 1) / 2.0 * (3 * w.dk + 3 * w.dv) + 6.0 * w.dk * w.dv)
    return float(b), f


def host_cores() -> dict:
    """The host CPUs this process may run on: the affinity mask, capped by a cgroup CPU
    quota when one is set, and the CPU model (from /proc/cpuinfo)."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
            if q != "max":
                quota = float(q) / float(per)
    except (OSError, ValueError):
        pass
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = affinity if quota is None else max(1, min(affinity, int(quota + 0.5)))
    return {"threads": threads, "affinity_cpus": affinity, "cgroup_cpu_quota": quota,
            "cpu_model": model}


def cpu_fields(hc: dict) -> dict:
    return {"cores": hc["threads"], "cpu_model": hc["cpu_model"],
            "affinity_cpus": hc["affinity_cpus"], "cgroup_cpu_quota": hc["cgroup_cpu_quota"]}


def kernel_name(w, bthd: bool = False) -> str:
    t = "__bf16" if w.dtype == "bf16" else "float"
    d = {"none": 0, "gamma": 1, "gate": 2, "token": 3}[w.decay]
    return f"chunk_fwd_kernel<{t}, {w.dk}, {w.chunk}, {d}, {str(w.normalize).lower()}, false, {'true' if bthd else 'false'}>"


def cpu_baseline(w, inp, out_gpu, fin_gpu, budget_s: float):
    """Time the fp64 oracle on a bounded sample: whole batches (every head and token), one
    after another until about budget_s of oracle time; also report the GPU's error on
    that sample."""
    import numpy as np
    import oracle
    from workloads import to_numpy_input

    hc = host_cores()
    threads = hc["threads"]

    def run(bs, hs):
        sl = (bs, hs)

        def part(t):
            return None if t is None else to_numpy_input(t[sl])

        dec = inp["decay"]
        dec_s = None if dec is None else (part(dec) if w.decay in ("gate", "token") else to_numpy_input(dec[hs]))
        q, k, v, ini = part(inp["q"]), part(inp["k"]), part(inp["v"]), part(inp["init"])
        t0 = time.perf_counter()
        ro, rf = oracle.fwd(q, k, v, dec_s, w.decay, ini, phi_elu1=w.phi_elu1,
                            normalize=w.normalize, nthreads=threads)
        dt = time.perf_counter() - t0
        o = out_gpu[sl].float().cpu().numpy().astype(np.float64)
        f = fin_gpu[sl].cpu().numpy().astype(np.float64)
        return dt, float(np.max(np.abs(o - ro))), float(np.max(np.abs(ro))), \
            float(np.max(np.abs(f - rf))), float(np.max(np.abs(rf)))

    # whole batches, one at a time, until about budget_s of oracle time
    dt = eo = mo = ef = mf = 0.0
    nbatch = 0
    while nbatch < w.B and (nbatch == 0 or dt < budget_s):
        r = run(slice(nbatch, nbatch + 1), slice(0, w.H))
        dt += r[0]
        eo, mo, ef, mf = max(eo, r[1]), max(mo, r[2]), max(ef, r[3]), max(mf, r[4])
        nbatch += 1
    token_heads = w.T * w.H * nbatch
    return {
        "value": token_heads / dt / w.H,   # tokens/s: H heads make one token
        "unit": "tokens/s",
        **cpu_fields(hc),
        "kind": "oracle",
        "sample": f"batches 0..{nbatch - 1} of {w.B}, all {w.H} heads, all {w.T} tokens "
                  f"({token_heads} token-heads, fp64 recurrence, {dt:.1f} s)",
    }, {"max_rel_err_out": eo / max(mo, 1e-300), "max_rel_err_final": ef / max(mf, 1e-300),
        "sample_batches": nbatch}


def cpu_baseline_bwd(w, inp, grads, got, budget_s: float):
    """The fp64 oracle's backward on whole batches until about budget_s, and the GPU's
    error on that sample (max |g - g_ref| / max |g_ref| per gradient)."""
    import numpy as np
    import oracle
    from workloads import to_numpy_input

    hc = host_cores()
    threads = hc["threads"]
    dt = 0.0
    nbatch = 0
    err, mag = {}, {}
    while nbatch < w.B and (nbatch == 0 or dt < budget_s):
        sl = slice(nbatch, nbatch + 1)

        def part(t):
            return None if t is None else to_numpy_input(t[sl])

        dec = inp["decay"]
        dec_s = None if dec is None else (part(dec) if w.decay in ("gate", "token")
                                          else to_numpy_input(dec))
        ini = part(inp["init"])
        t0 = time.perf_counter()
        ref = oracle.bwd(part(inp["q"]), part(inp["k"]), part(inp["v"]), part(grads["dout"]),
                         dec_s, w.decay, ini, part(grads["dfinal"]), phi_elu1=w.phi_elu1,
                         nthreads=threads)
        dt += time.perf_counter() - t0
        for n, t in got.items():
            if t is None or ref.get(n) is None:
                continue
            g = t[sl].double().cpu().numpy()
            err[n] = max(err.get(n, 0.0), float(np.max(np.abs(g - ref[n]))))
            mag[n] = max(mag.get(n, 0.0), float(np.max(np.abs(ref[n]))))
        nbatch += 1
    token_heads = w.T * w.H * nbatch
    return {
        "value": token_heads / dt / w.H,
        "unit": "tokens/s",
        **cpu_fields(hc),
        "kind": "oracle",
        "sample": f"batches 0..{nbatch - 1} of {w.B}, all {w.H} heads, all {w.T} tokens "
                  f"({token_heads} token-heads, fp64 back-propagation, {dt:.1f} s)",
    }, {f"max_rel_err_{n}": err[n] / max(mag[n], 1e-300) for n in err} | {"sample_batches": nbatch}


def timed(torch, step, steps, warmup, stream):
    """Warm-up (about a second of steps unless given), then `steps` steps with a HIP event
    on the launch stream before and after each.  Returns (mean ms per step over the timed
    region, warm-up steps, wall seconds, per-step stats {median, min, max} in ms)."""
    if warmup is None:
        warmup, t0 = 0, time.perf_counter()
        while True:
            step()
            warmup += 1
            if warmup % 8 == 0:
                torch.cuda.synchronize()
                if warmup >= 10 and time.perf_counter() - t0 >= 1.0:
                    break
    else:
        for _ in range(warmup):
            step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t_wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    mid = len(per) // 2
    median = per[mid] if len(per) % 2 else 0.5 * (per[mid - 1] + per[mid])
    stats = {"median": median, "min": per[0], "max": per[-1]}
    return evs[0].elapsed_time(evs[-1]) / steps, warmup, t_wall, stats


def measure_peaks(torch, fla, stream) -> dict:
    """What this GPU reaches with the library's plain probe kernels (include/fla_probe.h):
    HBM streaming rates (read only, copy, and five reads per write, the mix of the gated
    forward pass) over 2 GiB buffers, and the dense bf16 MFMA rate of register-only chains.
    Each is the best of several timed launches after a warm-up launch.  Running them
    first also brings the GPU clocks up before the warm-up steps."""
    nbytes = 2 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    dst = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    res = {}

    def best_ms(fn, reps):
        fn()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    ms = best_ms(lambda: fla.probe_stream(src, dst, nbytes, fla.PROBE_READ, stream), 8)
    res["hbm_read_GBs"] = nbytes / (ms * 1e-3) / 1e9
    half = nbytes // 2
    ms = best_ms(lambda: fla.probe_stream(src, dst, half, fla.PROBE_COPY, stream), 8)
    res["hbm_copy_GBs"] = 2 * half / (ms * 1e-3) / 1e9
    mix = (nbytes // 96) * 96            # 5/6 read from src, 1/6 written to dst
    ms = best_ms(lambda: fla.probe_stream(src, dst, mix, fla.PROBE_MIX5, stream), 8)
    res["hbm_read5_write1_GBs"] = mix / (ms * 1e-3) / 1e9
    del src, dst
    wgs, iters = 2048, 20000
    out = torch.empty(4 * wgs, dtype=torch.float32, device="cuda")
    flops = [0.0]

    def mf():
        flops[0] = fla.probe_mfma(out, wgs, iters, stream)

    ms = best_ms(mf, 5)
    res["mfma_bf16_TFLOPs"] = flops[0] / (ms * 1e-3) / 1e12
    res["probes"] = ("hand-written HIP: 16-byte non-temporal loads/stores, 8 in flight per "
                     "lane, grid-stride over 2 GiB; MFMA: 2048 workgroups x 4 waves x 4 "
                     "independent v_mfma_f32_32x32x16_bf16 chains")
    torch.cuda.synchronize()
    return res


def measure_chunk_pattern(torch, fla, inp, stream) -> float:
    """Rate (GB/s) of the forward pass's own access pattern with no arithmetic
    (fla_probe_chunk_pattern) on the workload's inputs: the best of several launches after
    a warm-up launch; bytes = q, k, gate, value slices read and outputs written once."""
    q, k, g, v = inp["q"], inp["k"], inp["decay"], inp["v"]
    out = torch.empty_like(v)
    B, H, T, dk = q.shape
    nbytes = B * H * T * (2 * dk * 2 + dk * 4 + 2 * v.shape[-1] * 2)
    fla.probe_chunk_pattern(q, k, g, v, out, stream)
    ts = []
    for _ in range(8):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fla.probe_chunk_pattern(q, k, g, v, out, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del out
    return nbytes / (min(ts) * 1e-3) / 1e9


def add_measured(roof: dict, peaks, dtype: str) -> dict:
    """Add the measured ceilings (measure_peaks) and the fractions of them to a roofline
    record; the nominal `peak` and `frac` stay as published."""
    if not peaks:
        roof["measured_peaks"] = None
        return roof
    roof["measured_peaks"] = peaks
    a = roof["achieved"]
    roof["frac_of_measured_read5_write1"] = a / peaks["hbm_read5_write1_GBs"]
    roof["frac_of_measured_copy"] = a / peaks["hbm_copy_GBs"]
    roof["frac_of_measured_read"] = a / peaks["hbm_read_GBs"]
    if peaks.get("hbm_chunk_pattern_GBs"):
        roof["frac_of_measured_chunk_pattern"] = a / peaks["hbm_chunk_pattern_GBs"]
    if dtype == "bf16":
        roof["mfma_frac_of_measured"] = roof["mfma_tflops"] / peaks["mfma_bf16_TFLOPs"]
    return roof


def bench_bwd(torch, fla, w, args):
    from workloads import generate_grads_torch, generate_torch

    inp = generate_torch(w, "cuda")
    grads = generate_grads_torch(w, "cuda")
    stream = torch.cuda.current_stream()
    got = {}

    def step():
        dq, dk, dv, dg, di = fla.bwd(inp["q"], inp["k"], inp["v"], grads["dout"], inp["decay"],
                                     decay_kind=w.decay, init_state=inp["init"],
                                     dfinal=grads["dfinal"], phi_elu1=w.phi_elu1,
                                     chunk=w.chunk, stream=stream)
        got.update(dq=dq, dk=dk, dv=dv, dgate=dg, dinit=di)

    ms, warmup, t_wall, per_step = timed(torch, step, args.steps, args.warmup, stream)
    alg_bytes, alg_flops = algorithmic_bwd(w)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "chunked linear-attn bwd tokens/s + roofline % (HBM), " + w.name,
        "value": w.B * w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "ms_per_step_median": per_step["median"],
        "ms_per_step_min": per_step["min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded torch generator on the GPU; shapes and distributions of the workload)",
        "config": {
            "workload": w.name, "pass": "backward", "B": w.B, "H": w.H, "T": w.T, "dk": w.dk,
            "dv": w.dv, "chunk": w.chunk, "decay": w.decay,
            "phi": "elu+1" if w.phi_elu1 else "identity", "init_state": w.init_sigma > 0,
            "global_batch": w.B, "seq_len": w.T, "parallelism": "single GPU",
        },
        "roofline": add_measured({
            "bound": "hbm",
            "kernel": "chunk_bwd_kernel: dq, dv, dk launches (+ per-token decay epilogue)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "algorithmic_bytes_per_launch": alg_bytes,
            "mfma_tflops": alg_flops / (ms * 1e-3) / 1e12,
            "mfma_frac": alg_flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype],
        }, args.peaks, w.dtype),
        "wall_s_timed_region": t_wall,
    }
    if not args.no_cpu_baseline:
        cb, parity = cpu_baseline_bwd(w, inp, grads, got, args.cpu_budget)
        res["cpu_baseline"] = cb
        res["parity_on_sample"] = parity
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_varlen(torch, fla, args):
    """Forward over packed variable-length sequences (one fla_linattn_fwd_varlen call)."""
    import numpy as np
    import oracle
    from workloads import generate_torch, to_numpy_input, varlen_workload

    w, lengths = varlen_workload(args.varlen)
    cu_h = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    n = len(lengths)
    inp = generate_torch(w, "cuda")       # [1, H, total, d]: one long draw, then packed
    packed = {k: inp[k][0].transpose(0, 1).contiguous() for k in ("q", "k", "v")}
    packed["decay"] = (inp["decay"][0].transpose(0, 1).contiguous()
                       if w.decay in ("gate", "token") else inp["decay"])
    cu = torch.from_numpy(cu_h).cuda()
    out = torch.empty((w.T, w.H, w.dv), dtype=inp["q"].dtype, device="cuda")
    fin = torch.empty((n, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fla.fwd_varlen(packed["q"], packed["k"], packed["v"], cu, packed["decay"],
                       decay_kind=w.decay, out=out, final_state=fin, chunk=w.chunk,
                       stream=stream)

    ms, warmup, t_wall, per_step = timed(torch, step, args.steps, args.warmup, stream)
    alg_bytes, alg_flops = algorithmic(w)
    alg_bytes += (n - 1) * w.H * w.dk * w.dv * 4  # one end state per sequence
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "chunked linear-attn fwd tokens/s + roofline % (HBM), packed sequences, " + w.name,
        "value": w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "ms_per_step_median": per_step["median"],
        "ms_per_step_min": per_step["min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded torch generator on the GPU; log-uniform sequence lengths)",
        "config": {
            "workload": w.name, "n_seqs": n, "total_tokens": int(w.T), "H": w.H, "dk": w.dk,
            "dv": w.dv, "chunk": w.chunk, "decay": w.decay, "layout": "packed [total][H][d]",
            "len_min": int(lengths.min()), "len_max": int(lengths.max()),
            "len_mean": float(lengths.mean()), "global_batch": n, "seq_len": int(lengths.max()),
            "parallelism": "single GPU",
        },
        "roofline": add_measured({
            "bound": "hbm",
            "kernel": kernel_name(w, True) + " [packed sequences]",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "algorithmic_bytes_per_launch": alg_bytes,
            "mfma_tflops": alg_flops / (ms * 1e-3) / 1e12,
            "mfma_frac": alg_flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype],
        }, args.peaks, w.dtype),
        "wall_s_timed_region": t_wall,
    }
    if not args.no_cpu_baseline:
        hc = host_cores()
        threads = hc["threads"]
        dt, eo, mo, ef, mf, done, toks = 0.0, 0.0, 0.0, 0.0, 0.0, 0, 0
        while done < n and (done == 0 or dt < args.cpu_budget):
            s0, s1 = int(cu_h[done]), int(cu_h[done + 1])
            part = lambda t: to_numpy_input(t[:, :, s0:s1])
            dec = inp["decay"]
            dec_s = part(dec) if w.decay in ("gate", "token") else (None if dec is None else to_numpy_input(dec))
            t0 = time.perf_counter()
            ro, rf = oracle.fwd(part(inp["q"]), part(inp["k"]), part(inp["v"]), dec_s, w.decay,
                                None, nthreads=threads)
            dt += time.perf_counter() - t0
            o = out[s0:s1].transpose(0, 1)[None].float().cpu().numpy().astype(np.float64)
            f = fin[done:done + 1].cpu().numpy().astype(np.float64)
            eo, mo = max(eo, float(np.max(np.abs(o - ro))) if s1 > s0 else 0.0), max(mo, float(np.max(np.abs(ro))) if s1 > s0 else 0.0)
            ef, mf = max(ef, float(np.max(np.abs(f - rf)))), max(mf, float(np.max(np.abs(rf))))
            toks += s1 - s0
            done += 1
        res["cpu_baseline"] = {"value": toks / dt, "unit": "tokens/s", **cpu_fields(hc),
                               "kind": "oracle",
                               "sample": f"sequences 0..{done - 1} of {n} ({toks} tokens, all "
                                         f"{w.H} heads, fp64 recurrence, {dt:.1f} s)"}
        res["parity_on_sample"] = {"max_rel_err_out": eo / max(mo, 1e-300),
                                   "max_rel_err_final": ef / max(mf, 1e-300),
                                   "sample_sequences": done}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_gdn(torch, fla, args):
    """Gated delta rule forward (one fla_gdn_fwd call per step)."""
    import numpy as np
    import oracle
    from workloads import GDN, generate_gdn_torch, to_numpy_input

    w = GDN[args.gdn]
    inp = generate_gdn_torch(w, "cuda")
    out = torch.empty((w.B, w.H, w.T, w.dv), dtype=inp["q"].dtype, device="cuda")
    fin = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fla.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                    init_state=inp["init"], out=out, final_state=fin, chunk=w.chunk,
                    stream=stream)

    ms, warmup, t_wall, per_step = timed(torch, step, args.steps, args.warmup, stream)
    s = 2 if w.dtype == "bf16" else 4
    th = w.B * w.H * w.T
    # q, k, v read, out written; alpha and beta read; end state written (start state read)
    alg_bytes = th * (2 * w.dk + 2 * w.dv) * s + th * 8 + w.B * w.H * w.dk * w.dv * 4 * (
        2 if w.init_sigma > 0 else 1)
    # per token-head: K^K^T and QK^T (causal halves, dk each), X = K^ H (dk dv), U = Tb W
    # and P U (causal halves, dv each), Q H and the state update (dk dv each)
    c = w.chunk
    alg_flops = th * 2.0 * ((c + 1) / 2.0 * (2 * w.dk + 2 * w.dv) + 3.0 * w.dk * w.dv)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    t = "__bf16" if w.dtype == "bf16" else "float"
    res = {
        "metric": "gated delta rule chunk fwd tokens/s + roofline % (HBM), " + w.name,
        "value": w.B * w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "ms_per_step_median": per_step["median"],
        "ms_per_step_min": per_step["min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded torch generator on the GPU; alpha = sigmoid(x)^(1/16), beta = sigmoid(y))",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
            "chunk": w.chunk, "init_state": w.init_sigma > 0, "global_batch": w.B,
            "seq_len": w.T, "parallelism": "single GPU",
        },
        "roofline": add_measured({
            "bound": "hbm",
            "kernel": f"gdn_prep_kernel<{t}, {w.dk}> + gdn_state_kernel<{t}, {w.dk}>",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(w.name),
            "algorithmic_bytes_per_launch": alg_bytes,
            "mfma_tflops": alg_flops / (ms * 1e-3) / 1e12,
            "mfma_frac": alg_flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype],
        }, args.peaks, w.dtype),
        "wall_s_timed_region": t_wall,
    }
    if not args.no_cpu_baseline:
        hc = host_cores()
        threads = hc["threads"]
        dt, eo, mo, ef, mf, nb = 0.0, 0.0, 0.0, 0.0, 0.0, 0
        while nb < w.B and (nb == 0 or dt < args.cpu_budget):
            sl = slice(nb, nb + 1)
            part = lambda x: None if x is None else to_numpy_input(x[sl])
            t0 = time.perf_counter()
            ro, rf = oracle.gdn_fwd(part(inp["q"]), part(inp["k"]), part(inp["v"]),
                                    part(inp["alpha"]), part(inp["beta"]), part(inp["init"]),
                                    nthreads=threads)
            dt += time.perf_counter() - t0
            o = out[sl].float().cpu().numpy().astype(np.float64)
            f = fin[sl].cpu().numpy().astype(np.float64)
            eo, mo = max(eo, float(np.max(np.abs(o - ro)))), max(mo, float(np.max(np.abs(ro))))
            ef, mf = max(ef, float(np.max(np.abs(f - rf)))), max(mf, float(np.max(np.abs(rf))))
            nb += 1
        res["cpu_baseline"] = {"value": w.T * nb / dt, "unit": "tokens/s", **cpu_fields(hc),
                               "kind": "oracle",
                               "sample": f"batches 0..{nb - 1} of {w.B}, all {w.H} heads, all "
                                         f"{w.T} tokens (fp64 recurrence, {dt:.1f} s)"}
        res["parity_on_sample"] = {"max_rel_err_out": eo / max(mo, 1e-300),
                                   "max_rel_err_final": ef / max(mf, 1e-300),
                                   "sample_batches": nb}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_proj(torch, fla, args):
    """The layer's input side: q, k, v projections with the feature map fused in, then the
    forward pass (one fla_linattn_fwd_proj call per step)."""
    import numpy as np
    import oracle
    from workloads import PROJ, generate_proj_torch, to_numpy_input

    sp = PROJ[args.proj]
    B, T, D, H, dk, dv = (sp[k] for k in ("B", "T", "hidden", "H", "dk", "dv"))
    inp = generate_proj_torch(sp, "cuda")
    dt = inp["x"].dtype
    out = torch.empty((B, T, H, dv), dtype=dt, device="cuda")
    fin = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fla.fwd_proj(inp["x"], inp["w_q"], inp["w_k"], inp["w_v"], H, inp["decay"],
                     decay_kind=sp["decay"], out=out, final_state=fin, chunk=sp["chunk"],
                     stream=stream)

    ms, warmup, t_wall, per_step = timed(torch, step, args.steps, args.warmup, stream)
    s = 2 if sp["dtype"] == "bf16" else 4
    M = B * T
    gemm_flops = 2.0 * M * D * H * (2 * dk + dv)
    attn_flops = M * H * 2.0 * ((sp["chunk"] + 1) / 2.0 * (dk + dv) + 2.0 * dk * dv)
    # the method's bytes: x and the weights in, the gate in, out and the final state out
    alg_bytes = (M * D + D * H * (2 * dk + dv)) * s + M * H * dv * s + B * H * dk * dv * 4
    alg_bytes += M * H * dk * 4 if sp["decay"] == "gate" else (M * H * 4 if sp["decay"] == "token" else 0)
    tflops = (gemm_flops + attn_flops) / (ms * 1e-3) / 1e12
    res = {
        "metric": "linear-attn layer input side + chunk fwd tokens/s + MFMA roofline, " + args.proj,
        "value": M / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "ms_per_step_median": per_step["median"],
        "ms_per_step_min": per_step["min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sp["dtype"],
        "data": "synthetic (seeded torch generator on the GPU; x ~ N(0,1), W scaled so q, k ~ N(0, 1/dk))",
        "config": {"workload": args.proj, "B": B, "T": T, "hidden": D, "H": H, "dk": dk, "dv": dv,
                   "chunk": sp["chunk"], "decay": sp["decay"], "layout": "[B][T][H][d]",
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "kernel": "proj_phi_kernel (q, k, v) + chunk_fwd_kernel (token-major)",
            "achieved": tflops,
            "peak": MFMA_PEAK_TFLOPS[sp["dtype"]],
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_PEAK_TFLOPS[sp["dtype"]],
            "traffic": measured_traffic(args.proj),
            "algorithmic_flops_per_step": gemm_flops + attn_flops,
            "algorithmic_bytes_per_step": alg_bytes,
            "hbm_GBs_algorithmic": alg_bytes / (ms * 1e-3) / 1e9,
        },
        "wall_s_timed_region": t_wall,
    }
    if args.peaks:
        res["roofline"]["measured_peaks"] = args.peaks
        if sp["dtype"] == "bf16":
            res["roofline"]["frac_of_measured_mfma"] = tflops / args.peaks["mfma_bf16_TFLOPs"]
    if not args.no_cpu_baseline:
        hc = host_cores()
        t0 = time.perf_counter()
        ro, rf = oracle.fwd_proj(to_numpy_input(inp["x"][:1]), to_numpy_input(inp["w_q"]),
                                 to_numpy_input(inp["w_k"]), to_numpy_input(inp["w_v"]), H,
                                 to_numpy_input(inp["decay"][:1]), sp["decay"],
                                 nthreads=hc["threads"])
        dt_s = time.perf_counter() - t0
        o = out[:1].float().cpu().numpy().astype(np.float64)
        res["cpu_baseline"] = {"value": T / dt_s, "unit": "tokens/s", **cpu_fields(hc),
                               "kind": "oracle",
                               "sample": f"batch row 0 of {B} ({T} tokens, all {H} heads; fp64 "
                                         f"projections (numpy) + recurrence, {dt_s:.1f} s)"}
        res["parity_on_sample"] = {"max_rel_err_out": float(np.max(np.abs(o - ro)) / np.max(np.abs(ro)))}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def copy_calibration(torch, steps, warmup):
    """A plain copy of 1 GiB: reads and writes exactly 2^30 bytes per launch."""
    n = 1 << 30
    src = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "ms_per_copy": ms, "copy_GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: as many as fill about "
                         "one second, so the GPU clocks have settled)")
    ap.add_argument("--workload", default=None, help="workload name (default: headline)")
    ap.add_argument("--mode", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward pass (default) or the chunkwise backward")
    ap.add_argument("--layout", choices=("bhtd", "bthd"), default="bhtd",
                    help="forward: [B][H][T][d] (default) or token-major [B][T][H][d] inputs")
    ap.add_argument("--gdn", default=None,
                    help="gated delta rule forward (workload name, e.g. gdn_d128)")
    ap.add_argument("--varlen", default=None,
                    help="forward over packed variable-length sequences (workload name, "
                         "e.g. varlen_gla_d128)")
    ap.add_argument("--proj", default=None,
                    help="the layer's input side: projections + feature map + forward "
                         "(workload name, e.g. gla_proj_d128)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--chunk", type=int, default=None,
                    help="evaluate the workload with this chunk size instead of its own "
                         "(tile sweeps; the forward pass's result does not depend on it)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured HBM / MFMA ceilings (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device copy instead (HBM reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters and the achievable copy rate)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards over (batch, head) or sequence segments across GPUs as "
              "described in the design notes, but no multi-GPU run is part of it.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch, args.steps, 20 if args.warmup is None else args.warmup)
        return

    import chunkwise_causal_linear_amd as fla
    from workloads import HEADLINE, WORKLOADS, generate_torch

    torch.cuda.set_device(0)
    args.peaks = None if args.no_probes else measure_peaks(torch, fla, torch.cuda.current_stream())
    if args.gdn:
        bench_gdn(torch, fla, args)
        return
    if args.varlen:
        bench_varlen(torch, fla, args)
        return
    if args.proj:
        bench_proj(torch, fla, args)
        return
    w = WORKLOADS[args.workload or HEADLINE]
    if args.chunk:
        # tile sweep: the same workload evaluated with another chunk size (the function
        # does not depend on it; the workload's own chunk is the one its config names)
        w = w.with_(chunk=args.chunk)
    if args.mode == "bwd":
        bench_bwd(torch, fla, w, args)
        return
    inp = generate_torch(w, "cuda")
    ncol = w.dv + (1 if w.normalize else 0)
    fin = torch.empty((w.B, w.H, w.dk, ncol), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    if args.layout == "bthd":
        # the same values in token-major order; the oracle leg reads [B][H][T][d] views
        tin = {n: (None if inp[n] is None else inp[n].transpose(1, 2).contiguous())
               for n in ("q", "k", "v")}
        tin["decay"] = (inp["decay"].transpose(1, 2).contiguous()
                        if w.decay in ("gate", "token") else inp["decay"])
        out_t = torch.empty((w.B, w.T, w.H, w.dv), dtype=inp["q"].dtype, device="cuda")
        out = out_t.transpose(1, 2)

        def step():
            fla.fwd(tin["q"], tin["k"], tin["v"], tin["decay"], decay_kind=w.decay,
                    init_state=inp["init"], out=out_t, final_state=fin, chunk=w.chunk,
                    phi_elu1=w.phi_elu1, normalize=w.normalize, layout="bthd", stream=stream)
    else:
        out = torch.empty((w.B, w.H, w.T, w.dv), dtype=inp["q"].dtype, device="cuda")

        def step():
            fla.fwd(inp["q"], inp["k"], inp["v"], inp["decay"], decay_kind=w.decay,
                    init_state=inp["init"], out=out, final_state=fin, chunk=w.chunk,
                    phi_elu1=w.phi_elu1, normalize=w.normalize, stream=stream)

    # timed region: HIP events on the stream the kernels are launched on
    ms, warmup, t_wall, per_step = timed(torch, step, args.steps, args.warmup, stream)

    # the ceiling of the kernel's own access pattern (gated bf16 forward, dk = 128, [B][H][T][d]),
    # measured after the timed region on the same inputs
    if args.peaks and args.layout == "bhtd" and w.decay == "gate" and w.dtype == "bf16" \
            and w.dk == 128 and w.dv % 64 == 0 and w.dv <= 256:
        args.peaks = dict(args.peaks)
        args.peaks["hbm_chunk_pattern_GBs"] = measure_chunk_pattern(torch, fla, inp, stream)
        args.peaks["chunk_pattern_probe"] = (
            "hand-written HIP: the forward pass's loads and stores (one workgroup per (b, h, "
            "64-wide value slice), chunks in order, one chunk of loads ahead) with no arithmetic")
    nseg = fla.segments_for(w.B, w.H, w.T, w.dk, w.dv, w.chunk,
                            fla.flags_for(inp["q"].dtype, w.decay, w.phi_elu1, w.normalize))
    alg_bytes, alg_flops = algorithmic(w)
    tokens = w.B * w.T
    achieved_gbs = alg_bytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name) if args.layout == "bhtd" else None

    res = {
        "metric": "chunked linear-attn fwd tokens/s + roofline % (MFMA/HBM), B8 H16 T16384 d128",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "ms_per_step_median": per_step["median"],
        "ms_per_step_min": per_step["min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded torch generator on the GPU; shapes and distributions of the workload)",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
            "chunk": w.chunk, "decay": w.decay, "phi": "elu+1" if w.phi_elu1 else "identity",
            "normalize": w.normalize, "init_state": w.init_sigma > 0, "segments": nseg,
            "layout": "[B][T][H][d]" if args.layout == "bthd" else "[B][H][T][d]",
            "global_batch": w.B, "seq_len": w.T, "parallelism": "single GPU",
        },
        "roofline": add_measured({
            "bound": "hbm",
            "kernel": kernel_name(w, args.layout == "bthd") + (" (+ segment passes)" if nseg > 1 else ""),
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes,
            "mfma_tflops": alg_flops / (ms * 1e-3) / 1e12,
            "mfma_frac": alg_flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype],
        }, args.peaks, w.dtype),
        "wall_s_timed_region": t_wall,
    }
    if not args.no_cpu_baseline:
        cb, parity = cpu_baseline(w, inp, out, fin, args.cpu_budget)
        res["cpu_baseline"] = cb
        res["parity_on_sample"] = parity
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
