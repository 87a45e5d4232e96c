#!/usr/bin/env python3
"""Throughput of the K-quant x int8 GEMM hot path on one MI355X.

One timed step is one LLaDA-8B denoising step's GEMM work at canvas L = 160
(heatdrop.ai card, "What it does": each step reruns the whole model over the
canvas, so the runtime is a stream of GEMMs; Architecture page, "A forward
pass"): for each of 32 layers, 4 activation quantizations (RMSNorm fused in
front of the one Q/K/V share and of the one gate/up share; O's input as is;
down's input, SiLU(gate) * up, which the gate/up GEMM forms in its epilogue)
and the 7 projections Q, K, V, O (4096 x 4096
Q4_K), gate, up (12288 x 4096 Q4_K) and down (4096 x 12288; Q6_K on odd
layers, Q4_K on even), then the output projection on 32 gathered canvas rows
(126,464 x 4096 Q6_K).  Q, K and V read the same quantized input, so their
weights are stacked at load time into one 12,288 x 4096 matrix and run as one
GEMM (same bytes and operations, two launches fewer per layer); gate and up
likewise share an input and run as one 24,576 x 4096 GEMM, their 16-row
tiles interleaved so that each workgroup holds matching gate and up columns.
Every layer
has its own seeded weights (4.6 GB in all, far above the 256 MB last-level
cache), resident in HBM before timing.

The timed steps replay the step captured as one HIP graph.  Prints one JSON
line: whole-step TOPS (value), HBM GB/s, the roofline of the dominant kernel
measured with HIP events around each of its launches (eager steps on the same
stream), and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "K-quant×int8 GEMM TOPS + HBM GB/s (% roofline) at LLaDA-8B step shapes"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA
L, K, F, V, LAYERS, ROWS = 160, 4096, 12288, 126464, 32, 32
EPS = 1e-5  # RMSNorm epsilon
Q4_K, Q6_K = 12, 14
BLOCK = {Q4_K: 144, Q6_K: 210}
COPY_MIB = 512
KERNEL_SOURCES = ["quantized_gemm_diffusion_amd/csrc/qgemm.hip",
                  "quantized_gemm_diffusion_amd/csrc/dq_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cpu-layers", type=int, default=16,
                   help="layers of the step the CPU oracle baseline runs on")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="oracle threads (default: every core this process may use, capped by "
                        "OMP_NUM_THREADS -- the job's CPU share)")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-configuration lines (Dream-7B, logits at 1 and 8 rows)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle timing (for profiler runs)")
    p.add_argument("--counters", action="store_true",
                   help="for hardware-counter runs: one eager step, then a plain copy of "
                        f"{COPY_MIB} MiB (the byte-count calibration), no timing")
    return p.parse_args()


def gemm_bytes(type_, M, N, K_):
    w = N * (K_ // 256) * BLOCK[type_]
    act = M * K_ + M * (K_ // 256) * 4 + (M * (K_ // 32) * 4 if type_ == Q4_K else 0)
    return w + act + M * N * 4


def quant_bytes(M, K_):
    return M * K_ * 4 + M * K_ + M * (K_ // 256) * 4 + M * (K_ // 32) * 4


def norm_quant_bytes(M, K_):  # the row, the norm weights, the quantized record
    return quant_bytes(M, K_) + K_ * 4


def source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def host_clocks():
    """GPU clocks as rocm-smi reports them, read in a child process before this
    process touches the GPU (None if the tool is missing)."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                             text=True, timeout=30)
        data = json.loads(out.stdout)
    except Exception:  # noqa: BLE001 -- the tool is optional
        return None
    res = {}
    for card, d in data.items():
        for k, v in d.items():
            if "sclk" in k.lower() or "mclk" in k.lower() or "fclk" in k.lower():
                res[f"{card} {k}"] = v
        break
    return res or None


def main():
    args = parse()
    if args.gpus != 1:
        log("bench.py measures one GPU: the library runs the hot path on a single MI355X and "
            "sharding across GPUs is described, not implemented, so --gpus must be 1.")
        sys.exit(2)
    # not in counters mode: under a counter profiler a child process would
    # initialise the GPU before its interpreter starts
    clocks_before = None if args.counters else host_clocks()

    import torch
    import quantized_gemm_diffusion_amd as dq

    lib = dq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------------------------------------------------------- inputs
    t0 = time.perf_counter()
    act_rng = np.random.default_rng(synth.seed(2, 0, 9))
    # the residual stream in front of attention and of the FFN, and attention's
    # output (attention is timed on its own, below, not inside the GEMM step); the
    # down projection's input is made by the step itself from the gate/up GEMM's
    # output
    acts = {"qkv": up(synth.activations(act_rng, L, K)), "o": up(synth.activations(act_rng, L, K)),
            "ffn": up(synth.activations(act_rng, L, K))}
    norm_rng = np.random.default_rng(synth.seed(2, 0, 8))
    gammas = [{n: up((1.0 + 0.1 * norm_rng.standard_normal(K)).astype(np.float32))
               for n in ("qkv", "ffn")} for _ in range(LAYERS)]
    qbuf = {kk: torch.empty(dq.act_size(L, kk), dtype=torch.uint8, device=dev) for kk in (K, F)}
    # the gate/up GEMM stores silu(gate) * up, L x F, in its epilogue
    outs = {name: torch.empty((L, N), dtype=torch.float32, device=dev)
            for name, N in (("qkv", 3 * K), ("o", K), ("gateup", F), ("down", K))}
    host_keep = {}
    packed = []
    for layer in range(LAYERS):
        mats = {}
        for p, (name, t, N, KK) in enumerate(synth.llada_layer(layer)):
            mats[name] = (t, N, KK, synth.weights(np.random.default_rng(synth.seed(2, layer, p)),
                                                  t, N, KK))
        # Q, K, V stacked along N: one 12288 x 4096 Q4_K matrix
        mats["qkv"] = (Q4_K, 3 * K, K, np.concatenate([mats.pop(n)[3] for n in "qkv"]))
        # gate and up stacked along N with their 16-row tiles interleaved: one
        # 24576 x 4096 Q4_K matrix, whose GEMM forms silu(gate) * up itself
        gate_w, up_w = mats.pop("gate")[3], mats.pop("up")[3]
        mats["gateup"] = (Q4_K, 2 * F, K, dq.interleave_gate_up(gate_w, up_w))
        lp = {}
        for name, (t, N, KK, W) in mats.items():
            if layer < args.cpu_layers:
                host_keep[(layer, name)] = W
            g = up(W.reshape(-1))
            lp[name] = (t, N, KK, dq.repack_weights(t, N, KK, g))
            del g
        packed.append(lp)
    Wout = synth.q6k_weights(np.random.default_rng(synth.seed(3, 0, 0)), V, K)
    out_packed = dq.repack_weights(Q6_K, V, K, up(Wout.reshape(-1)))
    canvas_np = synth.activations(np.random.default_rng(synth.seed(3, 0, 1)), L, K)
    idx_np = synth.row_index(np.random.default_rng(synth.seed(3, 0, 2)), L, ROWS)
    canvas, idx = up(canvas_np), up(idx_np)
    logits = torch.empty((ROWS, V), dtype=torch.float32, device=dev)
    ws = torch.empty(dq.qgemm_rows_workspace(ROWS, K), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM after {time.perf_counter() - t0:.1f} s")

    # ------------------------------------------------------- the step's calls
    calls = []  # (C function, args, kind, ops, algorithmic bytes)

    def quant(name):
        x = acts[name]
        kk = x.shape[1]
        buf = qbuf[kk]
        calls.append((lib.dq_quantize_act, (L, kk, x.data_ptr(), kk, buf.data_ptr()),
                      "quantize", 0, quant_bytes(L, kk)))
        return buf

    def norm_quant(li, name):
        x = acts[name]
        buf = qbuf[K]
        calls.append((lib.dq_rmsnorm_quantize_act,
                      (L, K, x.data_ptr(), K, gammas[li][name].data_ptr(), ctypes.c_float(EPS),
                       buf.data_ptr()),
                      "rmsnorm_quantize", 0, norm_quant_bytes(L, K)))
        return buf

    def down_quant():
        h = outs["gateup"]  # silu(gate) * up, from the gate/up GEMM's epilogue
        buf = qbuf[F]
        calls.append((lib.dq_quantize_act, (L, F, h.data_ptr(), F, buf.data_ptr()),
                      "quantize_down", 0, quant_bytes(L, F)))
        return buf

    def gemm(lp, name, buf):
        t, N, kk, pk = lp[name]
        y = outs[name]
        # one kind per GEMM shape: each kind is one kernel in a profile
        kind = f"qgemm_{'q4k' if t == Q4_K else 'q6k'}_{L}x{N}x{kk}"
        if name == "gateup":  # stores silu(gate) * up: N/2 outputs per row
            calls.append((lib.dq_qgemm_swiglu,
                          (t, L, N // 2, kk, buf.data_ptr(), pk.data_ptr(), y.data_ptr(), N // 2),
                          kind, 2 * L * N * kk, gemm_bytes(t, L, N, kk) - L * (N // 2) * 4))
            return
        calls.append((lib.dq_qgemm, (t, L, N, kk, buf.data_ptr(), pk.data_ptr(), y.data_ptr(), N),
                      kind, 2 * L * N * kk, gemm_bytes(t, L, N, kk)))

    for li, lp in enumerate(packed):
        gemm(lp, "qkv", norm_quant(li, "qkv"))
        gemm(lp, "o", quant("o"))
        gemm(lp, "gateup", norm_quant(li, "ffn"))
        gemm(lp, "down", down_quant())
    # gathered f32 rows and the index list stand in for pre-quantized activations
    rows_bytes = V * (K // 256) * BLOCK[Q6_K] + ROWS * K * 4 + ROWS * 4 + ROWS * V * 4
    calls.append((lib.dq_qgemm_rows,
                  (Q6_K, L, ROWS, V, K, canvas.data_ptr(), K, idx.data_ptr(),
                   out_packed.data_ptr(), logits.data_ptr(), V, ws.data_ptr(), ws.numel()),
                  "rows", 2 * ROWS * V * K, rows_bytes))
    step_ops = sum(c[3] for c in calls)
    step_bytes = sum(c[4] for c in calls)

    def run_calls(sh, brackets=None, kind=None):
        """Launch one step on stream handle sh; optionally record events around each
        launch of `kind` (on the same stream)."""
        for fn, a, k, _, _ in calls:
            if brackets is not None and k == kind:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                rc = fn(*a, sh)
                e1.record(stream)
                brackets.append((e0, e1))
            else:
                rc = fn(*a, sh)
            if rc:
                raise RuntimeError(f"{fn.__name__}: {lib.dq_last_error().decode()}")

    # ------------------------------------------------------ warmup, calibrate
    for _ in range(args.warmup):
        run_calls(sp)
    torch.cuda.synchronize()
    if args.counters:
        run_calls(sp)
        sampler_variants(lib, dq, torch, stream, sp, out_packed, canvas, idx, logits, ws, reps=0)
        attention_shapes(lib, dq, torch, stream, sp, up, reps=0)
        embedding_rows(lib, torch, stream, sp, up, reps=0)
        src = torch.ones(COPY_MIB << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"counters mode: one step, then a {COPY_MIB} MiB copy")
        # the kind of each call of a step, in launch order (the rows call makes two
        # launches: the gather-quantize, then the GEMM), so that per-dispatch
        # counters can be attributed to the step's GEMM shapes
        print(json.dumps({"counted_steps": args.warmup + 1,
                          "step_call_kinds": [c[2] for c in calls]}), flush=True)
        return
    per_kind = {}
    evs = []
    for fn, a, k, ops, nbytes in calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(*a, sp)
        e1.record(stream)
        evs.append((k, e0, e1, ops, nbytes))
    torch.cuda.synchronize()
    for k, e0, e1, ops, nbytes in evs:
        d = per_kind.setdefault(k, [0, 0.0, 0, 0])
        d[0] += 1
        d[1] += e0.elapsed_time(e1)
        d[2] += ops
        d[3] += nbytes
    dominant = max((k for k in per_kind if k.startswith("qgemm")), key=lambda k: per_kind[k][1])
    kernels = {k: {"calls_per_step": v[0], "avg_us": round(1e3 * v[1] / v[0], 3),
                   "TOPS": round(v[2] / (v[1] * 1e-3) / 1e12, 2) if v[2] else None,
                   "GB_s": round(v[3] / (v[1] * 1e-3) / 1e9, 1)}
               for k, v in per_kind.items()}
    log("per-kind (isolated launches):", json.dumps(kernels))
    sampler = sampler_variants(lib, dq, torch, stream, sp, out_packed, canvas, idx, logits, ws,
                               cpu=not args.no_cpu_baseline)
    log("output projection feeding the samplers:", json.dumps(sampler))
    attn = attention_shapes(lib, dq, torch, stream, sp, up, cpu=not args.no_cpu_baseline)
    log("canvas attention:", json.dumps(attn))
    emb = embedding_rows(lib, torch, stream, sp, up, cpu=not args.no_cpu_baseline)
    log("embedding rows:", json.dumps(emb))

    # ------------------------------------------ the step as one HIP graph
    # The step's launches are captured once and replayed: the host then
    # issues one launch per step instead of one per kernel.  The replay is
    # checked against the eager step (both deterministic) before timing.
    ref = {n: outs[n].clone() for n in ("qkv", "down")}
    ref["logits"] = logits.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_calls(torch.cuda.current_stream().cuda_stream)
    for t in list(outs.values()) + [logits]:
        t.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    got = {"qkv": outs["qkv"], "down": outs["down"], "logits": logits}
    for n, t in got.items():
        if not torch.equal(t, ref[n]):
            raise RuntimeError(f"graph replay differs from the eager step in {n}")

    # ------------------------------------------------------------- timed run
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = 1e3 * elapsed / args.steps

    # --------------------------------- dominant kernel, launch by launch
    # HIP events around every launch of the dominant kernel, on its stream,
    # over the same number of eager steps.
    brackets = []
    torch.cuda.synchronize()
    for _ in range(args.steps):
        run_calls(sp, brackets, dominant)
    torch.cuda.synchronize()
    dom_ms = sum(e0.elapsed_time(e1) for e0, e1 in brackets)
    dom_launches = per_kind[dominant][0] * args.steps
    dom_bytes = per_kind[dominant][3] / per_kind[dominant][0]  # per launch (average)
    dom_ops = per_kind[dominant][2] / per_kind[dominant][0]
    dom_avg_s = dom_ms * 1e-3 / dom_launches
    bound = "hbm" if dom_ops / dom_bytes < (INT8_PEAK_TOPS * 1e12) / (HBM_PEAK_GBS * 1e9) else "mfma"
    if bound == "hbm":
        achieved, peak, unit = dom_bytes / dom_avg_s / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = dom_ops / dom_avg_s / 1e12, INT8_PEAK_TOPS, "TOPS"
    traffic = stored_traffic(dominant)
    configs = None if args.no_configs else config_lines(lib, dq, torch, stream, sp, up,
                                                        out_packed, canvas)
    if configs:
        log("configurations:", json.dumps(configs))

    step_s = ms_per_step * 1e-3
    result = {
        "metric": METRIC,
        "value": round(step_ops / step_s / 1e12, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "LLaDA-8B denoising step at canvas L=160: 32 layers x (4 int8 "
                               "activation quantizations, two fused with RMSNorm + Q/K/V/O "
                               "4096x4096, gate/up 12288x4096 (stacked, SiLU(gate)*up formed "
                               "in the GEMM's epilogue), down 4096x12288 K-quant GEMMs; down "
                               "Q6_K on odd layers, Q4_K on even) + output projection on 32 of "
                               "160 gathered rows, 126464x4096 Q6_K",
                   "L": L, "K": K, "ffn": F, "vocab": V, "layers": LAYERS, "rows": ROWS,
                   "step_GOP": round(step_ops / 1e9, 2),
                   "step_algorithmic_MB": round(step_bytes / 1e6, 1)},
        "hbm_GBs": round(step_bytes / step_s / 1e9, 1),
        "hbm_frac": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(step_ops / step_s / 1e12 / INT8_PEAK_TOPS, 4),
        "roofline": {"kernel": dominant, "bound": bound, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "traffic_source": ("profiles/traffic.json: rocprofv3 FETCH_SIZE + "
                                        "WRITE_SIZE per launch of this kernel, calibrated by a "
                                        f"plain copy; taken on sources with hash "
                                        f"{source_hash()}" if traffic is not None else
                                        "none: the kernel's sources changed since the counters "
                                        "were taken"),
                     "avg_launch_us": round(dom_avg_s * 1e6, 3),
                     "algorithmic_bytes_per_launch": int(dom_bytes),
                     "ops_per_launch": int(dom_ops), "launches": dom_launches},
        "kernels_isolated": kernels,
        "sampler_output_projection": sampler,
        "attention": attn,
        "embedding_rows": emb,
        "configs": configs,
        "step_timing": f"HIP graph replay of the step's {len(calls)} launches",
        "device": device_info(torch, dev),
        "clocks_rocm_smi": clocks_before,
        "host_cores": {"os_cpu_count": os.cpu_count(), "usable": _usable_cores()},
    }

    # ------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, host_keep, Wout, canvas_np, idx_np, acts,
                                                gammas)
    print(json.dumps(result), flush=True)


def _usable_cores():
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count()


def device_info(torch, dev):
    """Name, architecture, compute units and peak shader clock (hipDeviceGetAttribute)."""
    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int()
        # hipDeviceAttributeClockRate: peak clock in kHz
        attr = 5
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev.index or 0) == 0:
            info["peak_sclk_MHz"] = v.value // 1000
    except OSError:
        pass
    return info


def config_lines(lib, dq, torch, stream, sp, up, out_packed, canvas, reps=10):
    """Per-configuration lines beside the LLaDA-8B step (whose shapes are configs
    2 and 3, and config 4 at 32 rows):
      * config 1, the single 16x256x512 Q4_K GEMM: a correctness configuration
        (launch-bound; its parity is in the tests), timed only;
      * config 4 at 1 and 8 gathered rows (126,464 x 4096 Q6_K logits);
      * config 5, Dream-7B at canvas L = 512 (K = 3584): Q/K/V stacked into one
        4608 x 3584 Q4_K matrix, O 3584 x 3584, gate/up stacked 37888 x 3584, down
        3584 x 18944 Q6_K, over 8 layers of seeded weights (1.2 GB, rotated so
        that HBM, not the 256 MB last-level cache, serves them), plus the output
        projection on 64 gathered rows (152,064 x 3584 Q6_K).
    HIP events around `reps` rounds of launches on the step's stream; per GEMM:
    us, TOPS, algorithmic GB/s and the fraction of the binding roofline
    (max of bytes / HBM peak and operations / int8 MFMA peak)."""
    dev = canvas.device

    def line(us, ops, nbytes, extra=None):
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = ops / (INT8_PEAK_TOPS * 1e12)
        d = {"us": round(us, 2), "TOPS": round(ops / us / 1e6, 2),
             "GB_s": round(nbytes / us / 1e3, 1), "bound": "hbm" if t_hbm >= t_mfma else "mfma",
             "bound_us": round(1e6 * max(t_hbm, t_mfma), 2),
             "roofline_frac": round(1e6 * max(t_hbm, t_mfma) / us, 4)}
        if extra:
            d.update(extra)
        return d

    def timed(fns):
        for f in fns:
            if f():
                raise RuntimeError(lib.dq_last_error().decode())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for f in fns:
                f()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / (reps * len(fns))

    res = {}
    # config 1
    rng = np.random.default_rng(0)
    x1 = up(synth.activations(rng, 16, 512))
    W1 = synth.q4k_weights(rng, 256, 512)
    p1 = dq.repack_weights(Q4_K, 256, 512, up(W1.reshape(-1)))
    a1 = dq.quantize_act(x1)
    y1 = torch.empty((16, 256), dtype=torch.float32, device=dev)
    us = timed([lambda: lib.dq_qgemm(Q4_K, 16, 256, 512, a1.buf.data_ptr(), p1.data_ptr(),
                                     y1.data_ptr(), 256, sp)])
    res["config1_q4k_16x256x512"] = line(us, 2 * 16 * 256 * 512, gemm_bytes(Q4_K, 16, 256, 512),
                                         {"note": "correctness configuration: launch-bound"})
    # config 4 at 1 and 8 rows
    for M in (1, 8):
        idx = up(synth.row_index(np.random.default_rng(synth.seed(3, 0, 2) + M), L, M))
        y = torch.empty((M, V), dtype=torch.float32, device=dev)
        wsr = torch.empty(dq.qgemm_rows_workspace(M, K), dtype=torch.uint8, device=dev)
        us = timed([lambda: lib.dq_qgemm_rows(Q6_K, L, M, V, K, canvas.data_ptr(), K,
                                              idx.data_ptr(), out_packed.data_ptr(),
                                              y.data_ptr(), V, wsr.data_ptr(), wsr.numel(), sp)])
        nbytes = V * (K // 256) * BLOCK[Q6_K] + M * K * 4 + M * 4 + M * V * 4
        res[f"config4_llada_logits_rows{M}"] = line(us, 2 * M * V * K, nbytes)
    # config 5
    D, LD = synth.DREAM, 512
    KD, FD, KVD, VD = D["K"], D["ffn"], D["kv"], D["vocab"]
    layers = 8
    xd = up(synth.activations(np.random.default_rng(synth.seed(4, 0, 9)), LD, KD))
    xf = up(synth.activations(np.random.default_rng(synth.seed(4, 0, 8)), LD, FD))
    ad, af = dq.quantize_act(xd), dq.quantize_act(xf)
    shapes = {"qkv": (Q4_K, KD + 2 * KVD, KD, ad), "o": (Q4_K, KD, KD, ad),
              "gateup": (Q4_K, 2 * FD, KD, ad), "down": (Q6_K, KD, FD, af)}
    mats = {n: [] for n in shapes}
    for layer in range(layers):
        for n, (t, N, KK, _) in shapes.items():
            W = synth.weights(np.random.default_rng(synth.seed(4, layer + 1, len(mats[n]) + 17)),
                              t, N, KK)
            mats[n].append(dq.repack_weights(t, N, KK, up(W.reshape(-1))))
            del W
    ys = {n: torch.empty((LD, shapes[n][1]), dtype=torch.float32, device=dev) for n in shapes}
    total_us = 0.0
    for n, (t, N, KK, a) in shapes.items():
        fns = [(lambda pk=pk, t=t, N=N, KK=KK, a=a, y=ys[n]:
                lib.dq_qgemm(t, LD, N, KK, a.buf.data_ptr(), pk.data_ptr(), y.data_ptr(), N, sp))
               for pk in mats[n]]
        us = timed(fns)
        total_us += us
        res[f"config5_dream_{n}_{LD}x{N}x{KK}_{'q4k' if t == Q4_K else 'q6k'}"] = line(
            us, 2 * LD * N * KK, gemm_bytes(t, LD, N, KK))
    ops = sum(2 * LD * N * KK for t, N, KK, _ in shapes.values())
    nbytes = sum(gemm_bytes(t, LD, N, KK) for t, N, KK, _ in shapes.values())
    res["config5_dream_layer_gemms"] = line(total_us, ops, nbytes,
                                            {"note": "Q/K/V + O + gate/up + down of one layer"})
    del mats
    Wd = synth.q6k_weights(np.random.default_rng(synth.seed(4, 0, 7)), VD, KD)
    pd = dq.repack_weights(Q6_K, VD, KD, up(Wd.reshape(-1)))
    del Wd
    cd = up(synth.activations(np.random.default_rng(synth.seed(4, 0, 6)), LD, KD))
    idx = up(synth.row_index(np.random.default_rng(synth.seed(4, 0, 5)), LD, 64))
    y = torch.empty((64, VD), dtype=torch.float32, device=dev)
    wsr = torch.empty(dq.qgemm_rows_workspace(64, KD), dtype=torch.uint8, device=dev)
    us = timed([lambda: lib.dq_qgemm_rows(Q6_K, LD, 64, VD, KD, cd.data_ptr(), KD,
                                          idx.data_ptr(), pd.data_ptr(), y.data_ptr(), VD,
                                          wsr.data_ptr(), wsr.numel(), sp)])
    nbytes = VD * (KD // 256) * BLOCK[Q6_K] + 64 * KD * 4 + 64 * 4 + 64 * VD * 4
    res["config5_dream_logits_rows64"] = line(us, 2 * 64 * VD * KD, nbytes)
    return res


def _oracle_seconds(fn):
    """Wall time of one call of an oracle function (its C code runs single-threaded)."""
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def sampler_variants(lib, dq, torch, stream, sp, out_packed, canvas, idx, logits, ws, reps=20,
                     cpu=False):
    # reps = 0: one call of each, untimed (the counter runs)
    """The step's output projection as the samplers consume it (not part of the
    timed step, whose projection stores the logits): per requested row the greedy
    token, maximum, log-partition, entropy and top probability of the logits,
    (a) formed in the GEMM's epilogue (dq_qgemm_rows_sample: no logits stored)
    and (b) by storing the logits and reducing them (dq_qgemm_rows, then
    dq_logits_stats).  HIP events around `reps` back-to-back calls of each on
    the step's stream; both read the 425 MB weight matrix from HBM every call
    (it is larger than the last-level cache)."""
    dev = canvas.device
    beta = ctypes.c_float(1.0 / 64)
    token = torch.empty(ROWS, dtype=torch.int32, device=dev)
    stats = torch.empty((ROWS, 4), dtype=torch.float32, device=dev)
    ws_f = torch.empty(dq.qgemm_rows_sample_workspace(ROWS, V, K), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(dq.logits_stats_workspace(ROWS, V), dtype=torch.uint8, device=dev)

    def fused():
        return lib.dq_qgemm_rows_sample(Q6_K, L, ROWS, V, K, canvas.data_ptr(), K, idx.data_ptr(),
                                        out_packed.data_ptr(), beta, token.data_ptr(),
                                        stats.data_ptr(), ws_f.data_ptr(), ws_f.numel(), sp)

    def unfused():
        return (lib.dq_qgemm_rows(Q6_K, L, ROWS, V, K, canvas.data_ptr(), K, idx.data_ptr(),
                                  out_packed.data_ptr(), logits.data_ptr(), V, ws.data_ptr(),
                                  ws.numel(), sp)
                or lib.dq_logits_stats(ROWS, V, logits.data_ptr(), V, beta, token.data_ptr(),
                                       stats.data_ptr(), ws_s.data_ptr(), ws_s.numel(), sp))

    weights = V * (K // 256) * BLOCK[Q6_K]
    rows_in = ROWS * K * 4 + ROWS * 4           # gathered f32 rows and their indices
    stats_out = ROWS * (4 + 16)                 # token and 4 statistics per row
    out = {"rows": ROWS, "vocab": V, "K": K, "beta": 1.0 / 64}
    for name, fn, nbytes in (("fused", fused, weights + rows_in + stats_out),
                             ("unfused", unfused, weights + rows_in + stats_out
                              + 2 * ROWS * V * 4)):  # logits written, then read back
        for _ in range(3 if reps else 1):
            if fn():
                raise RuntimeError(lib.dq_last_error().decode())
        torch.cuda.synchronize()
        if not reps:
            continue
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        out[f"{name}_us"] = round(us, 2)
        out[f"{name}_algorithmic_MB"] = round(nbytes / 1e6, 2)
        out[f"{name}_GB_s"] = round(nbytes / us / 1e3, 1)
    if not reps:
        return out
    # the fused result is the unfused one's, bit for bit in token and maximum
    tok_u, st_u = token.clone(), stats.clone()
    fused()
    torch.cuda.synchronize()
    if not (torch.equal(token, tok_u) and torch.equal(stats[:, 0], st_u[:, 0])):
        raise RuntimeError("fused and unfused sampler statistics differ")
    if cpu:
        # the oracle's statistics step on seeded logits of the same shape (its
        # projection is timed in cpu_baseline)
        import oracle
        y = np.random.default_rng(7).standard_normal((ROWS, V)) * 64.0
        out["cpu_oracle_stats_us"] = round(1e6 * _oracle_seconds(
            lambda: oracle.logits_stats(y, 1.0 / 64)), 1)
        out["cpu_oracle_cores"] = 1
    return out


def attention_shapes(lib, dq, torch, stream, sp, up, reps=20, cpu=False):
    """Bidirectional attention over the LLaDA-8B (L = 160, 32 heads, NORM RoPE) and
    Dream-7B (L = 512, 28 query heads over 4 kv heads, NEOX RoPE) canvases, on
    seeded Q/K/V rows: not part of the timed step (whose O projection reads a
    seeded input).  HIP events around `reps` back-to-back calls on the step's
    stream; algorithmic bytes are the f32 Q/K/V rows and RoPE table read and the
    f32 output written, operations 4 L^2 H D (two products)."""
    res = {}
    for name, cfg, mode in (("llada", synth.LLADA, 1), ("dream", synth.DREAM, 2)):
        Ln, H, Hkv, D = cfg["L"], cfg["heads"], cfg["kv_heads"], cfg["head_dim"]
        rng = np.random.default_rng(synth.seed(6, 0, mode))
        qkv = up(synth.qkv_rows(rng, Ln, H, Hkv, D))
        tab = up(synth.rope_table(Ln, D, cfg["rope_theta"]))
        out = torch.empty((Ln, H * D), dtype=torch.float32, device=qkv.device)
        wsa = torch.empty(dq.attention_workspace(Ln, H, Hkv, D), dtype=torch.uint8,
                          device=qkv.device)
        args = (Ln, H, Hkv, D, qkv.data_ptr(), qkv.shape[1], tab.data_ptr(), mode,
                out.data_ptr(), H * D, wsa.data_ptr(), wsa.numel(), sp)
        for _ in range(3 if reps else 1):
            if lib.dq_attention(*args):
                raise RuntimeError(lib.dq_last_error().decode())
        torch.cuda.synchronize()
        if not reps:
            continue
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            lib.dq_attention(*args)
        e1.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        nbytes = qkv.numel() * 4 + tab.numel() * 4 + out.numel() * 4
        flops = 4 * Ln * Ln * H * D
        res[name] = {"L": Ln, "heads": H, "kv_heads": Hkv, "us": round(us, 2),
                     "algorithmic_MB": round(nbytes / 1e6, 2), "GB_s": round(nbytes / us / 1e3, 1),
                     "TFLOPs": round(flops / us / 1e6, 2),
                     "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        if cpu:
            # the oracle on one kv head and its query heads, scaled to all of them
            import oracle
            G = H // Hkv
            q_np = synth.qkv_rows(np.random.default_rng(synth.seed(6, 0, mode)), Ln, H, Hkv, D)
            sub = np.concatenate([q_np[:, :G * D], q_np[:, H * D:(H + 1) * D],
                                  q_np[:, (H + Hkv) * D:(H + Hkv + 1) * D]], axis=1)
            tab_np = synth.rope_table(Ln, D, cfg["rope_theta"])
            sec = _oracle_seconds(lambda: oracle.attention(sub, G, 1, D, tab_np, mode))
            res[name]["cpu_oracle_us"] = round(1e6 * sec * Hkv, 1)
            res[name]["cpu_oracle_sample"] = f"1 of {Hkv} kv heads ({G} query heads), x{Hkv}"
            res[name]["cpu_oracle_cores"] = 1
    return res


def embedding_rows(lib, torch, stream, sp, up, reps=20, cpu=False):
    """The canvas's embedding rows: 160 token ids into the LLaDA-8B token table
    (126,464 x 4096 Q4_K, 291 MB, as stored in the GGUF file), decoded to f32 (not
    part of the timed step).  HIP events around `reps` calls; algorithmic bytes are
    the selected rows' blocks, the ids and the f32 output."""
    rng = np.random.default_rng(synth.seed(5, 0, 0))
    table_np = synth.q4k_weights(rng, V, K).reshape(V, -1)
    ids_np = rng.integers(0, V, L).astype(np.int32)
    table, ids = up(table_np.reshape(-1)), up(ids_np)
    out = torch.empty((L, K), dtype=torch.float32, device=table.device)
    flags = torch.empty(L, dtype=torch.int32, device=table.device)
    args = (Q4_K, V, K, table.data_ptr(), ids.data_ptr(), L, out.data_ptr(), K, flags.data_ptr(),
            sp)
    for _ in range(3 if reps else 1):
        if lib.dq_embed_rows(*args):
            raise RuntimeError(lib.dq_last_error().decode())
    torch.cuda.synchronize()
    if not reps:
        return None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        lib.dq_embed_rows(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / reps
    nbytes = L * (K // 256) * BLOCK[Q4_K] + L * 4 + L * K * 4
    res = {"rows": L, "table": f"{V}x{K} Q4_K", "us": round(us, 2),
           "algorithmic_MB": round(nbytes / 1e6, 3), "GB_s": round(nbytes / us / 1e3, 1),
           "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    if cpu:
        import oracle
        res["cpu_oracle_us"] = round(1e6 * _oracle_seconds(
            lambda: oracle.embed_rows(Q4_K, table_np, K, ids_np)), 1)
        res["cpu_oracle_cores"] = 1
    return res


def cpu_baseline(args, host_keep, Wout, canvas_np, idx_np, acts, gammas):
    """The oracle, as it stands, on the first layers of the step plus 1/4 of the vocab rows."""
    import oracle

    th = args.cpu_threads or oracle.host_threads()
    xs = {k: v.cpu().numpy() for k, v in acts.items()}
    ops = 0
    t0 = time.perf_counter()
    for layer in range(args.cpu_layers):
        g = {n: gammas[layer][n].cpu().numpy() for n in ("qkv", "ffn")}
        y_gu = None
        for name in ("qkv", "o", "gateup", "down"):
            W = host_keep[(layer, name)]
            t = Q6_K if W.shape[-1] == 210 else Q4_K
            N, KK = W.shape[0], W.shape[1] * 256
            if name == "qkv":
                q, d, b = oracle.rmsnorm_quantize_act(xs["qkv"], g["qkv"], EPS)
            elif name == "o":
                q, d, b = oracle.quantize_act(xs["o"])
            elif name == "gateup":
                q, d, b = oracle.rmsnorm_quantize_act(xs["ffn"], g["ffn"], EPS)
            else:
                q, d, b = oracle.swiglu_quantize_act(y_gu, F)
            y = oracle.qgemm_f32(t, q, d, b, W, N, threads=th)
            if name == "gateup":  # interleaved 16-row tiles -> [gate | up]
                yt = y.reshape(L, F // 16, 2, 16)
                y_gu = np.concatenate([yt[:, :, 0].reshape(L, F), yt[:, :, 1].reshape(L, F)], 1)
            ops += 2 * L * N * KK
    nv = V // 4
    gq, gd, gb = oracle.qgemm_rows_inputs(canvas_np, idx_np)
    oracle.qgemm_f32(Q6_K, gq, gd, gb, Wout.reshape(V, -1)[:nv], nv, threads=th)
    ops += 2 * ROWS * nv * K
    dt = time.perf_counter() - t0
    return {"value": round(ops / dt / 1e12, 5), "unit": "TOPS", "cores": th, "kind": "oracle",
            "sample": f"oracle RMSNorm/SwiGLU/plain quantize + integer-decomposition GEMM on "
                      f"{args.cpu_layers} of 32 "
                      f"layers (all projections, L=160) and 1/4 of the 126464 vocab rows at "
                      f"M=32: {ops / 1e9:.1f} GOP in {dt:.1f} s"}


if __name__ == "__main__":
    main()
