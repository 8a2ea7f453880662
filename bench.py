#!/usr/bin/env python3
"""Benchmark of the MI355X MoE feed-forward layer (DiffusionGemma 26B-A4B shape).

One step = one dg_moe_forward over one batch of T tokens: router, permutation, gate_up grouped GEMM,
down grouped GEMM and combine, on inputs already resident in HBM. The default workload is one layer
over a 256-token canvas, bf16, with the Zipf-skewed router bias; the weights rotate over several
resident copies so that no cache holds them from one step to the next. The expert weights are packed at
create into the GEMMs' fragment order (--borrow reads them in place, row-major).

Prints one JSON line: tokens/s, the roofline of the dominant kernel (the fused gate_up + down launch,
HBM-bound) measured with HIP events on the launch stream, and the CPU oracle timed on the host on a
bounded sample.

--workload head256 measures the canvas output stage instead (dg_head_forward: the tied LM head over a
256-position canvas, vocabulary 262144, fp32 logits written, plus the per-position softmax entropy), one
step = one call; the same JSON fields, with the logits kernel as the dominant one.

  python bench.py [--steps K] [--warmup W]
                  [--workload canvas256|encode2304|int4|q8|mxfp4|mxfp8|canvas32|stack30|head256]
"""
import argparse
import ctypes
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s per canvas step (T=256, bf16) + % of HBM/MFMA roofline"
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
F16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_NAMES = ("norm", "logits_topk", "permute", "gate_up", "down", "combine")
HEAD_METRIC = ("canvas output stage tokens/s (tied LM head, T=256 x vocab 262144, fp32 logits, softmax entropy) "
               "+ % of HBM roofline")
HEAD_KERNEL_NAMES = ("logits_partials", "merge", "mean")


class HipEvents:
    """hipEvent_t through the HIP runtime the process already runs (torch's, same soname)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e.value)
        return evs

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def expert_bytes(wl):
    D, F = wl.D, wl.F
    if wl.experts == "i4g128":
        gu = 2 * F * (D // 2) + 2 * F * (D // 128) * 2
        dn = D * (F // 2) + D * ((F + 127) // 128) * 2
    elif wl.experts == "q8_0":  # 34 bytes per block of 32 inputs
        gu = 2 * F * (D // 32) * 34
        dn = D * (F // 32) * 34
    elif wl.experts in ("mxfp4", "mxfp8"):  # 17 or 33 bytes per block of 32 inputs
        blk = 17 if wl.experts == "mxfp4" else 33
        gu = 2 * F * (D // 32) * blk
        dn = D * (F // 32) * blk
    else:
        gu = 2 * F * D * 2
        dn = D * F * 2
    return gu, dn


def algorithmic(wl, T, touched):
    """Bytes and FLOPs the method must move / compute for one forward; intermediates (h, the gated
    activations, the per-slot outputs) are excluded. Returns (layer bytes, layer FLOPs, bytes of the fused
    GEMM launch: the touched experts' weights and the input rows x, bytes of the gate_up GEMM alone)."""
    D, F, E, K = wl.D, wl.F, wl.E, wl.K
    act_b = 4 if wl.act == "f32" else 2
    rw_b = 4 if wl.router_w == "f32" else 2
    gu, dn = expert_bytes(wl)
    layer_bytes = touched * (gu + dn) + E * D * rw_b + 2 * D * 4 + E * 4 + 2 * T * D * act_b
    flops = T * K * 2 * 3 * D * F + T * 2 * E * D
    gemm_bytes = touched * (gu + dn) + T * D * act_b
    gate_up_bytes = touched * gu + T * D * act_b
    return layer_bytes, flops, gemm_bytes, gate_up_bytes


def _code_only(text):
    """Source text without its comments and blank lines (what the compiler sees of it)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_sources_digest():
    """Digest of the code of every source of the layer's library (the GEMMs, and the router, permutation and
    host code that set what they read), comments left out: counters taken on other code do not describe this
    build."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "expert_ffn_canvas_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "head.hip" or not name.endswith((".hip", ".h")):
            continue
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_counters(workload, kernel):
    """The committed rocprofv3 record of `kernel` for this workload (profiles/<workload>_gemm_counters.txt):
    HBM bytes per launch (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's reading) and the kernel's
    average duration in the kernel trace, if the record was taken on the current sources; else None."""
    path = os.path.join(PROFILES, f"{workload}_gemm_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if (kv.get("source_digest") != kernel_sources_digest() or kv.get("workload") != workload
            or kv.get("kernel") != kernel):
        return None
    out = {}
    for key in ("traffic_bytes_per_launch", "rocprof_avg_us"):
        try:
            out[key] = float(kv[key])
        except (KeyError, ValueError):
            out[key] = None
    return out


def host_cpu():
    """Model name of the host CPU (from /proc/cpuinfo) and the threads the OS offers."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


def percentiles(us):
    """Median, p10, p90, min, max of per-step times (us) and the spread p90 / p10."""
    import statistics
    v = sorted(us)
    q = lambda f: v[min(len(v) - 1, max(0, int(round(f * (len(v) - 1)))))]
    return {"median": round(statistics.median(v), 2), "p10": round(q(0.1), 2), "p90": round(q(0.9), 2),
            "min": round(v[0], 2), "max": round(v[-1], 2), "spread_p90_p10": round(q(0.9) / q(0.1), 4),
            "n": len(v)}


def _time_oracle(fn, budget_s, max_reps=64):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or reps >= max_reps:
            return reps, dt


def cpu_baseline(wl, x, w, threads):
    """The oracle, as it stands, on a bounded sample of this workload's batch on the host: all threads the
    host offers over 256 tokens (about ten seconds of work), and one thread over 16 tokens."""
    import oracle
    from expert_ffn_canvas_amd import synth

    wn = synth.weights_to_numpy(w)
    xn = synth.to_numpy_bits(x)
    T = x.shape[0]
    n_tok = min(T, 256)
    tok = list(range(n_tok))
    oracle.load()
    reps, dt = _time_oracle(lambda: oracle.moe_forward(wn, xn, wl.K, synth.RMS_EPS, tokens=tok, n_threads=threads),
                            10.0)
    tok1 = list(range(min(T, 16)))
    reps1, dt1 = _time_oracle(lambda: oracle.moe_forward(wn, xn, wl.K, synth.RMS_EPS, tokens=tok1, n_threads=1),
                              3.0)
    model, n_os = host_cpu()
    return {"value": round(reps * n_tok / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "threads": threads, "os_threads": n_os,
            "one_thread_value": round(reps1 * len(tok1) / dt1, 3),
            "sample": f"{n_tok} tokens of the {wl.name} batch (T={T}), all {wl.K} slots each, one layer, "
                      f"{reps} times on {threads} threads ({dt:.2f} s wall); one-thread leg: {len(tok1)} "
                      f"tokens, {reps1} times ({dt1:.2f} s wall). cores = the threads used (OpenMP), "
                      f"not physical cores"}


def head_cpu_baseline(hw, h, emb, threads):
    """The output-stage oracle, as it stands, on a bounded sample of positions of the batch."""
    import oracle
    from expert_ffn_canvas_amd import synth

    hb, eb = synth.to_numpy_bits(h.cpu()), synth.to_numpy_bits(emb.cpu())
    tok = [0, hw.T - 1]
    oracle.load()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.canvas_head(hb, eb, beta=1.0, tokens=tok, n_threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 64:
            break
    model, n_os = host_cpu()
    return {"value": round(reps * len(tok) / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "threads": threads, "os_threads": n_os,
            "sample": f"positions 0 and {hw.T - 1} of the {hw.name} batch, each against all {hw.V} vocabulary rows "
                      f"(logits, entropy, argmax), {reps} times on {threads} threads; {dt:.2f} s wall. cores = the "
                      f"threads used (OpenMP), not physical cores"}


def run_head(args, torch, dgmoe, synth):
    hw = synth.HEAD_WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    sp = torch.cuda.current_stream().cuda_stream
    t_setup = time.perf_counter()
    inp = synth.make_head_inputs(hw, device=dev)
    h, emb = inp["h"], inp["emb"]
    head = dgmoe.CanvasHead(emb, max_tokens=hw.T)
    T, V, D = hw.T, hw.V, hw.D
    logits = torch.empty((T, V), dtype=torch.float32, device=dev)
    ent = torch.empty((T,), dtype=torch.float32, device=dev)
    am = torch.empty((T,), dtype=torch.int32, device=dev)
    mean = torch.empty((1,), dtype=torch.float32, device=dev)
    ptrs = (logits.data_ptr(), ent.data_ptr(), am.data_ptr(), mean.data_ptr())
    print(f"[bench] {hw.name}: T={T} V={V} D={D} setup {time.perf_counter() - t_setup:.1f}s", file=sys.stderr,
          flush=True)

    def step():
        st = dgmoe.dg_head_forward(head.handle, h.data_ptr(), T, 1.0, *ptrs, sp)
        assert st == 0, dgmoe.dg_moe_last_error()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents()
    e0, e1 = ev.create(2)
    w0 = time.perf_counter()
    ev.record(e0, sp)
    for _ in range(args.steps):
        step()
    ev.record(e1, sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev.elapsed_ms(e0, e1)
    ms_per_step = gpu_ms / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall:.3f}s)", file=sys.stderr,
          flush=True)

    step_stats = None
    if not args.no_profile:
        evs = ev.create(2 * args.steps)
        for i in range(args.steps):
            ev.record(evs[2 * i], sp)
            step()
            ev.record(evs[2 * i + 1], sp)
        torch.cuda.synchronize()
        step_stats = percentiles([ev.elapsed_ms(evs[2 * i], evs[2 * i + 1]) * 1e3 for i in range(args.steps)])
        ev.destroy(evs)

    kern_us = None
    n_prof = 0 if args.no_profile else min(args.steps, 50)
    if n_prof:
        nk = len(HEAD_KERNEL_NAMES)
        evs = ev.create(2 * nk * n_prof)
        for i in range(n_prof):
            st = dgmoe.dg_head_forward_profiled(head.handle, h.data_ptr(), T, 1.0, *ptrs,
                                                evs[2 * nk * i:2 * nk * (i + 1)], sp)
            assert st == 0, dgmoe.dg_moe_last_error()
        torch.cuda.synchronize()
        tot = [0.0] * nk
        for i in range(n_prof):
            for k in range(nk):
                tot[k] += ev.elapsed_ms(evs[2 * nk * i + 2 * k], evs[2 * nk * i + 2 * k + 1])
        kern_us = {name: round(tot[k] / n_prof * 1e3, 2) for k, name in enumerate(HEAD_KERNEL_NAMES)}
        ev.destroy(evs)
    ev.destroy([e0, e1])

    # algorithmic work: the table and the hidden states read once, the logits written once
    stage_bytes = V * D * 2 + T * D * 2 + T * V * 4 + T * 4 * 2 + 4
    flops = 2 * T * V * D
    step_s = ms_per_step / 1e3
    roofline = None
    if kern_us:
        kbytes = V * D * 2 + T * D * 2 + T * V * 4
        ach = kbytes / (kern_us["logits_partials"] / 1e6) / 1e9
        roofline = {"bound": "hbm", "kernel": "logits_partials", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None,
                    "alg_bytes_per_launch": kbytes, "avg_launch_us": kern_us["logits_partials"],
                    "mfma_frac": round(flops / (kern_us["logits_partials"] / 1e6) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    result = {
        "metric": HEAD_METRIC,
        "value": round(T * args.steps / (gpu_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": hw.name, "T": T, "vocab": V, "d_model": D, "beta": 1.0,
                   "logits": "fp32, written", "table": "bf16 row-major, read in place"},
        "roofline": roofline,
        "stage": {"alg_bytes": stage_bytes, "alg_flops": flops,
                  "achieved_GBps": round(stage_bytes / step_s / 1e9, 1),
                  "hbm_frac": round(stage_bytes / step_s / 1e9 / HBM_PEAK_GBPS, 4),
                  "mfma_frac": round(flops / step_s / 1e12 / BF16_PEAK_TFLOPS, 4),
                  "mean_entropy": round(float(mean.item()), 5)},
        "step_us": step_stats,
        "kernels_us": kern_us,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        result["cpu_baseline"] = head_cpu_baseline(hw, h, emb, threads)
    head.close()
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="canvas256")
    ap.add_argument("--rotate", type=int, default=4, help="resident weight copies cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event pass")
    ap.add_argument("--borrow", action="store_true",
                    help="borrow the expert weights in their row-major layout instead of packing them at create")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this many MiB (3 times), so that a counter run "
                         "records HBM bytes for a transfer of known size")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU here; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from expert_ffn_canvas_amd import dgmoe, synth

    if args.workload in synth.HEAD_WORKLOADS:
        run_head(args, torch, dgmoe, synth)
        return
    wl = synth.WORKLOADS[args.workload]
    if args.borrow and wl.experts in ("q8_0", "mxfp4", "mxfp8"):
        print(json.dumps({"error": "Q8_0, MXFP4 and MXFP8 experts are read from the packed copy only; drop --borrow"}))
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    act = torch.float32 if wl.act == "f32" else torch.bfloat16
    T = wl.T
    t_setup = time.perf_counter()
    inp = synth.make_inputs(wl, device=dev)
    x = inp["x"]

    # handles: for a single layer, `rotate` copies of the weights; for the stack, its 30 layers
    if wl.layers > 1:
        sets = inp["layers"]
        rotate = 1
    else:
        base = inp["layers"][0]
        sets = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()}
                         for _ in range(max(args.rotate, 1) - 1)]
        rotate = len(sets)
    layers = [dgmoe.MoELayer(w, max_tokens=T, act_dtype=act, top_k=wl.K, pack=not args.borrow) for w in sets]
    out = torch.empty((T, wl.D), dtype=act, device=dev)
    bufs = [torch.empty_like(x), torch.empty_like(x)]
    deltas = inp["deltas"]

    def step(i):
        if wl.layers > 1:
            # x stays the stack input; the layers ping-pong between two buffers
            src = x
            for l, layer in enumerate(layers):
                dst = bufs[l % 2]
                st = dgmoe.dg_moe_forward(layer.handle, src.data_ptr(), dst.data_ptr(), T,
                                          deltas[l].data_ptr(), dgmoe.DG_FWD_ADD_INPUT, sp)
                assert st == 0, dgmoe.dg_moe_last_error()
                src = dst
        else:
            layer = layers[i % rotate]
            st = dgmoe.dg_moe_forward(layer.handle, x.data_ptr(), out.data_ptr(), T, None, 0, sp)
            assert st == 0, dgmoe.dg_moe_last_error()

    # routing statistics of the benchmark batch: every layer's touched experts (the bytes it must read)
    touched_l, max_load = [], 0
    src = x
    for l, layer in enumerate(layers if wl.layers > 1 else layers[:1]):
        c = layer.forward_debug(src)["counts"].cpu()
        touched_l.append(int((c > 0).sum()))
        max_load = max(max_load, int(c.max()))
        if wl.layers > 1:  # the next layer's input, as the timed steps form it
            src = layer.forward(src, addend=deltas[l], add_input=True)
    torch.cuda.synchronize()
    touched = touched_l[0]
    print(f"[bench] {wl.name}: T={T} touched={touched_l if wl.layers > 1 else touched} max_load={max_load} "
          f"rotate={rotate} setup {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    ev = HipEvents()
    e0, e1 = ev.create(2)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev.record(e0, sp)
    for i in range(args.steps):
        step(i)
    ev.record(e1, sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev.elapsed_ms(e0, e1)
    ms_per_step = gpu_ms / args.steps
    tokens_per_s = T * args.steps / (gpu_ms / 1e3)
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall:.3f}s)",
          file=sys.stderr, flush=True)

    # per-step distribution: a second pass of the same steps, an event pair around each
    step_stats = None
    if not args.no_profile:
        evs = ev.create(2 * args.steps)
        for i in range(args.steps):
            ev.record(evs[2 * i], sp)
            step(i)
            ev.record(evs[2 * i + 1], sp)
        torch.cuda.synchronize()
        step_stats = percentiles([ev.elapsed_ms(evs[2 * i], evs[2 * i + 1]) * 1e3 for i in range(args.steps)])
        ev.destroy(evs)

    # per-kernel durations: a third pass with events stamped by each kernel's dispatch (single-layer
    # workloads)
    kern_us, kern_stats = None, None
    n_prof = 0 if (args.no_profile or wl.layers > 1) else min(args.steps, 100)
    if n_prof:
        nk = len(KERNEL_NAMES)
        evs = ev.create(2 * nk * n_prof)
        for i in range(n_prof):
            layer = layers[i % rotate]
            st = dgmoe.dg_moe_forward_profiled(layer.handle, x.data_ptr(), out.data_ptr(), T, None, 0,
                                               evs[2 * nk * i:2 * nk * (i + 1)], sp)
            assert st == 0, dgmoe.dg_moe_last_error()
        torch.cuda.synchronize()
        per = [[ev.elapsed_ms(evs[2 * nk * i + 2 * k], evs[2 * nk * i + 2 * k + 1]) * 1e3 for i in range(n_prof)]
               for k in range(nk)]
        kern_us = {name: round(sum(per[k]) / n_prof, 2) for k, name in enumerate(KERNEL_NAMES)}
        kern_stats = {name: percentiles(per[k]) for k, name in enumerate(KERNEL_NAMES)}
        kern_us["norm"] = 0.0  # no norm kernel runs (the router writes h): its events bracket nothing
        kern_stats.pop("norm")
        if layers[0].gemms_fused:  # one launch ran both GEMMs: its time is under gate_up+down
            kern_us["gate_up+down"] = kern_us.pop("gate_up")
            kern_us.pop("down")
            kern_stats["gate_up+down"] = kern_stats.pop("gate_up")
            kern_stats.pop("down")
        ev.destroy(evs)
    ev.destroy([e0, e1])

    n_layers = wl.layers
    layer_bytes = 0
    for t_l in touched_l:
        lb, flops, gemm_bytes, gate_up_bytes = algorithmic(wl, T, t_l)
        layer_bytes += lb
    layer_bytes_1, flops, gemm_bytes, gate_up_bytes = algorithmic(wl, T, touched)
    step_s = ms_per_step / 1e3
    layer_gbps = layer_bytes / step_s / 1e9
    peak_tflops = F16_PEAK_TFLOPS if wl.experts in ("i4g128", "q8_0") else BF16_PEAK_TFLOPS
    roofline = None
    if kern_us:
        # the dominant launch: the fused launch of both GEMMs (or gate_up where they run apart); its
        # algorithmic bytes are the touched experts' weights and the input rows
        kname = "gate_up+down" if "gate_up+down" in kern_us else "gate_up"
        kbytes = gemm_bytes if kname == "gate_up+down" else gate_up_bytes
        ach = kbytes / (kern_us[kname] / 1e6) / 1e9
        rec = read_counters(wl.name, kname) or {}
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                    "traffic": rec.get("traffic_bytes_per_launch"), "alg_bytes_per_launch": kbytes,
                    "avg_launch_us": kern_us[kname]}
        if rec.get("rocprof_avg_us"):
            roofline["rocprof_avg_launch_us"] = rec["rocprof_avg_us"]
            roofline["frac_rocprof"] = round(kbytes / (rec["rocprof_avg_us"] / 1e6) / 1e9 / HBM_PEAK_GBPS, 4)

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"i4g128": "int4-g128 weights, f16 MFMA", "q8_0": "q8_0 weights, f16 MFMA",
                  "mxfp4": "mxfp4 weights, bf16 MFMA", "mxfp8": "mxfp8 weights, bf16 MFMA"}.get(wl.experts, "bf16"),
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "n_experts": wl.E, "top_k": wl.K, "d_model": wl.D,
                   "d_ff": wl.F, "experts": wl.experts, "act": wl.act, "router_bias": wl.bias or "none",
                   "layers": n_layers, "weight_copies_rotated": rotate,
                   "expert_weights": "borrowed row-major" if args.borrow else "packed at create"},
        "roofline": roofline,
        "layer": {"alg_bytes": layer_bytes, "alg_flops": flops * n_layers,
                  "achieved_GBps": round(layer_gbps, 1), "hbm_frac": round(layer_gbps / HBM_PEAK_GBPS, 4),
                  "mfma_frac": round(flops * n_layers / step_s / 1e12 / peak_tflops, 4),
                  "touched_experts": touched_l if n_layers > 1 else touched, "max_expert_load": max_load},
        "step_us": step_stats,
        "kernels_us": kern_us,
        "kernels_us_stats": kern_stats,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        w_host = inp["layers"][0]
        result["cpu_baseline"] = cpu_baseline(wl, x, w_host, threads)
    for layer in layers:
        layer.close()
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
