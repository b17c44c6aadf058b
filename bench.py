#!/usr/bin/env python3
"""Benchmark of the MoE indirect matmul hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--config lite|dec1|dec8|skew|v3|dec1x|dec8x|ppx|dec1n|dec8n|ppn|dec1s|dec8s|pps|rowids|gather]

A step is one full pass of the hot path -- row ids, gate/up grouped GEMM, down
grouped GEMM, fixed-order reduce (or the GEMV decode kernels) -- over one batch of
synthetic input already resident in HBM. The default workload is the
DeepSeek-Lite-shaped PP512 layer (E64 k6 + 2 shared, n_embd 2048, n_ff 1408,
Q8_0, 512 tokens). Weights are rotated through R copies so the set read per step
is not served from the 256 MB last-level cache.

Prints ONE JSON line: tokens/s (value), TFLOP/s, GB/s, a roofline entry for the
dominant kernel (timed with HIP events on the launch stream) and the CPU oracle
timed on a bounded sample of the same workload on this host. The same line carries,
under "workloads", the Zipf-skewed PP4096 prefill, the DeepSeek-V3-shaped PP8192 layer and
the GPT-OSS-20B-shaped decode batches of 1 and 8 tokens (--extra), each with its own
dominant-kernel roofline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA (the quantized-activation path)
Q8_BYTES = 34.0 / 32.0      # Q8_0: 32 int8 + one fp16 scale per 32 weights
MXFP4_BYTES = 17.0 / 32.0   # MXFP4: 32 four-bit codes + one E8M0 scale byte per 32 weights
IQ4NL_BYTES = 18.0 / 32.0   # IQ4_NL: 32 four-bit codes + one fp16 scale per 32 weights
IQ4XS_BYTES = 136.0 / 256.0  # IQ4_XS: 256 four-bit codes + one 8-byte record per 256 weights

STAGES = {1: ["row_ids", "gemm_gate_up", "gemm_down", "reduce"],
          2: ["gemv_gate_up", "gemv_down", "reduce"],
          3: ["row_ids", "quant_x", "gemm_gate_up", "quant_h", "gemm_down", "reduce"]}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed warm-up steps of the headline workload (default: at least 20 "
                        "steps and 0.2 s of them, so the GPU clocks have ramped up; the count is "
                        "reported). The further workloads (--extra) always warm up that long.")
    p.add_argument("--config", default="lite",
                   help="a workload of synth.CONFIGS, rowids, gather, or crossover (GEMV against GEMM)")
    p.add_argument("--rotate", type=int, default=0, help="weight copies (0 = auto)")
    p.add_argument("--path", type=int, default=0, help="0 auto, 1 GEMM, 2 GEMV")
    p.add_argument("--act-quant", type=int, default=0,
                   help="1: quantized activations (int8 MFMA grouped GEMM, Q8_0 experts)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--graph", type=int, default=0,
                   help="1: time replays of one HIP graph per weight copy (each graph holds one "
                        "step); 0: eager calls")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--extra", default="dec1,dec8,skew,v3",
                   help="further workloads reported on the same line under 'workloads' "
                        "(comma-separated, timed in this order before the headline one; "
                        "empty for none)")
    p.add_argument("--extra-cpu-seconds", type=float, default=3.0,
                   help="CPU oracle budget for each further workload")
    p.add_argument("--gather-shapes", default="skew,v3",
                   help="--config gather: the input shapes timed (skew, v3; the value is the last one)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="first run one device-to-device copy of this many MiB (a known-size "
                        "kernel for scaling HBM byte counters)")
    return p.parse_args()


def workload_stats(inp, cfg, h_bytes=2):
    """Algorithmic work of one step (flops, bytes) and per-kernel algorithmic bytes,
    counted by one rule: the weights of the experts the batch touches (each once) and
    the shared experts' weights, the layer input x read once, the layer output written
    once. Intermediates (h, the per-slot down results) are implementation traffic and
    are not credited; their bytes are reported beside ("intermediate_bytes")."""
    T, k = inp["ids"].shape
    E, n_embd, n_ff, S = cfg.n_experts, cfg.n_embd, cfg.n_ff, cfg.n_shared
    ids = inp["ids"].ravel()
    touched = len(np.unique(ids[(ids >= 0) & (ids < E)]))
    rows_routed = int(((ids >= 0) & (ids < E)).sum())
    rows = rows_routed + T * S                      # routed slots + shared-expert rows
    flops = 2.0 * rows * 3 * n_embd * n_ff
    wb = {"mxfp4": MXFP4_BYTES, "iq4_nl": IQ4NL_BYTES, "iq4_xs": IQ4XS_BYTES}.get(cfg.wtype, Q8_BYTES)
    w_gu = (touched + S) * 2 * n_ff * n_embd * wb
    w_dn = (touched + S) * n_embd * n_ff * wb
    x_b = T * n_embd * 2                            # bf16 input
    out_b = T * n_embd * 4                          # fp32 layer output
    h_b = rows * n_ff * h_bytes                     # silu(g)*u, written once and read once
    y_b = rows * n_embd * 4                         # per-slot fp32 down results
    return {
        "flops": flops, "bytes": w_gu + w_dn + x_b + out_b, "touched": touched,
        "gate_up": {"bytes": w_gu + x_b, "flops": 2.0 * rows * 2 * n_embd * n_ff,
                    "intermediate_bytes": h_b},
        "down": {"bytes": w_dn, "flops": 2.0 * rows * n_embd * n_ff,
                 "intermediate_bytes": h_b + y_b},
        # decode batches whose down GEMV also does the weighted reduce and writes out
        "down_reduce": {"bytes": w_dn + out_b, "flops": 2.0 * rows * n_embd * n_ff,
                        "intermediate_bytes": h_b},
        "reduce": {"bytes": out_b, "flops": 0.0, "intermediate_bytes": y_b},
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _omp_threads(n):
    """Set the OpenMP thread count of this process (the oracle's parallel loops)."""
    import ctypes
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


def cpu_baseline(inp, budget_s, flops_per_token, threads=None):
    """The oracle, as it stands, on a bounded token sample: tokens/s and fp64 GFLOP/s
    (the same algorithmic flops as the GPU figures) on this host. The sample grows until
    one pass takes about a quarter of the budget; when the whole batch is faster than
    that, whole-batch passes repeat until the budget."""
    import oracle
    oracle.lib()
    all_threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    used = threads or all_threads
    _omp_threads(used)
    try:
        T = inp["ids"].shape[0]
        n = min(T, 4)
        while True:
            rows = np.arange(n)
            t0 = time.perf_counter()
            oracle.ffn(inp, token_rows=rows)
            dt = time.perf_counter() - t0
            if dt >= budget_s / 4 or n >= T:
                break
            n = min(T, max(n * 2, int(n * budget_s / 4 / max(dt, 1e-3))))
        reps, total = 1, dt
        while total < budget_s and n >= T:
            t0 = time.perf_counter()
            oracle.ffn(inp, token_rows=np.arange(n))
            total += time.perf_counter() - t0
            reps += 1
    finally:
        _omp_threads(all_threads)
    tps = n * reps / total
    return {"value": tps, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "gflops_fp64": tps * flops_per_token / 1e9, "cpu_model": cpu_model(),
            "sample": "first %d of %d tokens x %d pass(es), full layer (all experts and shared), "
                      "fp64, %.1f s" % (n, T, reps, total)}


def measured_traffic(config, stage):
    """HBM bytes per launch of the dominant kernel, from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs summarised in profiles/hbm_traffic.md; None when no run covers this
    workload and kernel, or the kernel source changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    try:
        m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
        ent = json.loads(m.group(1)).get(config)
    except (OSError, AttributeError, ValueError):
        return None
    if not ent or ent.get("stage") != stage:
        return None
    src = open(os.path.join(ROOT, ent["source"]), "rb").read()
    if hashlib.sha256(src).hexdigest()[:16] != ent["source_sha256_16"]:
        return None
    return float(ent["bytes"])


class KernelEvent:
    """A HIP timing event without the end-of-record system-scope memory fence
    (hipEventDisableSystemFence). That fence makes every stop event wait for a
    system-wide cache write-back, which adds about 2 us to each timed interval,
    as much as an eighth of a decode GEMV. Without it the interval matches the
    kernel duration that rocprofv3 reports. The handle goes to the library, which
    records it on its own stream around each stage."""
    _hip = None
    FLAGS = 0x20000000   # hipEventDefault | hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        import torch  # noqa: F401  (loads the HIP runtime this process uses)
        if KernelEvent._hip is None:
            KernelEvent._hip = ctypes.CDLL("libamdhip64.so.7")
        h = ctypes.c_void_p()
        rc = KernelEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(self.FLAGS))
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        self.cuda_event = h.value

    def record(self, stream):
        import ctypes
        rc = KernelEvent._hip.hipEventRecord(ctypes.c_void_p(self.cuda_event), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        rc = KernelEvent._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                                  ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def __del__(self):
        import ctypes
        if KernelEvent._hip is not None and self.cuda_event:
            KernelEvent._hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))


def warm_up(run, n):
    """Untimed steps before the timed ones: exactly n if given, otherwise at least 20
    steps and at least 0.2 s of them (from idle, the GPU clocks take some milliseconds
    to ramp up, which a fixed handful of sub-millisecond steps does not cover).
    Returns the number of steps run."""
    import torch
    done, t0 = 0, time.perf_counter()
    while (done < n) if n is not None else (done < 20 or time.perf_counter() - t0 < 0.2):
        for _ in range(10 if n is None else n - done):
            run(done)
            done += 1
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    return done


def bench_row_ids(args):
    """The row-id pass alone at scale: T = 2^21 tokens, k = 8, E = 256, uniform ids
    (seed 6). Algorithmic bytes = ids read + the two maps written + the bounds."""
    import torch
    import indirect_expert_matmul_amd as moe
    import oracle
    import synth

    T, k, E = 1 << 21, 8, 256
    ids_np = synth.draw_ids_uniform(6, T, E, k)
    dev = torch.device("cuda:0")
    ids = torch.from_numpy(ids_np).to(dev)
    ws = torch.empty(moe.lib.moe_row_ids_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    args.warmup = warm_up(lambda i: moe.moe_row_ids(ids, E, workspace=ws, stream=stream), args.warmup)
    e0, e1 = KernelEvent(), KernelEvent()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        moe.moe_row_ids(ids, E, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    nbytes = 12.0 * T * k + 4.0 * (E + 1)
    gbs = nbytes / (ev_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu:
        # the oracle's enumeration on a bounded prefix of the same ids
        n = 1 << 15
        sub = np.ascontiguousarray(ids_np[:n])
        t1 = time.perf_counter()
        reps = 0
        while reps == 0 or time.perf_counter() - t1 < 2.0:
            oracle.row_ids(sub, E, 1)
            reps += 1
        sec = (time.perf_counter() - t1) / reps
        cpu = {"value": (12.0 * n * k + 4.0 * (E + 1)) / sec / 1e9, "unit": "GB/s",
               "cores": 1, "kind": "oracle",
               "sample": "first %d of %d tokens, %d pass(es), single thread" % (n, T, reps)}
    res = {
        "metric": "MoE row-id pass GB/s (T=2^21, k8, E256), 1 MI355X",
        "value": gbs, "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32", "data": "synthetic",
        "config": {"workload": "row ids: 2^21 tokens x 8 of 256 experts, uniform", "n_tokens": T,
                   "n_experts": E, "n_used": k, "parallelism": "single GPU"},
        "entries_per_s": T * k / (ev_ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("rowids", "row_ids"),
                     "kernel": "row_ids", "algorithmic_bytes": nbytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_gather(args):
    """The standalone row gather (moe_gather_rows) at the skewed PP4096 and the V3-shaped
    PP8192 shapes: the bf16 layer input copied into expert order by the row-id pass's first
    map. Algorithmic bytes = the T input rows read once + the T*k gathered rows written.
    The value is the V3-shaped rate; both shapes are on the line."""
    import torch
    import indirect_expert_matmul_amd as moe
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    shapes = {}
    names = [n for n in args.gather_shapes.split(",") if n]
    for name in names:
        cfg = synth.CONFIGS[name]
        T, k, E, K = cfg.n_tokens, cfg.n_used, cfg.n_experts, cfg.n_embd
        ids_np = (synth.draw_ids_zipf(cfg.seed, T, E, k, cfg.zipf_s) if cfg.routing == "zipf"
                  else synth.draw_ids_uniform(cfg.seed, T, E, k))
        x = torch.from_numpy(synth.gen.draw_x_bf16(cfg.seed, T, K).view(np.int16)).to(dev)
        s1, _, _ = moe.moe_row_ids(torch.from_numpy(ids_np).to(dev), E)
        outs = [torch.empty((T * k, K), dtype=x.dtype, device=dev) for _ in range(2)]
        shapes[name] = (cfg, T, k, K, x, s1, outs)
    torch.cuda.synchronize()
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    res_shapes = {}
    for name, (cfg, T, k, K, x, s1, outs) in shapes.items():
        run = lambda i: moe.moe_gather_rows(x, s1, out=outs[i % 2], stream=stream)
        warm = warm_up(run, args.warmup)
        e0, e1 = KernelEvent(), KernelEvent()
        e0.record(stream)
        for i in range(args.steps):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ev_ms = e0.elapsed_time(e1) / args.steps
        nbytes = (T + T * k) * K * 2.0
        gbs = nbytes / (ev_ms * 1e-3) / 1e9
        res_shapes[name] = {"workload": cfg.desc, "rows": T * k, "row_bytes": K * 2, "us": ev_ms * 1e3,
                            "gbps": gbs, "frac": gbs / HBM_PEAK_GBS, "warmup": warm,
                            "algorithmic_bytes": nbytes}
    v = res_shapes[names[-1]]
    res = {
        "metric": "MoE row gather GB/s (src1 rows into expert order), 1 MI355X",
        "value": v["gbps"], "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": v["warmup"], "ms_per_step": v["us"] * 1e-3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gather of the %s input (rows in expert order)" % shapes[names[-1]][0].desc,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": v["gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": v["frac"], "traffic": measured_traffic("gather_" + names[-1], "gather"),
                     "kernel": "gather",
                     "algorithmic_bytes": v["algorithmic_bytes"]},
        "shapes": res_shapes,
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def prepare_ffn_workload(args, name):
    """Inputs of one FFN workload drawn and made resident in HBM: the weights in R
    copies (rotated through by the steps, so the set a step reads is not served from
    the 256 MB last-level cache), x, ids, route_w, output and workspace."""
    import torch
    import indirect_expert_matmul_amd as moe
    import synth

    cfg = synth.CONFIGS[name]
    if cfg.kind != "ffn":
        raise SystemExit("bench.py: %s is not an FFN workload" % name)
    inp = synth.make_inputs(cfg)
    T, k = inp["ids"].shape
    dev = torch.device("cuda:0")

    def up(qs, d):
        return moe.weights_from_numpy(qs, d)

    wtype = {"q8_0": moe.MOE_Q8_0, "mxfp4": moe.MOE_MXFP4, "iq4_nl": moe.MOE_IQ4_NL,
             "iq4_xs": moe.MOE_IQ4_XS}[cfg.wtype]
    aq = args.act_quant
    path = moe.moe_select_path_typed(T, k, cfg.n_experts, max(cfg.n_embd, cfg.n_ff), wtype,
                                     path=args.path, act_quant=aq)
    st = workload_stats(inp, cfg, 4 if path == 2 else 2)
    R = args.rotate or (1 if st["bytes"] > 2e9 else max(4, int(np.ceil(1.2e9 / st["bytes"]))))
    sets = []
    base = [up(inp[n + "_qs"], inp[n + "_d"]) for n in ("gate", "up", "down")]
    sh = ([up(inp["sh_" + n + "_qs"], inp["sh_" + n + "_d"]) for n in ("gate", "up", "down")]
          if cfg.n_shared else None)
    for r in range(R):
        if r == 0:
            sets.append((base, sh))
        else:
            cl = lambda w: moe.Weights(w.data.clone(), w.scales.clone())
            sets.append(([cl(w) for w in base], [cl(w) for w in sh] if sh else None))
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev)
    ids = torch.from_numpy(inp["ids"]).to(dev)
    rw = torch.from_numpy(inp["route_w"]).to(dev)
    out = torch.empty((T, cfg.n_embd), dtype=torch.float32, device=dev)
    need = moe.moe_ffn_fused_workspace_size(base[0], sh[0] if sh else None, T, k, path=args.path,
                                            act_quant=aq)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(i, events=None):
        (g, u, d), s = sets[i % R]
        moe.moe_ffn_fused(g, u, d, x, ids, rw, shared=s, path=args.path, out=out, workspace=ws,
                          stream=stream, events=events, act_quant=aq)

    return {"name": name, "cfg": cfg, "inp": inp, "st": st, "path": path, "R": R, "sets": sets,
            "x": x, "ids": ids, "rw": rw, "out": out, "ws": ws, "stream": stream, "step": step}


def make_stage_events(W, steps):
    """The HIP events of a workload's per-stage pass (made before any timing starts)."""
    W["evs"] = [[KernelEvent() for _ in range(2 * len(STAGES[W["path"]]))] for _ in range(steps)]


def time_ffn_workload(args, W, steps, warmup):
    """Time a prepared FFN workload: warm-up, then `steps` timed steps (each one full
    layer call), then one pass with per-kernel HIP events recorded by the library on
    the stream its kernels run on. Only GPU work and its launches happen here (the
    events come from make_stage_events); finish_ffn_workload turns the result into
    measurements once all GPU timing is done, so the GPU does not idle between
    workloads."""
    import torch
    import indirect_expert_matmul_amd as moe

    name, cfg, inp, st, path, R, sets = (W[n] for n in ("name", "cfg", "inp", "st", "path", "R", "sets"))
    x, ids, rw, out, ws, stream, step = (W[n] for n in ("x", "ids", "rw", "out", "ws", "stream", "step"))
    aq = args.act_quant
    names = STAGES[path]
    evs = W["evs"]
    assert len(evs) == steps
    warmup = warm_up(step, warmup)
    run = step
    if args.graph:
        # one captured step per weight copy, replayed in the same rotation
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    (gw, uw, dw), sw_ = sets[r]
                    moe.moe_ffn_fused(gw, uw, dw, x, ids, rw, shared=sw_, path=args.path, out=out,
                                      workspace=ws, stream=cap, act_quant=aq)
            graphs.append(g)
        torch.cuda.synchronize()
        run = lambda i: graphs[i % R].replay()
        warm_up(run, warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / steps

    # per-kernel durations: HIP events recorded by the library around each stage, on
    # the stream the kernels run on
    for i in range(steps):
        step(i, events=[e.cuda_event for e in evs[i]])
    torch.cuda.synchronize()
    if moe.last_stage_count() < len(names):
        # small decode batches: the down GEMV does the weighted reduce itself
        names = names[:1] + ["gemv_down_reduce"]
    return {"W": W, "steps": steps, "warmup": warmup, "ms": ms, "evs": evs, "names": names}


def finish_ffn_workload(raw):
    """Measurements of a timed FFN workload (see time_ffn_workload) as a dict."""
    W, steps, warmup, ms, evs, names = (raw[n] for n in ("W", "steps", "warmup", "ms", "evs", "names"))
    name, cfg, inp, st, path, R, stream = (W[n] for n in ("name", "cfg", "inp", "st", "path", "R", "stream"))
    T = inp["ids"].shape[0]
    stage_ms = {n: float(np.mean([evs[i][2 * j].elapsed_time(evs[i][2 * j + 1])
                                  for i in range(steps)])) for j, n in enumerate(names)}
    dom = max(stage_ms, key=stage_ms.get)
    kern = {"gemm_gate_up": "gate_up", "gemv_gate_up": "gate_up", "gemm_down": "down",
            "gemv_down": "down", "gemv_down_reduce": "down_reduce", "reduce": "reduce"}.get(dom)
    mfma_bound = path in (1, 3) and st["flops"] / (BF16_PEAK_TFLOPS * 1e12) > st["bytes"] / (HBM_PEAK_GBS * 1e9)
    traffic = measured_traffic(name, dom)
    if kern is None:
        roof = {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": None, "traffic": None, "kernel": dom}
    elif mfma_bound:
        a = st[kern]["flops"] / (stage_ms[dom] * 1e-3) / 1e12
        pk, unit = (INT8_PEAK_TOPS, "TOP/s") if path == 3 else (BF16_PEAK_TFLOPS, "TFLOP/s")
        roof = {"bound": "mfma", "achieved": a, "peak": pk, "unit": unit,
                "frac": a / pk, "traffic": traffic, "kernel": dom,
                "algorithmic_bytes": st[kern]["bytes"], "intermediate_bytes": st[kern]["intermediate_bytes"]}
    else:
        a = st[kern]["bytes"] / (stage_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBS, "traffic": traffic, "kernel": dom,
                "algorithmic_bytes": st[kern]["bytes"], "intermediate_bytes": st[kern]["intermediate_bytes"]}

    res = {
        "workload": cfg.desc, "name": name, "n_tokens": T,
        "path": {1: "gemm", 2: "gemv", 3: "gemm, int8 activations"}[path],
        "weight_copies": R, "steps": steps, "warmup": warmup, "ms_per_step": ms,
        "tokens_per_s": T / (ms * 1e-3),
        "tflops": st["flops"] / (ms * 1e-3) / 1e12,
        "gbps": st["bytes"] / (ms * 1e-3) / 1e9,
        "stage_ms": stage_ms, "roofline": roof,
        "dtype": {1: "bf16", 2: "f32", 3: "int8"}[path],
        "cfg": cfg, "inp": inp, "stats": st, "stream": stream,
    }
    res["cpu_baseline"] = None
    return res


def attach_cpu_baseline(res, cpu_seconds, single_thread_cpu=False):
    """The oracle timed on the host for a measured workload (run after all GPU timing,
    so the GPU does not idle between its timed workloads while the host computes)."""
    if cpu_seconds <= 0:
        return
    inp, st = res["inp"], res["stats"]
    fpt = st["flops"] / res["n_tokens"]
    res["cpu_baseline"] = cpu_baseline(inp, cpu_seconds, fpt)
    if single_thread_cpu:
        res["cpu_baseline"]["single_thread"] = {
            k2: v for k2, v in cpu_baseline(inp, min(cpu_seconds, 3.0), fpt, threads=1).items()
            if k2 in ("value", "gflops_fp64", "sample")}


def time_router(cfg, stream, seconds=0.25, calls=64):
    """The router top-k that produces ids / route_w ahead of the layer (not part of the
    step), timed on logits of the workload's shape and reported beside the layer.
    One call is a few microseconds of GPU time, less than a Python call costs, so the
    calls are captured into a graph of `calls` back-to-back launches that is replayed
    for about `seconds`: the figure is GPU time per call, launch gaps inside the graph
    included. It runs first: from idle the GPU clocks take some milliseconds to ramp
    up, and the busy GPU keeps them up for the layer's warm-up."""
    import torch
    import indirect_expert_matmul_amd as moe
    import synth
    T, k = cfg.n_tokens, cfg.n_used
    dev = torch.device("cuda:0")
    lg = torch.from_numpy(synth.draw_router_logits(cfg.seed, T, cfg.n_experts)).to(dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    rw = torch.empty((T, k), dtype=torch.float32, device=dev)
    for _ in range(3):
        moe.moe_router_topk(lg, k, ids=ids, route_w=rw, stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(calls):
                moe.moe_router_topk(lg, k, ids=ids, route_w=rw, stream=cap)
    torch.cuda.synchronize()
    n_router, t0 = 0, time.perf_counter()
    r0, r1 = KernelEvent(), KernelEvent()
    r0.record(stream)
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            graph.replay()
        n_router += 8 * calls
        torch.cuda.synchronize()
    r1.record(stream)
    torch.cuda.synchronize()
    router_us = r0.elapsed_time(r1) * 1e3 / n_router
    del graph
    return {"us": router_us, "gbps": (T * cfg.n_experts * 4 + T * k * 8) / (router_us * 1e-6) / 1e9,
            "n_experts": cfg.n_experts, "n_used": k, "calls": n_router,
            "launch": "graph of %d back-to-back calls" % calls}


def _public(r):
    """The JSON-ready part of a workload result."""
    return {k: v for k, v in r.items() if k not in ("cfg", "inp", "stats", "stream")}


# Decode-to-small-prefill batches on which the automatic path choice was measured: each
# shape's GEMV (forced, where its bounds allow) against its grouped GEMM, per layer call.
CROSSOVER = ([("v3", 256, 8, T, 7168, 2048, 1, "q8_0") for T in (1, 2, 8, 16, 32)] +
             [("lite", 64, 6, T, 2048, 1408, 2, "q8_0") for T in (1, 4, 8, 10, 42)] +
             [("gptoss", 32, 4, T, 2880, 2880, 0, "q8_0") for T in (8, 16)] +
             [("gptoss", 32, 4, T, 2880, 2880, 0, "mxfp4") for T in (8, 12, 16)] +
             [("e128", 128, 8, T, 2048, 768, 0, "iq4_xs") for T in (4, 8)])


def bench_crossover(args):
    """GEMV against grouped GEMM per layer call on the CROSSOVER shapes (weights resident,
    only the experts each batch routes to drawn). One JSON line."""
    import torch
    import indirect_expert_matmul_amd as moe
    import synth
    wt = {"q8_0": moe.MOE_Q8_0, "mxfp4": moe.MOE_MXFP4, "iq4_xs": moe.MOE_IQ4_XS}
    dev = lambda a, dt, view=None: torch.from_numpy(np.ascontiguousarray(a, dtype=dt) if view is None
                                                    else np.ascontiguousarray(a, dtype=dt).view(view)).cuda()
    res = []
    for name, E, k, T, ne, nf, S, w in CROSSOVER:
        inp = synth.make_custom_ffn(600 + T, E, k, T, ne, nf, S, wtype=w, touched_only=True)
        W = [moe.weights_from_numpy(inp[n + "_qs"], inp[n + "_d"]) for n in ("gate", "up", "down")]
        sh = ([moe.weights_from_numpy(inp["sh_" + n + "_qs"], inp["sh_" + n + "_d"]) for n in ("gate", "up", "down")]
              if S else None)
        x, ids, rw = dev(inp["x"], np.uint16, np.int16), dev(inp["ids"], np.int32), dev(inp["route_w"], np.float32)
        call = lambda p: moe.moe_ffn_fused(W[0], W[1], W[2], x, ids, rw, shared=sh, path=p)
        row = {"shape": name, "wtype": w, "T": T, "slots": T * k,
               "auto": moe.moe_select_path_typed(T, k, E, max(ne, nf), wt[w])}
        for p, key in ((moe.PATH_GEMV, "gemv_us"), (moe.PATH_GEMM, "gemm_us")):
            try:
                moe.moe_select_path_typed(T, k, E, max(ne, nf), wt[w], path=p)
            except moe.MoeError:
                row[key] = None
                continue
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.3:
                for _ in range(10):
                    call(p)
                torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(50):
                call(p)
            b.record()
            torch.cuda.synchronize()
            row[key] = round(a.elapsed_time(b) * 1000 / 50, 1)
        print("crossover: %s" % json.dumps(row), file=sys.stderr, flush=True)
        res.append(row)
        del W, sh, x, ids, rw
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "MoE FFN layer call, GEMV against grouped GEMM", "unit": "us", "n_gpus": 1,
                      "data": "synthetic", "higher_is_better": False, "results": res}))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this implementation runs on one GPU; --gpus %d is not supported "
              "(the path would shard by expert with two all-to-all exchanges)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.config == "rowids":
        bench_row_ids(args)
        return
    if args.config == "gather":
        bench_gather(args)
        return
    if args.config == "crossover":
        bench_crossover(args)
        return
    import torch
    import indirect_expert_matmul_amd as moe
    import synth

    cfg = synth.CONFIGS[args.config]
    T, k = cfg.n_tokens, cfg.n_used
    stream = torch.cuda.current_stream()
    # Every workload's inputs are made resident first, then the GPU timing runs back
    # to back: the routers, the further workloads of the metric (PP4096 prefill, decode
    # batches of 1 and 8; each with its own dominant-kernel roofline), and the headline
    # workload last. From idle or light load the GPU clocks take about 10 ms to ramp up,
    # longer than a few warm-up steps of a 0.2 ms layer. The further workloads each warm
    # up for at least 20 steps and 0.2 s whatever --warmup says, so their figures are
    # steady-state ones; the headline runs exactly --warmup untimed steps, and timed
    # last, its warm-up starts from a GPU under load.
    names = [n for n in (args.extra.split(",") if args.extra else []) if n and n != args.config]
    prep = {n: prepare_ffn_workload(args, n) for n in names + [args.config]}
    routers = {n: time_router(prep[n]["cfg"], stream) for n in [args.config] + names}
    steps = {n: max(10, args.steps // 2) if n in ("skew", "v3") else args.steps for n in names}
    steps[args.config] = args.steps
    for n in steps:
        make_stage_events(prep[n], steps[n])
    raw = {n: time_ffn_workload(args, prep[n], steps[n], None) for n in names}
    r = finish_ffn_workload(time_ffn_workload(args, prep[args.config], steps[args.config], args.warmup))
    extras = {}
    for n in names:
        extras[n] = finish_ffn_workload(raw[n])
        extras[n]["router"] = routers[n]
    del raw
    router = routers[args.config]
    del prep
    torch.cuda.empty_cache()

    # the CPU oracle, once the GPU timing is done
    if not args.no_cpu:
        attach_cpu_baseline(r, args.cpu_seconds, single_thread_cpu=cfg.n_tokens <= 16)
        for n in names:
            attach_cpu_baseline(extras[n], args.extra_cpu_seconds,
                                single_thread_cpu=synth.CONFIGS[n].n_tokens <= 16)
    extras = {n: _public(e) for n, e in extras.items()}

    ms = r["ms_per_step"]
    res = {
        "metric": "MoE mul_mat_id tokens/s + TFLOP/s (PP512/PP4096) and decode GB/s, 1 MI355X",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": r["warmup"], "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic",
        "config": {"workload": cfg.desc, "n_tokens": T, "n_experts": cfg.n_experts,
                   "n_used": k, "n_shared": cfg.n_shared, "n_embd": cfg.n_embd, "n_ff": cfg.n_ff,
                   "path": r["path"], "weight_copies": r["weight_copies"],
                   "launch": "hip graph replay" if args.graph else "eager",
                   "parallelism": "single GPU"},
        "tflops": r["tflops"],
        "gbps": r["gbps"],
        "stage_ms": r["stage_ms"],
        "router": router,
        "roofline": r["roofline"],
        "cpu_baseline": r["cpu_baseline"],
        "workloads": extras,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
