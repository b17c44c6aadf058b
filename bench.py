#!/usr/bin/env python3
"""Benchmark of the MoE indirect matmul hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config lite|dec1|dec8|skew|v3|rowids]

A step is one full pass of the hot path -- row ids, gate/up grouped GEMM, down
grouped GEMM, fixed-order reduce (or the GEMV decode kernels) -- over one batch of
synthetic input already resident in HBM. The default workload is the
DeepSeek-Lite-shaped PP512 layer (E64 k6 + 2 shared, n_embd 2048, n_ff 1408,
Q8_0, 512 tokens). Weights are rotated through R copies so the set read per step
is not served from the 256 MB last-level cache.

Prints ONE JSON line: tokens/s (value), TFLOP/s, GB/s, a roofline entry for the
dominant kernel (timed with HIP events on the launch stream) and the CPU oracle
timed on a bounded sample of the same workload on this host.
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
Q8_BYTES = 34.0 / 32.0      # Q8_0: 32 int8 + one fp16 scale per 32 weights
MXFP4_BYTES = 17.0 / 32.0   # MXFP4: 32 four-bit codes + one E8M0 scale byte per 32 weights

STAGES = {1: ["row_ids", "gemm_gate_up", "gemm_down", "reduce"],
          2: ["gemv_gate_up", "gemv_down", "reduce"]}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed warm-up steps (default: at least 20 steps and 0.2 s of them, "
                        "so the GPU clocks have ramped up; the count is reported)")
    p.add_argument("--config", default="lite")
    p.add_argument("--rotate", type=int, default=0, help="weight copies (0 = auto)")
    p.add_argument("--path", type=int, default=0, help="0 auto, 1 GEMM, 2 GEMV")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--graph", type=int, default=0,
                   help="1: time replays of one HIP graph per weight copy (each graph holds one "
                        "step); 0: eager calls")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="first run one device-to-device copy of this many MiB (a known-size "
                        "kernel for scaling HBM byte counters)")
    return p.parse_args()


def workload_stats(inp, cfg, h_bytes=2):
    """Algorithmic work of one step (flops, bytes) and per-kernel bytes: the weights of
    the experts the batch touches (each once), activations read once, results written
    once."""
    T, k = inp["ids"].shape
    E, n_embd, n_ff, S = cfg.n_experts, cfg.n_embd, cfg.n_ff, cfg.n_shared
    ids = inp["ids"].ravel()
    touched = len(np.unique(ids[(ids >= 0) & (ids < E)]))
    rows_routed = int(((ids >= 0) & (ids < E)).sum())
    rows = rows_routed + T * S                      # routed slots + shared-expert rows
    flops = 2.0 * rows * 3 * n_embd * n_ff
    wb = MXFP4_BYTES if cfg.wtype == "mxfp4" else Q8_BYTES
    w_gu = (touched + S) * 2 * n_ff * n_embd * wb
    w_dn = (touched + S) * n_embd * n_ff * wb
    x_b = T * n_embd * 2                            # bf16 input
    out_b = T * n_embd * 4                          # fp32 layer output
    return {
        "flops": flops, "bytes": w_gu + w_dn + x_b + out_b, "touched": touched,
        # gate/up: weights + x in, h = silu(g)*u out (bf16 on the GEMM path, fp32 on
        # the GEMV path)
        "gate_up": {"bytes": w_gu + x_b + rows * n_ff * h_bytes,
                    "flops": 2.0 * rows * 2 * n_embd * n_ff},
        # down: weights + h in, per-row fp32 results out
        "down": {"bytes": w_dn + rows * n_ff * h_bytes + rows * n_embd * 4,
                 "flops": 2.0 * rows * n_embd * n_ff},
    }


def cpu_baseline(inp, budget_s):
    """The oracle, as it stands, on a bounded token sample: tokens/s on this host.
    The sample grows until one pass takes about a quarter of the budget; when the
    whole batch is faster than that, whole-batch passes repeat until the budget."""
    import oracle
    oracle.lib()
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
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    return {"value": n * reps / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
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
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "row_ids"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


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
    import torch
    import indirect_expert_matmul_amd as moe
    import synth

    cfg = synth.CONFIGS[args.config]
    if cfg.kind != "ffn":
        print("bench.py: --config must be an FFN workload", file=sys.stderr)
        sys.exit(2)
    inp = synth.make_inputs(cfg)
    T, k = inp["ids"].shape
    dev = torch.device("cuda:0")

    def up(qs, d):
        return moe.weights_from_numpy(qs, d)

    path = moe.moe_select_path(T, k, cfg.n_experts, max(cfg.n_embd, cfg.n_ff), path=args.path)
    st = workload_stats(inp, cfg, 2 if path == 1 else 4)
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
    need = moe.moe_ffn_fused_workspace_size(base[0], sh[0] if sh else None, T, k, path=args.path)
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
                          stream=stream, events=events)

    args.warmup = warm_up(step, args.warmup)
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
                                      workspace=ws, stream=cap)
            graphs.append(g)
        torch.cuda.synchronize()
        run = lambda i: graphs[i % R].replay()
        warm_up(run, args.warmup)
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps

    # per-kernel durations: HIP events recorded by the library around each stage
    names = STAGES[path]
    evs = [[KernelEvent() for _ in range(2 * len(names))] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, events=[e.cuda_event for e in evs[i]])
    torch.cuda.synchronize()
    if moe.last_stage_count() < len(names):
        # small decode batches: the down GEMV does the weighted reduce itself
        names = names[:1] + ["gemv_down_reduce"]
    stage_ms = {n: float(np.mean([evs[i][2 * j].elapsed_time(evs[i][2 * j + 1])
                                  for i in range(args.steps)])) for j, n in enumerate(names)}
    dom = max(stage_ms, key=stage_ms.get)
    kern = {"gemm_gate_up": "gate_up", "gemv_gate_up": "gate_up", "gemm_down": "down",
            "gemv_down": "down", "gemv_down_reduce": "down"}.get(dom)
    mfma_bound = path == 1 and st["flops"] / (BF16_PEAK_TFLOPS * 1e12) > st["bytes"] / (HBM_PEAK_GBS * 1e9)
    traffic = measured_traffic(args.config, dom)
    if kern is None:
        roof = {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": None, "traffic": None, "kernel": dom}
    elif mfma_bound:
        a = st[kern]["flops"] / (stage_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": a, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": a / BF16_PEAK_TFLOPS, "traffic": traffic, "kernel": dom}
    else:
        a = st[kern]["bytes"] / (stage_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBS, "traffic": traffic, "kernel": dom}

    # the router top-k that produces ids / route_w ahead of the layer (not part of the
    # step): timed on logits of the same shape, reported separately
    lg = torch.from_numpy(synth.draw_router_logits(cfg.seed, T, cfg.n_experts)).to(dev)
    for _ in range(3):
        moe.moe_router_topk(lg, k, stream=stream)
    r0, r1 = KernelEvent(), KernelEvent()
    r0.record(stream)
    n_router = 20
    for _ in range(n_router):
        moe.moe_router_topk(lg, k, stream=stream)
    r1.record(stream)
    torch.cuda.synchronize()
    router_us = r0.elapsed_time(r1) * 1e3 / n_router
    router = {"us": router_us, "gbps": (T * cfg.n_experts * 4 + T * k * 8) / (router_us * 1e-6) / 1e9,
              "n_experts": cfg.n_experts, "n_used": k}

    res = {
        "metric": "MoE mul_mat_id tokens/s + TFLOP/s (PP512/PP4096) and decode GB/s, 1 MI355X",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if path == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.desc, "n_tokens": T, "n_experts": cfg.n_experts,
                   "n_used": k, "n_shared": cfg.n_shared, "n_embd": cfg.n_embd, "n_ff": cfg.n_ff,
                   "path": "gemm" if path == 1 else "gemv", "weight_copies": R,
                   "launch": "hip graph replay" if args.graph else "eager",
                   "parallelism": "single GPU"},
        "tflops": st["flops"] / (ms * 1e-3) / 1e12,
        "gbps": st["bytes"] / (ms * 1e-3) / 1e9,
        "stage_ms": stage_ms,
        "router": router,
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu else cpu_baseline(inp, args.cpu_seconds),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
