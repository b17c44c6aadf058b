"""Helpers shared by the GPU tests: upload a synth workload to the device and
compare against the oracle with the normwise metric."""
import numpy as np
import torch

import indirect_expert_matmul_amd as moe

# Tolerances (normwise: max|got - ref| / max|ref| per output tensor).
TOL_MFMA = 2e-2   # bf16 MFMA path: bf16(d*q) weights and bf16 activations, fp32 accumulate
TOL_FP32 = 1e-5   # fp32 arithmetic: the fp32 mul_mat_id path and the GEMV (decode) path


def normwise(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()


def upload_ffn(inp: dict) -> dict:
    d = {
        "gate": moe.weights_from_numpy(inp["gate_qs"], inp["gate_d"]),
        "up": moe.weights_from_numpy(inp["up_qs"], inp["up_d"]),
        "down": moe.weights_from_numpy(inp["down_qs"], inp["down_d"]),
        "x": dev_bf16(inp["x"]),
        "ids": dev_i32(inp["ids"]),
        "route_w": dev_f32(inp["route_w"]),
        "shared": None,
    }
    if inp.get("sh_gate_qs") is not None:
        d["shared"] = [moe.weights_from_numpy(inp["sh_" + n + "_qs"], inp["sh_" + n + "_d"])
                       for n in ("gate", "up", "down")]
    return d


def run_ffn(dv: dict, **kw) -> torch.Tensor:
    return moe.moe_ffn_fused(dv["gate"], dv["up"], dv["down"], dv["x"], dv["ids"], dv["route_w"],
                             shared=dv["shared"], **kw)


def upload_mmid(inp: dict) -> dict:
    if inp["wtype"] == "f32":
        w = moe.weights_from_numpy(inp["w"])
        x = dev_f32(inp["x"])
    else:
        w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
        x = dev_bf16(inp["x"])
    return {"w": w, "x": x, "ids": dev_i32(inp["ids"]), "route_w": dev_f32(inp["route_w"])}
