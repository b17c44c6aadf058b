"""Seeded synthetic inputs for the MoE indirect matmul (mul_mat_id) workloads.

This module only draws inputs. It holds none of the arithmetic of the operation
itself (no products, no grouping of rows by expert); both the CPU oracle and the
GPU library consume what it returns, and the arrays it returns are the single
truth for both.

Workloads follow the shapes the pages discuss for mul_mat_id:
  * the op's operands: stacked expert weights [n_experts][rows][cols], activations,
    and an integer ids table naming each token's top-k experts
    ("CUDA: better MoE implementation", section 1.2);
  * Q8_0-style quantized experts (section 2.1 of the same page names Q8_0 as a
    type served by the quantized mul_mat_id path);
  * always-on shared experts fused beside the routed ones
    ("CUDA: fuse shared experts into MMVQ", release note b11370).

Storage conventions (row-major, last index contiguous):
  * Q8_0-style weights: ``qs`` int8 [E][rows][cols] with q uniform in [-127, 127],
    ``d`` float16 [E][rows][cols // 32] uniform in (0.5, 1.5) * 1e-3, value = d * q.
  * MXFP4 weights (the format GPT-OSS ships its experts in): ``qs`` uint8
    [E][rows][cols // 2], two 4-bit E2M1 codes per byte (column 2i in the low nibble,
    2i+1 in the high one), codes uniform over all 16; ``d`` uint8 [E][rows][cols // 32]
    E8M0 scales uniform in {118, ..., 121} (2^-9 .. 2^-6), value = fp4(code) * 2^(d-127).
  * IQ4_NL weights (the 4-bit codes of the IQ series): ``qs`` uint8 [E][rows][cols // 2]
    packed as MXFP4's, codes uniform over all 16; ``d`` float16 [E][rows][cols // 32]
    drawn as Q8_0's, value = d * level(code) with ggml's 16-level IQ4_NL table.
  * IQ4_XS weights: codes as IQ4_NL's; ``d`` uint8 [E][rows][cols // 256][8], one record per
    super-block of 256 columns: fp16 d (bytes 0-1) ~ U(0.5, 1.5) * 1e-4, then six uniform
    random bytes (scales_h, scales_l[4]: every bit pattern is a valid set of 6-bit
    sub-scales).
  * bf16 tensors are stored as their uint16 bit patterns (numpy has no bfloat16),
    rounded to nearest-even from float32.
  * ids int32 [T][k]; route_w float32 [T][k], softmax over each token's k picks
    (computed in float64, stored as float32).

Draw streams: every array has its own numpy SeedSequence child keyed by
(seed, stream id, ...), so large per-expert tensors can be drawn in parallel
threads and the result does not depend on scheduling.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

# Stream ids for SeedSequence spawn keys.
_S_IDS, _S_LOGITS, _S_ROUTED, _S_SHARED, _S_X, _S_ZIPF, _S_ROUTER = 0, 1, 2, 3, 4, 5, 6
_M_GATE, _M_UP, _M_DOWN = 0, 1, 2


@dataclass(frozen=True)
class Config:
    """One workload. ``kind`` is 'mmid' (single stacked weight, mul_mat_id only)
    or 'ffn' (gate + up + down experts, SiLU(gate) * up, optional shared experts)."""
    name: str
    kind: str
    n_experts: int
    n_used: int
    n_tokens: int
    n_embd: int
    n_ff: int
    n_shared: int = 0
    wtype: str = "q8_0"          # 'q8_0', 'mxfp4', 'iq4_nl', 'iq4_xs' or 'f32'
    routing: str = "uniform"     # 'uniform' or 'zipf'
    zipf_s: float = 1.1
    seed: int = 0
    desc: str = ""
    extra: dict = field(default_factory=dict)


CONFIGS = {
    # fp32 single up-projection: 8 experts, top-2, 16 tokens, 64 -> 32.
    "tiny": Config("tiny", "mmid", 8, 2, 16, 64, 32, wtype="f32", seed=1,
                   desc="E8 k2 T16 K64 N32 fp32 mul_mat_id"),
    # DeepSeek-Lite-shaped MoE FFN layer, PP512.
    "lite": Config("lite", "ffn", 64, 6, 512, 2048, 1408, n_shared=2, seed=2,
                   desc="DeepSeek-Lite-shaped: E64 k6 S2 T512 n_embd2048 n_ff1408 Q8_0"),
    # GPT-OSS-20B-shaped decode, batch 1 and batch 8.
    "dec1": Config("dec1", "ffn", 32, 4, 1, 2880, 2880, seed=3,
                   desc="GPT-OSS-20B-shaped decode: E32 k4 T1 n_embd=n_ff=2880 Q8_0"),
    "dec8": Config("dec8", "ffn", 32, 4, 8, 2880, 2880, seed=3,
                   desc="GPT-OSS-20B-shaped decode: E32 k4 T8 n_embd=n_ff=2880 Q8_0"),
    # The same decode shapes with MXFP4 experts (the format GPT-OSS ships them in).
    "dec1x": Config("dec1x", "ffn", 32, 4, 1, 2880, 2880, wtype="mxfp4", seed=3,
                    desc="GPT-OSS-20B-shaped decode: E32 k4 T1 n_embd=n_ff=2880 MXFP4"),
    "dec8x": Config("dec8x", "ffn", 32, 4, 8, 2880, 2880, wtype="mxfp4", seed=3,
                    desc="GPT-OSS-20B-shaped decode: E32 k4 T8 n_embd=n_ff=2880 MXFP4"),
    # GPT-OSS-20B-shaped prefill, PP4096, MXFP4 experts.
    "ppx": Config("ppx", "ffn", 32, 4, 4096, 2880, 2880, wtype="mxfp4", seed=7,
                  desc="GPT-OSS-20B-shaped prefill: E32 k4 T4096 n_embd=n_ff=2880 MXFP4"),
    # The GPT-OSS-20B shapes with IQ4_NL experts (the 4-bit codes of the IQ series).
    "dec1n": Config("dec1n", "ffn", 32, 4, 1, 2880, 2880, wtype="iq4_nl", seed=3,
                    desc="GPT-OSS-20B-shaped decode: E32 k4 T1 n_embd=n_ff=2880 IQ4_NL"),
    "dec8n": Config("dec8n", "ffn", 32, 4, 8, 2880, 2880, wtype="iq4_nl", seed=3,
                    desc="GPT-OSS-20B-shaped decode: E32 k4 T8 n_embd=n_ff=2880 IQ4_NL"),
    "ppn": Config("ppn", "ffn", 32, 4, 4096, 2880, 2880, wtype="iq4_nl", seed=7,
                  desc="GPT-OSS-20B-shaped prefill: E32 k4 T4096 n_embd=n_ff=2880 IQ4_NL"),
    # IQ4_XS experts (super-blocks of 256 columns) on a layer whose widths are multiples of
    # 256: E128 k8, n_embd 2048, n_ff 768 (the skewed layer's shape, uniform routing).
    "dec1s": Config("dec1s", "ffn", 128, 8, 1, 2048, 768, wtype="iq4_xs", seed=8,
                    desc="E128 k8 T1 n_embd2048 n_ff768 decode, IQ4_XS"),
    "dec8s": Config("dec8s", "ffn", 128, 8, 8, 2048, 768, wtype="iq4_xs", seed=8,
                    desc="E128 k8 T8 n_embd2048 n_ff768 decode, IQ4_XS"),
    "pps": Config("pps", "ffn", 128, 8, 4096, 2048, 768, wtype="iq4_xs", seed=9,
                  desc="E128 k8 T4096 n_embd2048 n_ff768 prefill, IQ4_XS"),
    # Zipf(1.1)-skewed prefill, PP4096.
    "skew": Config("skew", "ffn", 128, 8, 4096, 2048, 768, routing="zipf", seed=4,
                   desc="Skewed prefill: E128 k8 T4096 n_embd2048 n_ff768 Zipf(1.1) Q8_0"),
    # DeepSeek-V3-shaped single layer, PP8192.
    "v3": Config("v3", "ffn", 256, 8, 8192, 7168, 2048, n_shared=1, seed=5,
                 desc="DeepSeek-V3-shaped: E256 k8 S1 T8192 n_embd7168 n_ff2048 Q8_0"),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even), returned as uint16 bit patterns.
    Inputs here are finite; NaN handling is not needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_ids_uniform(seed: int, n_tokens: int, n_experts: int, n_used: int) -> np.ndarray:
    """k distinct experts per token, uniformly at random, in random order
    (Gumbel-top-k with equal popularities)."""
    if n_used > n_experts:
        raise ValueError("uniform draw without replacement needs n_used <= n_experts")
    g = _rng(seed, _S_IDS).gumbel(size=(n_tokens, n_experts))
    order = np.argsort(-g, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :n_used].astype(np.int32))


def zipf_popularity(seed: int, n_experts: int, s: float) -> np.ndarray:
    """p_e proportional to rank_e^-s, with rank_e = perm[e] + 1 from a seeded
    permutation of the experts."""
    perm = _rng(seed, _S_ZIPF).permutation(n_experts)
    p = (perm + 1.0) ** (-s)
    return p / p.sum()


def draw_ids_zipf(seed: int, n_tokens: int, n_experts: int, n_used: int, s: float) -> np.ndarray:
    """k distinct experts per token drawn without replacement from a Zipf(s)
    popularity (Gumbel-top-k, equivalent to successive renormalised draws)."""
    if n_used > n_experts:
        raise ValueError("draw without replacement needs n_used <= n_experts")
    logp = np.log(zipf_popularity(seed, n_experts, s))
    g = _rng(seed, _S_IDS).gumbel(size=(n_tokens, n_experts)) + logp[None, :]
    order = np.argsort(-g, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :n_used].astype(np.int32))


def draw_route_w(seed: int, n_tokens: int, n_used: int) -> np.ndarray:
    """Routing weights: softmax over each token's k picks of N(0,1) logits,
    in float64, stored as float32."""
    z = _rng(seed, _S_LOGITS).standard_normal((n_tokens, n_used))
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return np.ascontiguousarray((e / e.sum(axis=1, keepdims=True)).astype(np.float32))


def draw_router_logits(seed: int, n_tokens: int, n_experts: int, zipf_s: float = 0.0) -> np.ndarray:
    """Router logits float32 [T][E]: N(0,1), plus log of a Zipf(s) expert popularity
    over a seeded permutation when zipf_s > 0 (so top-k picks follow that popularity)."""
    z = _rng(seed, _S_ROUTER).standard_normal((n_tokens, n_experts))
    if zipf_s > 0:
        z = z + np.log(zipf_popularity(seed, n_experts, zipf_s))[None, :]
    return np.ascontiguousarray(z.astype(np.float32))


def draw_q8_0(rng: np.random.Generator, rows: int, cols: int):
    """One Q8_0-style matrix: qs int8 [rows][cols] ~ U{-127..127},
    d float16 [rows][cols/32] ~ U(0.5, 1.5) * 1e-3 (rounded to fp16)."""
    if cols % 32:
        raise ValueError("Q8_0 needs cols % 32 == 0")
    qs = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    d = (rng.uniform(0.5, 1.5, size=(rows, cols // 32)) * 1e-3).astype(np.float16)
    return qs, d


def draw_mxfp4(rng: np.random.Generator, rows: int, cols: int):
    """One MXFP4 matrix: packed codes uint8 [rows][cols/2] (two uniform 4-bit codes per
    byte), E8M0 scales uint8 [rows][cols/32] uniform in {118..121}."""
    if cols % 32:
        raise ValueError("MXFP4 needs cols % 32 == 0")
    qs = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    d = rng.integers(118, 122, size=(rows, cols // 32), dtype=np.uint8)
    return qs, d


def draw_iq4_nl(rng: np.random.Generator, rows: int, cols: int):
    """One IQ4_NL matrix: packed codes uint8 [rows][cols/2] (two uniform 4-bit codes per
    byte), d float16 [rows][cols/32] ~ U(0.5, 1.5) * 1e-3 (rounded to fp16)."""
    if cols % 32:
        raise ValueError("IQ4_NL needs cols % 32 == 0")
    qs = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    d = (rng.uniform(0.5, 1.5, size=(rows, cols // 32)) * 1e-3).astype(np.float16)
    return qs, d


def draw_iq4_xs(rng: np.random.Generator, rows: int, cols: int):
    """One IQ4_XS matrix: packed codes uint8 [rows][cols/2] (two uniform 4-bit codes per
    byte) and super-block records uint8 [rows][cols/256][8]: fp16 d ~ U(0.5, 1.5) * 1e-4,
    then six uniform bytes."""
    if cols % 256:
        raise ValueError("IQ4_XS needs cols % 256 == 0")
    qs = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    rec = rng.integers(0, 256, size=(rows, cols // 256, 8), dtype=np.uint8)
    d = (rng.uniform(0.5, 1.5, size=(rows, cols // 256)) * 1e-4).astype(np.float16)
    rec[:, :, 0:2] = d.view(np.uint8).reshape(rows, cols // 256, 2)
    return qs, rec


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def draw_q8_0_stack(seed: int, stream: int, which: int, n_mat: int, rows: int, cols: int,
                    qs_out: np.ndarray | None = None, d_out: np.ndarray | None = None,
                    wtype: str = "q8_0", only=None):
    """n_mat stacked Q8_0 (MXFP4, IQ4_NL) matrices; matrix e comes from stream
    (seed, stream, e, which). ``only`` (optional) lists the matrices to draw; the
    others are left zero (a drawn matrix has the same values either way)."""
    fp4 = wtype == "mxfp4"
    xs = wtype == "iq4_xs"
    nib = fp4 or xs or wtype == "iq4_nl"   # two 4-bit codes per byte
    alloc = np.empty if only is None else np.zeros
    qs = qs_out if qs_out is not None else (alloc((n_mat, rows, cols // 2), np.uint8) if nib
                                             else alloc((n_mat, rows, cols), np.int8))
    if d_out is not None:
        d = d_out
    elif xs:
        d = alloc((n_mat, rows, cols // 256, 8), np.uint8)
    else:
        d = alloc((n_mat, rows, cols // 32), np.uint8 if fp4 else np.float16)
    draw = draw_mxfp4 if fp4 else (draw_iq4_xs if xs else (draw_iq4_nl if nib else draw_q8_0))

    def one(e):
        q, s = draw(_rng(seed, stream, e, which), rows, cols)
        qs[e] = q
        d[e] = s

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(n_mat) if only is None else only))
    return qs, d


def draw_x_bf16(seed: int, n_tokens: int, n_embd: int) -> np.ndarray:
    """Activations N(0,1) rounded to bf16 (uint16 bits) [T][n_embd]."""
    x = _rng(seed, _S_X).standard_normal((n_tokens, n_embd), dtype=np.float32)
    return f32_to_bf16_bits(x)


def make_inputs(cfg: Config | str, seed: int | None = None, n_tokens: int | None = None,
                ids: np.ndarray | None = None, touched_only: bool = False) -> dict:
    """All inputs of one workload as numpy arrays (see module docstring).

    ``ids`` overrides the drawn routing table (shape [T][k]; entries may repeat or
    fall outside [0, E) for edge-case tests); everything else is drawn as usual.
    ``touched_only`` draws the routed experts' weights only for the experts the ids
    name and leaves the others zero (decode-sized batches of wide layers: nothing
    reads the untouched experts, and the touched ones get the same values)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.seed if seed is None else seed
    T = cfg.n_tokens if n_tokens is None else n_tokens
    E, k = cfg.n_experts, cfg.n_used
    out = {"cfg": cfg, "seed": seed, "n_tokens": T, "n_used": k, "n_experts": E}
    if ids is not None:
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(T, k))
        out["ids"] = ids
    elif cfg.routing == "zipf":
        out["ids"] = draw_ids_zipf(seed, T, E, k, cfg.zipf_s)
    else:
        out["ids"] = draw_ids_uniform(seed, T, E, k)
    out["route_w"] = draw_route_w(seed, T, k)
    if cfg.kind == "mmid":
        N, K = cfg.n_ff, cfg.n_embd
        if cfg.wtype == "f32":
            w = _rng(seed, _S_ROUTED, 0, 0).normal(0.0, 0.05, size=(E, N, K)).astype(np.float32)
            x = _rng(seed, _S_X).standard_normal((T, K), dtype=np.float32)
            out.update(w=w, x=x, wtype="f32", xtype="f32")
        else:
            qs, d = draw_q8_0_stack(seed, _S_ROUTED, 0, E, N, K, wtype=cfg.wtype)
            out.update(w_qs=qs, w_d=d, x=draw_x_bf16(seed, T, K), wtype=cfg.wtype, xtype="bf16")
        return out
    n_embd, n_ff, S = cfg.n_embd, cfg.n_ff, cfg.n_shared
    only = None
    if touched_only:
        v = out["ids"].ravel()
        only = sorted(set(v[(v >= 0) & (v < E)].tolist()))
    for name, which, rows, cols in (("gate", _M_GATE, n_ff, n_embd), ("up", _M_UP, n_ff, n_embd),
                                    ("down", _M_DOWN, n_embd, n_ff)):
        out[name + "_qs"], out[name + "_d"] = draw_q8_0_stack(seed, _S_ROUTED, which, E, rows, cols,
                                                              wtype=cfg.wtype, only=only)
        if S:
            out["sh_" + name + "_qs"], out["sh_" + name + "_d"] = draw_q8_0_stack(
                seed, _S_SHARED, which, S, rows, cols, wtype=cfg.wtype)
    out["x"] = draw_x_bf16(seed, T, n_embd)
    out.update(wtype=cfg.wtype, xtype="bf16")
    return out


def make_custom_ffn(seed: int, E: int, k: int, T: int, n_embd: int, n_ff: int, S: int = 0,
                    routing: str = "uniform", ids: np.ndarray | None = None,
                    wtype: str = "q8_0", touched_only: bool = False) -> dict:
    """An FFN workload of arbitrary shape (tests), same recipe as the named ones."""
    cfg = Config("custom", "ffn", E, k, T, n_embd, n_ff, n_shared=S, routing=routing, seed=seed,
                 wtype=wtype)
    return make_inputs(cfg, seed, ids=ids, touched_only=touched_only)


def make_custom_mmid(seed: int, E: int, k: int, T: int, K: int, N: int, wtype: str = "q8_0",
                     ids: np.ndarray | None = None) -> dict:
    """A mul_mat_id workload of arbitrary shape (tests)."""
    cfg = Config("custom", "mmid", E, k, T, K, N, wtype=wtype, seed=seed)
    return make_inputs(cfg, seed, ids=ids)
