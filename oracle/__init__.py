"""Python face of the CPU oracle (``oracle.c``) for MoE mul_mat_id.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU library never does, and the
two share no code. Every function takes and returns numpy arrays; results are
float64.

Parity of this oracle is pinned in tests/test_oracle.py against brute force,
invariants, numpy/torch library routines and hand-derived fixtures.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, Q8_0, MXFP4, IQ4_NL, IQ4_XS = 0, 1, 2, 3, 4, 5
_TYPES = {"f32": F32, "bf16": BF16, "q8_0": Q8_0}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2 -fopenmp, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp,
                               _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        _lib.oracle_half_to_double.restype = ctypes.c_double
        _lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        _lib.oracle_bf16_to_double.restype = ctypes.c_double
        _lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        _lib.oracle_e2m1_to_double.restype = ctypes.c_double
        _lib.oracle_e2m1_to_double.argtypes = [ctypes.c_int]
        _lib.oracle_e8m0_to_double.restype = ctypes.c_double
        _lib.oracle_e8m0_to_double.argtypes = [ctypes.c_int]
        _lib.oracle_iq4nl_level.restype = ctypes.c_double
        _lib.oracle_iq4nl_level.argtypes = [ctypes.c_int]
        _lib.oracle_iq4xs_block_scale.restype = ctypes.c_double
        _lib.oracle_iq4xs_block_scale.argtypes = [ctypes.c_void_p, ctypes.c_int]
        _lib.oracle_dequant.argtypes = [ctypes.c_int, P, P, I64, I64, I64, P]
        _lib.oracle_row_ids.argtypes = [P, I64, I32, I32, I32, P, P, P]
        _lib.oracle_mul_mat_id.argtypes = [ctypes.c_int, P, P, I64, I64, I64, P, ctypes.c_int, I32,
                                           P, I64, I32, P, P]
        _lib.oracle_ffn.argtypes = ([ctypes.c_int] + [P] * 6 + [I64] * 3 + [P] * 6 + [I64] * 2 +
                                    [P, ctypes.c_int, P, P, I64, I32, P])
        _lib.oracle_router_topk.argtypes = [P, I64, I32, I32, P, P]
        _lib.oracle_quantize_act.argtypes = [ctypes.c_int, P, I64, I64, P, P]
        _lib.oracle_mul_mat_id_q8act.argtypes = [ctypes.c_int, P, P, I64, I64, I64, P, P, I32, P, I64,
                                                 I32, P, P]
        _lib.oracle_ffn_q8act.argtypes = _lib.oracle_ffn.argtypes
        for f in (_lib.oracle_dequant, _lib.oracle_row_ids, _lib.oracle_mul_mat_id, _lib.oracle_ffn,
                  _lib.oracle_router_topk, _lib.oracle_quantize_act, _lib.oracle_mul_mat_id_q8act,
                  _lib.oracle_ffn_q8act):
            f.restype = ctypes.c_int
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(int(bits) & 0xFFFF)


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits) & 0xFFFF)


def e2m1_to_double(code: int) -> float:
    return lib().oracle_e2m1_to_double(int(code) & 15)


def e8m0_to_double(x: int) -> float:
    return lib().oracle_e8m0_to_double(int(x) & 0xFF)


def iq4nl_level(code: int) -> float:
    return lib().oracle_iq4nl_level(int(code))


def iq4xs_block_scale(record, j: int) -> float:
    """Scale of block j (0..7) of one IQ4_XS super-block record (8 bytes)."""
    r = np.ascontiguousarray(record, dtype=np.uint8)
    assert r.size == 8
    return lib().oracle_iq4xs_block_scale(_p(r), int(j))


def dequant(qs_or_w, d=None) -> np.ndarray:
    """Dequantize Q8_0 (qs int8 [..][rows][cols], d fp16 [..][rows][cols/32]), MXFP4
    (codes uint8 [..][rows][cols/2], E8M0 scales uint8 [..][rows][cols/32]) or IQ4_NL
    (codes uint8 [..][rows][cols/2], fp16 scales [..][rows][cols/32]), IQ4_XS (codes as
    IQ4_NL's, super-block records uint8 [..][rows][cols/256][8]), or widen float32 weights,
    to float64 [..][rows][cols]."""
    a = np.asarray(qs_or_w)
    if d is not None and a.dtype == np.uint8:
        shape = a.shape[:-1] + (2 * a.shape[-1],)
        a3 = _c(a.reshape((-1,) + a.shape[-2:]), np.uint8)
        out = np.empty((a3.shape[0], a3.shape[1], 2 * a3.shape[2]), np.float64)
        d = np.asarray(d)
        if d.dtype == np.uint8 and d.ndim == a.ndim + 1:   # IQ4_XS super-block records
            s = _c(d.reshape(a3.shape[0], a3.shape[1], -1), np.uint8)
            rc = lib().oracle_dequant(IQ4_XS, _p(a3), _p(s), out.shape[0], out.shape[1], out.shape[2],
                                      _p(out))
        elif d.dtype == np.float16:
            s = _c(d.view(np.uint16).reshape(a3.shape[0], a3.shape[1], -1), np.uint16)
            rc = lib().oracle_dequant(IQ4_NL, _p(a3), _p(s), out.shape[0], out.shape[1], out.shape[2],
                                      _p(out))
        else:
            s = _c(d.reshape(a3.shape[0], a3.shape[1], -1), np.uint8)
            rc = lib().oracle_dequant(MXFP4, _p(a3), _p(s), out.shape[0], out.shape[1], out.shape[2],
                                      _p(out))
        if rc:
            raise ValueError("oracle_dequant rejected its arguments (%d)" % rc)
        return out.reshape(shape)
    shape = a.shape
    a3 = a.reshape((-1,) + shape[-2:])
    out = np.empty(a3.shape, np.float64)
    if d is None:
        w = _c(a3, np.float32)
        rc = lib().oracle_dequant(F32, _p(w), None, a3.shape[0], a3.shape[1], a3.shape[2], _p(out))
    else:
        q = _c(a3, np.int8)
        s = _c(np.asarray(d).view(np.uint16).reshape(a3.shape[0], a3.shape[1], -1), np.uint16)
        rc = lib().oracle_dequant(Q8_0, _p(q), _p(s), a3.shape[0], a3.shape[1], a3.shape[2], _p(out))
    if rc:
        raise ValueError("oracle_dequant rejected its arguments (%d)" % rc)
    return out.reshape(shape)


def row_ids(ids: np.ndarray, n_experts: int, src1_rows_per_token: int = 1):
    """(ids_src1, ids_dst, expert_bounds) for ids int32 [T][k]."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    s1 = np.empty(T * k, np.int32)
    dd = np.empty(T * k, np.int32)
    b = np.empty(n_experts + 1, np.int32)
    rc = lib().oracle_row_ids(_p(ids), T, k, n_experts, src1_rows_per_token, _p(s1), _p(dd), _p(b))
    if rc:
        raise ValueError("oracle_row_ids rejected its arguments (%d)" % rc)
    return s1, dd, b


def _weights(qs_or_w, d):
    """(type, data, scales, logical shape). 4-bit codes come as uint8; their scales tell
    MXFP4 (uint8 E8M0, one per 32), IQ4_NL (float16) and IQ4_XS (uint8 records of 8 bytes
    per 256 columns, one more dimension) apart."""
    if d is None:
        w = _c(qs_or_w, np.float32)
        return F32, w, None, w.shape
    if np.asarray(qs_or_w).dtype == np.uint8:
        q = _c(qs_or_w, np.uint8)
        shape = q.shape[:-1] + (2 * q.shape[-1],)
        if np.asarray(d).dtype == np.float16:
            return IQ4_NL, q, _c(np.asarray(d).view(np.uint16), np.uint16), shape
        if np.asarray(d).ndim == q.ndim + 1:
            return IQ4_XS, q, _c(d, np.uint8), shape
        return MXFP4, q, _c(d, np.uint8), shape
    q = _c(qs_or_w, np.int8)
    return Q8_0, q, _c(np.asarray(d).view(np.uint16), np.uint16), q.shape


def mul_mat_id(w, w_d, src1, src1_type: str, ids, route_w=None, src1_rows_per_token: int = 1):
    """Per-slot dst float64 [T][k][N], or the route_w-weighted [T][N].
    ``w`` is float32 [E][N][K] (w_d None), Q8_0 qs [E][N][K] with scales w_d, or MXFP4
    (IQ4_NL) codes [E][N][K/2] with E8M0 (fp16) scales w_d. ``src1`` is [T*B][K] (float32, or bf16 bits
    as uint16)."""
    wt, wq, ws, (E, N, K) = _weights(w, w_d)
    ids = _c(ids, np.int32)
    T, k = ids.shape
    st = _TYPES[src1_type]
    src = _c(src1, np.float32 if st == F32 else np.uint16)
    rw = _c(route_w, np.float32)
    out = np.empty((T, N) if rw is not None else (T, k, N), np.float64)
    rc = lib().oracle_mul_mat_id(wt, _p(wq), _p(ws), E, N, K, _p(src), st, src1_rows_per_token,
                                 _p(ids), T, k, _p(rw), _p(out))
    if rc:
        raise ValueError("oracle_mul_mat_id rejected its arguments (%d)" % rc)
    return out


def quantize_act(x, src_type: str = "bf16"):
    """Quantized-activation format (per 32-column block: float32 scale d = max|x|/127,
    int8 codes rint(x/d), decisions in float32): (q int8 [rows][K], d float32
    [rows][K/32]) for x [rows][K] (bf16 bits as uint16, or float32)."""
    st = _TYPES[src_type]
    a = _c(x, np.float32 if st == F32 else np.uint16)
    rows, K = a.shape
    q = np.empty((rows, K), np.int8)
    d = np.empty((rows, K // 32), np.float32)
    rc = lib().oracle_quantize_act(st, _p(a), rows, K, _p(q), _p(d))
    if rc:
        raise ValueError("oracle_quantize_act rejected its arguments (%d)" % rc)
    return q, d


def mul_mat_id_q8act(w, w_d, q, d, ids, route_w=None, src1_rows_per_token: int = 1):
    """mul_mat_id with quantized activations (q int8 [T*B][K], d float32 [T*B][K/32]):
    per-slot float64 [T][k][N], or the route_w-weighted [T][N]."""
    wt, wq, ws, (E, N, K) = _weights(w, w_d)
    ids = _c(ids, np.int32)
    T, k = ids.shape
    qa, da = _c(q, np.int8), _c(d, np.float32)
    rw = _c(route_w, np.float32)
    out = np.empty((T, N) if rw is not None else (T, k, N), np.float64)
    rc = lib().oracle_mul_mat_id_q8act(wt, _p(wq), _p(ws), E, N, K, _p(qa), _p(da), src1_rows_per_token,
                                       _p(ids), T, k, _p(rw), _p(out))
    if rc:
        raise ValueError("oracle_mul_mat_id_q8act rejected its arguments (%d)" % rc)
    return out


def ffn(inp: dict, token_rows=None, act_quant: bool = False) -> np.ndarray:
    """Fused MoE FFN output float64 [T][n_embd] for a workload dict from ``synth``.
    ``token_rows`` (optional index array) restricts the computation to those tokens;
    every token's output depends only on its own row of x, ids and route_w.
    ``act_quant``: the quantized-activation path (x quantized before gate/up, each h
    rounded to bf16 and quantized before down)."""
    ids, rw, x = inp["ids"], inp["route_w"], inp["x"]
    if token_rows is not None:
        token_rows = np.asarray(token_rows)
        ids, rw, x = ids[token_rows], rw[token_rows], x[token_rows]
    ids = _c(ids, np.int32)
    T, k = ids.shape
    xt = _TYPES[inp.get("xtype", "bf16")]
    x = _c(x, np.float32 if xt == F32 else np.uint16)
    rw = _c(rw, np.float32)
    wt, g, gs, (E, n_ff, n_embd) = _weights(inp["gate_qs"], inp.get("gate_d"))
    _, u, us, _ = _weights(inp["up_qs"], inp.get("up_d"))
    _, dn, dns, _ = _weights(inp["down_qs"], inp.get("down_d"))
    S, n_ff_sh = 0, 0
    sg = sgs = su = sus = sd = sds = None
    if inp.get("sh_gate_qs") is not None:
        _, sg, sgs, (S, n_ff_sh, _) = _weights(inp["sh_gate_qs"], inp.get("sh_gate_d"))
        _, su, sus, _ = _weights(inp["sh_up_qs"], inp.get("sh_up_d"))
        _, sd, sds, _ = _weights(inp["sh_down_qs"], inp.get("sh_down_d"))
    out = np.empty((T, n_embd), np.float64)
    f = lib().oracle_ffn_q8act if act_quant else lib().oracle_ffn
    rc = f(wt, _p(g), _p(gs), _p(u), _p(us), _p(dn), _p(dns), E, n_ff, n_embd,
           _p(sg), _p(sgs), _p(su), _p(sus), _p(sd), _p(sds), S, n_ff_sh,
           _p(x), xt, _p(ids), _p(rw), T, k, _p(out))
    if rc:
        raise ValueError("oracle_ffn rejected its arguments (%d)" % rc)
    return out


def router_topk(logits: np.ndarray, n_used: int):
    """(ids int32 [T][k], weights float64 [T][k]) for router logits float32 [T][E]:
    the k largest logits per token (equal logits: lower index first), in descending
    order, weighted by a softmax over the picked logits."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, n_used), np.int32)
    w = np.empty((T, n_used), np.float64)
    rc = lib().oracle_router_topk(_p(lg), T, E, n_used, _p(ids), _p(w))
    if rc:
        raise ValueError("oracle_router_topk rejected its arguments (%d)" % rc)
    return ids, w
