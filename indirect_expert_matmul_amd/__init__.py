"""MI355X (gfx950) MoE indirect matrix multiplication -- Python binding of libmoe.

A thin ctypes layer over the C ABI in include/moe.h with the same entry-point
names. It only marshals arguments: torch tensors supply device memory (outputs and
the workspace are allocated with torch) and the current HIP stream; every step of
the computation runs in the library's HIP kernels. If libmoe.so is missing the
import fails -- there is no fallback.

    import indirect_expert_matmul_amd as moe
    out = moe.moe_ffn_fused(gate, up, down, x, ids, route_w, shared=(sg, su, sd))
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ELIMIT, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_Q8_0, MOE_MXFP4, MOE_IQ4_NL, MOE_IQ4_XS = 0, 1, 2, 3, 4, 5
PATH_AUTO, PATH_GEMM, PATH_GEMV = 0, 1, 2

# Every symbol include/moe.h declares.
EXPORTS = ("moe_row_ids", "moe_mul_mat_id", "moe_ffn_fused", "moe_router_topk",
           "moe_row_ids_workspace_size", "moe_mul_mat_id_workspace_size",
           "moe_ffn_fused_workspace_size", "moe_select_path", "moe_select_path_typed",
           "moe_status_string", "moe_last_error",
           "moe_last_stage_count", "moe_ffn_fused_noalloc", "moe_quantize_act", "moe_gather_rows")

NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (fn, _status_name(status), detail))


class c_moe_weights(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("n_mat", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class c_moe_options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("tau", ctypes.c_float), ("act_quant", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 5), ("timing_events", ctypes.POINTER(ctypes.c_void_p)),
                ("n_timing_events", ctypes.c_int32), ("reserved2", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmoe.so is not built (%s); run `python indirect_expert_matmul_amd/build.py`"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    W = ctypes.POINTER(c_moe_weights)
    O = ctypes.POINTER(c_moe_options)
    lib.moe_row_ids.argtypes = [P, I64, I32, I32, I32, P, P, P, P, SZ, P]
    lib.moe_mul_mat_id.argtypes = [W, P, ctypes.c_int, I32, P, I64, I32, P, P, O, P, SZ, P]
    lib.moe_ffn_fused.argtypes = [W, W, W, W, W, W, P, ctypes.c_int, P, P, I64, I32, P, O, P, SZ, P]
    lib.moe_router_topk.argtypes = [P, I64, I32, I32, P, P, P]
    lib.moe_ffn_fused_noalloc.argtypes = [W, W, W, W, W, W, P, ctypes.c_int, P, P, I64, I32, P, O, P]
    lib.moe_quantize_act.argtypes = [P, ctypes.c_int, I64, I64, P, P, P]
    lib.moe_gather_rows.argtypes = [P, ctypes.c_int, I64, I64, P, I64, P, P]
    for f in (lib.moe_row_ids, lib.moe_mul_mat_id, lib.moe_ffn_fused, lib.moe_router_topk,
              lib.moe_ffn_fused_noalloc, lib.moe_quantize_act, lib.moe_gather_rows):
        f.restype = ctypes.c_int
    lib.moe_row_ids_workspace_size.argtypes = [I64, I32, I32]
    lib.moe_mul_mat_id_workspace_size.argtypes = [W, ctypes.c_int, I32, I64, I32, O]
    lib.moe_ffn_fused_workspace_size.argtypes = [W, W, ctypes.c_int, I64, I32, O]
    for f in (lib.moe_row_ids_workspace_size, lib.moe_mul_mat_id_workspace_size,
              lib.moe_ffn_fused_workspace_size):
        f.restype = SZ
    lib.moe_select_path.argtypes = [I64, I32, I32, I64, O]
    lib.moe_select_path.restype = I32
    lib.moe_select_path_typed.argtypes = [I64, I32, I32, I64, ctypes.c_int, O]
    lib.moe_select_path_typed.restype = I32
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_stage_count.argtypes = []
    lib.moe_last_stage_count.restype = I32
    return lib


lib = _load()


def _status_name(s: int) -> str:
    return lib.moe_status_string(int(s)).decode()


def last_error() -> str:
    return lib.moe_last_error().decode()


def last_stage_count() -> int:
    """Kernels (timing-event pairs) the last mul_mat_id / ffn_fused call on this thread
    enqueued."""
    return int(lib.moe_last_stage_count())


def _check(status: int, fn: str):
    if status != MOE_OK:
        raise MoeError(status, fn, last_error())


@dataclass
class Weights:
    """Stacked expert matrices on the GPU. Q8_0: ``data`` int8 [n_mat][rows][cols] and
    ``scales`` float16 (or its uint16 bits) [n_mat][rows][cols/32]; MXFP4: ``data`` uint8
    [n_mat][rows][cols/2] (two E2M1 codes per byte, even column in the low nibble) and
    ``scales`` uint8 E8M0 [n_mat][rows][cols/32]; IQ4_NL: ``data`` uint8 codes packed as
    MXFP4's and ``scales`` float16 (or its 16 bits) [n_mat][rows][cols/32]; IQ4_XS: ``data``
    as IQ4_NL's and ``scales`` uint8 super-block records [n_mat][rows][cols/256][8]; F32:
    ``data`` float32 [n_mat][rows][cols] and ``scales`` None."""
    data: torch.Tensor
    scales: Optional[torch.Tensor] = None

    @property
    def type(self) -> int:
        if self.scales is None:
            return MOE_F32
        if self.data.dtype == torch.uint8:
            if self.scales.element_size() != 1:
                return MOE_IQ4_NL
            return MOE_IQ4_XS if self.scales.dim() == 4 else MOE_MXFP4
        return MOE_Q8_0

    @property
    def cols(self) -> int:
        return self.data.shape[2] * (2 if self.type in (MOE_MXFP4, MOE_IQ4_NL, MOE_IQ4_XS) else 1)

    def c(self) -> c_moe_weights:
        d = self.data
        if d.dim() != 3:
            raise ValueError("weights must be [n_mat][rows][cols]")
        if self.scales is None:
            if d.dtype != torch.float32:
                raise ValueError("float weights must be float32")
        else:
            if d.dtype == torch.uint8:
                if self.scales.dtype != torch.uint8 and self.scales.element_size() != 2:
                    raise ValueError("4-bit weights: uint8 codes with uint8 E8M0 (MXFP4), 16-bit "
                                     "fp16 (IQ4_NL) scales or uint8 super-block records (IQ4_XS)")
                if self.scales.dim() == 4 and (self.scales.dtype != torch.uint8 or
                                               tuple(self.scales.shape) != (d.shape[0], d.shape[1],
                                                                            2 * d.shape[2] // 256, 8)):
                    raise ValueError("IQ4_XS records must be uint8 [n_mat][rows][cols/256][8]")
            elif d.dtype != torch.int8 or self.scales.element_size() != 2:
                raise ValueError("Q8_0 weights: int8 qs with 16-bit scales")
            if not self.scales.is_contiguous():
                raise ValueError("scales must be contiguous")
        if not d.is_contiguous():
            raise ValueError("weights must be contiguous")
        return c_moe_weights(self.type, d.data_ptr(),
                             None if self.scales is None else self.scales.data_ptr(),
                             d.shape[0], d.shape[1], self.cols)


def _options(path: int = PATH_AUTO, tau: float = 0.0, events: Optional[Sequence[int]] = None,
             act_quant: int = 0):
    o = c_moe_options()
    o.path = path
    o.tau = tau
    o.act_quant = act_quant
    if events:
        arr = (ctypes.c_void_p * len(events))(*events)
        o.timing_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        o.n_timing_events = len(events)
        o._keep = arr
    return o


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _dev_check(*tensors):
    for t in tensors:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("all tensors must be contiguous device tensors")


def _xtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return MOE_BF16
    raise ValueError("activations must be float32 or bfloat16 (or its 16-bit patterns)")


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor], stream=None):
    """The caller's workspace, or a temporary one. A temporary is allocated by torch's
    caching allocator on its current stream; when the kernels run on another stream it
    is marked as used there (record_stream), so its memory is not handed out again
    before those kernels have finished with it."""
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small: need %d bytes" % nbytes)
        return ws
    t = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _keep_alive(stream, t)
    return t


def _keep_alive(stream, *tensors):
    """Mark torch-allocated tensors as in use on ``stream`` when it is not torch's current
    stream (the kernels are enqueued there, asynchronously)."""
    if stream is None:
        return
    cur = torch.cuda.current_stream(tensors[0].device if tensors else None)
    if stream.cuda_stream != cur.cuda_stream:
        for t in tensors:
            if t is not None:
                t.record_stream(stream)


def _check_ids(ids: torch.Tensor, route_w: Optional[torch.Tensor] = None):
    """ids must be int32 [T][k] (torch.topk gives int64, which would be read as wrong
    experts), route_w float32 of the same shape."""
    if ids.dtype != torch.int32 or ids.dim() != 2:
        raise ValueError("ids must be int32 [n_tokens][n_used] (got %s of shape %s)"
                         % (ids.dtype, tuple(ids.shape)))
    if route_w is not None and (route_w.dtype != torch.float32 or tuple(route_w.shape) != tuple(ids.shape)):
        raise ValueError("route_w must be float32 [n_tokens][n_used] like ids (got %s of shape %s)"
                         % (route_w.dtype, tuple(route_w.shape)))


def _check_out(out: Optional[torch.Tensor], shape):
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != tuple(shape)):
        raise ValueError("out must be float32 of shape %s (got %s of shape %s)"
                         % (tuple(shape), out.dtype, tuple(out.shape)))


def moe_select_path(n_tokens: int, n_used: int, n_experts: int, act_width: int,
                    path: int = PATH_AUTO, tau: float = 0.0) -> int:
    r = lib.moe_select_path(n_tokens, n_used, n_experts, act_width, ctypes.byref(_options(path, tau)))
    if r < 0:
        raise MoeError(r, "moe_select_path", last_error())
    return r


def moe_select_path_typed(n_tokens: int, n_used: int, n_experts: int, act_width: int, weight_type: int,
                          path: int = PATH_AUTO, tau: float = 0.0, act_quant: int = 0) -> int:
    r = lib.moe_select_path_typed(n_tokens, n_used, n_experts, act_width, weight_type,
                                  ctypes.byref(_options(path, tau, act_quant=act_quant)))
    if r < 0:
        raise MoeError(r, "moe_select_path_typed", last_error())
    return r


def moe_row_ids(ids: torch.Tensor, n_experts: int, src1_rows_per_token: int = 1, stream=None,
                workspace: Optional[torch.Tensor] = None):
    """(ids_src1, ids_dst, expert_bounds) for ids int32 [T][k] on the GPU."""
    _check_ids(ids)
    _dev_check(ids)
    T, k = ids.shape
    dev = ids.device
    s1 = torch.empty(T * k, dtype=torch.int32, device=dev)
    dd = torch.empty(T * k, dtype=torch.int32, device=dev)
    b = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    _keep_alive(stream, s1, dd, b)
    need = lib.moe_row_ids_workspace_size(T, k, n_experts)
    ws = _workspace(need, dev, workspace, stream)
    _check(lib.moe_row_ids(ids.data_ptr(), T, k, n_experts, src1_rows_per_token, s1.data_ptr(),
                           dd.data_ptr(), b.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                           _stream(stream)), "moe_row_ids")
    return s1, dd, b


def moe_gather_rows(src1: torch.Tensor, ids_src1: torch.Tensor, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """dst[j] = src1[ids_src1[j]] for src1 [rows][K] (bf16 or its 16-bit patterns, or
    float32) and int32 ids_src1 [n] (moe_row_ids' first map): the rows in expert order."""
    if src1.dim() != 2:
        raise ValueError("src1 must be [rows][K]")
    if ids_src1.dtype != torch.int32 or ids_src1.dim() != 1:
        raise ValueError("ids_src1 must be int32 [n]")
    _dev_check(src1)
    _dev_check(ids_src1)
    if not src1.is_contiguous() or not ids_src1.is_contiguous():
        raise ValueError("src1 and ids_src1 must be contiguous")
    rows, K = src1.shape
    n = ids_src1.numel()
    if out is None:
        out = torch.empty((n, K), dtype=src1.dtype, device=src1.device)
    elif out.dtype != src1.dtype or tuple(out.shape) != (n, K) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [n][K] tensor of src1's dtype")
    _keep_alive(stream, out)
    _check(lib.moe_gather_rows(src1.data_ptr(), _xtype(src1), rows, K, ids_src1.data_ptr(), n,
                               out.data_ptr(), _stream(stream)), "moe_gather_rows")
    return out


def moe_quantize_act(x: torch.Tensor, stream=None):
    """(q int8 [rows][K], d float32 [rows][K/32]) for activations x [rows][K] (bf16 or its
    16-bit patterns, or float32): the quantized-activation format of the int8 path."""
    if x.dim() != 2 or x.shape[1] % 32:
        raise ValueError("x must be [rows][K] with K % 32 == 0")
    _dev_check(x)
    rows, K = x.shape
    q = torch.empty((rows, K), dtype=torch.int8, device=x.device)
    d = torch.empty((rows, K // 32), dtype=torch.float32, device=x.device)
    _keep_alive(stream, q, d)
    _check(lib.moe_quantize_act(x.data_ptr(), _xtype(x), rows, K, q.data_ptr(), d.data_ptr(),
                                _stream(stream)), "moe_quantize_act")
    return q, d


def moe_router_topk(logits: torch.Tensor, n_used: int, ids: Optional[torch.Tensor] = None,
                    route_w: Optional[torch.Tensor] = None, stream=None):
    """(ids int32 [T][k], route_w float32 [T][k]) from router logits float32 [T][E]:
    the k largest logits per token (equal logits: lower index first), weighted by a
    softmax over the picked logits."""
    if logits.dtype != torch.float32 or logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be contiguous float32 [n_tokens][n_experts]")
    _dev_check(logits)
    T, E = logits.shape
    dev = logits.device
    if ids is None:
        ids = torch.empty((T, n_used), dtype=torch.int32, device=dev)
        _keep_alive(stream, ids)
    if route_w is None:
        route_w = torch.empty((T, n_used), dtype=torch.float32, device=dev)
        _keep_alive(stream, route_w)
    if ids.shape != (T, n_used) or ids.dtype != torch.int32 or route_w.shape != (T, n_used) \
            or route_w.dtype != torch.float32:
        raise ValueError("ids / route_w must be int32 / float32 [n_tokens][n_used]")
    _dev_check(ids, route_w)
    _check(lib.moe_router_topk(logits.data_ptr(), T, E, n_used, ids.data_ptr(), route_w.data_ptr(),
                               _stream(stream)), "moe_router_topk")
    return ids, route_w


def moe_mul_mat_id_workspace_size(w: Weights, src1_type: int, src1_rows_per_token: int,
                                  n_tokens: int, n_used: int, path: int = PATH_AUTO,
                                  tau: float = 0.0, act_quant: int = 0) -> int:
    cw = w.c()
    return lib.moe_mul_mat_id_workspace_size(ctypes.byref(cw), src1_type, src1_rows_per_token,
                                             n_tokens, n_used,
                                             ctypes.byref(_options(path, tau, act_quant=act_quant)))


def moe_mul_mat_id(w: Weights, src1: torch.Tensor, ids: torch.Tensor,
                   route_w: Optional[torch.Tensor] = None, src1_rows_per_token: int = 1,
                   path: int = PATH_AUTO, tau: float = 0.0, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None, events=None,
                   act_quant: int = 0):
    """GGML_OP_MUL_MAT_ID: float32 [T][k][N] per slot, or [T][N] weighted by route_w.
    ``act_quant=1``: the quantized-activation (int8 MFMA) grouped GEMM, Q8_0 experts."""
    _check_ids(ids, route_w)
    T, k = ids.shape
    cw = w.c()
    N = cw.rows
    shape = (T, N) if route_w is not None else (T, k, N)
    _check_out(out, shape)
    if src1.dim() < 2 or src1.numel() != T * src1_rows_per_token * cw.cols:
        raise ValueError("src1 must hold [n_tokens][src1_rows_per_token][K] = %d x %d x %d elements"
                         % (T, src1_rows_per_token, cw.cols))
    _dev_check(src1, ids, route_w, out)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=ids.device)
        _keep_alive(stream, out)
    st = _xtype(src1)
    opt = _options(path, tau, events, act_quant)
    need = lib.moe_mul_mat_id_workspace_size(ctypes.byref(cw), st, src1_rows_per_token, T, k,
                                             ctypes.byref(opt))
    ws = _workspace(need, ids.device, workspace, stream)
    _check(lib.moe_mul_mat_id(ctypes.byref(cw), src1.data_ptr(), st, src1_rows_per_token,
                              ids.data_ptr(), T, k,
                              None if route_w is None else route_w.data_ptr(), out.data_ptr(),
                              ctypes.byref(opt), ws.data_ptr(), ws.numel() * ws.element_size(),
                              _stream(stream)), "moe_mul_mat_id")
    return out


def moe_ffn_fused_workspace_size(gate: Weights, sh_gate: Optional[Weights], n_tokens: int,
                                 n_used: int, path: int = PATH_AUTO, tau: float = 0.0,
                                 act_quant: int = 0) -> int:
    cg = gate.c()
    cs = sh_gate.c() if sh_gate is not None else None
    return lib.moe_ffn_fused_workspace_size(ctypes.byref(cg), ctypes.byref(cs) if cs else None,
                                            MOE_BF16, n_tokens, n_used,
                                            ctypes.byref(_options(path, tau, act_quant=act_quant)))


def moe_ffn_fused(gate: Weights, up: Weights, down: Weights, x: torch.Tensor, ids: torch.Tensor,
                  route_w: torch.Tensor, shared: Optional[Sequence[Weights]] = None,
                  path: int = PATH_AUTO, tau: float = 0.0, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None, events=None,
                  act_quant: int = 0):
    """Fused MoE FFN: float32 [T][n_embd]. ``act_quant=1``: the quantized-activation
    (int8 MFMA) grouped GEMMs, Q8_0 experts."""
    _check_ids(ids, route_w)
    T, k = ids.shape
    cg, cu, cd = gate.c(), up.c(), down.c()
    _check_out(out, (T, cg.cols))
    if x.dim() != 2 or tuple(x.shape) != (T, cg.cols):
        raise ValueError("x must be [n_tokens][n_embd] = [%d][%d] (got %s)" % (T, cg.cols, tuple(x.shape)))
    _dev_check(x, ids, route_w, out)
    cs = [s.c() for s in shared] if shared else [None, None, None]
    if out is None:
        out = torch.empty((T, cg.cols), dtype=torch.float32, device=x.device)
        _keep_alive(stream, out)
    opt = _options(path, tau, events, act_quant)
    need = lib.moe_ffn_fused_workspace_size(ctypes.byref(cg),
                                            ctypes.byref(cs[0]) if cs[0] is not None else None,
                                            MOE_BF16, T, k, ctypes.byref(opt))
    ws = _workspace(need, x.device, workspace, stream)
    ref = [ctypes.byref(c) if c is not None else None for c in cs]
    _check(lib.moe_ffn_fused(ctypes.byref(cg), ctypes.byref(cu), ctypes.byref(cd), ref[0], ref[1],
                             ref[2], x.data_ptr(), _xtype(x), ids.data_ptr(), route_w.data_ptr(), T,
                             k, out.data_ptr(), ctypes.byref(opt), ws.data_ptr(),
                             ws.numel() * ws.element_size(), _stream(stream)), "moe_ffn_fused")
    return out


def moe_ffn_fused_noalloc(gate: Weights, up: Weights, down: Weights, x: torch.Tensor,
                          ids: torch.Tensor, route_w: torch.Tensor,
                          shared: Optional[Sequence[Weights]] = None, path: int = PATH_AUTO,
                          tau: float = 0.0, out: Optional[torch.Tensor] = None, stream=None,
                          events=None, act_quant: int = 0):
    """The fused MoE FFN with the library's own fixed scratch array as workspace (the C
    call allocates nothing; pass ``out`` to allocate nothing here either). Calls that
    overlap in time on one device share that array and race."""
    _check_ids(ids, route_w)
    T, k = ids.shape
    cg, cu, cd = gate.c(), up.c(), down.c()
    _check_out(out, (T, cg.cols))
    if x.dim() != 2 or tuple(x.shape) != (T, cg.cols):
        raise ValueError("x must be [n_tokens][n_embd] = [%d][%d] (got %s)" % (T, cg.cols, tuple(x.shape)))
    _dev_check(x, ids, route_w, out)
    cs = [s.c() for s in shared] if shared else [None, None, None]
    if out is None:
        out = torch.empty((T, cg.cols), dtype=torch.float32, device=x.device)
        _keep_alive(stream, out)
    opt = _options(path, tau, events, act_quant)
    ref = [ctypes.byref(c) if c is not None else None for c in cs]
    _check(lib.moe_ffn_fused_noalloc(ctypes.byref(cg), ctypes.byref(cu), ctypes.byref(cd), ref[0], ref[1],
                                     ref[2], x.data_ptr(), _xtype(x), ids.data_ptr(), route_w.data_ptr(),
                                     T, k, out.data_ptr(), ctypes.byref(opt), _stream(stream)),
           "moe_ffn_fused_noalloc")
    return out


def weights_from_numpy(qs_or_w, d=None, device="cuda") -> Weights:
    """Upload numpy weights (from ``synth``) as a Weights pair: float32; Q8_0 (int8 qs,
    fp16 scales); MXFP4 (uint8 codes, uint8 E8M0 scales); IQ4_NL (uint8 codes, fp16
    scales); or IQ4_XS (uint8 codes, uint8 records [..][cols/256][8])."""
    import numpy as np
    if d is None:
        return Weights(torch.from_numpy(np.ascontiguousarray(qs_or_w, dtype=np.float32)).to(device))
    if np.asarray(qs_or_w).dtype == np.uint8 and np.asarray(d).dtype == np.float16:
        q = torch.from_numpy(np.ascontiguousarray(qs_or_w, dtype=np.uint8)).to(device)
        return Weights(q, torch.from_numpy(np.ascontiguousarray(np.asarray(d).view(np.int16))).to(device))
    if np.asarray(qs_or_w).dtype == np.uint8:
        q = torch.from_numpy(np.ascontiguousarray(qs_or_w, dtype=np.uint8)).to(device)
        return Weights(q, torch.from_numpy(np.ascontiguousarray(d, dtype=np.uint8)).to(device))
    q = torch.from_numpy(np.ascontiguousarray(qs_or_w, dtype=np.int8)).to(device)
    s = torch.from_numpy(np.ascontiguousarray(np.asarray(d).view(np.int16))).to(device)
    return Weights(q, s)
