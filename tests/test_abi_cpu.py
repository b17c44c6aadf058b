"""CPU-side checks of the C ABI (include/moe.h): the library loads without a GPU,
exports every declared symbol, and rejects bad arguments before any HIP call
(validation is pure host code). No compute call is made here."""
import ctypes
import os
import re

import pytest

import indirect_expert_matmul_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(moe.EXPORTS)
    for n in names:
        assert hasattr(moe.lib, n), n


def test_status_strings():
    assert moe.lib.moe_status_string(0) == b"MOE_OK"
    for s in (-1, -2, -3, -4):
        assert moe.lib.moe_status_string(s).startswith(b"MOE_E")


def _w(n_mat=8, rows=64, cols=128, typ=moe.MOE_Q8_0, data=FAKE, scales=FAKE):
    return moe.c_moe_weights(typ, data, scales if typ in (moe.MOE_Q8_0, moe.MOE_MXFP4, moe.MOE_IQ4_NL,
                                                           moe.MOE_IQ4_XS) else None,
                             n_mat, rows, cols)


def _ffn(gate=None, up=None, down=None, sh=(None, None, None), T=16, k=2, x_type=moe.MOE_BF16,
         ws_bytes=1 << 40, ids=FAKE, out=FAKE, path=0, aq=0):
    gate = gate or _w()
    up = up or _w()
    down = down or _w(rows=128, cols=64)
    ref = lambda w: ctypes.byref(w) if w is not None else None
    opt = moe._options(path, act_quant=aq)
    return moe.lib.moe_ffn_fused(ref(gate), ref(up), ref(down), ref(sh[0]), ref(sh[1]), ref(sh[2]),
                                 FAKE, x_type, ids, FAKE, T, k, out, ctypes.byref(opt), FAKE,
                                 ws_bytes, None)


def test_ffn_validation():
    assert _ffn(T=1 << 22) == moe.MOE_ELIMIT
    assert _ffn(k=1024) == moe.MOE_ELIMIT
    assert _ffn(T=-1) == moe.MOE_EINVAL
    assert _ffn(k=0) == moe.MOE_EINVAL
    assert _ffn(gate=_w(n_mat=1025), up=_w(n_mat=1025), down=_w(n_mat=1025, rows=128, cols=64)) == moe.MOE_ELIMIT
    assert _ffn(gate=_w(cols=100), up=_w(cols=100), down=_w(rows=100, cols=64)) == moe.MOE_ELIMIT
    assert _ffn(down=_w(rows=64, cols=128)) == moe.MOE_EINVAL          # wrong down shape
    assert _ffn(x_type=moe.MOE_F32) == moe.MOE_EINVAL
    assert _ffn(gate=_w(scales=None)) == moe.MOE_EINVAL
    assert _ffn(gate=_w(data=None)) == moe.MOE_EINVAL
    assert _ffn(gate=_w(typ=moe.MOE_F32)) == moe.MOE_EINVAL
    assert _ffn(sh=(_w(n_mat=1, rows=32), None, None)) == moe.MOE_EINVAL    # partial shared set
    assert _ffn(ids=None) == moe.MOE_EINVAL
    assert _ffn(out=None) == moe.MOE_EINVAL
    assert _ffn(ws_bytes=16) == moe.MOE_EWORKSPACE
    assert _ffn(path=7) == moe.MOE_EINVAL
    assert _ffn(T=100, k=8, path=2) == moe.MOE_EINVAL                     # GEMV forced past its bound
    assert "n_used" in moe.last_error() or "GEMV" in moe.last_error()
    assert _ffn(T=0) == moe.MOE_OK                                         # empty batch: no-op
    assert moe.last_stage_count() == 0                                     # ... that timed nothing


def test_mul_mat_id_validation():
    def call(w=None, st=moe.MOE_BF16, B=1, T=16, k=2, ws=1 << 40, dst=FAKE):
        w = w or _w()
        return moe.lib.moe_mul_mat_id(ctypes.byref(w), FAKE, st, B, FAKE, T, k, None, dst,
                                      None, FAKE, ws, None)
    assert call(B=3) == moe.MOE_EINVAL
    assert call(st=moe.MOE_F32) == moe.MOE_EINVAL
    assert call(w=_w(typ=moe.MOE_F32), st=moe.MOE_BF16) == moe.MOE_EINVAL
    assert call(dst=None) == moe.MOE_EINVAL
    assert call(ws=8) == moe.MOE_EWORKSPACE
    assert call(T=1 << 22) == moe.MOE_ELIMIT
    assert call(T=0) == moe.MOE_OK


def test_mxfp4_validation():
    """MXFP4 experts: both paths validate (the calls stop at the workspace check here);
    the GEMV path forced past its wave-kernel bound and mixed weight types are refused."""
    fp4 = lambda **kw: _w(typ=moe.MOE_MXFP4, **kw)
    dn = lambda **kw: fp4(rows=128, cols=64, **kw)
    assert _ffn(gate=fp4(), up=fp4(), down=dn(), T=4, k=2, ws_bytes=16) == moe.MOE_EWORKSPACE
    assert _ffn(gate=fp4(), up=fp4(), down=dn(), T=40, k=2, ws_bytes=16) == moe.MOE_EWORKSPACE
    assert _ffn(gate=fp4(), up=fp4(), down=dn(), T=4, k=2, path=1, ws_bytes=16) == moe.MOE_EWORKSPACE
    assert _ffn(gate=fp4(), up=fp4(), down=dn(), T=40, k=2, path=2) == moe.MOE_EINVAL   # 80 slots
    assert "MXFP4" in moe.last_error()
    assert _ffn(gate=fp4(), up=_w(), down=dn(), T=4, k=2) == moe.MOE_EINVAL       # mixed types
    assert _ffn(gate=fp4(scales=None), up=fp4(), down=dn(), T=4, k=2) == moe.MOE_EINVAL
    assert _ffn(gate=fp4(cols=100), up=fp4(cols=100), down=fp4(rows=100, cols=64), T=4, k=2) == moe.MOE_ELIMIT
    sh = (fp4(n_mat=1), fp4(n_mat=1), dn(n_mat=1))
    assert _ffn(gate=fp4(), up=fp4(), down=dn(), sh=sh, T=4, k=2, ws_bytes=16) == moe.MOE_EWORKSPACE
    shq = (_w(n_mat=1), _w(n_mat=1), _w(n_mat=1, rows=128, cols=64))
    assert _ffn(gate=fp4(), up=fp4(), down=dn(), sh=shq, T=4, k=2) == moe.MOE_EINVAL
    w = fp4()
    mm = moe.lib.moe_mul_mat_id_workspace_size
    assert mm(ctypes.byref(w), moe.MOE_BF16, 1, 100, 2, None) > 0              # the GEMM path
    assert moe.lib.moe_mul_mat_id(ctypes.byref(w), FAKE, moe.MOE_F32, 1, FAKE, 4, 2, None, FAKE,
                                  None, FAKE, 1 << 30, None) == moe.MOE_EINVAL   # needs BF16 src1


def test_iq4nl_validation():
    """IQ4_NL experts: both paths validate (the calls stop at the workspace check here),
    the GEMV path forced past its wave-kernel bound, mixed types, missing scales, cols not
    a multiple of 32 and float32 src1 are refused."""
    nl = lambda **kw: _w(typ=moe.MOE_IQ4_NL, **kw)
    dn = lambda **kw: nl(rows=128, cols=64, **kw)
    assert _ffn(gate=nl(), up=nl(), down=dn(), T=4, k=2, ws_bytes=16) == moe.MOE_EWORKSPACE
    assert _ffn(gate=nl(), up=nl(), down=dn(), T=40, k=2, ws_bytes=16) == moe.MOE_EWORKSPACE
    assert _ffn(gate=nl(), up=nl(), down=dn(), T=40, k=2, path=2) == moe.MOE_EINVAL   # 80 slots
    assert "IQ4_NL" in moe.last_error()
    assert _ffn(gate=nl(), up=_w(typ=moe.MOE_MXFP4), down=dn(), T=4, k=2) == moe.MOE_EINVAL
    assert _ffn(gate=nl(scales=None), up=nl(), down=dn(), T=4, k=2) == moe.MOE_EINVAL
    assert _ffn(gate=nl(cols=100), up=nl(cols=100), down=nl(rows=100, cols=64), T=4, k=2) == moe.MOE_ELIMIT
    assert _ffn(gate=nl(), up=nl(), down=dn(), T=4, k=2, aq=1) == moe.MOE_EINVAL     # act_quant: Q8_0 only
    w = nl()
    mm = moe.lib.moe_mul_mat_id_workspace_size
    assert mm(ctypes.byref(w), moe.MOE_BF16, 1, 100, 2, None) > 0
    assert moe.lib.moe_mul_mat_id(ctypes.byref(w), FAKE, moe.MOE_F32, 1, FAKE, 4, 2, None, FAKE,
                                  None, FAKE, 1 << 30, None) == moe.MOE_EINVAL
    assert "IQ4_NL" in moe.last_error()


def test_iq4xs_validation():
    """IQ4_XS experts: widths must be multiples of 256 (MOE_ELIMIT), the super-block records
    8-byte aligned (MOE_EINVAL); both paths validate otherwise (the calls stop at the
    workspace check here), the GEMV path forced past its bound and float32 src1 are refused."""
    xs = lambda **kw: _w(typ=moe.MOE_IQ4_XS, cols=kw.pop("cols", 256), **kw)
    dn = lambda **kw: xs(rows=256, cols=64 * 4, **kw)
    g = lambda **kw: xs(rows=256, **kw)
    assert _ffn(gate=g(), up=g(), down=dn(), T=4, k=2, ws_bytes=16) == moe.MOE_EWORKSPACE
    assert _ffn(gate=g(), up=g(), down=dn(), T=40, k=2, ws_bytes=16) == moe.MOE_EWORKSPACE
    assert _ffn(gate=g(), up=g(), down=dn(), T=40, k=2, path=2) == moe.MOE_EINVAL   # 80 slots
    assert _ffn(gate=g(cols=128), up=g(cols=128), down=xs(rows=128, cols=256), T=4, k=2) == moe.MOE_ELIMIT
    assert "IQ4_XS" in moe.last_error() and "256" in moe.last_error()
    assert _ffn(gate=g(scales=FAKE + 4), up=g(), down=dn(), T=4, k=2) == moe.MOE_EINVAL
    assert "aligned" in moe.last_error()
    assert _ffn(gate=g(), up=_w(typ=moe.MOE_IQ4_NL, rows=256, cols=256), down=dn(), T=4, k=2) == moe.MOE_EINVAL
    w = g()
    assert moe.lib.moe_mul_mat_id_workspace_size(ctypes.byref(w), moe.MOE_BF16, 1, 100, 2, None) > 0
    assert moe.lib.moe_mul_mat_id(ctypes.byref(w), FAKE, moe.MOE_F32, 1, FAKE, 4, 2, None, FAKE,
                                  None, FAKE, 1 << 30, None) == moe.MOE_EINVAL


def test_gather_validation():
    g = moe.lib.moe_gather_rows
    assert g(FAKE, moe.MOE_Q8_0, 10, 64, FAKE, 5, FAKE, None) == moe.MOE_EINVAL      # type
    assert g(FAKE, moe.MOE_BF16, 0, 64, FAKE, 5, FAKE, None) == moe.MOE_EINVAL       # no rows
    assert g(FAKE, moe.MOE_BF16, 10, 64, None, 5, FAKE, None) == moe.MOE_EINVAL      # NULL map
    assert g(FAKE, moe.MOE_F32, 1 << 31, 64, FAKE, 5, FAKE, None) == moe.MOE_ELIMIT
    assert g(None, moe.MOE_BF16, 10, 64, None, 0, None, None) == moe.MOE_OK         # n = 0


def test_row_ids_validation():
    f = moe.lib.moe_row_ids
    assert f(FAKE, 16, 2, 8, 3, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == moe.MOE_EINVAL
    assert f(FAKE, 16, 2, 0, 1, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == moe.MOE_EINVAL
    assert f(FAKE, 16, 2, 2000, 1, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == moe.MOE_ELIMIT
    assert f(None, 16, 2, 8, 1, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == moe.MOE_EINVAL
    big = moe.lib.moe_row_ids_workspace_size(1 << 21, 8, 256)
    assert big > 0 and moe.lib.moe_row_ids_workspace_size(512, 6, 64) == 0
    assert f(FAKE, 1 << 21, 8, 256, 1, FAKE, FAKE, FAKE, FAKE, big - 1, None) == moe.MOE_EWORKSPACE


def test_path_selection():
    assert moe.moe_select_path(512, 6, 64, 2048) == moe.PATH_GEMM        # DeepSeek-Lite-shaped prefill
    assert moe.moe_select_path(1, 4, 32, 2880) == moe.PATH_GEMV          # decode, batch 1
    assert moe.moe_select_path(8, 4, 32, 2880) == moe.PATH_GEMV          # decode, batch 8
    assert moe.moe_select_path(4096, 8, 128, 2048) == moe.PATH_GEMM
    assert moe.moe_select_path(16, 2, 8, 64) == moe.PATH_GEMM            # T/E = 2
    assert moe.moe_select_path(8, 4, 32, 2880, path=moe.PATH_GEMM) == moe.PATH_GEMM
    assert moe.moe_select_path(64, 2, 64, 2048, path=moe.PATH_GEMV) == moe.PATH_GEMV
    assert moe.moe_select_path(64, 2, 16, 2048) == moe.PATH_GEMM                 # T >= tau*E
    assert moe.moe_select_path(20, 4, 32, 2880, tau=0.5) == moe.PATH_GEMM
    # automatic GEMV: wave kernels up to 48 slots, the block kernel for one token only
    assert moe.moe_select_path(16, 4, 32, 2880) == moe.PATH_GEMM         # 64 slots
    assert moe.moe_select_path(8, 6, 64, 2048) == moe.PATH_GEMV          # 48 slots
    assert moe.moe_select_path(10, 6, 64, 2048) == moe.PATH_GEMM         # 60 slots
    assert moe.moe_select_path(42, 6, 64, 2048) == moe.PATH_GEMM
    assert moe.moe_select_path(1, 8, 256, 7168) == moe.PATH_GEMV         # width > 4096, one token
    assert moe.moe_select_path(2, 8, 256, 7168) == moe.PATH_GEMM
    assert moe.moe_select_path(42, 6, 64, 2048, path=moe.PATH_GEMV) == moe.PATH_GEMV
    assert moe.moe_select_path(8, 8, 256, 7168, path=moe.PATH_GEMV) == moe.PATH_GEMV
    # by weight type: 4-bit experts use the wave kernels only (MXFP4 up to 32 slots, the
    # IQ formats up to 64); quantized activations need Q8_0
    typed = moe.moe_select_path_typed
    assert typed(8, 8, 128, 2048, moe.MOE_IQ4_XS) == moe.PATH_GEMV       # 64 slots
    assert typed(8, 8, 128, 2048, moe.MOE_Q8_0) == moe.PATH_GEMM
    assert typed(8, 4, 32, 2880, moe.MOE_MXFP4) == moe.PATH_GEMV         # 32 slots
    assert typed(12, 4, 32, 2880, moe.MOE_MXFP4) == moe.PATH_GEMM
    assert typed(12, 4, 32, 2880, moe.MOE_IQ4_NL) == moe.PATH_GEMV
    assert typed(1, 8, 256, 7168, moe.MOE_IQ4_NL) == moe.PATH_GEMM       # width > 4096
    assert typed(1, 8, 256, 7168, moe.MOE_Q8_0) == moe.PATH_GEMV
    assert typed(8, 4, 32, 2880, moe.MOE_Q8_0, act_quant=1) == 3
    for bad in ((8, 4, 32, 2880, moe.MOE_MXFP4), (8, 4, 32, 2880, moe.MOE_F32)):
        with pytest.raises(moe.MoeError):
            typed(*bad, act_quant=1 if bad[4] == moe.MOE_MXFP4 else 0)
    with pytest.raises(moe.MoeError):
        typed(1, 8, 256, 7168, moe.MOE_IQ4_XS, path=moe.PATH_GEMV)
    with pytest.raises(moe.MoeError):
        moe.moe_select_path(100, 8, 256, 7168, path=moe.PATH_GEMV)


def test_workspace_sizes_are_positive_and_monotone():
    g = _w(n_mat=64, rows=1408, cols=2048)
    s = _w(n_mat=2, rows=1408, cols=2048)
    a = moe.lib.moe_ffn_fused_workspace_size(ctypes.byref(g), ctypes.byref(s), moe.MOE_BF16, 512, 6, None)
    b = moe.lib.moe_ffn_fused_workspace_size(ctypes.byref(g), ctypes.byref(s), moe.MOE_BF16, 1024, 6, None)
    assert 0 < a < b
    assert moe.lib.moe_ffn_fused_workspace_size(ctypes.byref(g), None, moe.MOE_F32, 512, 6, None) == 0
    w = _w(n_mat=8, rows=32, cols=64, typ=moe.MOE_F32)
    assert moe.lib.moe_mul_mat_id_workspace_size(ctypes.byref(w), moe.MOE_F32, 1, 16, 2, None) > 0


def test_router_validation():
    f = moe.lib.moe_router_topk
    assert f(FAKE, 16, 8, 9, FAKE, FAKE, None) == moe.MOE_EINVAL     # n_used > n_experts
    assert f(FAKE, 16, 8, 0, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert f(FAKE, 16, 0, 1, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert f(FAKE, 16, 2048, 8, FAKE, FAKE, None) == moe.MOE_ELIMIT
    assert f(FAKE, 1 << 22, 64, 8, FAKE, FAKE, None) == moe.MOE_ELIMIT
    assert f(None, 16, 64, 8, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert f(FAKE, 16, 64, 8, FAKE, None, None) == moe.MOE_EINVAL
    assert f(None, 0, 64, 8, None, None, None) == moe.MOE_OK                # empty batch: no-op


def test_gathered_activation_limit_and_f32_path():
    """The grouped GEMM gathers activation rows through 32-bit byte offsets from the
    tensor's start: a gathered tensor of 4 GiB or more is MOE_ELIMIT, caught before
    anything is enqueued. h (the down projection's input, read in order) has no such
    limit. A float32 mul_mat_id has only the grouped fp32 product: forcing the GEMV
    path (or an unknown path) is MOE_EINVAL."""
    g = _w(n_mat=1, rows=64, cols=1024)
    d = _w(n_mat=1, rows=1024, cols=64)
    assert _ffn(gate=g, up=_w(n_mat=1, rows=64, cols=1024), down=d, T=1 << 21, k=1) == moe.MOE_ELIMIT
    assert "4 GiB" in moe.last_error()
    # just under: the same layer with one token fewer gets past the limit checks
    # (it then fails on the fake workspace size)
    assert _ffn(gate=g, up=_w(n_mat=1, rows=64, cols=1024), down=d, T=(1 << 21) - 1, k=1,
                ws_bytes=16) == moe.MOE_EWORKSPACE
    w = _w(n_mat=1, rows=64, cols=1024)
    assert moe.lib.moe_mul_mat_id(ctypes.byref(w), FAKE, moe.MOE_BF16, 1, FAKE, 1 << 21, 1, None, FAKE,
                                  None, FAKE, 1 << 40, None) == moe.MOE_ELIMIT
    f32 = _w(n_mat=8, rows=32, cols=64, typ=moe.MOE_F32)
    for path, want in ((2, moe.MOE_EINVAL), (5, moe.MOE_EINVAL), (1, moe.MOE_EWORKSPACE)):
        opt = moe._options(path)
        assert moe.lib.moe_mul_mat_id(ctypes.byref(f32), FAKE, moe.MOE_F32, 1, FAKE, 16, 2, None, FAKE,
                                      ctypes.byref(opt), FAKE, 16, None) == want, path
        size = moe.lib.moe_mul_mat_id_workspace_size(ctypes.byref(f32), moe.MOE_F32, 1, 16, 2,
                                                      ctypes.byref(opt))
        assert (size > 0) == (want != moe.MOE_EINVAL), path


def test_binding_rejects_wrong_dtypes_and_shapes():
    """The Python binding checks dtypes and shapes before anything reaches the library:
    int64 ids (what torch.topk returns), float64 routing weights, an output of the wrong
    shape or dtype, and activations of the wrong size."""
    import torch
    w = moe.Weights(torch.zeros((4, 32, 64), dtype=torch.int8), torch.zeros((4, 32, 2), dtype=torch.int16))
    x = torch.zeros((8, 64), dtype=torch.int16)
    ids = torch.zeros((8, 2), dtype=torch.int32)
    rw = torch.zeros((8, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="ids must be int32"):
        moe.moe_ffn_fused(w, w, w, x, ids.long(), rw)
    with pytest.raises(ValueError, match="route_w must be float32"):
        moe.moe_ffn_fused(w, w, w, x, ids, rw.double())
    with pytest.raises(ValueError, match="route_w must be float32"):
        moe.moe_mul_mat_id(w, x, ids, route_w=rw[:4])
    with pytest.raises(ValueError, match="out must be float32"):
        moe.moe_mul_mat_id(w, x, ids, out=torch.zeros((8, 32), dtype=torch.float32))
    with pytest.raises(ValueError, match="out must be float32"):
        moe.moe_mul_mat_id(w, x, ids, route_w=rw, out=torch.zeros((8, 32), dtype=torch.float16))
    with pytest.raises(ValueError, match="src1 must hold"):
        moe.moe_mul_mat_id(w, x[:4], ids)
    with pytest.raises(ValueError, match="ids must be int32"):
        moe.moe_row_ids(ids.long(), 4)
    with pytest.raises(ValueError, match="x must be"):
        moe.moe_ffn_fused(w, w, moe.Weights(torch.zeros((4, 64, 32), dtype=torch.int8),
                                            torch.zeros((4, 64, 1), dtype=torch.int16)), x[:5], ids, rw)


def test_act_quant_validation():
    """Quantized activations: Q8_0 experts only, the grouped GEMM only (path 0 or 1),
    act_quant 0 or 1; moe_quantize_act needs K % 32 == 0 and a bf16 or float32 input."""
    fp4 = lambda **kw: _w(typ=moe.MOE_MXFP4, **kw)

    def ffn(gate=None, up=None, down=None, path=0, aq=1, ws=16):
        gate = gate or _w()
        up = up or _w()
        down = down or _w(rows=128, cols=64)
        opt = moe._options(path, act_quant=aq)
        return moe.lib.moe_ffn_fused(ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down), None, None,
                                     None, FAKE, moe.MOE_BF16, FAKE, FAKE, 16, 2, FAKE, ctypes.byref(opt),
                                     FAKE, ws, None)
    assert ffn() == moe.MOE_EWORKSPACE                  # valid: stops at the fake workspace
    assert ffn(path=1) == moe.MOE_EWORKSPACE
    assert ffn(path=2) == moe.MOE_EINVAL
    assert ffn(aq=2) == moe.MOE_EINVAL
    assert ffn(gate=fp4(), up=fp4(), down=fp4(rows=128, cols=64)) == moe.MOE_EINVAL
    g = _w(n_mat=64, rows=1408, cols=2048)
    a = moe.lib.moe_ffn_fused_workspace_size(ctypes.byref(g), None, moe.MOE_BF16, 512, 6,
                                              ctypes.byref(moe._options(0, act_quant=1)))
    b = moe.lib.moe_ffn_fused_workspace_size(ctypes.byref(g), None, moe.MOE_BF16, 512, 6, None)
    assert a > b > 0
    f32 = _w(n_mat=8, rows=32, cols=64, typ=moe.MOE_F32)
    opt = moe._options(0, act_quant=1)
    assert moe.lib.moe_mul_mat_id(ctypes.byref(f32), FAKE, moe.MOE_F32, 1, FAKE, 16, 2, None, FAKE,
                                  ctypes.byref(opt), FAKE, 1 << 30, None) == moe.MOE_EINVAL
    q = moe.lib.moe_quantize_act
    assert q(FAKE, moe.MOE_BF16, 4, 100, FAKE, FAKE, None) == moe.MOE_ELIMIT
    assert q(FAKE, moe.MOE_Q8_0, 4, 64, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert q(None, moe.MOE_BF16, 4, 64, FAKE, FAKE, None) == moe.MOE_EINVAL
    assert q(None, moe.MOE_BF16, 0, 64, None, None, None) == moe.MOE_OK
