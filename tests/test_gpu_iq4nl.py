"""GPU parity of IQ4_NL experts (ggml's 4-bit non-linear IQ-series codes: 16 fixed
levels, one fp16 scale per 32 weights) against the fp64 oracle, on both paths.

GEMV path (n_tokens * n_used <= 64, widths <= 4096): the levels are exact small
integers and the scale multiplies each block's fp32 partial sum, so the error is fp32
rounding only (gate 1e-5). Grouped GEMM path: bf16(d * level) rounded to nearest-even,
as Q8_0's bf16(d * q), with bf16 activations and h (gate 2e-2). Tolerances are the
normwise max relative errors the op's accuracy contract states.
"""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import oracle
import synth
from moe_testutil import TOL_FP32, TOL_MFMA, dev_bf16, dev_f32, dev_i32, normwise, run_ffn, upload_ffn

pytestmark = pytest.mark.gpu

W = "iq4_nl"


# ------------------------------------------------------------------------- GEMV path

@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S", [
    (8, 2, 1, 2880, 2880, 0),     # single token: register rows; K = 2880 ends inside the second piece
    (8, 2, 1, 512, 256, 2),       # shared experts, fused reduce
    (16, 4, 6, 448, 1056, 1),     # several tokens: LDS ring, two slots per pass; separate reduce
    (4, 3, 5, 2048, 2080, 0),     # duplicate experts inside tokens; K exactly one piece / just past it
])
def test_ffn_iq4nl_gemv(E, k, T, n_embd, n_ff, S):
    ids = np.random.default_rng(T * 11 + E).integers(0, E, size=(T, k)).astype(np.int32)
    inp = synth.make_custom_ffn(151 + E, E, k, T, n_embd, n_ff, S, ids=ids, wtype=W)
    dv = upload_ffn(inp)
    assert dv["gate"].type == moe.MOE_IQ4_NL
    got = run_ffn(dv, path=moe.PATH_GEMV)
    torch.cuda.synchronize()
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_FP32


def test_ffn_iq4nl_gemv_zero_scales_and_invalid_ids():
    E, k, T, n_embd, n_ff = 6, 2, 3, 256, 128
    ids = synth.draw_ids_uniform(4, T, E, k)
    ids[1, 0] = -2
    ids[2, 1] = E + 5
    inp = synth.make_custom_ffn(161, E, k, T, n_embd, n_ff, 1, ids=ids, wtype=W)
    inp["gate_d"][0, :, 0] = 0
    inp["down_d"][2, 5, :] = 0
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMV)
    torch.cuda.synchronize()
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_FP32


@pytest.mark.parametrize("path,E,k,T,K,N,B_is_k,bad", [
    (moe.PATH_GEMV, 6, 3, 9, 96, 40, False, True),     # one 2048 piece, mostly past K; invalid ids
    (moe.PATH_GEMV, 8, 4, 5, 3008, 70, True, False),   # one src1 row per slot, K in the second piece
    (moe.PATH_GEMM, 6, 3, 9, 96, 40, False, True),     # the same shapes on the grouped GEMM
    (moe.PATH_GEMM, 8, 4, 5, 3008, 70, True, False),
    (moe.PATH_GEMM, 6, 3, 50, 96, 45, False, True),    # single partial stage, odd N
    (moe.PATH_GEMM, 8, 2, 200, 640, 200, True, False), # one src1 row per slot, ragged last stage
])
def test_iq4nl_mul_mat_id(path, E, k, T, K, N, B_is_k, bad):
    rng = np.random.default_rng(E * 100 + T + K)
    ids = synth.draw_ids_uniform(5, T, E, k)
    if bad:
        ids[0, 0], ids[T - 1, k - 1] = -1, E + 1
    inp = synth.make_custom_mmid(117, E, k, T, K, N, wtype=W, ids=ids)
    B = k if B_is_k else 1
    x = synth.f32_to_bf16_bits(rng.standard_normal((T * B, K)).astype(np.float32))
    w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
    assert w.type == moe.MOE_IQ4_NL and w.cols == K
    got = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), src1_rows_per_token=B, path=path)
    gotw = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), route_w=dev_f32(inp["route_w"]),
                              src1_rows_per_token=B, path=path)
    torch.cuda.synchronize()
    ref = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, None, B)
    refw = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, inp["route_w"], B)
    tol = TOL_FP32 if path == moe.PATH_GEMV else TOL_MFMA
    g = got.cpu().numpy()
    assert normwise(g, ref) <= tol
    assert normwise(gotw.cpu().numpy(), refw) <= tol
    assert np.all(g[(ids < 0) | (ids >= E)] == 0.0)


@pytest.mark.parametrize("name", ["dec1n", "dec8n"])
def test_decode_iq4nl_full(name):
    """GPT-OSS-20B-shaped decode (E32 k4, n_embd = n_ff = 2880) with IQ4_NL experts, every
    output compared."""
    inp = synth.make_inputs(name)
    got = run_ffn(upload_ffn(inp))
    torch.cuda.synchronize()
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    print("%s normwise error %.3g" % (name, err))
    assert err <= TOL_FP32


# ------------------------------------------------------------------------- grouped GEMM

@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S,routing", [
    (8, 2, 40, 256, 192, 1, "uniform"),   # 64-row tiles; down K = 192 ends inside a stage; ragged N
    (4, 2, 300, 512, 160, 0, "uniform"),  # 128-row tiles; down K = 160
    (6, 3, 100, 96, 64, 2, "uniform"),    # single partial stages both ways, duplicate experts
    (16, 4, 200, 384, 224, 1, "zipf"),    # skewed segments: empty, tiny and oversized experts
])
def test_ffn_iq4nl_gemm(E, k, T, n_embd, n_ff, S, routing):
    ids = (synth.draw_ids_zipf(35, T, E, k, 1.1) if routing == "zipf"
           else np.random.default_rng(T + E + 1).integers(0, E, size=(T, k)).astype(np.int32))
    inp = synth.make_custom_ffn(171 + E, E, k, T, n_embd, n_ff, S, ids=ids, wtype=W)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    assert moe.last_stage_count() == 4
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_MFMA


def test_ffn_iq4nl_gemm_segments_at_tile_edges_and_invalid_ids():
    """Expert segments of 0-200 rows around the 64- and 128-row tiles, one slot per token,
    every segment checked on its own; plus out-of-range ids and zero scales."""
    seg = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200]
    ids = np.repeat(np.arange(len(seg), dtype=np.int32), seg)
    np.random.default_rng(5).shuffle(ids)
    ids = ids.reshape(-1, 1)
    ids[7, 0], ids[100, 0] = -1, len(seg) + 2
    E, T = len(seg), ids.shape[0]
    inp = synth.make_custom_ffn(181, E, 1, T, 256, 192, 1, ids=ids, wtype=W)
    inp["up_d"][3, :, 1] = 0
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    g, ref = got.cpu().numpy(), oracle.ffn(inp)
    assert normwise(g, ref) <= TOL_MFMA
    for e in range(E):
        sel = ids[:, 0] == e
        if sel.any():
            assert normwise(g[sel], ref[sel]) <= TOL_MFMA, e


def test_ffn_iq4nl_gemm_large_grid_sampled():
    """64-row tiles with 2048 or more 8-wave tiles: gate/up runs 256 weight rows per block
    with a three-slot ring."""
    E, k, T, n_embd, n_ff = 128, 2, 2048, 512, 2048
    inp = synth.make_custom_ffn(191, E, k, T, n_embd, n_ff, 0, wtype=W)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    rows = np.array(sorted(set(np.random.default_rng(3).choice(T, 64, replace=False).tolist()) | {0, T - 1}))
    err = normwise(got.cpu().numpy()[rows], oracle.ffn(inp, token_rows=rows))
    assert err <= TOL_MFMA
    assert torch.isfinite(got).all()


def test_ppn_full_size_segments():
    """GPT-OSS-20B-shaped PP4096 prefill with IQ4_NL experts (128-row tiles): the oracle
    runs on the tokens holding the first and last row of every 128-row stretch of every
    expert's segment, plus random tokens."""
    inp = synth.make_inputs("ppn")
    got = run_ffn(upload_ffn(inp)).cpu().numpy()
    ids = inp["ids"]
    _, dst, bounds = oracle.row_ids(ids, inp["n_experts"], 1)
    k = ids.shape[1]
    pick = set(np.random.default_rng(2).choice(ids.shape[0], 32, replace=False).tolist())
    for e in range(inp["n_experts"]):
        lo, hi = int(bounds[e]), int(bounds[e + 1])
        for a in range(lo, hi, 128):
            pick.add(int(dst[a]) // k)
            pick.add(int(dst[min(a + 128, hi) - 1]) // k)
    rows = np.array(sorted(pick))
    err = normwise(got[rows], oracle.ffn(inp, token_rows=rows))
    print("ppn normwise error %.3g over %d tokens" % (err, len(rows)))
    assert err <= TOL_MFMA
    assert np.isfinite(got).all()


def _scales_off_by_one_half(w):
    """The same weights with the fp16 scales moved 2 bytes past a 4-byte boundary (a view
    one element into a larger buffer)."""
    flat = w.scales.reshape(-1)
    buf = torch.empty(flat.numel() + 1, dtype=flat.dtype, device=flat.device)
    buf[1:].copy_(flat)
    return moe.Weights(w.data, buf[1:].view(w.scales.shape))


@pytest.mark.parametrize("n_ff", [256, 320])
def test_ffn_iq4nl_gemm_128_row_tiles_both_kernels(n_ff):
    """128-row tiles with K % 64 == 0 run the wide kernel when the scale tensors are 4-byte
    aligned (with the 160-row last tiles when both widths qualify), the narrow one
    otherwise; both take the same k groups in the same order, so the outputs agree bit for
    bit."""
    E, k, T, n_embd = 4, 2, 300, 512
    ids = synth.draw_ids_uniform(14, T, E, k)
    inp = synth.make_custom_ffn(193, E, k, T, n_embd, n_ff, 1, ids=ids, wtype=W)
    dv = upload_ffn(inp)
    wide = run_ffn(dv, path=moe.PATH_GEMM)
    odd = dict(dv)
    for n in ("gate", "up", "down"):
        odd[n] = _scales_off_by_one_half(dv[n])
        assert odd[n].scales.data_ptr() % 4 == 2
    odd["shared"] = [_scales_off_by_one_half(w) for w in dv["shared"]]
    narrow = run_ffn(odd, path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    ref = oracle.ffn(inp)
    assert normwise(wide.cpu().numpy(), ref) <= TOL_MFMA
    assert normwise(narrow.cpu().numpy(), ref) <= TOL_MFMA
    assert torch.equal(wide, narrow)
