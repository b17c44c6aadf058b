"""GPU parity of IQ4_XS experts (ggml's super-block form of the IQ4_NL codes: 256 weights
share an fp16 d, each block of 32 a 6-bit sub-scale, value = d * (ls - 32) * level) against
the fp64 oracle, on both paths. Widths are multiples of 256.

GEMV path: exact levels and block scales, fp32 accumulate (gate 1e-5). Grouped GEMM:
bf16(scale * level) rounded to nearest-even, bf16 activations and h (gate 2e-2). The
tolerances are the normwise max relative errors of the op's accuracy contract.
"""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import oracle
import synth
from moe_testutil import TOL_FP32, TOL_MFMA, dev_bf16, dev_f32, dev_i32, normwise, run_ffn, upload_ffn

pytestmark = pytest.mark.gpu

W = "iq4_xs"


@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S", [
    (8, 2, 1, 2048, 1024, 0),     # single token: register rows; K = 2048 is one whole piece
    (8, 2, 1, 512, 256, 2),       # shared experts, fused reduce
    (16, 4, 6, 768, 1280, 1),     # several tokens: LDS ring, two slots per pass; separate reduce
    (4, 3, 5, 2048, 2304, 0),     # duplicate experts inside tokens; K just past one piece
])
def test_ffn_iq4xs_gemv(E, k, T, n_embd, n_ff, S):
    ids = np.random.default_rng(T * 13 + E).integers(0, E, size=(T, k)).astype(np.int32)
    inp = synth.make_custom_ffn(251 + E, E, k, T, n_embd, n_ff, S, ids=ids, wtype=W)
    dv = upload_ffn(inp)
    assert dv["gate"].type == moe.MOE_IQ4_XS
    got = run_ffn(dv, path=moe.PATH_GEMV)
    torch.cuda.synchronize()
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_FP32


@pytest.mark.parametrize("path", [moe.PATH_GEMV, moe.PATH_GEMM])
def test_ffn_iq4xs_zero_scales_and_invalid_ids(path):
    E, k, T, n_embd, n_ff = 6, 2, 3 if path == moe.PATH_GEMV else 90, 256, 512
    ids = synth.draw_ids_uniform(4, T, E, k)
    ids[1, 0] = -2
    ids[2, 1] = E + 5
    inp = synth.make_custom_ffn(261, E, k, T, n_embd, n_ff, 1, ids=ids, wtype=W)
    inp["gate_d"][0, :, 0, 0:2] = 0       # d = 0: the whole super-block contributes nothing
    inp["down_d"][2, 5, :, 2:] = 0        # every sub-scale 0: block scales -32 d
    got = run_ffn(upload_ffn(inp), path=path)
    torch.cuda.synchronize()
    tol = TOL_FP32 if path == moe.PATH_GEMV else TOL_MFMA
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= tol


@pytest.mark.parametrize("path,E,k,T,K,N,B_is_k,bad", [
    (moe.PATH_GEMV, 6, 3, 9, 256, 40, False, True),
    (moe.PATH_GEMV, 8, 4, 5, 3072, 70, True, False),   # K in the second piece
    (moe.PATH_GEMM, 6, 3, 9, 256, 40, False, True),
    (moe.PATH_GEMM, 8, 4, 5, 3072, 70, True, False),
    (moe.PATH_GEMM, 6, 3, 50, 512, 45, False, True),   # odd N
    (moe.PATH_GEMM, 8, 2, 200, 768, 200, True, False), # one src1 row per slot
])
def test_iq4xs_mul_mat_id(path, E, k, T, K, N, B_is_k, bad):
    rng = np.random.default_rng(E * 100 + T + K)
    ids = synth.draw_ids_uniform(5, T, E, k)
    if bad:
        ids[0, 0], ids[T - 1, k - 1] = -1, E + 1
    inp = synth.make_custom_mmid(217, E, k, T, K, N, wtype=W, ids=ids)
    B = k if B_is_k else 1
    x = synth.f32_to_bf16_bits(rng.standard_normal((T * B, K)).astype(np.float32))
    w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
    assert w.type == moe.MOE_IQ4_XS and w.cols == K
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


@pytest.mark.parametrize("name", ["dec1s", "dec8s"])
def test_decode_iq4xs_full(name):
    """E128 k8 decode (n_embd 2048, n_ff 768) with IQ4_XS experts, every output compared."""
    inp = synth.make_inputs(name)
    got = run_ffn(upload_ffn(inp))
    torch.cuda.synchronize()
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    print("%s normwise error %.3g" % (name, err))
    assert err <= TOL_FP32


@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S,routing", [
    (8, 2, 40, 256, 512, 1, "uniform"),   # 64-row tiles
    (4, 2, 300, 512, 256, 0, "uniform"),  # 128-row tiles
    (6, 3, 100, 256, 256, 2, "uniform"),  # single stage pairs, duplicate experts
    (16, 4, 200, 768, 512, 1, "zipf"),    # skewed segments: empty, tiny and oversized experts
])
def test_ffn_iq4xs_gemm(E, k, T, n_embd, n_ff, S, routing):
    ids = (synth.draw_ids_zipf(37, T, E, k, 1.1) if routing == "zipf"
           else np.random.default_rng(T + E + 2).integers(0, E, size=(T, k)).astype(np.int32))
    inp = synth.make_custom_ffn(271 + E, E, k, T, n_embd, n_ff, S, ids=ids, wtype=W)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    assert moe.last_stage_count() == 4
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_MFMA


def test_ffn_iq4xs_gemm_segments_at_tile_edges():
    """Expert segments of 0-200 rows around the 64- and 128-row tiles, one slot per token,
    every segment checked on its own."""
    seg = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200]
    ids = np.repeat(np.arange(len(seg), dtype=np.int32), seg)
    np.random.default_rng(6).shuffle(ids)
    ids = ids.reshape(-1, 1)
    E, T = len(seg), ids.shape[0]
    inp = synth.make_custom_ffn(281, E, 1, T, 256, 256, 1, ids=ids, wtype=W)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    g, ref = got.cpu().numpy(), oracle.ffn(inp)
    assert normwise(g, ref) <= TOL_MFMA
    for e in range(E):
        sel = ids[:, 0] == e
        if sel.any():
            assert normwise(g[sel], ref[sel]) <= TOL_MFMA, e


def test_ffn_iq4xs_gemm_large_grid_sampled():
    """64-row tiles with 2048 or more 8-wave tiles (256 weight rows per block)."""
    E, k, T, n_embd, n_ff = 128, 2, 2048, 512, 2048
    inp = synth.make_custom_ffn(291, E, k, T, n_embd, n_ff, 0, wtype=W)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    rows = np.array(sorted(set(np.random.default_rng(4).choice(T, 64, replace=False).tolist()) | {0, T - 1}))
    err = normwise(got.cpu().numpy()[rows], oracle.ffn(inp, token_rows=rows))
    assert err <= TOL_MFMA
    assert torch.isfinite(got).all()


def test_pps_full_size_segments():
    """E128 k8 PP4096 prefill with IQ4_XS experts (128-row tiles): the oracle runs on the
    tokens holding the first and last row of every 128-row stretch of every expert's
    segment, plus random tokens."""
    inp = synth.make_inputs("pps")
    got = run_ffn(upload_ffn(inp)).cpu().numpy()
    ids = inp["ids"]
    _, dst, bounds = oracle.row_ids(ids, inp["n_experts"], 1)
    k = ids.shape[1]
    pick = set(np.random.default_rng(3).choice(ids.shape[0], 32, replace=False).tolist())
    for e in range(inp["n_experts"]):
        lo, hi = int(bounds[e]), int(bounds[e + 1])
        for a in range(lo, hi, 128):
            pick.add(int(dst[a]) // k)
            pick.add(int(dst[min(a + 128, hi) - 1]) // k)
    rows = np.array(sorted(pick))
    err = normwise(got[rows], oracle.ffn(inp, token_rows=rows))
    print("pps normwise error %.3g over %d tokens" % (err, len(rows)))
    assert err <= TOL_MFMA
    assert np.isfinite(got).all()
