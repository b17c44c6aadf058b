"""GPU parity of moe_mul_mat_id and moe_ffn_fused against the fp64 oracle.

Tolerances (normwise max relative error per output tensor, as the op's accuracy
contract states): 2e-2 on the bf16-MFMA grouped GEMM path, 1e-5 on the fp32 paths
(fp32 mul_mat_id and the fp32 GEMV decode path). Expected errors are about 2e-3 and
1e-6; the gates leave room for rounding-order differences only.
"""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import oracle
import synth
from moe_testutil import (TOL_FP32, TOL_MFMA, dev_bf16, dev_f32, dev_i32, normwise, run_ffn,
                          upload_ffn, upload_mmid)

pytestmark = pytest.mark.gpu


def _tol(path):
    return TOL_MFMA if path == moe.PATH_GEMM else TOL_FP32


# ------------------------------------------------------------------ mul_mat_id

def test_tiny_fp32_mul_mat_id():
    inp = synth.make_inputs("tiny")
    dv = upload_mmid(inp)
    per_slot = moe.moe_mul_mat_id(dv["w"], dv["x"], dv["ids"])
    weighted = moe.moe_mul_mat_id(dv["w"], dv["x"], dv["ids"], route_w=dv["route_w"])
    torch.cuda.synchronize()
    ref = oracle.mul_mat_id(inp["w"], None, inp["x"], "f32", inp["ids"])
    refw = oracle.mul_mat_id(inp["w"], None, inp["x"], "f32", inp["ids"], inp["route_w"])
    assert per_slot.shape == (16, 2, 32)
    assert normwise(per_slot.cpu().numpy(), ref) <= TOL_FP32
    assert normwise(weighted.cpu().numpy(), refw) <= TOL_FP32


@pytest.mark.parametrize("path", [moe.PATH_GEMM, moe.PATH_GEMV])
@pytest.mark.parametrize("E,k,T,K,N,B_is_k,bad", [
    (6, 3, 9, 96, 40, False, False),     # K tail (96 = 64 + 32), ragged N
    (6, 3, 9, 96, 40, True, True),       # one src1 row per slot, invalid ids
    (16, 2, 50, 256, 300, False, False), # several N tiles plus a ragged one
    (4, 4, 60, 128, 64, False, True),    # k = E, several M tiles per expert
    (5, 2, 7, 96, 45, False, False),     # odd N and K/32: rows of scales start at 2 mod 4
    (8, 2, 64, 512, 200, False, True),   # 64-row tiles with scale groups (K % 512 == 0)
])
def test_q8_mul_mat_id(path, E, k, T, K, N, B_is_k, bad):
    if path == moe.PATH_GEMV and T * k > 256:
        pytest.skip("GEMV path bound")
    rng = np.random.default_rng(E * 1000 + T)
    ids = synth.draw_ids_uniform(3, T, E, k)
    if bad:
        ids[0, 0], ids[T // 2, k - 1] = -1, E + 3
    inp = synth.make_custom_mmid(7, E, k, T, K, N, ids=ids)
    B = k if B_is_k else 1
    x = synth.f32_to_bf16_bits(rng.standard_normal((T * B, K)).astype(np.float32))
    w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
    got = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), src1_rows_per_token=B, path=path)
    gotw = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), route_w=dev_f32(inp["route_w"]),
                              src1_rows_per_token=B, path=path)
    torch.cuda.synchronize()
    ref = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, None, B)
    refw = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, inp["route_w"], B)
    g = got.cpu().numpy()
    assert normwise(g, ref) <= _tol(path)
    assert normwise(gotw.cpu().numpy(), refw) <= _tol(path)
    invalid = (ids < 0) | (ids >= E)
    assert np.all(g[invalid] == 0.0)


# Shapes whose segments average more than 64 rows take 128-row tiles: the wide
# kernel (K % 64 == 0; scale groups of four stages when K % 256 == 0, else one scale
# word per stage) or, for other K, the 128-row kernel with 256-row N tiles.
@pytest.mark.parametrize("E,k,T,K,N,bad", [
    (3, 2, 200, 192, 600, False),   # scale word per stage, N ragged over 512-row tiles
    (5, 3, 300, 512, 520, True),    # scale groups, ragged N, partly filled sub-tiles, bad ids
    (2, 2, 150, 96, 130, False),    # K % 64 != 0: the 128-row fallback
])
def test_q8_mul_mat_id_tall_tiles(E, k, T, K, N, bad):
    ids = synth.draw_ids_uniform(17, T, E, k)
    if bad:
        ids[3, 1], ids[T - 1, 0] = -2, E
    inp = synth.make_custom_mmid(19, E, k, T, K, N, ids=ids)
    x = synth.f32_to_bf16_bits(np.random.default_rng(T).standard_normal((T, K)).astype(np.float32))
    w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
    got = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), path=moe.PATH_GEMM)
    gotw = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), route_w=dev_f32(inp["route_w"]),
                              path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    ref = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, None, 1)
    refw = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, inp["route_w"], 1)
    g = got.cpu().numpy()
    assert normwise(g, ref) <= TOL_MFMA
    assert normwise(gotw.cpu().numpy(), refw) <= TOL_MFMA
    invalid = (ids < 0) | (ids >= E)
    assert np.all(g[invalid] == 0.0)


def test_q8_mul_mat_id_many_chunks():
    """160000 rows (T = 20000, k = 8, E = 64): more than 128 chunks, so the row-id pass
    runs its scan over chunks and its place kernel writes the bounds and the tile table
    the GEMM reads; invalid ids included."""
    E, k, T, K, N = 64, 8, 20000, 64, 72
    ids = synth.draw_ids_uniform(23, T, E, k)
    ids[5, 2], ids[T - 3, 7] = -1, E + 1
    inp = synth.make_custom_mmid(29, E, k, T, K, N, ids=ids)
    x = synth.f32_to_bf16_bits(np.random.default_rng(31).standard_normal((T, K)).astype(np.float32))
    w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
    got = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), route_w=dev_f32(inp["route_w"]),
                             path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    ref = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, inp["route_w"], 1)
    assert normwise(got.cpu().numpy(), ref) <= TOL_MFMA


# Segment lengths around the 128-row tile and its last-tile allowance of 32 more rows
# (128-row tiles, the last one holding up to 160): 160 rows make one tile, 161 two,
# 288 two, 289 three. One expert per length, in a seeded token order, k = 1.
_SEG_ROWS = [0, 1, 31, 32, 33, 127, 128, 129, 159, 160, 161, 255, 256, 257, 287, 288, 289, 416]


def _ids_with_segments(seed):
    ids = np.repeat(np.arange(len(_SEG_ROWS), dtype=np.int32), _SEG_ROWS)
    np.random.default_rng(seed).shuffle(ids)
    return ids.reshape(-1, 1)


@pytest.mark.parametrize("wtype,K,N", [("q8_0", 256, 200), ("q8_0", 192, 72), ("mxfp4", 256, 200)])
def test_mul_mat_id_segment_lengths_at_tile_edges(wtype, K, N):
    ids = _ids_with_segments(41)
    E, T = len(_SEG_ROWS), ids.shape[0]
    inp = synth.make_custom_mmid(43, E, 1, T, K, N, wtype=wtype, ids=ids)
    x = synth.f32_to_bf16_bits(np.random.default_rng(47).standard_normal((T, K)).astype(np.float32))
    w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
    got = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), route_w=dev_f32(inp["route_w"]),
                             path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    ref = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, inp["route_w"], 1)
    g = got.cpu().numpy()
    assert normwise(g, ref) <= TOL_MFMA
    # every segment, the last tile's rows included, on its own
    for e in range(E):
        sel = ids[:, 0] == e
        if sel.any():
            assert normwise(g[sel], ref[sel]) <= TOL_MFMA, e


@pytest.mark.parametrize("wtype", ["q8_0", "mxfp4"])
def test_ffn_segment_lengths_at_tile_edges(wtype):
    ids = _ids_with_segments(53)
    E, T = len(_SEG_ROWS), ids.shape[0]
    inp = synth.make_custom_ffn(59, E, 1, T, 256, 192, 1, ids=ids, wtype=wtype)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    g, ref = got.cpu().numpy(), oracle.ffn(inp)
    assert normwise(g, ref) <= TOL_MFMA
    for e in range(E):
        sel = ids[:, 0] == e
        if sel.any():
            assert normwise(g[sel], ref[sel]) <= TOL_MFMA, e


# ------------------------------------------------------------------------- FFN

@pytest.mark.parametrize("path", [moe.PATH_GEMM, moe.PATH_GEMV])
@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S", [
    (8, 2, 12, 96, 64, 0),       # K tails on both projections
    (8, 3, 20, 128, 96, 2),      # shared experts, ragged N tiles
    (32, 4, 8, 256, 160, 1),
    (4, 6, 10, 64, 32, 1),       # n_used > n_experts: duplicate experts inside tokens
    (16, 1, 1, 320, 192, 2),     # a single token
    (8, 2, 24, 512, 160, 1),     # gate/up with scale groups on 64-row tiles, down without
])
def test_ffn_small_shapes(path, E, k, T, n_embd, n_ff, S):
    if path == moe.PATH_GEMV and T * k > 256:
        pytest.skip("GEMV path bound")
    ids = np.random.default_rng(T * 31 + E).integers(0, E, size=(T, k)).astype(np.int32)
    inp = synth.make_custom_ffn(11 + E, E, k, T, n_embd, n_ff, S, ids=ids)
    got = run_ffn(upload_ffn(inp), path=path)
    torch.cuda.synchronize()
    if path == moe.PATH_GEMM:
        assert moe.last_stage_count() == 4   # row ids, gate/up, down, reduce
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= _tol(path)


@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S,routing", [
    (4, 2, 300, 256, 320, 1, "uniform"),   # gate/up with scale groups, down with words, ragged N
    (6, 2, 400, 512, 768, 2, "zipf"),      # skewed segments: empty, tiny and oversized experts
])
def test_ffn_tall_tiles(E, k, T, n_embd, n_ff, S, routing):
    ids = (synth.draw_ids_zipf(23, T, E, k, 1.1) if routing == "zipf"
           else synth.draw_ids_uniform(23, T, E, k))
    inp = synth.make_custom_ffn(29, E, k, T, n_embd, n_ff, S, ids=ids)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_MFMA


def test_ffn_invalid_ids_and_shared_width():
    """Out-of-range ids contribute nothing; shared experts of a different width."""
    E, k, T, n_embd, n_ff = 8, 3, 24, 128, 64
    ids = synth.draw_ids_uniform(5, T, E, k)
    ids[1, 0], ids[7, 2], ids[20, 1] = -5, E, 1 << 20
    inp = synth.make_custom_ffn(5, E, k, T, n_embd, n_ff, 0, ids=ids)
    sh = synth.make_custom_ffn(6, 2, 1, T, n_embd, 96, 0)
    for n in ("gate", "up", "down"):
        inp["sh_" + n + "_qs"], inp["sh_" + n + "_d"] = sh[n + "_qs"], sh[n + "_d"]
    ref = oracle.ffn(inp)
    dv = upload_ffn(inp)
    for path in (moe.PATH_GEMM, moe.PATH_GEMV):
        got = run_ffn(dv, path=path)
        torch.cuda.synchronize()
        assert normwise(got.cpu().numpy(), ref) <= _tol(path), path


@pytest.mark.parametrize("S", [0, 1])
@pytest.mark.parametrize("which", ["some", "all"])
def test_ffn_gemv_invalid_ids(S, which):
    """Decode-sized batches (the GEMV path; without shared experts here the down launch
    also does the weighted reduce): out-of-range ids contribute nothing; with every id
    out of range the routed part is zero and only the shared experts remain."""
    E, k, T, n_embd, n_ff = 8, 4, 6, 192, 128
    ids = synth.draw_ids_uniform(9, T, E, k)
    if which == "some":
        ids[0, 1], ids[3, 0], ids[5, 3] = -1, E, 1 << 30
    else:
        ids[:] = -7
    inp = synth.make_custom_ffn(21, E, k, T, n_embd, n_ff, S, ids=ids)
    ref = oracle.ffn(inp)
    dv = upload_ffn(inp)
    for path in (moe.PATH_GEMV, moe.PATH_GEMM):
        got = run_ffn(dv, path=path)
        torch.cuda.synchronize()
        g = got.cpu().numpy()
        if which == "all" and S == 0:
            assert np.all(g == 0.0), path
        else:
            assert normwise(g, ref) <= _tol(path), path


# Decode-sized batches whose routed experts plus shared experts fit two per wave run the
# down projection and the weighted reduce in one launch (a block owns a chunk of output
# rows for every expert and sums the slots through LDS). The cases vary the shared
# experts (several tokens, a width of their own), output widths that leave a short last
# chunk of rows, and two experts per wave.
@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S,n_ff_sh", [
    (4, 2, 3, 224, 96, 2, 96),       # shared experts on three tokens, one row per block
    (6, 2, 2, 1120, 160, 1, 224),    # shared width of its own; 3-row chunks, last one short
    (16, 8, 1, 2624, 256, 0, 0),     # eight experts, two per wave; 6-row chunks, last one short
    (8, 4, 2, 640, 1056, 0, 0),      # K = 1056: two K pieces, the second mostly past K
])
def test_ffn_gemv_fused_reduce(E, k, T, n_embd, n_ff, S, n_ff_sh):
    ids = np.stack([np.random.default_rng(100 + t).permutation(E)[:k] for t in range(T)]).astype(np.int32)
    inp = synth.make_custom_ffn(41 + E, E, k, T, n_embd, n_ff, 0, ids=ids)
    if S:
        sh = synth.make_custom_ffn(43, S, 1, T, n_embd, n_ff_sh, 0)
        for n in ("gate", "up", "down"):
            inp["sh_" + n + "_qs"], inp["sh_" + n + "_d"] = sh[n + "_qs"], sh[n + "_d"]
    ref = oracle.ffn(inp)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMV)
    torch.cuda.synchronize()
    assert moe.last_stage_count() == 2   # gate/up GEMV, down GEMV with the reduce
    assert normwise(got.cpu().numpy(), ref) <= TOL_FP32


def test_lite_full():
    inp = synth.make_inputs("lite")
    got = run_ffn(upload_ffn(inp))
    torch.cuda.synchronize()
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    print("lite normwise error %.3g" % err)
    assert err <= TOL_MFMA


@pytest.mark.parametrize("name", ["dec1", "dec8"])
@pytest.mark.parametrize("path", [moe.PATH_AUTO, moe.PATH_GEMM])
def test_decode_full(name, path):
    inp = synth.make_inputs(name)
    got = run_ffn(upload_ffn(inp), path=path)
    torch.cuda.synchronize()
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    print("%s path %d normwise error %.3g" % (name, path, err))
    assert err <= (TOL_FP32 if path == moe.PATH_AUTO else TOL_MFMA)


def _sample_tokens(ids, n, seed):
    """Tokens for sampled checks: random ones plus the first tokens of the largest
    and smallest expert segments and the first and last token."""
    T = ids.shape[0]
    rng = np.random.default_rng(seed)
    cnt = np.bincount(ids.ravel()[ids.ravel() >= 0])
    pick = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    for e in (int(np.argmax(cnt)), int(np.argmin(np.where(cnt > 0, cnt, 1 << 30)))):
        pick.add(int(np.nonzero((ids == e).any(axis=1))[0][0]))
    return np.array(sorted(pick))


def test_skew_full():
    """Zipf-skewed PP4096 layer (empty, tiny and oversized expert segments), every
    token compared."""
    inp = synth.make_inputs("skew")
    got = run_ffn(upload_ffn(inp))
    torch.cuda.synchronize()
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    print("skew normwise error %.3g" % err)
    assert err <= TOL_MFMA


def _segment_tokens(ids, n_experts, block=128):
    """Tokens of the first and last row of every block-row stretch of every expert
    segment, in the row-id order (token, then slot): every M tile of 64 or 128 rows of
    every expert, its first and its last, holds a row of one of these tokens."""
    _, dst, bounds = oracle.row_ids(ids, n_experts, 1)
    k = ids.shape[1]
    pick = set()
    for e in range(n_experts):
        lo, hi = int(bounds[e]), int(bounds[e + 1])
        for a in range(lo, hi, block):
            b = min(a + block, hi) - 1
            pick.add(int(dst[a]) // k)
            pick.add(int(dst[b]) // k)
    return pick


def test_v3_full_size_stratified():
    """DeepSeek-V3-shaped PP8192 layer. The oracle runs on the tokens holding the first
    and last row of every 128-row stretch of every expert's segment (so every M tile of
    every expert, including each expert's partly filled last tile, has rows checked),
    plus random tokens; the shared expert is part of every token's output."""
    inp = synth.make_inputs("v3")
    dv = upload_ffn(inp)
    got = run_ffn(dv).cpu().numpy()
    rows = _segment_tokens(inp["ids"], 256) | set(_sample_tokens(inp["ids"], 64, 2).tolist())
    rows = np.array(sorted(rows))
    ref = oracle.ffn(inp, token_rows=rows)
    err = normwise(got[rows], ref)
    print("v3 normwise error %.3g over %d tokens" % (err, len(rows)))
    assert len(rows) > 500
    assert err <= TOL_MFMA
    assert np.isfinite(got).all()


@pytest.mark.parametrize("T", [1, 8])
def test_v3_shaped_decode_wide(T):
    """Decode batches of a DeepSeek-V3-shaped layer (n_embd 7168 > 4096) on the GEMV
    path's block kernel for widths past the wave kernels' 4096: automatic selection
    takes it for one token, and it is forced for eight. Only the experts the batch
    routes to are drawn (nothing reads the others)."""
    inp = synth.make_custom_ffn(71 + T, 256, 8, T, 7168, 2048, 1, touched_only=True)
    assert moe.moe_select_path(T, 8, 256, 7168) == (moe.PATH_GEMV if T == 1 else moe.PATH_GEMM)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMV)
    torch.cuda.synchronize()
    assert moe.last_stage_count() == 3   # gate/up GEMV, down GEMV, reduce
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    print("v3-shaped decode T=%d normwise error %.3g" % (T, err))
    assert err <= TOL_FP32


@pytest.mark.parametrize("T", [11, 16, 42])
def test_lite_widths_gemv_block_kernel(T):
    """DeepSeek-Lite-shaped layer (shared experts included) at batches of 64 < T*k <=
    256 slots: the GEMV path (forced; automatic selection takes the grouped GEMM here)
    past the wave kernels' 64 slots runs the block kernel."""
    inp = synth.make_custom_ffn(90 + T, 64, 6, T, 2048, 1408, 2, touched_only=True)
    assert moe.moe_select_path(T, 6, 64, 2048) == moe.PATH_GEMM
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMV)
    torch.cuda.synchronize()
    assert moe.last_stage_count() == 3
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    print("lite widths T=%d (%d slots) normwise error %.3g" % (T, 6 * T, err))
    assert err <= TOL_FP32


@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S", [
    (64, 6, 8, 2048, 1408, 2),    # Lite-shaped, 48 slots: shared units split in rows and run first
    (64, 6, 10, 2048, 1408, 2),   # 60 slots: shared units split, in the usual order
    (32, 4, 5, 2880, 2880, 1),    # odd T: three passes of two tokens per shared unit
    (16, 2, 3, 512, 256, 3),      # three shared experts, two passes each
])
def test_ffn_gemv_shared_units_split(E, k, T, n_embd, n_ff, S):
    """Wave-kernel GEMV with shared experts over several tokens: a shared unit serves
    every token in several passes, so it gets fewer rows than a routed unit (and, up
    to 8 tokens, the first waves). Every output row compared with the oracle."""
    inp = synth.make_custom_ffn(130 + T, E, k, T, n_embd, n_ff, S, touched_only=True)
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMV)
    torch.cuda.synchronize()
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    print("gemv shared split E%d k%d T%d S%d normwise error %.3g" % (E, k, T, S, err))
    assert err <= TOL_FP32


# ------------------------------------------------------------------------- MXFP4 experts
# GEMV path only (n_tokens * n_used <= 64, widths <= 4096). Weights are exact (E2M1 code
# times a power of two); bf16 activations meet them in bf16 pair dot products with fp32
# accumulation, fp32 activations (the down projection's h) in fp32 FMAs.

@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S", [
    (8, 2, 1, 2880, 2880, 0),     # single token: register rows; K = 2880 ends inside the second piece
    (8, 2, 1, 512, 256, 2),       # shared experts, fused reduce (2 + 2 units)
    (16, 4, 6, 448, 1056, 1),     # several tokens: LDS ring, two slots per pass; 17 units: separate reduce
    (4, 3, 5, 2048, 2080, 0),     # duplicate experts inside tokens; K exactly one piece / just past it
])
def test_ffn_mxfp4_gemv(E, k, T, n_embd, n_ff, S):
    ids = np.random.default_rng(T * 7 + E).integers(0, E, size=(T, k)).astype(np.int32)
    inp = synth.make_custom_ffn(51 + E, E, k, T, n_embd, n_ff, S, ids=ids, wtype="mxfp4")
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMV)
    torch.cuda.synchronize()
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_FP32


def test_ffn_mxfp4_extreme_scales_and_invalid_ids():
    """Scale byte 0 (the subnormal 2^-127) and large scales, plus out-of-range ids."""
    E, k, T, n_embd, n_ff = 6, 2, 3, 256, 128
    ids = synth.draw_ids_uniform(4, T, E, k)
    ids[1, 0] = -2
    ids[2, 1] = E + 5
    inp = synth.make_custom_ffn(61, E, k, T, n_embd, n_ff, 1, ids=ids, wtype="mxfp4")
    inp["gate_d"][0, :, 0] = 0
    inp["up_d"][1, ::3, 2] = 140
    inp["down_d"][2, 5, :] = 0
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMV)
    torch.cuda.synchronize()
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_FP32


@pytest.mark.parametrize("E,k,T,K,N,B_is_k,bad", [
    (6, 3, 9, 96, 40, False, True),      # one 2048 piece, mostly past K; invalid ids
    (8, 4, 5, 3008, 70, True, False),    # one src1 row per slot, K in the second piece
])
def test_mxfp4_mul_mat_id_gemv(E, k, T, K, N, B_is_k, bad):
    rng = np.random.default_rng(E * 100 + T)
    ids = synth.draw_ids_uniform(5, T, E, k)
    if bad:
        ids[0, 0], ids[T - 1, k - 1] = -1, E + 1
    inp = synth.make_custom_mmid(17, E, k, T, K, N, wtype="mxfp4", ids=ids)
    B = k if B_is_k else 1
    x = synth.f32_to_bf16_bits(rng.standard_normal((T * B, K)).astype(np.float32))
    w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
    assert w.type == moe.MOE_MXFP4
    got = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), src1_rows_per_token=B)
    gotw = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), route_w=dev_f32(inp["route_w"]),
                              src1_rows_per_token=B)
    torch.cuda.synchronize()
    ref = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, None, B)
    refw = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, inp["route_w"], B)
    g = got.cpu().numpy()
    assert normwise(g, ref) <= TOL_FP32
    assert normwise(gotw.cpu().numpy(), refw) <= TOL_FP32
    assert np.all(g[(ids < 0) | (ids >= E)] == 0.0)


@pytest.mark.parametrize("T,want_gemm", [(8, False), (12, True)])
def test_mxfp4_automatic_path_bound(T, want_gemm):
    """MXFP4 experts take the GEMV automatically up to 32 slots, the grouped GEMM
    beyond (GPT-OSS-shaped layer, n_used 4)."""
    inp = synth.make_custom_ffn(140 + T, 32, 4, T, 640, 512, 0, wtype="mxfp4", touched_only=True)
    got = run_ffn(upload_ffn(inp))
    torch.cuda.synchronize()
    stages = moe.last_stage_count()
    assert (stages == 4) == want_gemm   # GEMM: row ids, gate/up, down, reduce
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    assert err <= (TOL_MFMA if want_gemm else TOL_FP32)


@pytest.mark.parametrize("name", ["dec1x", "dec8x"])
def test_decode_mxfp4_full(name):
    inp = synth.make_inputs(name)
    got = run_ffn(upload_ffn(inp))
    torch.cuda.synchronize()
    err = normwise(got.cpu().numpy(), oracle.ffn(inp))
    print("%s normwise error %.3g" % (name, err))
    assert err <= TOL_FP32


# MXFP4 on the grouped GEMM: weights are exact in bf16, so the error is that of the bf16
# activations and the bf16 h, as on the Q8_0 GEMM path.
@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S,routing", [
    (8, 2, 40, 256, 192, 1, "uniform"),   # 64-row tiles; down K = 192 ends inside a stage; ragged N
    (4, 2, 300, 512, 160, 0, "uniform"),  # 128-row tiles; down K = 160
    (6, 3, 100, 96, 64, 2, "uniform"),    # single partial stages both ways, duplicate experts
    (16, 4, 200, 384, 224, 1, "zipf"),    # skewed segments: empty, tiny and oversized experts
])
def test_ffn_mxfp4_gemm(E, k, T, n_embd, n_ff, S, routing):
    ids = (synth.draw_ids_zipf(33, T, E, k, 1.1) if routing == "zipf"
           else np.random.default_rng(T + E).integers(0, E, size=(T, k)).astype(np.int32))
    inp = synth.make_custom_ffn(71 + E, E, k, T, n_embd, n_ff, S, ids=ids, wtype="mxfp4")
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    assert moe.last_stage_count() == 4
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_MFMA


def _odd_offset_scales(w):
    """The same weights with the scale bytes moved to an odd address (a view one byte
    into a larger buffer)."""
    flat = w.scales.reshape(-1)
    buf = torch.empty(flat.numel() + 1, dtype=torch.uint8, device=flat.device)
    buf[1:].copy_(flat)
    return moe.Weights(w.data, buf[1:].view(w.scales.shape))


def test_ffn_mxfp4_gemm_128_row_tiles_both_kernels():
    # 128-row tiles with K % 64 == 0 run the wide kernel when the scale rows start at even
    # addresses, the narrow one otherwise; both take the same k groups in the same order
    E, k, T, n_embd, n_ff = 4, 2, 300, 512, 256
    ids = synth.draw_ids_uniform(12, T, E, k)
    inp = synth.make_custom_ffn(93, E, k, T, n_embd, n_ff, 1, ids=ids, wtype="mxfp4")
    dv = upload_ffn(inp)
    wide = run_ffn(dv, path=moe.PATH_GEMM)
    odd = dict(dv)
    for n in ("gate", "up", "down"):
        odd[n] = _odd_offset_scales(dv[n])
        assert odd[n].scales.data_ptr() % 2 == 1
    odd["shared"] = [_odd_offset_scales(w) for w in dv["shared"]]
    narrow = run_ffn(odd, path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    ref = oracle.ffn(inp)
    assert normwise(wide.cpu().numpy(), ref) <= TOL_MFMA
    assert normwise(narrow.cpu().numpy(), ref) <= TOL_MFMA
    assert torch.equal(wide, narrow)


def test_ffn_mxfp4_gemm_invalid_ids_and_scale_zero():
    E, k, T, n_embd, n_ff = 8, 2, 70, 128, 96
    ids = synth.draw_ids_uniform(8, T, E, k)
    ids[3, 0], ids[40, 1], ids[69, 0] = -1, E, 1 << 20
    inp = synth.make_custom_ffn(81, E, k, T, n_embd, n_ff, 1, ids=ids, wtype="mxfp4")
    inp["gate_d"][2, :, 1] = 0          # scale 2^-127: those blocks contribute ~nothing
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    assert normwise(got.cpu().numpy(), oracle.ffn(inp)) <= TOL_MFMA


@pytest.mark.parametrize("E,k,T,K,N,B_is_k", [(6, 3, 50, 96, 45, False), (8, 2, 200, 640, 200, True)])
def test_mxfp4_mul_mat_id_gemm(E, k, T, K, N, B_is_k):
    rng = np.random.default_rng(E + T)
    ids = synth.draw_ids_uniform(6, T, E, k)
    ids[1, 0] = -3
    inp = synth.make_custom_mmid(19, E, k, T, K, N, wtype="mxfp4", ids=ids)
    B = k if B_is_k else 1
    x = synth.f32_to_bf16_bits(rng.standard_normal((T * B, K)).astype(np.float32))
    w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
    got = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), src1_rows_per_token=B, path=moe.PATH_GEMM)
    gotw = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), route_w=dev_f32(inp["route_w"]),
                              src1_rows_per_token=B, path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    ref = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, None, B)
    refw = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, inp["route_w"], B)
    g = got.cpu().numpy()
    assert normwise(g, ref) <= TOL_MFMA
    assert normwise(gotw.cpu().numpy(), refw) <= TOL_MFMA
    assert np.all(g[(ids < 0) | (ids >= E)] == 0.0)


def test_ppx_full_size_sampled():
    """GPT-OSS-20B-shaped PP4096 prefill with MXFP4 experts (128-row tiles)."""
    inp = synth.make_inputs("ppx")
    got = run_ffn(upload_ffn(inp))
    torch.cuda.synchronize()
    assert moe.last_stage_count() == 4
    rows = _sample_tokens(inp["ids"], 96, 2)
    err = normwise(got.cpu().numpy()[rows], oracle.ffn(inp, token_rows=rows))
    print("ppx sampled normwise error %.3g" % err)
    assert err <= TOL_MFMA
    assert torch.isfinite(got).all()


def test_ffn_mxfp4_gemm_large_grid_sampled():
    """64-row tiles with a grid of 2048 or more 8-wave tiles: gate/up runs 256 weight
    rows per block with a three-slot ring; down (few N tiles) stays on 4 waves."""
    E, k, T, n_embd, n_ff = 128, 2, 2048, 512, 2048
    inp = synth.make_custom_ffn(91, E, k, T, n_embd, n_ff, 0, wtype="mxfp4")
    got = run_ffn(upload_ffn(inp), path=moe.PATH_GEMM)
    torch.cuda.synchronize()
    rows = _sample_tokens(inp["ids"], 64, 3)
    err = normwise(got.cpu().numpy()[rows], oracle.ffn(inp, token_rows=rows))
    assert err <= TOL_MFMA
    assert torch.isfinite(got).all()
