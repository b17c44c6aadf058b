"""GPU parity of the quantized-activation path (the MMQ-style grouped GEMM: int8
activation codes with one float32 scale per 32-column block, Q8_0 experts, int8 MFMA
with the per-block scales applied in float32) against the oracle.

Bars:
  * the activation codes and scales (moe_quantize_act) are bit-exact: both sides take
    the float32 decisions of the format's definition;
  * mul_mat_id on quantized activations: within 1e-5 (normwise) of the oracle on the
    same codes -- each block's integer dot product is exact, only the float32 scale
    products and the block sum round;
  * the fused FFN: within 2e-3 of the oracle's quantized-activation FFN. The GPU's h
    (float32 sums, rounded to bf16) can differ from the oracle's in its last bit, and
    such an h can then round to a neighbouring code (one step of max|h|/127 in one
    element); a few such steps stay far below 2e-3. Both paths also stay within the
    2e-2 gate of the bf16 paths against the unquantized oracle.
"""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import oracle
import synth
from moe_testutil import TOL_MFMA, dev_bf16, dev_f32, dev_i32, normwise, run_ffn, upload_ffn

pytestmark = pytest.mark.gpu

TOL_Q_MMID = 1e-5
TOL_Q_FFN = 2e-3


def _x_with_edge_blocks(rows, K, seed):
    """bf16-exact activations: random rows plus blocks of zeros, blocks whose values sit
    on code ties (d = 4: x/4 = k + 1/2), a block with one huge and many tiny values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)).astype(np.float32) * rng.uniform(0.01, 30, size=(rows, 1)).astype(np.float32)
    blocks = [(r, b) for r in range(rows) for b in range(K // 32)]
    if len(blocks) > 1:
        x[blocks[0][0], 32 * blocks[0][1]:32 * blocks[0][1] + 32] = 0.0
    if len(blocks) > 2:
        tie = np.array([508.0] + [4.0 * (i + 0.5) for i in range(31)], np.float32)
        r, b = blocks[1]
        x[r, 32 * b:32 * b + 32] = tie * np.where(np.arange(32) % 2 == 0, 1, -1)
    if len(blocks) > 3:
        r, b = blocks[2]
        x[r, 32 * b:32 * b + 32] = np.float32(1e-3)
        x[r, 32 * b + 5] = np.float32(3e4)
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("rows,K", [(1, 32), (7, 96), (300, 2048), (4096, 7168)])
def test_quantize_act_bit_exact(rows, K):
    x = _x_with_edge_blocks(rows, K, rows + K)
    q, d = moe.moe_quantize_act(dev_bf16(x))
    torch.cuda.synchronize()
    rq, rd = oracle.quantize_act(x, "bf16")
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), rd.view(np.uint32))
    xf = synth.bf16_bits_to_f32(x) * np.float32(1.0001)          # float32 input, off the bf16 grid
    q, d = moe.moe_quantize_act(dev_f32(xf))
    torch.cuda.synchronize()
    rq, rd = oracle.quantize_act(xf, "f32")
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), rd.view(np.uint32))


@pytest.mark.parametrize("E,k,T,K,N,B_is_k,routing,bad", [
    (6, 3, 9, 96, 40, False, "uniform", True),      # K ends inside a stage; ragged N; invalid ids
    (16, 2, 50, 256, 300, True, "uniform", False),  # one src1 row per slot; several N tiles
    (4, 4, 300, 512, 520, False, "uniform", True),  # several M tiles per expert, partly filled sub-tiles
    (8, 2, 400, 1024, 256, False, "zipf", False),   # skewed segments: empty, tiny and oversized
    (3, 2, 1, 64, 64, False, "uniform", False),     # a single token
])
def test_mul_mat_id_q8act(E, k, T, K, N, B_is_k, routing, bad):
    ids = synth.draw_ids_zipf(3, T, E, k, 1.1) if routing == "zipf" else synth.draw_ids_uniform(3, T, E, k)
    if bad:
        ids[0, 0], ids[T - 1, k - 1] = -1, E + 2
    inp = synth.make_custom_mmid(K + N, E, k, T, K, N, ids=ids)
    B = k if B_is_k else 1
    x = _x_with_edge_blocks(T * B, K, T + K)
    w = moe.weights_from_numpy(inp["w_qs"], inp["w_d"])
    got = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), src1_rows_per_token=B, act_quant=1)
    gotw = moe.moe_mul_mat_id(w, dev_bf16(x), dev_i32(ids), route_w=dev_f32(inp["route_w"]),
                              src1_rows_per_token=B, act_quant=1)
    torch.cuda.synchronize()
    assert moe.last_stage_count() == 4   # row ids, quantize, int8 GEMM, reduce
    q, d = oracle.quantize_act(x, "bf16")
    ref = oracle.mul_mat_id_q8act(inp["w_qs"], inp["w_d"], q, d, ids, None, B)
    refw = oracle.mul_mat_id_q8act(inp["w_qs"], inp["w_d"], q, d, ids, inp["route_w"], B)
    g = got.cpu().numpy()
    assert normwise(g, ref) <= TOL_Q_MMID
    assert normwise(gotw.cpu().numpy(), refw) <= TOL_Q_MMID
    assert np.all(g[(ids < 0) | (ids >= E)] == 0.0)
    plain = oracle.mul_mat_id(inp["w_qs"], inp["w_d"], x, "bf16", ids, None, B)
    assert normwise(g, plain) <= TOL_MFMA


@pytest.mark.parametrize("E,k,T,n_embd,n_ff,S,routing", [
    (8, 2, 12, 96, 64, 0, "uniform"),       # K tails on both projections
    (8, 3, 40, 256, 160, 2, "uniform"),     # shared experts, ragged N tiles
    (6, 2, 400, 512, 768, 1, "zipf"),       # skewed segments, several M tiles
    (4, 6, 10, 64, 32, 1, "uniform"),       # n_used > n_experts: duplicate experts
])
def test_ffn_q8act_small(E, k, T, n_embd, n_ff, S, routing):
    ids = (synth.draw_ids_zipf(23, T, E, k, 1.1) if routing == "zipf"
           else np.random.default_rng(T * 31 + E).integers(0, E, size=(T, k)).astype(np.int32))
    inp = synth.make_custom_ffn(11 + E, E, k, T, n_embd, n_ff, S, ids=ids)
    got = run_ffn(upload_ffn(inp), act_quant=1).cpu().numpy()
    assert moe.last_stage_count() == 6   # row ids, quantize x, gate/up, quantize h, down, reduce
    err = normwise(got, oracle.ffn(inp, act_quant=True))
    print("q8act ffn error %.3g" % err)
    assert err <= TOL_Q_FFN
    assert normwise(got, oracle.ffn(inp)) <= TOL_MFMA


def test_ffn_q8act_lite_full():
    inp = synth.make_inputs("lite")
    got = run_ffn(upload_ffn(inp), act_quant=1).cpu().numpy()
    err = normwise(got, oracle.ffn(inp, act_quant=True))
    err_plain = normwise(got, oracle.ffn(inp))
    print("lite q8act error %.3g (vs unquantized %.3g)" % (err, err_plain))
    assert err <= TOL_Q_FFN
    assert err_plain <= TOL_MFMA


def test_ffn_q8act_skew_sampled_and_repeatable():
    inp = synth.make_inputs("skew")
    dv = upload_ffn(inp)
    outs = [run_ffn(dv, act_quant=1) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
    rows = np.unique(np.concatenate([np.arange(0, 4096, 37), [4095]]))
    got = outs[0].cpu().numpy()[rows]
    err = normwise(got, oracle.ffn(inp, token_rows=rows, act_quant=True))
    print("skew q8act error %.3g" % err)
    assert err <= TOL_Q_FFN


def test_ffn_q8act_decode_batch_takes_the_int8_gemm():
    """act_quant = 1 runs the int8 grouped GEMM for any batch, also where automatic
    selection would pick the GEMV path."""
    inp = synth.make_inputs("dec8")
    got = run_ffn(upload_ffn(inp), act_quant=1).cpu().numpy()
    assert moe.last_stage_count() == 6
    assert normwise(got, oracle.ffn(inp, act_quant=True)) <= TOL_Q_FFN
