"""GPU parity of moe_router_topk (the step ahead of the op: ids and routing weights
from router logits) against the oracle: ids bit-exact, weights within 1e-6 of the
float64 softmax over the picks (float32 exp and division), bit-identical reruns."""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import oracle
import synth
from moe_testutil import TOL_FP32, dev_f32, normwise, run_ffn, upload_ffn

pytestmark = pytest.mark.gpu

TOL_W = 1e-6


def _check(lg, k):
    ids, w = moe.moe_router_topk(dev_f32(lg), k)
    torch.cuda.synchronize()
    rid, rw = oracle.router_topk(lg, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.abs(w.cpu().numpy().astype(np.float64) - rw).max() <= TOL_W
    return ids, w


@pytest.mark.parametrize("name", ["lite", "dec1", "dec8", "skew", "v3"])
def test_router_config_shapes(name):
    cfg = synth.CONFIGS[name]
    zs = cfg.zipf_s if cfg.routing == "zipf" else 0.0
    lg = synth.draw_router_logits(cfg.seed, cfg.n_tokens, cfg.n_experts, zs)
    _check(lg, cfg.n_used)


@pytest.mark.parametrize("T,E,k,seed", [
    (37, 1, 1, 1),        # one expert
    (50, 33, 33, 2),      # k = E, E not a multiple of 64
    (20, 64, 1, 3),
    (11, 1024, 32, 4),    # the largest expert count
    (9, 130, 70, 5),      # picks spill into a second register slot
    (3, 1000, 999, 6),
])
def test_router_random_shapes(T, E, k, seed):
    _check(synth.draw_router_logits(seed, T, E), k)


def test_router_ties_and_nan():
    rng = np.random.default_rng(8)
    lg = rng.integers(0, 3, size=(64, 100)).astype(np.float32)   # many equal logits
    _check(lg, 16)
    lg2 = synth.draw_router_logits(9, 16, 40)
    lg2[0, 5] = np.nan
    lg2[3, :] = np.nan
    lg2[3, 7] = -1.0
    ids, _ = _check(lg2, 4)
    assert ids.cpu().numpy()[3, 0] == 7


def test_router_non_finite_rows():
    """NaN strictly below -inf, all-NaN and all -inf rows (weight 1/k on every pick),
    +inf picks sharing the weight, and -0 equal to +0 (a tie: lower index first)."""
    nan, inf = np.nan, np.inf
    lg = np.zeros((8, 70), np.float32)
    lg[0, :6] = [nan, 1.0, 2.0, 3.0, 4.0, -inf]
    lg[0, 6:] = -inf
    lg[1, :] = nan
    lg[2, :] = -inf
    lg[2, 65] = nan
    lg[3, 1], lg[3, 66] = inf, inf
    lg[4, :] = -1.0
    lg[4, 3], lg[4, 2] = 0.0, -0.0
    lg[5, ::2] = nan
    lg[5, 1::2] = -inf
    lg[6] = synth.draw_router_logits(13, 1, 70)[0]
    lg[6, 64:] = nan
    lg[7, 0] = np.float32(1e-40)                # a subnormal above +0
    for k in (1, 3, 6, 70):
        ids, w = _check(lg, k)
    ids = ids.cpu().numpy()
    assert ids[0, :6].tolist() == [4, 3, 2, 1, 5, 6]
    assert ids[0, 69] == 0                        # the NaN comes after every -inf
    assert ids[4, :2].tolist() == [2, 3]          # -0 == +0: lower index first
    assert ids[7, 0] == 0


def test_router_empty_and_repeatable():
    ids, w = moe.moe_router_topk(torch.zeros((0, 16), dtype=torch.float32, device="cuda"), 4)
    assert ids.shape == (0, 4)
    lg = dev_f32(synth.draw_router_logits(10, 4096, 256))
    a = moe.moe_router_topk(lg, 8)
    for _ in range(9):
        b = moe.moe_router_topk(lg, 8)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_router_feeds_the_layer():
    """Router -> fused MoE layer on the device, against the oracle's router feeding the
    oracle's layer: the whole MoE FFN from logits without host involvement."""
    E, k, T, n_embd, n_ff, S = 16, 4, 24, 128, 96, 1
    lg = synth.draw_router_logits(12, T, E)
    rid, rw = oracle.router_topk(lg, k)
    inp = synth.make_custom_ffn(13, E, k, T, n_embd, n_ff, S, ids=rid)
    inp["route_w"] = rw.astype(np.float32)
    ref = oracle.ffn(inp)
    dv = upload_ffn(inp)
    dv["ids"], dv["route_w"] = moe.moe_router_topk(dev_f32(lg), k)
    for path in (moe.PATH_GEMM, moe.PATH_GEMV):
        got = run_ffn(dv, path=path)
        torch.cuda.synchronize()
        tol = 2e-2 if path == moe.PATH_GEMM else TOL_FP32
        assert normwise(got.cpu().numpy(), ref) <= tol, path
