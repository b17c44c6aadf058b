"""GPU checks of moe_gather_rows (the src1 rows copied into expert order by the row-id
pass's first map): bit-exact against x[ids_src1] taken on the host with the oracle's maps
("CUDA: better MoE implementation", section 2.1: ids_src1 names the src1 row each position
of the expert-grouped buffer reads)."""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["skew", "v3"])
def test_gather_full_shapes_bit_exact(name):
    """The skewed PP4096 (Zipf ids) and the V3-shaped PP8192 inputs, the maps from the GPU
    row-id pass (bit-exact to the oracle's, checked here too), every gathered row compared."""
    cfg = synth.CONFIGS[name]
    T, k, E, K = cfg.n_tokens, cfg.n_used, cfg.n_experts, cfg.n_embd
    ids = (synth.draw_ids_zipf(cfg.seed, T, E, k, cfg.zipf_s) if cfg.routing == "zipf"
           else synth.draw_ids_uniform(cfg.seed, T, E, k))
    x = synth.gen.draw_x_bf16(cfg.seed, T, K)
    s1_ref, _, _ = oracle.row_ids(ids, E, 1)
    s1, _, _ = moe.moe_row_ids(torch.from_numpy(ids).cuda(), E)
    got = moe.moe_gather_rows(torch.from_numpy(x.view(np.int16)).cuda(), s1)
    torch.cuda.synchronize()
    assert np.array_equal(s1.cpu().numpy(), s1_ref)
    assert np.array_equal(got.cpu().numpy().view(np.uint16), x[s1_ref])


@pytest.mark.parametrize("K,dtype", [(17, np.uint16), (8, np.float32), (2048, np.uint16), (1, np.float32)])
def test_gather_row_sizes_and_invalid_indices(K, dtype):
    """Rows of 34 bytes (the 2-byte path), 32 and 8192 bytes (16-byte chunks, a tail of
    whole chunks), 4-byte float rows; indices -1 and src1_rows give zero rows."""
    rng = np.random.default_rng(K)
    rows, n = 37, 300
    if dtype == np.uint16:
        x = synth.f32_to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
        xt = torch.from_numpy(x.view(np.int16)).cuda()
    else:
        x = rng.standard_normal((rows, K)).astype(np.float32)
        xt = torch.from_numpy(x).cuda()
    idx = rng.integers(0, rows, size=n).astype(np.int32)
    idx[5], idx[77] = -1, rows
    got = moe.moe_gather_rows(xt, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    g = g.view(np.uint16) if dtype == np.uint16 else g
    ok = (idx >= 0) & (idx < rows)
    assert np.array_equal(g[ok], x[idx[ok]])
    assert np.all(g[~ok] == 0)


def test_gather_empty_and_repeatable():
    x = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    out = moe.moe_gather_rows(x, torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 64)
    cfg = synth.CONFIGS["lite"]
    xs = torch.from_numpy(synth.gen.draw_x_bf16(2, 512, 2048).view(np.int16)).cuda()
    s1, _, _ = moe.moe_row_ids(torch.from_numpy(synth.draw_ids_uniform(2, 512, 64, 6)).cuda(), cfg.n_experts)
    a = [moe.moe_gather_rows(xs, s1) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(a[0], b) for b in a[1:])
