"""GPU parity of the row-id pass (moe_row_ids) against the oracle: the three maps
of "CUDA: better MoE implementation", section 2.1, must match bit for bit."""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import oracle
import synth
from moe_testutil import dev_i32

pytestmark = pytest.mark.gpu


def _gpu_maps(ids, E, B):
    s1, dd, b = moe.moe_row_ids(dev_i32(ids), E, B)
    torch.cuda.synchronize()
    return s1.cpu().numpy(), dd.cpu().numpy(), b.cpu().numpy()


def _cfg_ids(name):
    cfg = synth.CONFIGS[name]
    if cfg.routing == "zipf":
        return synth.draw_ids_zipf(cfg.seed, cfg.n_tokens, cfg.n_experts, cfg.n_used, cfg.zipf_s), cfg
    return synth.draw_ids_uniform(cfg.seed, cfg.n_tokens, cfg.n_experts, cfg.n_used), cfg


@pytest.mark.parametrize("name", ["tiny", "lite", "dec1", "dec8", "skew", "v3"])
@pytest.mark.parametrize("B_is_k", [False, True])
def test_row_ids_configs_bit_exact(name, B_is_k):
    ids, cfg = _cfg_ids(name)
    B = cfg.n_used if B_is_k else 1
    got = _gpu_maps(ids, cfg.n_experts, B)
    ref = oracle.row_ids(ids, cfg.n_experts, B)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    assert got[2][-1] == cfg.n_tokens * cfg.n_used


@pytest.mark.parametrize("E,T,k,lo,hi,seed", [
    (1, 100, 1, 0, 1, 1),        # one expert
    (3, 50, 5, 0, 3, 2),         # n_used > n_experts: duplicates inside tokens
    (7, 33, 7, -2, 9, 3),        # out-of-range ids on both sides
    (512, 97, 12, 0, 512, 4),
    (1024, 40, 64, -1, 1025, 5), # the largest expert count, k not a specialised size
    (64, 3000, 12, 0, 64, 6),    # 36000 entries: the multi-workgroup pass
    (256, 9000, 8, -3, 260, 7),  # multi-workgroup with invalid ids
    (5, 1, 3, 0, 5, 8),          # a single token
    (64, 512, 8, -1, 65, 9),     # 4096 entries: the largest one-workgroup input (4 batches a wave)
    (1024, 1024, 4, 0, 1024, 10),  # 4096 entries over 1025 buckets: 17 buckets per lane in the scan
    (64, 4097, 1, 0, 64, 11),    # 4097 entries: the smallest multi-workgroup input
    (64, 20000, 8, -2, 66, 12),     # 160000 entries: more than 128 chunks (the scan over chunks runs)
    (1024, 40000, 4, -1, 1025, 13), # the same with the most buckets: the count pass's largest LDS
    (1, 150000, 1, 0, 1, 14),       # one expert: every entry in one bucket, across chunks
])
def test_row_ids_random_shapes(E, T, k, lo, hi, seed):
    ids = np.random.default_rng(seed).integers(lo, hi, size=(T, k)).astype(np.int32)
    for B in sorted({1, k}):
        got = _gpu_maps(ids, E, B)
        ref = oracle.row_ids(ids, E, B)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r)


def test_row_ids_empty():
    ids = np.zeros((0, 4), np.int32)
    b = moe.moe_row_ids(torch.zeros((0, 4), dtype=torch.int32, device="cuda"), 16)[2]
    torch.cuda.synchronize()
    assert np.array_equal(b.cpu().numpy(), oracle.row_ids(ids, 16, 1)[2])


def test_row_ids_scaled_2M_tokens_by_invariants():
    """T = 2^21, k = 8, E = 256 (16.7M entries): the oracle's enumeration is too slow
    at this size, so the maps are checked by the properties that define them
    uniquely: bounds = exclusive prefix of the per-expert counts, ids_dst a
    bijection whose segment e holds exactly the entries with id e in increasing
    order, ids_src1 = ids_dst // k; plus the oracle on a 4096-token prefix."""
    T, k, E = 1 << 21, 8, 256
    ids = synth.draw_ids_uniform(6, T, E, k)
    s1, dd, b = _gpu_maps(ids, E, 1)
    flat = ids.reshape(-1)
    cnt = np.bincount(flat, minlength=E)
    assert np.array_equal(b, np.concatenate([[0], np.cumsum(cnt)]))
    assert np.array_equal(dd, np.argsort(flat, kind="stable"))
    assert np.array_equal(s1, dd // k)
    small = ids[:4096]
    got = _gpu_maps(small, E, 1)
    for g, r in zip(got, oracle.row_ids(small, E, 1)):
        assert np.array_equal(g, r)


def test_row_ids_repeatable():
    ids, cfg = _cfg_ids("v3")
    first = _gpu_maps(ids, cfg.n_experts, 1)
    for _ in range(9):
        again = _gpu_maps(ids, cfg.n_experts, 1)
        for a, b in zip(first, again):
            assert np.array_equal(a, b)
