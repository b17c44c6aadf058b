"""Capture into a HIP graph (torch.cuda.CUDAGraph is a HIP graph on ROCm) and replay:
the router and the fused MoE layer enqueue only kernels (no memset nodes, no host
reads), so a captured layer must give, on every replay, the bytes the eager call
gives. Replays are interleaved with the program's own eager work and syncs."""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import synth
from moe_testutil import dev_f32, run_ffn, upload_ffn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,path", [("lite", moe.PATH_AUTO), ("dec1", moe.PATH_AUTO),
                                       ("dec8", moe.PATH_GEMM)])
def test_graph_replays_match_eager(name, path):
    inp = synth.make_inputs(name)
    cfg = inp["cfg"]
    dv = upload_ffn(inp)
    T, k = inp["ids"].shape
    logits = dev_f32(synth.draw_router_logits(cfg.seed, T, cfg.n_experts))
    need = moe.moe_ffn_fused_workspace_size(dv["gate"], dv["shared"][0] if dv["shared"] else None,
                                            T, k, path=path)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    rw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, cfg.n_embd), dtype=torch.float32, device="cuda")

    def layer():   # router logits -> ids, weights -> MoE layer, all on the device
        moe.moe_router_topk(logits, k, ids=ids, route_w=rw)
        dv["ids"], dv["route_w"] = ids, rw
        run_ffn(dv, path=path, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # eager warm-up: kernel attributes, allocator
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = out.clone()
    ref_ids = ids.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for _ in range(5):
        out.fill_(float("nan"))
        ids.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids)
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
        scratch = torch.randn(1 << 20, device="cuda").sum()   # the program's own work
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
