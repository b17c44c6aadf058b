"""moe_ffn_fused_noalloc (the fused FFN on the library's fixed scratch array, for
callers that cannot allocate) against moe_ffn_fused with a caller workspace: the
same kernels on the same inputs, so the outputs must be bit-identical. Two calls in a
row on each path, the second with a smaller batch, so the second runs on whatever the
first left in the array. A call that needs more scratch than the array holds is
refused with MOE_ELIMIT and leaves its output untouched."""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import synth
from moe_testutil import upload_ffn

pytestmark = pytest.mark.gpu


def _same_bytes(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _both(dv, path):
    T = dv["ids"].shape[0]
    ref = moe.moe_ffn_fused(dv["gate"], dv["up"], dv["down"], dv["x"], dv["ids"], dv["route_w"],
                            shared=dv["shared"], path=path)
    out = torch.full((T, dv["x"].shape[1]), np.nan, dtype=torch.float32, device="cuda")
    got = moe.moe_ffn_fused_noalloc(dv["gate"], dv["up"], dv["down"], dv["x"], dv["ids"], dv["route_w"],
                                    shared=dv["shared"], path=path, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    return ref, got


@pytest.mark.parametrize("path", [moe.PATH_GEMM, moe.PATH_GEMV])
def test_noalloc_matches_workspace_call_twice(path):
    big = synth.make_custom_ffn(31, 16, 4, 60 if path == moe.PATH_GEMM else 40, 512, 384, 1)
    small = synth.make_custom_ffn(32, 16, 4, 9, 512, 384, 1)
    for inp in (big, small):
        ref, got = _both(upload_ffn(inp), path)
        assert torch.isfinite(got).all()
        assert _same_bytes(got, ref)


def test_noalloc_lite_then_decode():
    """The DeepSeek-Lite-shaped PP512 layer (about 45 MB of scratch), then a decode batch
    of the GPT-OSS-20B shape on the same array."""
    for name in ("lite", "dec8"):
        ref, got = _both(upload_ffn(synth.make_inputs(name)), moe.PATH_AUTO)
        assert _same_bytes(got, ref), name


def test_noalloc_refuses_calls_beyond_the_array():
    inp = synth.make_custom_ffn(33, 8, 8, 4096, 512, 1024, 0, touched_only=True)
    dv = upload_ffn(inp)
    need = moe.moe_ffn_fused_workspace_size(dv["gate"], None, 4096, 8)
    assert need > moe.NOALLOC_SCRATCH_BYTES
    out = torch.full((4096, 512), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_ffn_fused_noalloc(dv["gate"], dv["up"], dv["down"], dv["x"], dv["ids"], dv["route_w"],
                                  out=out)
    assert ei.value.status == moe.MOE_ELIMIT
    assert "scratch" in moe.last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


@pytest.mark.parametrize("name,path", [("dec8", moe.PATH_AUTO), ("lite", moe.PATH_GEMM)])
def test_noalloc_under_graph_capture(name, path):
    """The callers it is for: the call captured into a HIP graph (no allocation happens
    during capture) and replayed five times, with eager writes to the output and syncs
    between replays; every replay must reproduce the workspace call's bytes."""
    dv = upload_ffn(synth.make_inputs(name))
    T, n_embd = dv["x"].shape
    ref = moe.moe_ffn_fused(dv["gate"], dv["up"], dv["down"], dv["x"], dv["ids"], dv["route_w"],
                            shared=dv["shared"], path=path)
    out = torch.empty((T, n_embd), dtype=torch.float32, device="cuda")
    args = (dv["gate"], dv["up"], dv["down"], dv["x"], dv["ids"], dv["route_w"])
    moe.moe_ffn_fused_noalloc(*args, shared=dv["shared"], path=path, out=out)   # first call on the device
    torch.cuda.synchronize()
    assert _same_bytes(out, ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            moe.moe_ffn_fused_noalloc(*args, shared=dv["shared"], path=path, out=out, stream=side)
    torch.cuda.synchronize()
    for _ in range(5):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same_bytes(out, ref)
