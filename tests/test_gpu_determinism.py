"""Run-to-run bit identity: the pages' reproducibility problem (same model, input and
seed gave different outputs, "CUDA: better MoE implementation", section 1.1) must not
exist here. Ten calls per workload, with the workspace overwritten by 0xFF bytes
(NaN patterns) before every call, must give byte-identical outputs."""
import numpy as np
import pytest
import torch

import indirect_expert_matmul_amd as moe
import synth
from moe_testutil import run_ffn, upload_ffn, upload_mmid

pytestmark = pytest.mark.gpu


def _same_bytes(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("name,path", [("lite", moe.PATH_AUTO), ("dec1", moe.PATH_AUTO),
                                       ("dec8", moe.PATH_AUTO), ("dec8", moe.PATH_GEMM),
                                       ("skew", moe.PATH_AUTO), ("v3", moe.PATH_AUTO),
                                       ("dec1x", moe.PATH_AUTO), ("dec8x", moe.PATH_AUTO),
                                       ("ppx", moe.PATH_AUTO), ("dec1n", moe.PATH_AUTO),
                                       ("dec8n", moe.PATH_AUTO), ("ppn", moe.PATH_AUTO),
                                       ("dec1s", moe.PATH_AUTO), ("dec8s", moe.PATH_AUTO),
                                       ("pps", moe.PATH_AUTO)])
def test_ffn_ten_runs_bit_identical(name, path):
    inp = synth.make_inputs(name)
    dv = upload_ffn(inp)
    T, k = inp["ids"].shape
    need = moe.moe_ffn_fused_workspace_size(dv["gate"], dv["shared"][0] if dv["shared"] else None,
                                            T, k, path=path)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(10):
        ws.fill_(255)
        outs.append(run_ffn(dv, path=path, workspace=ws))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    for o in outs[1:]:
        assert _same_bytes(o, outs[0])


@pytest.mark.parametrize("weighted", [False, True])
def test_tiny_ten_runs_bit_identical(weighted):
    inp = synth.make_inputs("tiny")
    dv = upload_mmid(inp)
    rw = dv["route_w"] if weighted else None
    outs = [moe.moe_mul_mat_id(dv["w"], dv["x"], dv["ids"], route_w=rw) for _ in range(10)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert _same_bytes(o, outs[0])


def test_streams_interleaved_calls_stay_identical():
    """Many calls queued back to back on two streams with separate workspaces (the
    stream-order lifetime question the pages discuss in section 5): every result must
    equal the single-call result."""
    inp = synth.make_inputs("lite")
    dv = upload_ffn(inp)
    ref = run_ffn(dv)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(20):
        st = s1 if i % 2 == 0 else s2
        with torch.cuda.stream(st):
            outs.append(run_ffn(dv, stream=st))
    torch.cuda.synchronize()
    for o in outs:
        assert _same_bytes(o, ref)


_CHILD = r"""
import hashlib, sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import indirect_expert_matmul_amd as moe
import synth
from moe_testutil import run_ffn, upload_ffn
out = run_ffn(upload_ffn(synth.make_inputs(sys.argv[2])))
torch.cuda.synchronize()
print("SHA256", hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest(), flush=True)
"""


@pytest.mark.parametrize("name", ["lite", "v3"])
def test_second_process_gives_the_same_bits(name):
    """Identity across processes, not only inside one: a fresh Python process (its own
    HIP context, workspace and allocations) computes the same layer and must print the
    same SHA-256 of the output bytes."""
    import hashlib
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    out = run_ffn(upload_ffn(synth.make_inputs(name)))
    torch.cuda.synchronize()
    mine = hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest()
    del out
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([root, here]))
    r = subprocess.run([sys.executable, "-c", _CHILD, root, name], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-2000:]
    theirs = [l.split()[1] for l in r.stdout.splitlines() if l.startswith("SHA256 ")]
    assert theirs == [mine]


def test_non_current_stream_without_workspace():
    """Calls on a stream other than torch's current one, with no workspace given: the
    binding's temporary workspace and output are marked as used on that stream, so
    allocations made meanwhile on the current stream cannot take their memory. Every
    result must equal the plain call's."""
    inp = synth.make_inputs("lite")
    dv = upload_ffn(inp)
    ref = run_ffn(dv)
    mm = upload_mmid(synth.make_custom_mmid(3, 16, 4, 300, 512, 256))
    ref_mm = moe.moe_mul_mat_id(mm["w"], mm["x"], mm["ids"], route_w=mm["route_w"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs, outs_mm = [], []
    for _ in range(8):
        outs.append(run_ffn(dv, stream=side))
        outs_mm.append(moe.moe_mul_mat_id(mm["w"], mm["x"], mm["ids"], route_w=mm["route_w"], stream=side))
        # allocations and writes on the current stream while the side stream still runs
        junk = torch.full((1 << 24,), -1, dtype=torch.int32, device="cuda")
        del junk
    torch.cuda.synchronize()
    for o in outs:
        assert _same_bytes(o, ref)
    for o in outs_mm:
        assert _same_bytes(o, ref_mm)
