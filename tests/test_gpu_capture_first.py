"""The first int4 expert-FFN call of a process made under HIP graph capture.

With int4 weights and T > 32 the library runs the grouped GEMM on a second
stream of the device, which it creates on the first such call made outside
graph capture; a call made while the caller's stream is capturing, before
that, stays on the caller's stream.  A child process (so that its first call
is the captured one) captures moe_expert_ffn as its first FFN call at T = 100
(E = 8, H = 256, FF = 128: every group in the grouped GEMM), replays the graph
three times with eager work between the replays, and compares every replay
with an eager call made afterwards (which does use the second stream) bit for
bit."""
import os
import subprocess
import sys
import textwrap

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent("""
    import sys
    import numpy as np
    import torch
    sys.path.insert(0, {root!r})
    import bench
    import expert_ffn_amd as lib
    import synth
    from expert_ffn_amd.layer import MoeLayer
    lib.lib()
    dev = torch.device("cuda")
    E, k, H, FF, T = 8, 2, 256, 128, 100
    pool, sb, slots = bench.build_stack(lib, 5, 1, E, H, FF, lib.W_INT4_G64, dev)
    slot_d = torch.from_numpy(slots[0].astype(np.int32)).to(dev)
    logits = torch.from_numpy(synth.logits(6, 0, T, E)).to(dev)
    x = torch.from_numpy(synth.x_bf16(6, 0, T, H).view(np.int16)).to(dev).view(torch.bfloat16)
    ml = MoeLayer(E, k, H, FF, lib.W_INT4_G64, T, device=dev).bind(pool, sb, slot_d)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ml.route(logits, stream=s)
        s.synchronize()
        m = np.diff(ml.offsets.cpu().numpy())
        assert (m > 8).all(), m            # every group is the grouped GEMM's
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            ml.ffn(x, stream=s)            # the process's first FFN call
        kept = int(ml.offsets[E].item())
        replays = []
        for rep in range(3):
            ml.out_routes.fill_(-1.0)
            g.replay()
            s.synchronize()
            replays.append(ml.out_routes[:kept].clone())
        ml.out_routes.fill_(-2.0)
        ml.ffn(x, stream=s)                # eager: the second stream is used from here on
        s.synchronize()
        want = ml.out_routes[:kept].clone()
        assert torch.isfinite(want).all()
        for rep, got in enumerate(replays):
            assert torch.equal(got, want), f"replay {{rep}} differs from the eager call"
    print(f"capture-first: {{kept}} routes, 3 replays identical to the eager call", flush=True)
""")


def test_first_ffn_call_under_capture():
    code = CHILD.format(root=ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240, cwd=ROOT)
    print(r.stdout[-2000:], r.stderr[-4000:], flush=True)
    assert r.returncode == 0, f"child failed ({r.returncode})"
    assert "3 replays identical" in r.stdout
