"""Launches captured in a HIP graph give the eager results on every replay.

The short-kernel workloads (image-model rows, one-token decode) are launch
bound, so their timed steps are replayed from a captured graph.  Each case
here captures six launches that cycle through three buffer sets on a side
stream, replays the graph three times with eager work and a synchronisation
between replays (the outputs are overwritten with NaN and unrelated matrix
products run before each replay), and requires every replay to reproduce
the eager outputs bit for bit.  The kernels are deterministic, so any
difference is a capture or replay fault.
"""
import numpy as np
import pytest

import exact_attention_127_amd as A
from seeded_inputs import W4Workload, make_w4a16_inputs, random_inputs

pytestmark = pytest.mark.gpu

SETS = 3
LAUNCHES = 6
REPLAYS = 3


def _replays_match(launchers, outputs, side):
    """side: the stream the launchers were built on, which the capture uses."""
    import torch
    ref = []
    for launch, outs in zip(launchers, outputs):
        launch()
        torch.cuda.synchronize()
        ref.append([t.clone() for t in outs])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(LAUNCHES):
            launchers[i % SETS]()
    torch.cuda.synchronize()
    for outs in outputs:                      # capture alone writes nothing
        for t in outs:
            t.fill_(float("nan"))
    a = torch.randn(512, 512, device="cuda")
    for rep in range(REPLAYS):
        for outs in outputs:
            for t in outs:
                t.fill_(float("nan"))
        b = a @ a
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s, (outs, want) in enumerate(zip(outputs, ref)):
            for t, w in zip(outs, want):
                assert torch.equal(t, w), f"replay {rep}, buffer set {s}"
        assert torch.isfinite(b).all()


@pytest.mark.parametrize("B,H,N,d,causal,dtype", [
    (4, 12, 196, 64, False, "bf16"),     # image-model rows: the one-tile-at-a-time kernel
    (1, 8, 777, 128, True, "bf16"),      # the pipelined kernel, causal, ragged last block
    (1, 12, 196, 64, False, "f32"),      # the float32 kernel
])
def test_forward_graph_replays_match_eager(gpu, B, H, N, d, causal, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    side = torch.cuda.Stream()
    launchers, outputs = [], []
    for s in range(SETS):
        inp = random_inputs(B, H, N, d, dtype, causal, seed=900 + s)
        q, k, v = (torch.from_numpy(inp[x]).to(gpu).to(tdt).contiguous() for x in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=gpu)
        launchers.append(A.attn_fwd_launcher(q, k, v, o, lse, scale=inp["scale"], causal=causal, stream=side))
        outputs.append((o, lse, q, k, v))
    torch.cuda.synchronize()
    _replays_match(launchers, [(o, lse) for (o, lse, *_) in outputs], side)


@pytest.mark.parametrize("M", [1, 16])
def test_w4a16_graph_replays_match_eager(gpu, M):
    import torch
    side = torch.cuda.Stream()
    launchers, outputs, keep = [], [], []
    for s in range(SETS):
        inp = make_w4a16_inputs(W4Workload(f"graph_{M}_{s}", M, 384, 1024, 128, seed=700 + s))
        x = torch.from_numpy(np.ascontiguousarray(inp["x"])).to(gpu)
        qw = torch.from_numpy(np.ascontiguousarray(inp["qweight"]).view(np.int32)).to(gpu)
        sc = torch.from_numpy(np.ascontiguousarray(inp["scales"])).to(gpu)
        z = torch.from_numpy(np.ascontiguousarray(inp["zeros"])).to(gpu)
        y = torch.empty((M, 384), dtype=torch.float16, device=gpu)
        launchers.append(A.w4a16_gemm_launcher(x, qw, sc, z, y, stream=side))
        outputs.append((y,))
        keep.append((x, qw, sc, z))
    torch.cuda.synchronize()
    _replays_match(launchers, outputs, side)
