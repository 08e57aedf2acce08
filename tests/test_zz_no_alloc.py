"""attn_bwd_static, the backward entry point that allocates nothing, against
attn_bwd through the C ABI: identical gradients on two calls in a row (the
second smaller, so it runs on what the first left in the fixed scratch
array), no change in device memory allocated during the call, and sizes
beyond the array rejected before any HIP call."""
import ctypes

import numpy as np
import pytest

import exact_attention_127_amd as A
from seeded_inputs import make_output_grad, random_inputs
from tests.helpers import to_device

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def test_static_matches_attn_bwd_on_two_calls(gpu):
    import torch
    L = A.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = [(2, 4, 1000, 128, True, 71), (1, 3, 300, 64, False, 72)]   # the second is smaller
    for B, H, N, d, causal, seed in cases:
        inp = random_inputs(B, H, N, d, "bf16", causal, seed=seed)
        do = make_output_grad(inp["workload"])
        q, k, v, dout = (to_device(x, torch.bfloat16, gpu) for x in (inp["q"], inp["k"], inp["v"], do))
        o, lse = A.attn_fwd(q, k, v, scale=inp["scale"], causal=causal)
        ref = [torch.empty_like(q) for _ in range(3)]
        delta = torch.empty_like(lse)
        st = L.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta),
                        *map(_ptr, ref), B, H, N, d, inp["scale"], int(causal), 1, stream)
        assert st == 0
        got = [torch.full_like(q, 7.0) for _ in range(3)]
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        st = L.attn_bwd_static(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                               *map(_ptr, got), B, H, N, d, inp["scale"], int(causal), 1, stream)
        torch.cuda.synchronize()
        assert st == 0, A.attn_strerror(st)
        assert torch.cuda.memory_allocated() == before
        for g, r in zip(got, ref):
            assert torch.equal(g, r)
            assert torch.isfinite(g.float()).all()


def test_static_binding_and_size_limit(gpu):
    import torch
    inp = random_inputs(1, 2, 200, 128, "bf16", True, seed=73)
    do = make_output_grad(inp["workload"])
    q, k, v, dout = (to_device(x, torch.bfloat16, gpu) for x in (inp["q"], inp["k"], inp["v"], do))
    o, lse = A.attn_fwd(q, k, v, scale=inp["scale"], causal=True)
    a = A.attn_bwd(q, k, v, o, dout, lse, scale=inp["scale"], causal=True)
    b = A.attn_bwd_static(q, k, v, o, dout, lse, scale=inp["scale"], causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # one row more than the array holds: rejected on the host
    L = A.lib()
    n = A.STATIC_SCRATCH_FLOATS + 1
    fake = ctypes.c_void_p(0x10000)
    assert L.attn_bwd_static(*([fake] * 9), 1, 1, n, 128, 0.1, 0, 1, None) == -4
