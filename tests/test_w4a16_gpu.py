"""W4A16 product on the GPU (w4a16_gemm, w4a16_dequantize) against the
float64 oracle.

* The fp16 weights (w4a16_dequantize) equal oracle.dequantize bit for bit:
  fp16(s (q - z)) is one rounding of an exact product on both sides.
* Y = fp16(S), S the float32 sum of the K exact products x*w, in any order:
  |S - Y_ref| <= K 2^-24 sum_k |x||w| and the output rounding adds
  2^-11 |S|, so the gate is |Y - Y_ref| <= 2^-11 |Y_ref| + 1.01 K 2^-24
  sum|x||w| + 2^-25 (half the smallest fp16 subnormal), element by element.
* A one-hot X selects one fp16 weight column exactly; q = z gives Y = 0.
"""
import numpy as np
import pytest

import exact_attention_127_amd as A
import oracle
from seeded_inputs import W4_WORKLOADS, W4Workload, make_w4a16_inputs

pytestmark = pytest.mark.gpu


def _dev(inp, gpu):
    import torch
    return (torch.from_numpy(np.ascontiguousarray(inp["x"])).to(gpu),
            torch.from_numpy(np.ascontiguousarray(inp["qweight"]).view(np.int32)).to(gpu),
            torch.from_numpy(np.ascontiguousarray(inp["scales"])).to(gpu),
            torch.from_numpy(np.ascontiguousarray(inp["zeros"])).to(gpu))


def _gemm(inp, gpu):
    import torch
    y = A.w4a16_gemm(*_dev(inp, gpu))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def _gate(y, inp, cols=None):
    args = (inp["x"], inp["qweight"], inp["scales"], inp["zeros"], inp["G"])
    ref = oracle.w4a16_gemm(*args) if cols is None else oracle.w4a16_rows(*args, cols)
    sa = oracle.w4a16_sum_abs(*args, cols=cols)
    K = inp["x"].shape[1]
    bound = 2.0 ** -11 * np.abs(ref) + 1.01 * K * 2.0 ** -24 * sa + 2.0 ** -25
    got = y if cols is None else y[:, cols]
    err = np.abs(got - ref)
    return err, bound, ref


def _case(M, N, K, seed):
    return make_w4a16_inputs(W4Workload(f"w4_{M}x{N}x{K}", M, N, K, 128, seed))


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (50, 640), (96, 1024), (33, 256)])
def test_dequantize_bit_exact(gpu, N, K):
    import torch
    inp = _case(1, N, K, 7 * N + K)
    _, q, s, z = _dev(inp, gpu)
    w = A.w4a16_dequantize(q, s, z, K)
    torch.cuda.synchronize()
    want = oracle.dequantize(inp["qweight"], inp["scales"], inp["zeros"], K, 128).astype(np.float16)
    assert np.array_equal(w.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("M", [1, 2, 3, 7, 16])
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (50, 640), (96, 1024), (37, 1152)])
def test_gemm_matches_the_oracle(gpu, M, N, K):
    inp = _case(M, N, K, 100 * M + N + K)
    y = _gemm(inp, gpu)
    err, bound, ref = _gate(y, inp)
    assert y.shape == (M, N) and np.isfinite(y).all()
    assert np.all(err <= bound), (float((err / bound).max()), M, N, K)


@pytest.mark.parametrize("M,N,K", [(16, 64, 28672), (5, 40, 32768), (16, 72, 4096), (4, 64, 28672)])
def test_gemm_long_rows(gpu, M, N, K):
    # long weight rows: 224 and 256 groups (the staged scales near their LDS
    # limit, and the launch's choice between 2 and 4 row tiles per wave)
    inp = _case(M, N, K, M + N + K)
    y = _gemm(inp, gpu)
    err, bound, ref = _gate(y, inp)
    assert np.all(err <= bound), (float((err / bound).max()), M, N, K)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (16, 1, 256), (2, 3, 128), (16, 17, 128), (9, 5, 512)])
def test_gemm_tiny_outputs(gpu, M, N, K):
    # fewer output rows than one 16-row tile, N not a multiple of 4 (element stores)
    inp = _case(M, N, K, 5 * M + N + K)
    y = _gemm(inp, gpu)
    err, bound, ref = _gate(y, inp)
    assert y.shape == (M, N)
    assert np.all(err <= bound), (float((err / bound).max()), M, N, K)


def test_one_hot_selects_a_weight_column(gpu):
    inp = _case(4, 40, 512, 3)
    K = 512
    x = np.zeros((4, K), np.float16)
    ks = [0, 129, 300, 511]
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    inp["x"] = x
    y = _gemm(inp, gpu)
    w = oracle.dequantize(inp["qweight"], inp["scales"], inp["zeros"], K, 128)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], w[:, k])


def test_zero_weights_and_zero_activations(gpu):
    inp = _case(3, 32, 256, 4)
    q = oracle.unpack_int4(inp["qweight"], 256)
    inp["zeros"] = q[:, ::128][:, :2].copy()            # make every group's zero equal to its first q ...
    qz = np.repeat(inp["zeros"], 128, axis=1)
    inp["qweight"] = oracle.pack_int4(qz)                # ... and every q equal to its group's zero
    assert not np.any(_gemm(inp, gpu))
    inp2 = _case(3, 32, 256, 5)
    inp2["x"] = np.zeros_like(inp2["x"])
    assert not np.any(_gemm(inp2, gpu))


def test_deterministic(gpu):
    inp = _case(16, 96, 1024, 9)
    assert np.array_equal(_gemm(inp, gpu), _gemm(inp, gpu))


def test_launcher_matches_w4a16_gemm(gpu):
    """w4a16_gemm_launcher checks once and relaunches w4a16_gemm on the same buffers."""
    import torch
    inp = _case(3, 96, 1024, 12)
    args = _dev(inp, gpu)
    y1 = A.w4a16_gemm(*args)
    y2 = torch.full_like(y1, 7)
    launch = A.w4a16_gemm_launcher(*args, y2)
    launch()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y2.fill_(7)
    launch()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("name", ["w4a16_decode_70b", "w4a16_batch16_70b"])
def test_full_size_sampled_columns(gpu, name):
    inp = make_w4a16_inputs(name)
    w = inp["workload"]
    y = _gemm(inp, gpu)
    rng = np.random.default_rng(11)
    cols = np.unique(np.concatenate([[0, 1, 15, 16, w.N - 1], rng.integers(0, w.N, 59)]))
    err, bound, ref = _gate(y, inp, cols)
    print(f"{name}: max err/bound {(err / bound).max():.3f}, max |err| {err.max():.3e}, "
          f"max |Y| {np.abs(ref).max():.3f}")
    assert np.all(err <= bound)
