"""GPU parity of the group-128 scale path ("Day 6 — Quantize It Yourself", The mechanism,
block 1: one scale per group of 128 weights along the input dimension): the group quantizer
(codes and scales bitwise equal to the oracle's) and the weight-only GEMM with group scales
(float tolerance as for W8A16, tests/parity.py)."""
import numpy as np
import pytest
import torch

import int8_quantized_linear_amd as i8
from int8_quantized_linear_amd import workloads as wl
from parity import check_float, host, sentinel, w8a16_tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    i8.load_library()
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
    if torch.cuda.is_available():
        torch.cuda.synchronize()


def group_quant_vs_ref(ref, dev, t, view, dtype):
    q, s = i8.quantize_per_group_int8(t.to(dev))
    qr, sr = ref.quantize_groups(view, dtype)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    return q, s, qr, sr


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 128), (3, 256), (37, 1024), (130, 2560), (9, 12288)])
def test_group_quantizer(ref, dev, dtype, shape):
    g = wl.rng(140 + shape[0])
    w = wl.weight(g, *shape)
    w[0, :128] = 0.0                                   # an all-zero group
    if shape[0] > 2:
        w[1, 128:256] *= np.float32(1e-30) if dtype == "f32" else np.float32(1.0)  # tiny scales
        w[2, 5] = 40.0                                 # an outlier in one group
    t, view = host(dtype, w)
    group_quant_vs_ref(ref, dev, t, view, dtype)


def test_group_quantizer_decoder_weights(ref, dev):
    g = wl.rng(149)
    t, view = host("bf16", wl.weight(g, 4096, 4096))
    group_quant_vs_ref(ref, dev, t, view, "bf16")


def run_g128(ref, dev, g, m, n, k, bias, out_dtype):
    t, view = host("bf16", wl.weight(g, n, k))
    q, s, qr, sr = group_quant_vs_ref(ref, dev, t, view, "bf16")
    xt, xv = host("bf16", wl.activations(g, m, k))
    b = (g.standard_normal(n, dtype=np.float32) * 0.02).astype(np.float32) if bias else None
    y = i8.w8a16_gemm_g128(xt.to(dev), q, s, None if b is None else torch.from_numpy(b).to(dev),
                           out_dtype=out_dtype, out=sentinel((m, n), out_dtype, dev))
    yref = ref.w8a16_grouped_scales(xv, qr, sr, 128, b)
    deq = np.repeat(sr.astype(np.float64), 128, axis=1) * np.abs(qr.astype(np.float64))
    absdot = np.abs(xt.double().numpy()) @ deq.T
    check_float(y, yref, w8a16_tol(yref, absdot, k, b), f"w8a16 g128 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (1, 40, 4096), (4, 200, 4096), (8, 96, 12288),
                                   (37, 72, 1024), (100, 48, 2560)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_w8a16_g128_small(ref, dev, m, n, k, out_dtype):
    run_g128(ref, dev, wl.rng(150 + m), m, n, k, m % 2 == 0, out_dtype)


@pytest.mark.parametrize("m", [1, 4, 8])
@pytest.mark.parametrize("n,k", [(4096, 4096), (4096, 12288)])
def test_w8a16_g128_dense_8b_decode(ref, dev, m, n, k):
    run_g128(ref, dev, wl.rng(160 + m), m, n, k, False, torch.bfloat16)


def test_w8a16_g128_rejects_a_bias_of_the_wrong_length(dev):
    q = torch.zeros((32, 256), dtype=torch.int8, device=dev)
    s = torch.ones((32, 2), dtype=torch.float32, device=dev)
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        i8.w8a16_gemm_g128(x, q, s, torch.zeros(31, dtype=torch.float32, device=dev))
