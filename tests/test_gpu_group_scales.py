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


# one activation row: the one-row kernel's group-scale form (a group's 8 chunks summed
# across 8 lanes), ragged in the last 64-chunk block, at 8 chunks per lane, and past it
@pytest.mark.parametrize("n,k", [(7, 1152), (33, 8192), (5, 8320), (3, 128)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_w8a16_g128_one_row(ref, dev, n, k, out_dtype):
    run_g128(ref, dev, wl.rng(170 + n), 1, n, k, True, out_dtype)


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


# ---------------------------------------------------------------------------------------
# W8A8 with group-128 weight scales ("Day 6 — Quantize It Yourself", The mechanism, blocks 1
# and 5): codes and scales bitwise against the oracle; outputs within the float32 bound of
# the kernel's arithmetic.  Each group's int32 partial is exact; the kernel adds the G = k/128
# scaled partials with one rounding each, then multiplies by the token scale and adds the
# bias, so |y - ref| <= (G + 3) u s_x sum_g |part_g| s_w[g] + 2 u |bias|, and
# sum_g |part_g| s_w[g] <= (|q_x| @ (|q_w| * s_w per element).T).

U32 = 2.0 ** -24
GS_CONFIGS = [c for c in range(i8.W8A8_NUM_CONFIGS) if i8.w8a8_gemm_config_info(c)[4]]


def w8a8_g128_tol(qx, sx, qw, sw, bias):
    k = qx.shape[1]
    wabs = np.abs(qw.astype(np.float64)) * np.repeat(sw.astype(np.float64), 128, axis=1)
    tol = np.empty((qx.shape[0], qw.shape[0]), np.float64)
    for r0 in range(0, qx.shape[0], 1024):
        a = np.abs(qx[r0:r0 + 1024].astype(np.float64)) @ wabs.T
        tol[r0:r0 + 1024] = (k // 128 + 3) * U32 * sx[r0:r0 + 1024, None].astype(np.float64) * a
    if bias is not None:
        tol += 2 * U32 * np.abs(bias.astype(np.float64))[None, :]
    return tol


def run_w8a8_g128(ref, dev, m, n, k, bias, seed, out_dtypes=(torch.bfloat16, torch.float32),
                  config=-1, frac=0.001, rows=None):
    g = wl.rng(seed)
    w = wl.weight(g, n, k)
    w[:, g.choice(k, 1)] *= np.float32(50.0)          # an outlier input column
    wt, wv = host("bf16", w)
    xt, xv = host("bf16", wl.activations(g, m, k, outlier_frac=frac))
    qw, sw, qwr, swr = group_quant_vs_ref(ref, dev, wt, wv, "bf16")
    qx, sx = i8.quantize_per_token_int8(xt.to(dev))
    b_np = (g.standard_normal(n, dtype=np.float32) * np.float32(0.02)) if bias else None
    b = torch.from_numpy(b_np).to(dev) if bias else None
    ys = {od: i8.w8a8_gemm_g128(qx, sx, qw, sw, b, out_dtype=od, out=sentinel((m, n), od, dev),
                                config=config) for od in out_dtypes}
    if rows is None:
        qxr, sxr = ref.quantize_rows(xv, "bf16")
        np.testing.assert_array_equal(qx.cpu().numpy(), qxr)
        np.testing.assert_array_equal(sx.cpu().numpy(), sxr)
    else:
        for y in ys.values():
            assert not torch.isnan(y).any()           # every element written
        qxr, sxr = ref.quantize_rows(xv[rows], "bf16")
        idx = torch.from_numpy(rows).to(dev)
        np.testing.assert_array_equal(qx[idx].cpu().numpy(), qxr)
        ys = {od: y[idx] for od, y in ys.items()}
    yref = ref.w8a8_grouped_scales(qxr, sxr, qwr, swr, 128, b_np)
    tol = w8a8_g128_tol(qxr, sxr, qwr, swr, b_np)
    for od, y in ys.items():
        check_float(y, yref, tol, f"w8a8 g128 {m}x{n}x{k} {od}")


@pytest.mark.parametrize("config", GS_CONFIGS)
def test_w8a8_g128_every_config(ref, dev, config):
    """Each group-scale configuration, forced: ragged tiles in both directions, one to 24
    groups, more than one group of eight tile rows; an odd N takes the per-element epilogue."""
    bm, bn = i8.w8a8_gemm_config_info(config)[:2]
    for (m, n, k) in [(2 * bm + 37, 2 * bn + 24, 384), (bm - 3, bn + 19, 128),
                      (9 * bm + 5, 3 * bn + 8, 3072)]:
        print(f"w8a8 g128 config {config} ({bm}x{bn}): {m}x{n}x{k}", flush=True)
        run_w8a8_g128(ref, dev, m, n, k, bias=(m % 2 == 1), seed=config * 13 + m, config=config)


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (4, 256, 512), (130, 200, 384),
                                   (300, 33, 2560), (257, 385, 1024), (1000, 1500, 4096)])
def test_w8a8_g128_small(ref, dev, m, n, k):
    run_w8a8_g128(ref, dev, m, n, k, bias=(n % 2 == 0), seed=m + n + k)


G128_4B = [(m, n, k) for m in wl.PREFILL_4B_TOKENS for (n, k) in sorted(set(wl.DENSE_4B.values()))]
G128_8B = [(m, n, k) for m in wl.PREFILL_8B_TOKENS for (n, k) in sorted(set(wl.DENSE_8B.values()))]


@pytest.mark.parametrize("m,n,k", G128_4B)
def test_w8a8_g128_dense_4b_prefill_full(ref, dev, m, n, k):
    run_w8a8_g128(ref, dev, m, n, k, bias=False, seed=m + n + k)


@pytest.mark.parametrize("m,n,k", G128_8B)
def test_w8a8_g128_dense_8b_prefill_full(ref, dev, m, n, k):
    rows = None
    if m > 4096:  # the 16384-token shapes: first and last 8 rows and 256 seeded random rows
        g = wl.rng(m + n)
        rows = np.array(sorted(set(range(8)) | set(range(m - 8, m)) |
                               set(g.choice(m, 256, replace=False).tolist())))
    run_w8a8_g128(ref, dev, m, n, k, bias=True, seed=m + n + k, frac=0.01, rows=rows)


def test_w8a8_g128_equal_group_scales_match_per_channel(dev):
    """Equal scales in all groups of a row: the same values as w8a8_gemm with that scale up to
    the float32 summation of the group partials (here exact: every partial times a power of
    two, sums below 2^24 of the scale's unit)."""
    g = wl.rng(170)
    m, n, k = 300, 260, 1024
    qx = torch.from_numpy(g.integers(-127, 128, (m, k), dtype=np.int8)).to(dev)
    qw = torch.from_numpy(g.integers(-127, 128, (n, k), dtype=np.int8)).to(dev)
    sx = torch.full((m,), 2.0 ** -7, device=dev)
    sw = torch.full((n,), 2.0 ** -9, device=dev)
    swg = sw[:, None].repeat(1, k // 128).contiguous()
    y1 = i8.w8a8_gemm(qx, sx, qw, sw, out_dtype=torch.float32)
    y2 = i8.w8a8_gemm_g128(qx, sx, qw, swg, out_dtype=torch.float32)
    assert torch.equal(y1, y2)


def test_w8a8_g128_rejects_bad_arguments(dev):
    q = torch.zeros((4, 256), dtype=torch.int8, device=dev)
    s = torch.ones(4, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        i8.w8a8_gemm_g128(q, s, q, torch.ones((4, 3), device=dev))
    with pytest.raises(i8.I8qlError, match="I8QL_ERR_ARG"):
        i8.w8a8_gemm_g128(q, s, q, torch.ones((4, 2), device=dev), config=0)  # not a GS config
