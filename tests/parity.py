"""Comparison rules of the GPU parity tests (test-side helpers; no method arithmetic).

* int8 codes, scales and int32 accumulators: bitwise equality.
* float outputs: the GPU value y must lie within ``tol`` of the oracle's float64 value r,
  where ``tol`` is stated per operation in the tests (1e-3 relative, plus a floor derived
  from float32 rounding for values that cancel).
* bfloat16 outputs: y must be a value that round-to-nearest-even can produce from some
  float32 in [r - tol, r + tol], i.e. rne(lo) <= y <= rne(hi) (rounding is monotone).

Also the small input/output helpers the GPU parity modules share (host tensors with the
oracle's view of them, sentinel-filled outputs, the quantize-and-compare step).
"""
from __future__ import annotations

import numpy as np
import torch

import int8_quantized_linear_amd as i8
from int8_quantized_linear_amd import workloads as wl

U32 = 2.0 ** -24  # float32 unit roundoff


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy()


def bf16_rne(a: np.ndarray) -> np.ndarray:
    """float64 -> the bf16 values (as float64) that rne produces, going through float32
    conservatively (caller passes already-widened bounds)."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).double().numpy()


def check_float(y: torch.Tensor, ref: np.ndarray, tol: np.ndarray, what: str = "") -> None:
    got = to_np(y).astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if y.dtype == torch.float32:
        bad = np.abs(got - ref) > tol
    elif y.dtype == torch.bfloat16:
        lo = np.nextafter((ref - tol).astype(np.float32), np.float32(-np.inf))
        hi = np.nextafter((ref + tol).astype(np.float32), np.float32(np.inf))
        bad = (got < bf16_rne(lo)) | (got > bf16_rne(hi))
        # aggregate: against the oracle rounded to bf16, 1e-3 relative in Frobenius norm
        rb = bf16_rne(ref)
        fro = np.linalg.norm(got - rb) / max(np.linalg.norm(ref), 1e-30)
        assert fro <= 1e-3, f"{what}: Frobenius relative error {fro:.3e} vs rne(ref)"
    else:
        raise TypeError(y.dtype)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        msg = ", ".join(f"{tuple(i)}: got {got[tuple(i)]!r} ref {ref[tuple(i)]!r} tol {tol[tuple(i)]!r}"
                        for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; {msg}")


def w8a8_tol(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray, bias) -> np.ndarray:
    """Bound on |fp32 epilogue - exact| for ((float)acc * sx) * sw (+ b): four roundings."""
    p = np.abs(acc.astype(np.float64) * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :])
    b = 0.0 if bias is None else np.abs(bias.astype(np.float64))[None, :]
    return 8 * U32 * (p + b)


def w8a16_tol(ref: np.ndarray, absdot: np.ndarray, k: int, bias=None) -> np.ndarray:
    """1e-3 relative to the oracle, plus the float32 summation floor
    (k/8 + 64) * u * sum|scaled products| (+ 2u|b|) for values that cancel."""
    floor = (k / 8 + 64) * U32 * absdot
    if bias is not None:
        floor = floor + 2 * U32 * np.abs(bias.astype(np.float64))[None, :]
    return 1e-3 * np.abs(ref) + floor


def host(dtype, a32):
    """Host tensor of the given dtype from float32 numpy + the oracle's view of it."""
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a32, np.float32))
        return t, t.numpy()
    t = wl.to_bf16(a32) if dtype == "bf16" else wl.to_f16(a32)
    return t, wl.bits16(t)


def sentinel(shape, dtype, dev):
    """Output buffer pre-filled so that an element the kernel fails to write cannot match:
    NaN for float outputs, the 0xAAAAAAAA pattern for int32."""
    if dtype == torch.int32:
        return torch.full(shape, -0x55555556, dtype=torch.int32, device=dev)
    return torch.full(shape, float("nan"), dtype=dtype, device=dev)


def quant_gpu_vs_ref(ref, dev, t, view, dtype, per_token=False):
    """Quantize on the GPU and with the oracle; codes and scales must be bitwise equal."""
    fn = i8.quantize_per_token_int8 if per_token else i8.quantize_per_channel_int8
    q, s = fn(t.to(dev))
    qr, sr = ref.quantize_rows(view, dtype)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    return q, s, qr, sr


def moe_stack(ref, dev, g, n, k, e):
    """A stacked [e, n, k] expert weight quantized on both sides (checked bitwise)."""
    w = wl.moe_weights(g, n, k, experts=e).reshape(e * n, k)
    wt, wv = host("bf16", w)
    qw, sw, qwr, swr = quant_gpu_vs_ref(ref, dev, wt, wv, "bf16")
    return qw.view(e, n, k), sw.view(e, n), qwr.reshape(e, n, k), swr.reshape(e, n)
