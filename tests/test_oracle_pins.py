"""Pins of the CPU oracle: checks against facts the pages and the mathematics fix.

None of these re-types the oracle's formulas: they use exact rational brute force, Python
big integers, numpy's independent float64/int64 matmuls, closed forms printed on the pages
(tests/golden/), metamorphic identities, and deliberately wrong oracle builds (mutants)
that the pins must reject.  Pages cited by title and section:

* "Day 6 — Quantize It Yourself", The mechanism, block 1 (q = clamp(round(w/s)), s = absmax
  over the largest code, w ~ s*q) and block 5 (W8A8 vs weight-only);
* "Phase 5a: int8 weight-only quantization", Summary (float32 arithmetic fix with its
  "1.5x the ideal bound", the all-zero-channel guard fix, 49.89% expert memory reduction);
* "feat(quantization): support compressed-tensors W8A8 and mixed modules", Design and
  Supported Execution Scheme (per-channel weights, per-token activations);
* the mixture-of-experts block of "Phase 5a" around its grouped GEMM (routing, SiLU·mul,
  combine: readings, pinned against scipy's softmax/expit, brute-force sorting and einsum).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from int8_quantized_linear_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
H = 0.5 + 2.0 ** -16  # rounding bound in units of s: 1/2 plus the float32 quotient's slack


# ---------------------------------------------------------------------------------------
# exact helpers (rational arithmetic, independent of the oracle)

def nearest_f32(fr: Fraction) -> np.float32:
    """The float32 nearest to the rational ``fr``, ties to the even significand."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - fr),
                                     int(np.array(v, np.float32).view(np.uint32)) & 1))


def brute_row(row32: np.ndarray, all_codes: bool = True):
    """Quantize one row by exhaustive search: correctly rounded float32 scale and quotient,
    then the code nearest to the quotient among all 255 codes, ties to the even code."""
    vals = [Fraction(float(v)) for v in row32]
    amax = max(abs(v) for v in vals)
    s = nearest_f32(amax / 127)
    if s == 0:
        return np.zeros(len(vals), np.int8), np.float32(1.0)
    S = Fraction(float(s))
    out = []
    for v in vals:
        T = Fraction(float(nearest_f32(v / S)))
        if all_codes:
            codes = range(-127, 128)
        else:
            f = int(np.floor(float(T)))
            codes = [c for c in range(f - 1, f + 3) if -127 <= c <= 127] or [127 if T > 0 else -127]
        out.append(min(codes, key=lambda c: (abs(T - c), c & 1)))
    return np.array(out, np.int8), s


def widen(a, dtype):
    if dtype == "f32":
        return np.asarray(a, np.float32)
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(a, np.uint16).view(np.float16).astype(np.float32)


def as_dtype(x32: np.ndarray, dtype: str):
    if dtype == "f32":
        return x32.astype(np.float32)
    if dtype == "bf16":
        return wl.bits16(wl.to_bf16(x32))
    return wl.bits16(wl.to_f16(x32))


# ---------------------------------------------------------------------------------------
# P1  brute force on tiny rows

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_p1_brute_force_all_codes(ref, dtype):
    g = wl.rng(11)
    rows = as_dtype(g.standard_normal((48, 12), dtype=np.float32) *
                    np.exp(g.uniform(-6, 3, size=(48, 1))).astype(np.float32), dtype)
    q, s = ref.quantize_rows(rows, dtype)
    w = widen(rows, dtype)
    for r in range(w.shape[0]):
        bq, bs = brute_row(w[r], all_codes=True)
        assert s[r] == bs, r
        np.testing.assert_array_equal(q[r], bq)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_p1_brute_force_many_rows(ref, dtype):
    g = wl.rng(12)
    x = g.standard_normal((600, 24), dtype=np.float32)
    x[::7] *= 1e-3
    x[::11, 3] *= 100.0
    rows = as_dtype(x, dtype)
    q, s = ref.quantize_rows(rows, dtype)
    w = widen(rows, dtype)
    for r in range(w.shape[0]):
        bq, bs = brute_row(w[r], all_codes=False)
        assert s[r] == bs, r
        np.testing.assert_array_equal(q[r], bq)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p1_exact_ties_go_to_even(ref, dtype):
    # amax = 127 * 2^-7 makes s = 2^-7 exactly, so (c + 1/2) * 2^-7 gives quotient c + 1/2.
    s = 2.0 ** -7
    halves = np.array([0.5, 1.5, 2.5, 3.5, 62.5, 63.5, 125.5, 126.5], np.float64)
    row = np.concatenate([[127.0], halves, -halves]) * s
    rows = as_dtype(row[None, :].astype(np.float32), dtype)
    assert np.array_equal(widen(rows, dtype)[0], row.astype(np.float32))
    q, sc = ref.quantize_rows(rows, dtype)
    assert sc[0] == np.float32(s)
    even = np.array([0, 2, 2, 4, 62, 64, 126, 126])
    np.testing.assert_array_equal(q[0], np.concatenate([[127], even, -even]))
    bq, _ = brute_row(widen(rows, dtype)[0])
    np.testing.assert_array_equal(q[0], bq)


def test_p1_near_ties_and_tiny_scales(ref):
    s = np.float32(2.0 ** -7)
    near = []
    for c in (0.5, 1.5, 64.5, 126.5):
        v = np.float32(c * float(s))
        near += [np.nextafter(v, np.float32(-1)), np.nextafter(v, np.float32(2))]
    rows = [np.array([127 * float(s)] + near, np.float32)]
    # subnormal magnitudes: scale underflows to zero (guard) or stays a tiny subnormal
    rows.append(np.array([1e-44, -5e-45] + [0.0] * 8, np.float32))
    rows.append(np.array([3 * 2.0 ** -126, -2.0 ** -127] + [1e-40] * 8, np.float32))
    for row in rows:
        q, sc = ref.quantize_rows(row[None, :], "f32")
        bq, bs = brute_row(row)
        assert sc[0] == bs
        np.testing.assert_array_equal(q[0], bq)


def test_f16_and_bf16_widening_is_exact(ref):
    # every finite binary16 pattern, as rows: the oracle's own decoding must agree with
    # numpy's binary16 -> binary32 conversion bit for bit.
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(pats.view(np.float16))
    pats = pats[finite][: (finite.sum() // 64) * 64].reshape(-1, 64)
    q1, s1 = ref.quantize_rows(pats, "f16")
    q2, s2 = ref.quantize_rows(pats.view(np.float16).astype(np.float32), "f32")
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)
    b = wl.bits16(wl.to_bf16(wl.rng(3).standard_normal((64, 64), dtype=np.float32)))
    q1, s1 = ref.quantize_rows(b, "bf16")
    q2, s2 = ref.quantize_rows(widen(b, "bf16"), "f32")
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)


# ---------------------------------------------------------------------------------------
# P2 round-trip bound, P3 largest code, P6 scale invariance

def _matrix(dtype, seed=5, r=256, k=1024):
    g = wl.rng(seed)
    w = wl.weight(g, r, k)
    w[:, g.choice(k, 3, replace=False)] *= 50.0
    w[[0, 77, r - 1]] = 0.0
    w[5] *= 1e-3
    return as_dtype(w, dtype)


def round_trip_ratio(a, q, s):
    """max over nonzero rows of |w - s*q| / s, in float64 (exact here)."""
    w = a.astype(np.float64)
    sc = s.astype(np.float64)[:, None]
    nz = np.abs(w).max(axis=1) > 0
    return float((np.abs(w - sc * q)[nz] / sc[nz]).max())


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_p2_round_trip_bound(ref, dtype):
    rows = _matrix(dtype)
    q, s = ref.quantize_rows(rows, dtype)
    assert round_trip_ratio(widen(rows, dtype), q, s) <= H
    assert q.min() >= -127 and q.max() <= 127


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_p3_largest_code_and_sign(ref, dtype):
    rows = _matrix(dtype, seed=6)
    q, s = ref.quantize_rows(rows, dtype)
    w = widen(rows, dtype)
    for r in range(w.shape[0]):
        amax = np.abs(w[r]).max()
        if amax == 0:
            continue
        at = np.abs(w[r]) == amax
        assert np.all(np.abs(q[r][at]) == 127)
        assert np.all(np.sign(q[r][at]) == np.sign(w[r][at]))
    nz = q != 0
    assert np.all(np.sign(q[nz]) == np.sign(w[nz]))


@pytest.mark.parametrize("j", [-20, -3, 4, 30])
def test_p6_power_of_two_invariance(ref, j):
    w = wl.weight(wl.rng(7), 64, 300, std=1.0)
    q1, s1 = ref.quantize_rows(w, "f32")
    q2, s2 = ref.quantize_rows(np.ldexp(w, j).astype(np.float32), "f32")
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(np.ldexp(s1, j).astype(np.float32), s2)


# ---------------------------------------------------------------------------------------
# P4 / P5: the two precision bugs of the Phase 5a page, as mutants the pins reject

def test_p4_bf16_arithmetic_mutant_hits_one_and_a_half_bound(ref, mutant):
    gold = json.load(open(os.path.join(GOLDEN, "bf16_arith_bound.json")))
    bad = mutant("REF_MUTANT_BF16_ARITH")
    rows = as_dtype(wl.rng(8).standard_normal((256, 2048), dtype=np.float32), "bf16")
    w = widen(rows, "bf16")
    q, s = ref.quantize_rows(rows, "bf16")
    assert round_trip_ratio(w, q, s) <= H
    qb, sb = bad.quantize_rows(rows, "bf16")
    ratio = round_trip_ratio(w, qb, sb) / gold["ideal_bound_in_scale_units"]
    # the mutant breaks the ideal bound, and by no more than the page's 1.5x
    assert ratio > 1.25
    assert ratio <= gold["bf16_worst_ratio"] + 2.0 ** -14
    # brute force sides with the oracle on a row where the two disagree
    r = int(np.flatnonzero((q != qb).any(axis=1) | (s != sb))[0])
    bq, bs = brute_row(w[r], all_codes=False)
    assert bs == s[r] and np.array_equal(bq, q[r])
    assert not (bs == sb[r] and np.array_equal(bq, qb[r]))


def test_p5_zero_channels_and_floor_mutant(ref, mutant):
    t = wl.tiny_w8a8(0)
    q, s = ref.quantize_rows(t["w"], "f32")
    for r in t["zero_rows"]:
        assert s[r] == 1.0 and not np.any(q[r])
    assert np.all(np.isfinite(s))
    # small but nonzero fp16 channels must keep the full int8 range (the guard is only for
    # all-zero channels); a floored scale loses it and fails the largest-code pin.
    g = wl.rng(9)
    small = (g.standard_normal((16, 256), dtype=np.float32) * 1e-5).astype(np.float32)
    rows = as_dtype(small, "f16")
    q, s = ref.quantize_rows(rows, "f16")
    assert np.all(np.abs(q).max(axis=1) == 127)
    qb, sb = mutant("REF_MUTANT_FLOOR_SCALE").quantize_rows(rows, "f16")
    assert np.any(np.abs(qb).max(axis=1) < 127)


# ---------------------------------------------------------------------------------------
# P7 exact integer GEMM, P8 epilogue special case, P9 a-priori error

def test_p7_big_int_triple_loop(ref):
    g = wl.rng(10)
    xq = g.integers(-127, 128, size=(3, 48), dtype=np.int8)
    wq = g.integers(-127, 128, size=(5, 48), dtype=np.int8)
    acc, _ = ref.w8a8(xq, None, wq, None, want_y=False)
    for i in range(3):
        for j in range(5):
            assert acc[i, j] == sum(int(xq[i, c]) * int(wq[j, c]) for c in range(48))


def test_p7_numpy_int64_matmul(ref):
    g = wl.rng(13)
    xq = g.integers(-127, 128, size=(37, 1040), dtype=np.int8)
    wq = g.integers(-127, 128, size=(53, 1040), dtype=np.int8)
    acc, _ = ref.w8a8(xq, None, wq, None, want_y=False)
    np.testing.assert_array_equal(acc, xq.astype(np.int64) @ wq.astype(np.int64).T)


def test_p7_int32_limit(ref):
    k = 133144
    xq = np.full((2, k), 127, np.int8)
    wq = np.stack([np.full(k, 127, np.int8), np.full(k, -127, np.int8)])
    acc, _ = ref.w8a8(xq, None, wq, None, want_y=False)
    assert acc[0, 0] == 2147479576 and acc[0, 1] == -2147479576
    with pytest.raises(OverflowError):
        ref.w8a8(np.full((1, k + 16), 127, np.int8), None, np.full((1, k + 16), 127, np.int8),
                 None, want_y=False)


def test_p8_unit_scales_give_the_accumulator(ref):
    g = wl.rng(14)
    xq = g.integers(-127, 128, size=(9, 4096), dtype=np.int8)
    wq = g.integers(-127, 128, size=(11, 4096), dtype=np.int8)
    one_m, one_n = np.ones(9, np.float32), np.ones(11, np.float32)
    acc, y = ref.w8a8(xq, one_m, wq, one_n)
    np.testing.assert_array_equal(y, acc.astype(np.float64))
    b = np.linspace(-3, 3, 11).astype(np.float32)
    _, yb = ref.w8a8(xq, one_m, wq, one_n, bias=b)
    np.testing.assert_array_equal(yb, acc.astype(np.float64) + b.astype(np.float64))


def apriori_bound(qx, sx, qw, sw):
    """|x.w - y| <= sx*sw*sum(|qx|*h + h*|qw| + h*h) with h the per-element rounding bound."""
    ax = np.abs(qx.astype(np.float64))
    aw = np.abs(qw.astype(np.float64))
    k = qx.shape[1]
    core = ax.sum(1)[:, None] * H + H * aw.sum(1)[None, :] + k * H * H
    return core * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]


def test_p9_tiny_workload_error_is_within_the_quantization_bound(ref):
    t = wl.tiny_w8a8(0)
    qw, sw = ref.quantize_rows(t["w"], "f32")
    qx, sx = ref.quantize_rows(t["x"], "f32")
    acc, y = ref.w8a8(qx, sx, qw, sw)
    exact = t["x"].astype(np.float64) @ t["w"].astype(np.float64).T
    bound = apriori_bound(qx, sx, qw, sw) * (1 + 1e-9)
    assert np.all(np.abs(y - exact) <= bound)
    for r in t["zero_rows"]:
        assert np.all(y[:, r] == 0.0)
    # a mistake that drops the weight scale or transposes an operand is far outside it
    assert np.any(np.abs(y / sw[None, :] - exact) > bound)


def test_p9_bf16_outlier_activations(ref):
    g = wl.rng(15)
    w = wl.to_bf16(wl.weight(g, 96, 2560))
    x = wl.to_bf16(wl.activations(g, 17, 2560, outlier_frac=0.001))
    qw, sw = ref.quantize_rows(wl.bits16(w), "bf16")
    qx, sx = ref.quantize_rows(wl.bits16(x), "bf16")
    _, y = ref.w8a8(qx, sx, qw, sw)
    exact = x.double().numpy() @ w.double().numpy().T
    assert np.all(np.abs(y - exact) <= apriori_bound(qx, sx, qw, sw) * (1 + 1e-9))


# ---------------------------------------------------------------------------------------
# P10 closed form printed on the Phase 5a page

def test_p10_expert_memory_reduction_matches_the_page(ref):
    gold = json.load(open(os.path.join(GOLDEN, "expert_footprint.json")))
    g = wl.rng(16)
    before = after = 0
    for name, (n, k) in gold["expert_projections"].items():
        w = wl.bits16(wl.to_bf16(wl.weight(g, n, k)))
        q, s = ref.quantize_rows(w, "bf16")
        before += n * k * gold["bf16_bytes_per_weight"]
        after += q.nbytes + s.nbytes
    pct = round(100.0 * (1 - after / before), gold["decimals"])
    assert pct == gold["printed_reduction_percent"]
    # a 2-byte scale would print a different number: the page pins float32 scales
    alt = sum(n * k + 2 * n for n, k in gold["expert_projections"].values())
    assert round(100.0 * (1 - alt / before), 2) != gold["printed_reduction_percent"]


# ---------------------------------------------------------------------------------------
# P11 weight-only and grouped products against numpy's float64 matmul

def _w8a16_case(ref, g, m, n, k, bias):
    x = wl.to_bf16(wl.activations(g, m, k))
    q, s = ref.quantize_rows(wl.bits16(wl.to_bf16(wl.weight(g, n, k))), "bf16")
    b = (g.standard_normal(n, dtype=np.float32) * 0.02).astype(np.float32) if bias else None
    return x, q, s, b


@pytest.mark.parametrize("m,n,k,bias", [(1, 64, 512, False), (8, 200, 4096, True), (5, 33, 48, True)])
def test_p11_w8a16_is_x_times_dequantized_weight(ref, m, n, k, bias):
    g = wl.rng(17)
    x, q, s, b = _w8a16_case(ref, g, m, n, k, bias)
    y = ref.w8a16(wl.bits16(x), q, s, b)
    deq = s.astype(np.float64)[:, None] * q.astype(np.float64)
    xd = x.double().numpy()
    want = xd @ deq.T + (0.0 if b is None else b.astype(np.float64))
    scale = np.abs(xd) @ np.abs(deq).T + 1.0
    assert np.all(np.abs(y - want) <= 1e-12 * scale)
    # dropping the last 16 input channels is visible at this tolerance
    short = xd[:, :-16] @ deq[:, :-16].T + (0.0 if b is None else b.astype(np.float64))
    assert np.any(np.abs(short - y) > 1e-6 * scale)


def test_p11_grouped_reduces_to_w8a16_and_per_expert_matmul(ref):
    g = wl.rng(18)
    e, n, k, t, topk = 7, 40, 256, 9, 3
    wf = wl.moe_weights(g, n, k, experts=e)
    q, s = ref.quantize_rows(wl.bits16(wl.to_bf16(wf.reshape(e * n, k))), "bf16")
    q, s = q.reshape(e, n, k), s.reshape(e, n)
    ids = np.stack([g.choice(e, topk, replace=False) for _ in range(t)]).astype(np.int32)
    ids[2, 1] = -1
    ids[4, 0] = e  # out of range
    for per_assign in (0, 1):
        x = wl.to_bf16(wl.activations(g, t * topk if per_assign else t, k))
        y = ref.grouped_w8a16(wl.bits16(x), per_assign, q, s, ids)
        xd = x.double().numpy()
        for p in range(t * topk):
            ex = ids.flat[p]
            if not 0 <= ex < e:
                assert np.all(y[p] == 0.0)
                continue
            xr = xd[p if per_assign else p // topk]
            want = (s[ex].astype(np.float64)[:, None] * q[ex].astype(np.float64)) @ xr
            np.testing.assert_allclose(y[p], want, rtol=1e-12, atol=1e-12)
    # one expert, one slot: the grouped product is the plain weight-only product
    x = wl.to_bf16(wl.activations(g, 6, k))
    yg = ref.grouped_w8a16(wl.bits16(x), 0, q[:1], s[:1], np.zeros((6, 1), np.int32))
    np.testing.assert_array_equal(yg, ref.w8a16(wl.bits16(x), q[0], s[0]))


def test_p11_grouped_token_permutation(ref):
    g = wl.rng(19)
    e, n, k, t, topk = 5, 24, 128, 8, 2
    q, s = ref.quantize_rows(wl.bits16(wl.to_bf16(wl.weight(g, e * n, k))), "bf16")
    q, s = q.reshape(e, n, k), s.reshape(e, n)
    ids = g.integers(0, e, size=(t, topk), dtype=np.int32)
    x = wl.bits16(wl.to_bf16(wl.activations(g, t, k)))
    perm = g.permutation(t)
    y = ref.grouped_w8a16(x, 0, q, s, ids).reshape(t, topk, n)
    yp = ref.grouped_w8a16(x[perm], 0, q, s, ids[perm]).reshape(t, topk, n)
    np.testing.assert_array_equal(yp, y[perm])


# ---------------------------------------------------------------------------------------
# P12–P14 the mixture-of-experts steps around the grouped GEMM.  "Phase 5a: int8 weight-only
# quantization" (Summary) measures the block but does not spell these steps out; the
# readings (softmax top-k routing with unrenormalized weights and shared experts appended,
# h = silu(gate) * up, routing-weighted combine) are pinned here against independent
# definitions: brute-force sorting, scipy's softmax and expit, numpy einsum.

def _route_brute(logits, k_routed, n_shared):
    from scipy.special import softmax
    t, e = logits.shape
    ids = np.empty((t, k_routed + n_shared), np.int64)
    w = np.empty((t, k_routed + n_shared))
    for i in range(t):
        order = sorted(range(e), key=lambda j: (-float(logits[i, j]), j))[:k_routed]
        p = softmax(logits[i].astype(np.float64))
        ids[i, :k_routed] = order
        w[i, :k_routed] = p[order]
        ids[i, k_routed:] = np.arange(e, e + n_shared)
        w[i, k_routed:] = 1.0
    return ids, w


@pytest.mark.parametrize("t,e,k,ns", [(9, 64, 6, 2), (3, 5, 5, 0), (4, 200, 17, 3), (1, 1, 1, 1)])
def test_p12_routing_is_softmax_top_k(ref, t, e, k, ns):
    g = wl.rng(60 + e)
    logits = g.standard_normal((t, e), dtype=np.float32) * np.float32(2.0)
    ids, w = ref.moe_route_topk(logits, k, ns)
    bids, bw = _route_brute(logits, k, ns)
    np.testing.assert_array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=1e-13, atol=0)


def test_p12_routing_ties_shift_and_shared(ref):
    # equal logits: the lower index first, every weight 1/e
    ids, w = ref.moe_route_topk(np.zeros((2, 64), np.float32), 6, 2)
    assert ids.tolist() == [[0, 1, 2, 3, 4, 5, 64, 65]] * 2
    np.testing.assert_allclose(w[:, :6], 1.0 / 64, rtol=1e-15)
    assert np.all(w[:, 6:] == 1.0)
    # ties inside the selection and at its boundary
    l = np.array([[1, 3, 3, 2, 3, 2, 0]], np.float32)
    ids, _ = ref.moe_route_topk(l, 4, 0)
    assert ids.tolist() == [[1, 2, 4, 3]]
    # softmax is shift invariant: integer logits (exact in float32) moved by 7
    g = wl.rng(64)
    li = g.integers(-20, 20, size=(5, 64)).astype(np.float32)
    a_ids, a_w = ref.moe_route_topk(li, 6, 2)
    b_ids, b_w = ref.moe_route_topk(li + np.float32(7), 6, 2)
    np.testing.assert_array_equal(a_ids, b_ids)
    np.testing.assert_allclose(a_w, b_w, rtol=1e-13)
    # the routed weights are probabilities of distinct experts: positive, summing below 1
    assert np.all(a_w[:, :6] > 0) and np.all(a_w[:, :6].sum(axis=1) <= 1.0 + 1e-15)
    assert all(len(set(r)) == len(r) for r in a_ids.tolist())


def _silu_case(ref, g, e, n, k):
    wf = wl.moe_weights(g, 2 * n, k, experts=e)
    q, s = ref.quantize_rows(wl.bits16(wl.to_bf16(wf.reshape(e * 2 * n, k))), "bf16")
    return q.reshape(e, 2 * n, k), s.reshape(e, 2 * n)


def test_p13_silu_mul_of_the_gate_and_up_products(ref):
    from scipy.special import expit
    g = wl.rng(65)
    e, n, k, t, topk = 6, 24, 192, 7, 3
    q, s = _silu_case(ref, g, e, n, k)
    ids = np.stack([g.choice(e, topk, replace=False) for _ in range(t)]).astype(np.int32)
    ids[3, 2] = e   # invalid: zero row
    for per_assign in (0, 1):
        x = wl.bits16(wl.to_bf16(wl.activations(g, t * topk if per_assign else t, k)))
        h = ref.grouped_w8a16_silu(x, per_assign, q, s, ids)
        gate = ref.grouped_w8a16(x, per_assign, q[:, :n], s[:, :n], ids)
        up = ref.grouped_w8a16(x, per_assign, q[:, n:], s[:, n:], ids)
        want = gate * expit(gate) * up
        np.testing.assert_allclose(h, want, rtol=1e-12, atol=1e-15)
        assert np.all(h[3 * topk + 2] == 0.0)
        # swapping the halves (up as gate) is a different function: the layout is pinned
        swapped = up * expit(up) * gate
        assert np.max(np.abs(swapped - h)) > 1e-3 * np.max(np.abs(h))


def test_p13_silu_special_values(ref):
    g = wl.rng(66)
    e, n, k, t = 2, 16, 64, 3
    q, s = _silu_case(ref, g, e, n, k)
    ids = np.zeros((t, 1), np.int32)
    x = wl.bits16(wl.to_bf16(wl.activations(g, t, k)))
    # a zero gate row: silu(0) = 0 exactly, whatever the up row
    qz = q.copy()
    qz[0, 5] = 0
    h = ref.grouped_w8a16_silu(x, 0, qz, s, ids)
    assert np.all(h[:, 5] == 0.0)
    # odd part: silu(-v) = silu(v) - v, so negating the gate codes gives (silu(v) - v) * up
    qn = q.copy()
    qn[0, :n] = -qn[0, :n]
    hp = ref.grouped_w8a16_silu(x, 0, q, s, ids)
    hn = ref.grouped_w8a16_silu(x, 0, qn, s, ids)
    gate = ref.grouped_w8a16(x, 0, q[:, :n], s[:, :n], ids)
    up = ref.grouped_w8a16(x, 0, q[:, n:], s[:, n:], ids)
    np.testing.assert_allclose(hn, hp - gate * up, rtol=1e-10, atol=1e-14)


def test_p14_combine_is_the_weighted_sum(ref):
    g = wl.rng(67)
    t, topk, n = 5, 8, 96
    d = g.standard_normal((t * topk, n), dtype=np.float32)
    w = g.random((t, topk), dtype=np.float32)
    y = ref.moe_combine(d, w)
    want = np.einsum("tj,tjc->tc", w.astype(np.float64),
                     d.reshape(t, topk, n).astype(np.float64))
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-14)
    # one-hot weights pick the slot's row exactly; the wrong slot would be visible
    oh = np.zeros((t, topk), np.float32)
    oh[np.arange(t), np.arange(t) % topk] = 1.0
    y1 = ref.moe_combine(d, oh)
    for i in range(t):
        np.testing.assert_array_equal(y1[i], d[i * topk + i % topk].astype(np.float64))
        assert not np.array_equal(y1[i], d[i * topk + (i + 1) % topk].astype(np.float64))


# ---------------------------------------------------------------------------------------
# P15–P16 one scale per group of 128 input channels ("Day 6 — Quantize It Yourself", The
# mechanism, block 1: a scale can cover a tensor, a row, or 128 consecutive input channels;
# with groups, an outlier coarsens only the codes of its own group).

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_p15_group_quantizer_is_the_row_rule_per_group(ref, dtype):
    g = wl.rng(130)
    r, k, grp = 7, 1024, 128
    w = wl.weight(g, r, k)
    w[2, 128:256] = 0.0                       # an all-zero group: scale 1, codes 0
    w[4, 5] = 3.0                             # an outlier inside the first group
    if dtype == "f32":
        a = w
    else:
        a = wl.bits16(wl.to_bf16(w) if dtype == "bf16" else wl.to_f16(w))
    q, s = ref.quantize_groups(a, dtype, grp)
    qr, sr = ref.quantize_rows(np.ascontiguousarray(a).reshape(r * k // grp, grp), dtype)
    np.testing.assert_array_equal(q, qr.reshape(r, k))
    np.testing.assert_array_equal(s.view(np.uint32), sr.reshape(r, k // grp).view(np.uint32))
    assert s[2, 1] == 1.0 and np.all(q[2, 128:256] == 0)
    # one group spanning the row is the per-channel quantizer
    q1, s1 = ref.quantize_groups(a, dtype, k)
    qc, sc = ref.quantize_rows(a, dtype)
    np.testing.assert_array_equal(q1, qc)
    np.testing.assert_array_equal(s1[:, 0], sc)


def test_p15_an_outlier_costs_only_its_group(ref):
    g = wl.rng(131)
    k = 1024
    w = wl.weight(g, 1, k)
    wo = w.copy()
    wo[0, 700] = 50.0                          # group 5 (640..767)
    q, s = ref.quantize_groups(w, "f32")
    qo, so = ref.quantize_groups(wo, "f32")
    other = np.ones(k, bool)
    other[640:768] = False
    np.testing.assert_array_equal(qo[0, other], q[0, other])   # other groups untouched
    assert np.count_nonzero(qo[0, 640:768]) < np.count_nonzero(q[0, 640:768])
    # per-channel: the same outlier zeroes most codes of the whole row
    qc, _ = ref.quantize_rows(wo, "f32")
    assert np.count_nonzero(qc[0, other]) < 0.1 * np.count_nonzero(q[0, other])
    # the round-trip bound holds per group
    d = np.abs(wo.astype(np.float64) - np.repeat(so.astype(np.float64), 128, axis=1) * qo)
    assert np.all(d <= np.repeat(so.astype(np.float64), 128, axis=1) * H)


@pytest.mark.parametrize("m,n,k,bias", [(1, 64, 512, False), (8, 40, 4096, True), (3, 17, 128, True)])
def test_p16_w8a16_group_scales_against_numpy(ref, m, n, k, bias):
    g = wl.rng(132)
    x = wl.to_bf16(wl.activations(g, m, k))
    q, s = ref.quantize_groups(wl.bits16(wl.to_bf16(wl.weight(g, n, k))), "bf16")
    b = (g.standard_normal(n, dtype=np.float32) * 0.02).astype(np.float32) if bias else None
    y = ref.w8a16_grouped_scales(wl.bits16(x), q, s, 128, b)
    deq = np.repeat(s.astype(np.float64), 128, axis=1) * q.astype(np.float64)
    xd = x.double().numpy()
    want = xd @ deq.T + (0.0 if b is None else b.astype(np.float64))
    mag = np.abs(xd) @ np.abs(deq).T + 1.0
    assert np.all(np.abs(y - want) <= 1e-12 * mag)
    # a scale applied to the wrong group is visible
    s2 = s.copy()
    s2[:, [0, -1]] = s2[:, [-1, 0]]
    if s.shape[1] > 1:
        y2 = ref.w8a16_grouped_scales(wl.bits16(x), q, s2, 128, b)
        assert np.max(np.abs(y2 - y)) > 1e-6 * np.max(np.abs(y))
    # one group over the whole row is the per-channel product
    qc, sc = ref.quantize_rows(wl.bits16(wl.to_bf16(wl.weight(g, n, k))), "bf16")
    np.testing.assert_array_equal(
        ref.w8a16_grouped_scales(wl.bits16(x), qc, sc[:, None], k, b), ref.w8a16(wl.bits16(x), qc, sc, b))


# ---------------------------------------------------------------------------------------
# P17 W8A8 with group-128 weight scales ("Day 6 — Quantize It Yourself", The mechanism,
# block 1: one scale per group of input channels; block 5: both operands int8).

def w8a8_g128_case(ref, g, m, n, k, bias):
    w = wl.weight(g, n, k)
    w[:, g.choice(k, 1)] *= np.float32(50.0)     # one outlier input column
    x = wl.activations(g, m, k, outlier_frac=0.01)
    qw, sw = ref.quantize_groups(wl.bits16(wl.to_bf16(w)), "bf16")
    qx, sx = ref.quantize_rows(wl.bits16(wl.to_bf16(x)), "bf16")
    b = (g.standard_normal(n, dtype=np.float32) * 0.02).astype(np.float32) if bias else None
    return qx, sx, qw, sw, b


def test_p17_w8a8_group_scales_exact_rational_brute_force(ref):
    g = wl.rng(140)
    m, n, k = 3, 5, 384
    qx, sx, qw, sw, b = w8a8_g128_case(ref, g, m, n, k, True)
    y = ref.w8a8_grouped_scales(qx, sx, qw, sw, 128, b)
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for gi in range(k // 128):
                part = sum(int(qx[i, c]) * int(qw[j, c]) for c in range(128 * gi, 128 * gi + 128))
                tot += Fraction(float(sw[j, gi])) * part
            want = Fraction(float(sx[i])) * tot + Fraction(float(b[j]))
            assert abs(Fraction(y[i, j]) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


@pytest.mark.parametrize("m,n,k,bias", [(4, 64, 512, False), (16, 40, 4096, True), (2, 9, 128, True)])
def test_p17_w8a8_group_scales_against_numpy(ref, m, n, k, bias):
    g = wl.rng(141 + k)
    qx, sx, qw, sw, b = w8a8_g128_case(ref, g, m, n, k, bias)
    y = ref.w8a8_grouped_scales(qx, sx, qw, sw, 128, b)
    xd = qx.astype(np.float64) * sx.astype(np.float64)[:, None]
    wd = qw.astype(np.float64) * np.repeat(sw.astype(np.float64), 128, axis=1)
    want = xd @ wd.T + (0.0 if b is None else b.astype(np.float64))
    mag = np.abs(xd) @ np.abs(wd).T + 1.0
    assert np.all(np.abs(y - want) <= 1e-12 * mag)
    # the group scales of two groups exchanged, or applied per output channel transposed,
    # are visible
    if sw.shape[1] > 1:
        s2 = sw.copy()
        s2[:, [0, -1]] = s2[:, [-1, 0]]
        y2 = ref.w8a8_grouped_scales(qx, sx, qw, s2, 128, b)
        assert np.max(np.abs(y2 - y)) > 1e-6 * np.max(np.abs(y))


def test_p17_w8a8_group_scales_reduce_to_per_channel(ref):
    """Equal scales in every group of a row: the per-channel W8A8 value (the exact int32 sum
    times both scales); and the result does not depend on the order of the groups."""
    g = wl.rng(142)
    m, n, k = 6, 20, 1024
    qx, sx, qw, _, b = w8a8_g128_case(ref, g, m, n, k, True)
    qc, sc = ref.quantize_rows(wl.bits16(wl.to_bf16(wl.weight(g, n, k))), "bf16")
    same = np.repeat(sc[:, None], k // 128, axis=1)
    y = ref.w8a8_grouped_scales(qx, sx, qc, same, 128, b)
    _, y1 = ref.w8a8(qx, sx, qc, sc, b)
    assert np.all(np.abs(y - y1) <= 1e-14 * (np.abs(y1) + 1e-30))
    # permuting the groups of k (codes of both operands and the weight scales together)
    perm = g.permutation(k // 128)
    cols = (perm[:, None] * 128 + np.arange(128)[None, :]).reshape(-1)
    _, sw = ref.quantize_groups(wl.bits16(wl.to_bf16(wl.weight(g, n, k))), "bf16")
    ya = ref.w8a8_grouped_scales(qx, sx, qc, sw, 128, b)
    yb = ref.w8a8_grouped_scales(np.ascontiguousarray(qx[:, cols]), sx,
                                 np.ascontiguousarray(qc[:, cols]),
                                 np.ascontiguousarray(sw[:, perm]), 128, b)
    assert np.all(np.abs(ya - yb) <= 1e-13 * (np.abs(ya) + 1e-30))


def test_p17_w8a8_group_scales_quantization_error_bound(ref):
    """Against the unquantized float64 product: per element, the quantization of each operand
    moves a product term by at most half a code step of that operand's scale."""
    g = wl.rng(143)
    m, n, k = 8, 32, 2048
    w = wl.weight(g, n, k)
    x = wl.activations(g, m, k, outlier_frac=0.01)
    wb, xb = wl.to_bf16(w), wl.to_bf16(x)
    qw, sw = ref.quantize_groups(wl.bits16(wb), "bf16")
    qx, sx = ref.quantize_rows(wl.bits16(xb), "bf16")
    y = ref.w8a8_grouped_scales(qx, sx, qw, sw, 128, None)
    wd, xd = wb.double().numpy(), xb.double().numpy()
    exact = xd @ wd.T
    swf = np.repeat(sw.astype(np.float64), 128, axis=1)     # [n, k] weight scale per element
    sxf = sx.astype(np.float64)[:, None]                   # [m, 1]
    # x = sx*qx + ex, w = sw*qw + ew with |ex| <= H*sx, |ew| <= H*sw, so per term
    # |xw - (sx qx)(sw qw)| <= |sx qx| H sw + H sx |sw qw| + H^2 sx sw
    bound = (np.abs(qx * sxf) @ (H * swf).T
             + (H * sxf) * np.abs(qw * swf).sum(axis=1)[None, :]
             + (H * sxf) * (H * swf).sum(axis=1)[None, :])
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-9) + 1e-12)


# ---------------------------------------------------------------------------------------
# P18: the RMS norm that produces a quantized projection's input (reading in oracle/ref.c;
# pinned against numpy float64 with an explicit bf16 rounding, exact power-of-two rows,
# scale invariance and torch's own bfloat16 addition)

def bf16_round_f64(v: np.ndarray):
    """Round float64 values to the bfloat16 grid (normal range), ties to even, and flag the
    values within 2^-12 of a bfloat16 ulp of a rounding midpoint (ambiguous at float32
    precision)."""
    v = np.asarray(v, np.float64)
    out = np.zeros_like(v)
    amb = np.zeros(v.shape, bool)
    nz = v != 0
    e = np.floor(np.log2(np.abs(v[nz])))
    ulp = np.exp2(e - 7)
    q = v[nz] / ulp
    frac = np.abs(q - np.floor(q) - 0.5)
    out[nz] = np.rint(q) * ulp
    amb[nz] = frac < 2.0 ** -12
    return out, amb


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _norm_case(g, m, k, scale=1.0, residual=False):
    x = wl.bits16(wl.to_bf16(wl.activations(g, m, k, outlier_frac=0.01) * np.float32(scale)))
    gamma = wl.bits16(wl.to_bf16(wl.norm_weight(g, k)))
    res = wl.bits16(wl.to_bf16(wl.activations(g, m, k) * np.float32(scale))) if residual else None
    return x, gamma, res


@pytest.mark.parametrize("m,k,scale,eps,residual", [
    (64, 4096, 1.0, 1e-6, False), (16, 2560, 1.0, 1e-6, True), (32, 12288, 1.0, 1e-5, True),
    (8, 1024, 1e-3, 1e-6, False),   # mean square ~ eps: eps changes the result by ~1/sqrt(2)
    (8, 1024, 3e-4, 1e-6, True), (5, 48, 1.0, 0.0, False)])
def test_p18_rmsnorm_against_numpy_float64(ref, m, k, scale, eps, residual):
    g = wl.rng(41)
    x, gamma, res = _norm_case(g, m, k, scale, residual)
    h, res_out = ref.rmsnorm(x, gamma, eps, res)
    if residual:
        u_bits = wl.bits16(torch_bf16_sum(x, res))
        np.testing.assert_array_equal(res_out, u_bits)
    else:
        assert res_out is None
        u_bits = x
    u = bf16_values(u_bits)
    want = u / np.sqrt(np.mean(u * u, axis=1, keepdims=True) + eps) * bf16_values(gamma)[None]
    want_bf16, amb = bf16_round_f64(want)
    got = bf16_values(h)
    assert amb.mean() < 1e-2
    np.testing.assert_array_equal(got[~amb], want_bf16[~amb])
    assert np.all(np.abs(got - want) <= (2.0 ** -8 + 2.0 ** -20) * np.abs(want))


def torch_bf16_sum(a_bits, b_bits):
    """torch's own bfloat16 addition of two bf16 bit-pattern arrays."""
    import torch
    a = torch.from_numpy(a_bits.astype(np.int16)).view(torch.bfloat16)
    b = torch.from_numpy(b_bits.astype(np.int16)).view(torch.bfloat16)
    return a + b


def test_p18_rmsnorm_of_power_of_two_rows_is_gamma(ref):
    # |u| = 2^j for every element: mean square 4^j exactly, r = 2^-j exactly (eps = 0), so
    # h = sign(u) * gamma with no rounding at all
    g = wl.rng(43)
    m, k = 6, 256
    gamma = wl.bits16(wl.to_bf16(wl.norm_weight(g, k)))
    js = np.array([-20, -3, 0, 1, 7, 30], np.float32)
    signs = np.where(g.random((m, k)) < 0.5, -1.0, 1.0).astype(np.float32)
    x = wl.bits16(wl.to_bf16(signs * np.exp2(js)[:, None]))
    h, _ = ref.rmsnorm(x, gamma, 0.0)
    np.testing.assert_array_equal(bf16_values(h), signs * bf16_values(gamma)[None])
    # the same through the residual add: x + x = 2x, still a power of two
    h2, res_out = ref.rmsnorm(x, gamma, 0.0, x)
    np.testing.assert_array_equal(bf16_values(res_out), 2.0 * bf16_values(x))
    np.testing.assert_array_equal(h2, h)


def test_p18_rmsnorm_scale_invariance_and_zero_rows(ref):
    g = wl.rng(47)
    x, gamma, _ = _norm_case(g, 16, 2048)
    h, _ = ref.rmsnorm(x, gamma, 0.0)
    for j in (-8, 5):
        xs = wl.bits16(wl.to_bf16(bf16_values(x).astype(np.float32) * np.float32(2.0 ** j)))
        np.testing.assert_array_equal(ref.rmsnorm(xs, gamma, 0.0)[0], h)
    # an all-zero row with eps > 0 normalizes to zeros and quantizes with the zero guard
    x[3] = 0
    q, s, _ = ref.rmsnorm_quantize(x, gamma, 1e-6)
    assert np.all(ref.rmsnorm(x, gamma, 1e-6)[0][3] == 0)
    assert s[3] == 1.0 and np.all(q[3] == 0)


def test_p18_rmsnorm_residual_is_the_normalized_sum(ref):
    g = wl.rng(53)
    x, gamma, res = _norm_case(g, 12, 4096, residual=True)
    h, res_out = ref.rmsnorm(x, gamma, 1e-6, res)
    h_direct, none = ref.rmsnorm(res_out, gamma, 1e-6)
    assert none is None
    np.testing.assert_array_equal(h, h_direct)
    # columns permuted together with gamma permute the output (the sum of squares is
    # order-free at double precision here)
    perm = g.permutation(4096)
    hp, _ = ref.rmsnorm(x[:, perm], gamma[perm], 1e-6, res[:, perm])
    np.testing.assert_array_equal(hp, h[:, perm])
    # the fused quantization is the row quantizer on the normalized rows
    q, s, _ = ref.rmsnorm_quantize(x, gamma, 1e-6, res)
    q2, s2 = ref.quantize_rows(h, "bf16")
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s, s2)


# ---------------------------------------------------------------------------------------
# P19: SiLU·mul producing the down projection's input (reading in oracle/ref.c), pinned
# against a 60-digit decimal evaluation with exact bf16 rounding by rational comparison

def _bf16_nearest_exact(v):
    """(nearest bf16 as float, the other neighbour, relative distance to the halfway point)
    of a decimal value, by exact rational arithmetic."""
    from decimal import Decimal
    fr = Fraction(v)
    if fr == 0:
        return 0.0, 0.0, None
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - 7)           # bf16: 8 significant bits (normal range)
    lo = (a // ulp) * ulp
    hi = lo + ulp
    mid = (lo + hi) / 2
    if lo == a:
        return float(sign * lo), float(sign * lo), None
    if a < mid or (a == mid and (lo / ulp) % 2 == 0):
        near, other = lo, hi
    else:
        near, other = hi, lo
    return float(sign * near), float(sign * other), float(abs(a - mid) / a)


def test_p19_silu_mul_against_high_precision(ref):
    import decimal
    from decimal import Decimal
    decimal.getcontext().prec = 60
    g = wl.rng(59)
    n = 1500
    gate = np.concatenate([g.standard_normal(n - 12).astype(np.float32) * np.float32(4.0),
                           np.array([0.0, -0.0, 1e-3, -1e-3, 30.0, -30.0, 80.0, -80.0, 0.5,
                                     -0.5, 7.25, -7.25], np.float32)])
    up = g.standard_normal(n).astype(np.float32) * np.float32(3.0)
    gb = wl.bits16(wl.to_bf16(gate))
    ub = wl.bits16(wl.to_bf16(up))
    gu = np.concatenate([gb, ub])[None, :]
    h, other, amb = ref.silu_mul(gu, rel=2.0 ** -17)
    hv = bf16_values(h[0])
    ov = bf16_values(other[0])
    gv, uv = bf16_values(gb), bf16_values(ub)
    for j in range(n):
        x = Decimal(float(gv[j]))
        v = x / (1 + (-x).exp()) * Decimal(float(uv[j]))
        near, oth, dist = _bf16_nearest_exact(v)
        assert hv[j] == near, (j, gv[j], uv[j], hv[j], near)
        if dist is not None:
            assert ov[j] == oth
            assert amb[0, j] == (dist <= 2.0 ** -17)
        else:
            assert not amb[0, j]
    # silu(0) * u = 0 and g * u of one sign for a positive gate
    assert np.all(hv[gv == 0] == 0)
    pos = gv > 0
    assert np.all(np.sign(hv[pos]) * np.sign(uv[pos]) >= 0)


def test_p19_codes_with_scale_is_the_quantizer_code_step(ref):
    g = wl.rng(61)
    a = wl.bits16(wl.to_bf16(wl.activations(g, 40, 1024, outlier_frac=0.01)))
    q, s = ref.quantize_rows(a, "bf16")
    np.testing.assert_array_equal(ref.codes_with_scale(a, s), q)
