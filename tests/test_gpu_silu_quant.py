"""GPU parity of SiLU·mul fused with the per-token quantization (the producer of a decoder
MLP's down-projection input) and of the unfused SiLU·mul, through the C ABI against the CPU
oracle on the same seeded inputs.

The activation involves an exponential, which float32 evaluates to within a few ulps, so the
bf16 value of an element may round either way when the exact value lies within 2^-17
(relative) of the halfway point between two bf16 values: the oracle (float64) gives both
neighbours and flags those elements.  Everywhere else the GPU's bf16 activations must equal
the oracle's bitwise.  For the codes, the oracle gives each row's possible scales (from the
smaller- and larger-magnitude choices at flagged elements); the GPU's scale must be one of
them, and each code must be the oracle's code under that scale of the oracle's value, or,
at a flagged element, of its other neighbour.  The fused call's codes and scales must also
be bitwise those of quantize_per_token_int8 of the unfused call's output."""
import numpy as np
import pytest
import torch

import int8_quantized_linear_amd as i8
from int8_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu
REL = 2.0 ** -17


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


def bits_tensor(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).astype(np.int16)).view(torch.bfloat16).to(dev)


def gpu_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def mag(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).__abs__()


def gate_up(seed, m, n, scale_g=4.0, scale_u=3.0):
    """[m, 2n] bf16 bits: gate ~ N(0, scale_g^2) with 1% of the columns x10 (outlier
    channels), up ~ N(0, scale_u^2)."""
    g = wl.rng(seed)
    gate = g.standard_normal((m, n), dtype=np.float32) * np.float32(scale_g)
    cols = g.choice(n, max(1, n // 100), replace=False)
    gate[:, cols] *= np.float32(10.0)
    up = g.standard_normal((m, n), dtype=np.float32) * np.float32(scale_u)
    return wl.bits16(wl.to_bf16(np.concatenate([gate, up], axis=1)))


def check(ref, dev, gu, rows=None, max_flagged=5e-3):
    """Run both entry points on gu and compare (all rows, or the listed rows); at most
    max_flagged of the elements may be flagged (about 2^-9 of random values are)."""
    m, n2 = gu.shape
    n = n2 // 2
    d = bits_tensor(gu, dev)
    hb = torch.full((m * n + 64,), -7.0, dtype=torch.bfloat16, device=dev)
    h = hb[:m * n].view(m, n)
    i8.silu_mul_bf16(d, h_out=h)
    qb = torch.full((m * n + 64,), 0x55, dtype=torch.int8, device=dev)
    sb = torch.full((m + 16,), float("nan"), dtype=torch.float32, device=dev)
    q, s = qb[:m * n].view(m, n), sb[:m]
    i8.silu_mul_quantize_per_token_int8(d, q_out=q, scale_out=s)
    assert torch.all(hb[m * n:] == -7.0) and torch.all(qb[m * n:] == 0x55)
    assert torch.all(torch.isnan(sb[m:]))
    q2, s2 = i8.quantize_per_token_int8(h)
    assert torch.equal(q2, q) and torch.equal(s2, s), "fused != quantize(unfused)"
    sel = np.arange(m) if rows is None else np.asarray(rows)
    near, other, amb = ref.silu_mul(gu[sel], rel=REL)
    hg, qg, sg = gpu_bits(h)[sel], q.cpu().numpy()[sel], s.cpu().numpy()[sel]
    # activations: bitwise where unambiguous, either neighbour where flagged
    bad = (hg != near) & ~(amb & (hg == other))
    assert not bad.any(), f"{int(bad.sum())} activations differ; first at {np.argwhere(bad)[:3]}"
    assert amb.mean() <= max_flagged
    # scales: one of the two extremes of the flagged choices
    alt = np.where(amb, other, near)
    small = np.where(mag(near) <= mag(alt), near, alt)
    large = np.where(mag(near) <= mag(alt), alt, near)
    _, s_lo = ref.quantize_rows(small, "bf16")
    _, s_hi = ref.quantize_rows(large, "bf16")
    okscale = (sg == s_lo) | (sg == s_hi)
    assert okscale.all(), f"scales differ in rows {sel[~okscale][:5]}"
    s_sel = np.where(sg == s_lo, s_lo, s_hi)
    c_near = ref.codes_with_scale(near, s_sel)
    c_alt = ref.codes_with_scale(alt, s_sel)
    badq = (qg != c_near) & ~(amb & (qg == c_alt))
    assert not badq.any(), f"{int(badq.sum())} codes differ; first at {np.argwhere(badq)[:3]}"
    return amb


@pytest.mark.parametrize("m,n", [(1, 8), (3, 4096), (130, 1000), (1100, 6144), (1030, 6152),
                                 (7, 24576), (2000, 12288)])
def test_silu_mul_quantize_small_and_ragged(ref, dev, m, n):
    check(ref, dev, gate_up(m + n, m, n))


@pytest.mark.parametrize("m", wl.PREFILL_4B_TOKENS)
def test_silu_mul_quantize_dense_4b_full(ref, dev, m):
    check(ref, dev, gate_up(3 + m, m, wl.DENSE_4B["gate"][0]))


def test_silu_mul_quantize_dense_8b_full(ref, dev):
    m, n = 4096, wl.DENSE_8B["gate"][0]
    check(ref, dev, gate_up(5, m, n))


def test_silu_mul_quantize_dense_8b_16384_sampled_rows(ref, dev):
    m, n = 16384, wl.DENSE_8B["gate"][0]
    g = wl.rng(9)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(m - 8, m),
                                     g.choice(m, 256, replace=False)]))
    check(ref, dev, gate_up(7, m, n), rows=rows)


def test_silu_mul_special_values(ref, dev):
    # zeros, gates far below -80 (float64 path), products below 2^-120, large gates
    # (silu(g) = g to float32), an all-zero row (the zero guard) and rows of a single sign
    m, n = 8, 512
    gu = gate_up(11, m, n)
    f = (gu.astype(np.uint32) << 16).view(np.float32).copy()
    f[0, :n] = 0.0
    f[1, :64] = -85.0
    f[1, 64:128] = -100.0
    f[1, 128:192] = -300.0
    f[2, n:] = np.float32(1e-30)
    f[2, :n] = -20.0
    f[3, :n] = np.float32(50.0)
    f[4, :n] = np.abs(f[4, :n])
    f[4, n:] = np.abs(f[4, n:])
    f[5, n:] = 0.0
    gu2 = wl.bits16(wl.to_bf16(f))
    check(ref, dev, gu2, max_flagged=0.05)  # (rows of one repeated value flag together)


def test_silu_mul_binding_checks(dev):
    gu = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        i8.silu_mul_quantize_per_token_int8(torch.zeros((4, 63), dtype=torch.bfloat16, device=dev))
    with pytest.raises(TypeError):
        i8.silu_mul_bf16(gu.float())
    with pytest.raises(i8.I8qlError, match="I8QL_ERR_SHAPE"):
        i8.silu_mul_bf16(torch.zeros((4, 60), dtype=torch.bfloat16, device=dev))
    q, s = i8.silu_mul_quantize_per_token_int8(gu)
    assert torch.all(q == 0) and torch.all(s == 1.0)
