"""GPU parity of the RMS norm fused with the per-token quantization (the producer of a
decoder layer's q/k/v and gate/up inputs) and of the unfused norm, through the C ABI against
the CPU oracle on the same seeded inputs: codes, scales, the bf16 norm output and the updated
residual are compared bitwise.  Shapes span both work layouts (one or four wavefronts per
row), ragged row counts, the largest row the kernel takes and the decoder workloads at full
size (the 4B layer's 128/512/2048 tokens at hidden 2560, the 8B layer's 4096/16384 tokens at
hidden 4096)."""
import numpy as np
import pytest
import torch

import int8_quantized_linear_amd as i8
from int8_quantized_linear_amd import workloads as wl

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


def bits_tensor(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(dev)


def gpu_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def norm_inputs(seed, m, k, residual, outlier_frac=0.01, scale=1.0):
    g = wl.rng(seed)
    x = wl.bits16(wl.to_bf16(wl.activations(g, m, k, outlier_frac=outlier_frac) *
                             np.float32(scale)))
    gamma = wl.bits16(wl.to_bf16(wl.norm_weight(g, k)))
    res = wl.bits16(wl.to_bf16(wl.activations(g, m, k) * np.float32(scale))) if residual else None
    return x, gamma, res


def run_case(ref, dev, m, k, residual, eps=1e-6, seed=0, x=None, gamma=None, res=None,
             both=True):
    if x is None:
        x, gamma, res = norm_inputs(seed, m, k, residual)
    q_ref, s_ref, res_ref = ref.rmsnorm_quantize(x, gamma, eps, res)
    xd, gd = bits_tensor(x, dev), bits_tensor(gamma, dev)
    # outputs in sentinel-filled buffers with a guard band past the end
    q_buf = torch.full((m * k + 64,), 0x55, dtype=torch.int8, device=dev)
    s_buf = torch.full((m + 16,), float("nan"), dtype=torch.float32, device=dev)
    q_out, s_out = q_buf[:m * k].view(m, k), s_buf[:m]
    rd = bits_tensor(res, dev) if res is not None else None
    i8.rmsnorm_quantize_per_token_int8(xd, gd, eps, rd, q_out=q_out, scale_out=s_out)
    np.testing.assert_array_equal(q_out.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s_out.cpu().numpy(), s_ref)
    assert torch.all(q_buf[m * k:] == 0x55) and torch.all(torch.isnan(s_buf[m:]))
    if res is not None:
        np.testing.assert_array_equal(gpu_bits(rd), res_ref)
    if both:
        # the unfused producer: bitwise the oracle's norm, and quantize_per_token_int8 of it
        # gives the fused call's codes
        h_ref, _ = ref.rmsnorm(x, gamma, eps, res)
        rd2 = bits_tensor(res, dev) if res is not None else None
        h_buf = torch.full((m * k + 64,), -7.0, dtype=torch.bfloat16, device=dev)
        h = h_buf[:m * k].view(m, k)
        i8.rmsnorm_bf16(xd, gd, eps, rd2, y_out=h)
        np.testing.assert_array_equal(gpu_bits(h), h_ref)
        assert torch.all(h_buf[m * k:] == -7.0)
        if res is not None:
            np.testing.assert_array_equal(gpu_bits(rd2), res_ref)
        q2, s2 = i8.quantize_per_token_int8(h)
        assert torch.equal(q2, q_out) and torch.equal(s2, s_out)


@pytest.mark.parametrize("m,k", [(1, 8), (3, 2560), (5, 4096), (130, 1000), (1100, 4096),
                                 (1027, 6144), (1030, 6152), (7, 24576), (2000, 12288)])
@pytest.mark.parametrize("residual", [False, True])
def test_rmsnorm_quantize_small_and_ragged(ref, dev, m, k, residual):
    run_case(ref, dev, m, k, residual, seed=m + k)


@pytest.mark.parametrize("m", wl.PREFILL_4B_TOKENS)
def test_rmsnorm_quantize_dense_4b_full(ref, dev, m):
    run_case(ref, dev, m, wl.DENSE_4B["q"][1], True, seed=7 + m)


@pytest.mark.parametrize("m", wl.PREFILL_8B_TOKENS)
def test_rmsnorm_quantize_dense_8b_full(ref, dev, m):
    run_case(ref, dev, m, wl.DENSE_8B["q"][1], True, eps=1e-5, seed=11 + m, both=m <= 4096)


def test_rmsnorm_quantize_special_rows(ref, dev):
    # all-zero rows (zero guard), power-of-two rows (exact normalization), rows whose mean
    # square is near eps, and a row holding one huge outlier
    m, k = 12, 2048
    x, gamma, _ = norm_inputs(5, m, k, False, outlier_frac=0.0)
    xf = (x.astype(np.uint32) << 16).view(np.float32).copy()
    xf[0] = 0.0
    xf[5] = 0.0
    xf[1] = np.where(xf[1] < 0, -4.0, 4.0)
    xf[2] = np.where(xf[2] < 0, -2.0 ** -40, 2.0 ** -40)
    xf[3] *= np.float32(1e-3)
    xf[4, 17] = np.float32(3e4)
    x2 = wl.bits16(wl.to_bf16(xf))
    for eps in (1e-6, 1e-30):
        run_case(ref, dev, m, k, False, eps=eps, x=x2, gamma=gamma, res=None)
    # with a residual that cancels the input exactly: u = 0 everywhere in that row
    res = x2.copy()
    res[7] = x2[7] ^ np.uint16(0x8000)
    run_case(ref, dev, m, k, True, x=x2, gamma=gamma, res=res)


def test_rmsnorm_quantize_deterministic_and_graph_replay(ref, dev):
    m, k = 512, 2560
    x, gamma, _ = norm_inputs(3, m, k, False)
    q_ref, s_ref, _ = ref.rmsnorm_quantize(x, gamma, 1e-6, None)
    xd, gd = bits_tensor(x, dev), bits_tensor(gamma, dev)
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    s = torch.empty((m,), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        i8.rmsnorm_quantize_per_token_int8(xd, gd, 1e-6, None, q_out=q, scale_out=s)  # warm
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        i8.rmsnorm_quantize_per_token_int8(xd, gd, 1e-6, None, q_out=q, scale_out=s)
    for _ in range(3):
        q.fill_(0)
        s.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
        np.testing.assert_array_equal(s.cpu().numpy(), s_ref)


def test_rmsnorm_binding_checks(dev):
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev)
    g = torch.ones((64,), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        i8.rmsnorm_quantize_per_token_int8(x, g[:32])
    with pytest.raises(TypeError):
        i8.rmsnorm_quantize_per_token_int8(x.float(), g)
    with pytest.raises(i8.I8qlError, match="I8QL_ERR_SHAPE"):
        i8.rmsnorm_bf16(torch.zeros((4, 60), dtype=torch.bfloat16, device=dev), g[:60])
    with pytest.raises(i8.I8qlError, match="I8QL_ERR_ARG"):
        i8.rmsnorm_bf16(x, g, eps=0.0)
