"""GPU: decoder layers with per-module schemes ("feat(quantization): support
compressed-tensors W8A8 and mixed modules", Design and Supported Execution Scheme), each fused
projection in the scheme its modules resolved to, against the oracle: W8A8 codes and int32
sums exact and the outputs within the float32 epilogue bound; W8A8-g128 and W8A16 within their
float32 summation bounds; the unquantized BF16 projection (a bf16 library GEMM, not on the int8
path) within the float32 summation bound of a K-long dot product."""
import numpy as np
import pytest
import torch

import int8_quantized_linear_amd as i8
from int8_quantized_linear_amd import layer
from int8_quantized_linear_amd import workloads as wl
from parity import U32, check_float, w8a16_tol, w8a8_tol

pytestmark = pytest.mark.gpu
P = "model.layers.0"


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


def build(g, m, dev):
    names = {"q_proj": "q", "k_proj": "k", "v_proj": "v", "o_proj": "o", "gate_proj": "gate",
             "up_proj": "up", "down_proj": "down"}
    w = {mod: wl.to_bf16(wl.weight(g, *wl.DENSE_4B[s])) for mod, s in names.items()}
    kin = {"attn_in": 2560, "attn_out": 4096, "mlp_in": 2560, "mlp_mid": 9728}
    x = {key: wl.to_bf16(wl.activations(g, m, k, 0.001)) for key, k in kin.items()}
    return w, x


def check(ref, scheme, fused, y, w_cat, x, bias=None):
    xb, wb = wl.bits16(x), wl.bits16(w_cat)
    k = x.shape[1]
    if scheme == layer.W8A8:
        qw, sw = ref.quantize_rows(wb, "bf16")
        qx, sx = ref.quantize_rows(xb, "bf16")
        acc, yref = ref.w8a8(qx, sx, qw, sw, bias)
        check_float(y, yref, w8a8_tol(acc, sx, sw, bias), f"{fused} w8a8")
    elif scheme == layer.W8A8_G128:
        qw, sw = ref.quantize_groups(wb, "bf16")
        qx, sx = ref.quantize_rows(xb, "bf16")
        yref = ref.w8a8_grouped_scales(qx, sx, qw, sw, 128, bias)
        wabs = np.abs(qw.astype(np.float64)) * np.repeat(sw.astype(np.float64), 128, axis=1)
        tol = (k // 128 + 3) * U32 * sx[:, None] * (np.abs(qx.astype(np.float64)) @ wabs.T)
        check_float(y, yref, tol, f"{fused} w8a8_g128")
    elif scheme == layer.W8A16:
        qw, sw = ref.quantize_rows(wb, "bf16")
        yref = ref.w8a16(xb, qw, sw, bias)
        absdot = np.abs(x.double().numpy()) @ (np.abs(qw.astype(np.float64)) * sw[:, None]).T
        check_float(y, yref, w8a16_tol(yref, absdot, k, bias), f"{fused} w8a16")
    else:
        xd, wd = x.double().numpy(), w_cat.double().numpy()
        yref = xd @ wd.T
        tol = (k + 8) * U32 * (np.abs(xd) @ np.abs(wd).T)
        check_float(y, yref, tol, f"{fused} bf16")


@pytest.mark.parametrize("case", ["hybrid_w8a8_bf16_o", "g128_with_w8a16_down", "all_bf16"])
def test_mixed_layer_against_the_oracle(ref, dev, case):
    groups = {"hybrid_w8a8_bf16_o": ([layer.QuantGroup("group_0", layer.W8A8, ["Linear"])],
                                     [f"{P}.self_attn.o_proj", "lm_head"]),
              "g128_with_w8a16_down": ([layer.QuantGroup("g", layer.W8A8_G128, ["Linear"]),
                                        layer.QuantGroup("d", layer.W8A16,
                                                         [r"re:.*\.down_proj"])], []),
              "all_bf16": ([], [])}[case]
    schemes = layer.resolve_layer(P, *groups)
    g = wl.rng(200)
    m = 96
    w, x = build(g, m, dev)
    dl = layer.DecoderLinears(schemes, {k: v.to(dev) for k, v in w.items()})
    out = dl.run({k: v.to(dev) for k, v in x.items()})
    for fused, parts in layer.FUSED.items():
        w_cat = torch.cat([w[p] for p in parts])
        check(ref, schemes[fused], fused, out[fused], w_cat, x[layer.FUSED_INPUT[fused]])
    if case == "hybrid_w8a8_bf16_o":
        assert schemes == {"qkv": "w8a8", "o": "bf16", "gate_up": "w8a8", "down": "w8a8"}
