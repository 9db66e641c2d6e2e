"""The allocation-free W8A8 entry point (w8a8_gemm_noalloc, the library's static scratch as
the workspace) through the C ABI, against the entry point it varies (w8a8_gemm_with_plan with
a caller workspace of the same size) and the oracle: two calls in a row, the second with a
smaller input, both on shapes whose plan splits k (so the scratch is used)."""
import numpy as np
import pytest
import torch

import int8_quantized_linear_amd as i8
from int8_quantized_linear_amd import workloads as wl
from parity import check_float, host, quant_gpu_vs_ref, sentinel, w8a8_tol

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


def test_noalloc_matches_the_workspace_entry_point(ref, dev):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ws = torch.zeros(i8.W8A8_SCRATCH_BYTES, dtype=torch.uint8, device=dev)
    # the 4B down projection at 512, then at 128 tokens (smaller), both split plans
    for m, n, k in ((512, 2560, 9728), (128, 2560, 9728)):
        print(f"noalloc {m}x{n}x{k}", flush=True)
        plan = i8.w8a8_gemm_choose_plan(m, n, k, cus, i8.W8A8_SCRATCH_BYTES)
        assert plan[1] > 1, plan
        g = wl.rng(m + n + k)
        wt, wv = host("bf16", wl.weight(g, n, k))
        xt, xv = host("bf16", wl.activations(g, m, k, outlier_frac=0.001))
        qw, sw, qwr, swr = quant_gpu_vs_ref(ref, dev, wt, wv, "bf16")
        qx, sx, qxr, sxr = quant_gpu_vs_ref(ref, dev, xt, xv, "bf16", per_token=True)
        b_np = (g.standard_normal(n, dtype=np.float32) * np.float32(0.02)).astype(np.float32)
        b = torch.from_numpy(b_np).to(dev)
        acc, yref = ref.w8a8(qxr, sxr, qwr, swr, b_np)
        yi = i8.w8a8_gemm_noalloc(qx, None, qw, None, out_dtype=torch.int32,
                                  out=sentinel((m, n), torch.int32, dev))
        yi_ws = i8.w8a8_gemm_with_plan(-1, -1, qx, None, qw, None, out_dtype=torch.int32,
                                       workspace=ws)
        np.testing.assert_array_equal(yi.cpu().numpy(), acc)
        assert torch.equal(yi, yi_ws)
        for od in (torch.bfloat16, torch.float32):
            y = i8.w8a8_gemm_noalloc(qx, sx, qw, sw, b, out_dtype=od,
                                     out=sentinel((m, n), od, dev))
            y_ws = i8.w8a8_gemm_with_plan(-1, -1, qx, sx, qw, sw, b, out_dtype=od, workspace=ws)
            check_float(y, yref, w8a8_tol(acc, sxr, swr, b_np), f"noalloc {m}x{n}x{k} {od}")
            assert torch.equal(y, y_ws)
        # an explicit plan that needs more than the scratch is rejected before any launch
        big = (6, 8)
        assert i8.w8a8_gemm_workspace_size(m * 16, n, k, cus, *big) > i8.W8A8_SCRATCH_BYTES
        qbig = torch.zeros((m * 16, k), dtype=torch.int8, device=dev)
        with pytest.raises(i8.I8qlError, match="I8QL_ERR_WORKSPACE"):
            i8.w8a8_gemm_noalloc(qbig, None, qw, None, out_dtype=torch.int32, config=big[0],
                                 splits=big[1])
