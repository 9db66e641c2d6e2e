"""GPU parity of the mixture-of-experts steps around the grouped GEMM: top-k routing, the
gate/up grouped GEMM with SiLU·mul fused, and the weighted combine, each through the C ABI
against the CPU oracle on the same inputs, and the whole block chained at the 16B MoE shapes
(each stage checked on the GPU's own output of the stage before).

Routing ids are decided by exact comparisons of the logits, so they must be equal; the
float outputs carry tolerances derived below from float32 rounding, as tests/parity.py
states for the other operations."""
import numpy as np
import pytest
import torch

import int8_quantized_linear_amd as i8
from int8_quantized_linear_amd import workloads as wl
from parity import U32, check_float, moe_stack, quant_gpu_vs_ref, sentinel, to_np, w8a16_tol

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


# ---------------------------------------------------------------------------------------
# routing

def route_tol(w_ref: np.ndarray) -> np.ndarray:
    """float32 softmax weight: the shifted logit (one rounding, |v - max| <= 64 here, so an
    absolute 64u inside exp), exp (a few ulp), a 256-term float32 sum (256u) and a division:
    400u relative covers all of it."""
    return 400 * U32 * np.abs(w_ref)


def run_route(ref, dev, logits32, k_routed, n_shared, dtype=torch.float32):
    t, e = logits32.shape
    lg = torch.from_numpy(logits32).to(dtype)
    lg_seen = lg.float().numpy()  # the values the kernel reads (bf16-rounded when bf16)
    ids = torch.full((t, k_routed + n_shared), -7, dtype=torch.int32, device=dev)
    w = sentinel((t, k_routed + n_shared), torch.float32, dev)
    i8.moe_route_topk(lg.to(dev), k_routed, n_shared, ids_out=ids, weights_out=w)
    rids, rw = ref.moe_route_topk(lg_seen, k_routed, n_shared)
    np.testing.assert_array_equal(ids.cpu().numpy(), rids)
    check_float(w, rw, route_tol(rw), f"route t={t} e={e} k={k_routed}")
    return ids, w


@pytest.mark.parametrize("t", [1, 4, 16, 64, 1000, 4097])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_route_16b(ref, dev, t, dtype):
    g = wl.rng(70 + t)
    run_route(ref, dev, wl.router_logits(g, t), wl.MOE_TOP, wl.MOE_SHARED, dtype)


@pytest.mark.parametrize("e,k,ns", [(256, 32, 32), (5, 5, 0), (1, 1, 1), (100, 8, 0),
                                    (200, 17, 3), (65, 6, 2), (128, 1, 0)])
def test_route_other_sizes(ref, dev, e, k, ns):
    g = wl.rng(80 + e)
    logits = g.standard_normal((37, e), dtype=np.float32) * np.float32(3.0)
    run_route(ref, dev, logits, k, ns)


def test_route_ties(ref, dev):
    # all equal; integer logits with many ties, inside and at the edge of the selection
    z = np.zeros((3, 64), np.float32)
    ids, _ = run_route(ref, dev, z, 6, 2)
    assert ids.cpu().numpy().tolist() == [[0, 1, 2, 3, 4, 5, 64, 65]] * 3
    g = wl.rng(90)
    li = g.integers(-3, 3, size=(50, 64)).astype(np.float32)
    run_route(ref, dev, li, 6, 2)
    run_route(ref, dev, g.integers(0, 2, size=(9, 200)).astype(np.float32), 17, 3)


# ---------------------------------------------------------------------------------------
# grouped gate/up with SiLU·mul

def silu_tol(gate, up, tg, tu, h_ref):
    """|d silu(g)/dg| <= 1.1, |silu(g)| <= |g| + 0.28: the gate and up errors propagate
    through silu(g) * u, plus float32 rounding of the epilogue (exp, division, products)."""
    sg = np.abs(gate) * (1.0 / (1.0 + np.exp(-np.clip(gate, -700, 700))))
    return 1.1 * np.abs(up) * tg + (sg + 1e-30) * tu + 8 * U32 * np.abs(h_ref)


def run_silu(ref, dev, qw, sw, qwr, swr, ids, xt, xv, per_assign, out_dtype):
    """qw [E, 2n, K] on the GPU, qwr/swr the oracle's; returns the GPU h."""
    e, n2, k = qwr.shape
    n = n2 // 2
    t, topk = ids.shape
    h = i8.grouped_w8a16_silu_gemm(xt.to(dev), qw, sw, torch.from_numpy(ids).to(dev),
                                   x_per_assignment=per_assign, out_dtype=out_dtype,
                                   out=sentinel((t * topk, n), out_dtype, dev))
    href = ref.grouped_w8a16_silu(xv, per_assign, qwr, swr, ids)
    gate = ref.grouped_w8a16(xv, per_assign, qwr[:, :n], swr[:, :n], ids)
    up = ref.grouped_w8a16(xv, per_assign, qwr[:, n:], swr[:, n:], ids)
    xd = np.abs(xt.double().numpy())
    dg = np.zeros_like(gate)
    du = np.zeros_like(up)
    for p in range(t * topk):
        ex = ids.flat[p]
        if 0 <= ex < e:
            xr = xd[p if per_assign else p // topk]
            dg[p] = (np.abs(qwr[ex, :n].astype(np.float64)) * swr[ex, :n, None]) @ xr
            du[p] = (np.abs(qwr[ex, n:].astype(np.float64)) * swr[ex, n:, None]) @ xr
    tol = silu_tol(gate, up, w8a16_tol(gate, dg, k), w8a16_tol(up, du, k), href)
    check_float(h, href, tol, f"silu e={e} n={n} k={k} t={t}")
    hc = to_np(h)
    for p in range(t * topk):
        if not 0 <= ids.flat[p] < e:
            assert np.all(hc[p] == 0.0)
    return h


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_silu_small_edge_cases(ref, dev, out_dtype):
    g = wl.rng(91)
    e, n, k = 7, 40, 272
    qw, sw, qwr, swr = moe_stack(ref, dev, g, 2 * n, k, e)
    ids = np.stack([g.choice(e, 3, replace=False) for _ in range(11)]).astype(np.int32)
    ids[2, 1] = -1
    ids[4, 0] = e
    ids[5] = 6
    for per_assign in (False, True):
        xt, xv = _bf16_rows(g, 33 if per_assign else 11, k)
        run_silu(ref, dev, qw, sw, qwr, swr, ids, xt, xv, per_assign, out_dtype)


def test_silu_few_tokens_and_long_k(ref, dev):
    """Fewer assignments than experts (the expert is picked from the bitmap) and a k that
    takes several batches per wavefront (4 wavefronts per tile at most)."""
    g = wl.rng(92)
    e, n, k = 20, 48, 6144
    qw, sw, qwr, swr = moe_stack(ref, dev, g, 2 * n, k, e)
    ids = np.array([[3, 17, 9], [9, 0, 19]], dtype=np.int32)
    xt, xv = _bf16_rows(g, 2, k)
    run_silu(ref, dev, qw, sw, qwr, swr, ids, xt, xv, False, torch.bfloat16)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_silu_one_token(ref, dev, out_dtype):
    """One token: the per-assignment kernel with gate and up rows together (ragged k), an
    invalid id and a repeated expert."""
    g = wl.rng(95)
    e, n, k = 6, 36, 1040
    qw, sw, qwr, swr = moe_stack(ref, dev, g, 2 * n, k, e)
    ids = np.array([[5, 2, -1, 2, 0]], dtype=np.int32)
    for per_assign in (False, True):
        xt, xv = _bf16_rows(g, 5 if per_assign else 1, k)
        run_silu(ref, dev, qw, sw, qwr, swr, ids, xt, xv, per_assign, out_dtype)


def test_silu_few_tokens(ref, dev):
    """Three tokens: the few-token kernel with gate and up rows together, an invalid id and
    an expert shared by every token."""
    g = wl.rng(96)
    e, n, k = 8, 20, 1040
    qw, sw, qwr, swr = moe_stack(ref, dev, g, 2 * n, k, e)
    ids = np.array([[7, 1, 4], [7, -1, 1], [7, 3, 3]], dtype=np.int32)
    for per_assign in (False, True):
        xt, xv = _bf16_rows(g, 9 if per_assign else 3, k)
        run_silu(ref, dev, qw, sw, qwr, swr, ids, xt, xv, per_assign, torch.bfloat16)


@pytest.mark.parametrize("e,n,k,t,topk", [(20, 13, 8192, 4, 16), (6, 24, 512, 2, 33),
                                          (9, 30, 2064, 3, 4), (40, 24, 2048, 8, 8),
                                          (12, 20, 1040, 6, 5), (30, 16, 256, 9, 6)])
def test_silu_few_tokens_shapes(ref, dev, e, n, k, t, topk):
    """The few-token kernel's SiLU·mul form at its longest k (8 chunks per lane), 4 chunks,
    64 assignments, and 66 (past it: the tiled kernel); 6 and 8 tokens, and 9 (past the
    token limit); invalid and repeated ids."""
    g = wl.rng(97 + k)
    qw, sw, qwr, swr = moe_stack(ref, dev, g, 2 * n, k, e)
    ids = np.stack([g.choice(e, topk, replace=topk > e) for _ in range(t)]).astype(np.int32)
    ids[0, 0] = -1
    ids[1, :2] = ids[0, 1]
    xt, xv = _bf16_rows(g, t, k)
    run_silu(ref, dev, qw, sw, qwr, swr, ids, xt, xv, False, torch.float32)


def test_silu_later_passes_split(ref, dev):
    """More tokens than two passes of 8 rows: later passes on extra rows of workgroups."""
    g = wl.rng(94)
    e, n, k = 5, 24, 256
    qw, sw, qwr, swr = moe_stack(ref, dev, g, 2 * n, k, e)
    ids = np.stack([g.choice(e, 2, replace=False) for _ in range(48)]).astype(np.int32)
    ids[9, 1] = e
    xt, xv = _bf16_rows(g, 48, k)
    run_silu(ref, dev, qw, sw, qwr, swr, ids, xt, xv, False, torch.bfloat16)


@pytest.mark.parametrize("t", wl.MOE_TOKENS)
def test_silu_moe_16b_full(ref, dev, t):
    g = wl.rng(93 + t)
    n, k = wl.MOE_16B["gate"]
    e = wl.MOE_ROUTED + wl.MOE_SHARED
    qw, sw, qwr, swr = moe_stack(ref, dev, g, 2 * n, k, e)
    ids = wl.moe_expert_ids(g, t)
    xt, xv = _bf16_rows(g, t, k)
    run_silu(ref, dev, qw, sw, qwr, swr, ids, xt, xv, False, torch.bfloat16)


def _bf16_rows(g, rows, k):
    xt = wl.to_bf16(wl.activations(g, rows, k))
    return xt, wl.bits16(xt)


# ---------------------------------------------------------------------------------------
# combine

def combine_tol(d64, w32, topk):
    """float32 accumulation of topk products in order: (topk + 2) u * sum_j |w_j d_j|."""
    t = w32.shape[0]
    mag = np.einsum("tj,tjc->tc", np.abs(w32.astype(np.float64)),
                    np.abs(d64).reshape(t, topk, -1))
    return (topk + 2) * U32 * mag + 1e-30


def run_combine(ref, dev, d, w, out_dtype, out=None):
    t, topk = w.shape
    y = i8.moe_combine(d, w, out_dtype=out_dtype,
                       out=out if out is not None else sentinel((t, d.shape[1]), out_dtype, dev))
    d64 = to_np(d).astype(np.float64)
    w32 = w.cpu().numpy()
    yr = ref.moe_combine(d64.astype(np.float32), w32)
    check_float(y, yr, combine_tol(d64, w32, topk), f"combine t={t} topk={topk}")
    return y


@pytest.mark.parametrize("t", wl.MOE_TOKENS)
@pytest.mark.parametrize("d_dtype,y_dtype", [(torch.bfloat16, torch.bfloat16),
                                             (torch.float32, torch.float32),
                                             (torch.bfloat16, torch.float32)])
def test_combine_16b(ref, dev, t, d_dtype, y_dtype):
    g = wl.rng(100 + t)
    topk, n = wl.MOE_TOP + wl.MOE_SHARED, wl.MOE_16B["down"][0]
    d = torch.from_numpy(g.standard_normal((t * topk, n), dtype=np.float32)).to(d_dtype).to(dev)
    w = torch.from_numpy(g.random((t, topk), dtype=np.float32)).to(dev)
    run_combine(ref, dev, d, w, y_dtype)


def test_combine_element_path(ref, dev):
    """Rows that are not whole 16-byte chunks, and a misaligned output, take the element
    path; the results agree with the 16-byte path's."""
    g = wl.rng(110)
    t, topk, n = 5, 3, 1001
    d = torch.from_numpy(g.standard_normal((t * topk, n), dtype=np.float32)).to(
        torch.bfloat16).to(dev)
    w = torch.from_numpy(g.random((t, topk), dtype=np.float32)).to(dev)
    run_combine(ref, dev, d, w, torch.bfloat16)
    n = 1024
    d = torch.from_numpy(g.standard_normal((t * topk, n), dtype=np.float32)).to(dev)
    w = torch.from_numpy(g.random((t, topk), dtype=np.float32)).to(dev)
    y_vec = run_combine(ref, dev, d, w, torch.float32)
    buf = torch.full((t * n + 1,), float("nan"), dtype=torch.float32, device=dev)
    y_mis = run_combine(ref, dev, d, w, torch.float32, out=buf[1:].view(t, n))
    assert torch.equal(y_vec, y_mis)


# ---------------------------------------------------------------------------------------
# the block, chained at the 16B MoE shapes

@pytest.mark.parametrize("t", [1, 4, 16, 64])
def test_moe_block_chain_16b(ref, dev, t):
    """logits -> route -> gate/up with SiLU·mul -> down -> combine, each stage against the
    oracle on the GPU's output of the stage before."""
    g = wl.rng(120 + t)
    e = wl.MOE_ROUTED + wl.MOE_SHARED
    n_i, hid = wl.MOE_16B["gate"]          # intermediate 1408, hidden 2048
    qgu, sgu, qgur, sgur = moe_stack(ref, dev, g, 2 * n_i, hid, e)
    qd, sd, qdr, sdr = moe_stack(ref, dev, g, hid, n_i, e)
    ids, w = run_route(ref, dev, wl.router_logits(g, t), wl.MOE_TOP, wl.MOE_SHARED)
    ids_np = ids.cpu().numpy()
    xt, xv = _bf16_rows(g, t, hid)
    h = run_silu(ref, dev, qgu, sgu, qgur, sgur, ids_np, xt, xv, False, torch.bfloat16)
    # down: one row per assignment, the GPU's h as input
    hb = h.cpu()
    d = i8.grouped_w8a16_gemm(h, qd, sd, ids, x_per_assignment=True,
                              out=sentinel((t * ids_np.shape[1], hid), torch.bfloat16, dev))
    hv = wl.bits16(hb)
    dref = ref.grouped_w8a16(hv, 1, qdr, sdr, ids_np)
    hd = np.abs(hb.double().numpy())
    absdot = np.stack([(np.abs(qdr[ids_np.flat[p]].astype(np.float64))
                        * sdr[ids_np.flat[p]][:, None]) @ hd[p]
                       for p in range(ids_np.size)])
    check_float(d, dref, w8a16_tol(dref, absdot, n_i), f"down t={t}")
    run_combine(ref, dev, d, w, torch.bfloat16)


# ---------------------------------------------------------------------------------------
# the block and the group-scale path replayed from a HIP graph

def test_graph_replays_of_the_grouped_row_paths_match_eager(ref, dev):
    """The one-token kernel (plain and SiLU·mul), the few-token kernel (SiLU·mul, 3 tokens)
    and the later-pass split with the occupancy-sized tile walk (40 tokens), captured in one
    graph and replayed three times with eager work between the replays."""
    g = wl.rng(171)
    e, n_i, hid = 6, 32, 256
    qgu, sgu, _, _ = moe_stack(ref, dev, g, 2 * n_i, hid, e)
    qd, sd, _, _ = moe_stack(ref, dev, g, hid, n_i, e)
    cases = []
    for t, topk in ((1, 4), (3, 4), (40, 4)):
        ids = torch.from_numpy(np.stack([g.choice(e, topk, replace=False)
                                         for _ in range(t)]).astype(np.int32)).to(dev)
        x = wl.to_bf16(wl.activations(g, t, hid)).to(dev)
        h = torch.empty((t * topk, n_i), dtype=torch.bfloat16, device=dev)
        d = torch.empty((t * topk, hid), dtype=torch.bfloat16, device=dev)
        yp = torch.empty((t * topk, n_i), dtype=torch.float32, device=dev)
        cases.append((ids, x, h, d, yp))

    def path():
        for ids, x, h, d, yp in cases:
            i8.grouped_w8a16_silu_gemm(x, qgu, sgu, ids, out=h)
            i8.grouped_w8a16_gemm(h, qd, sd, ids, x_per_assignment=True, out=d)
            i8.grouped_w8a16_gemm(x, qgu[:, :n_i].contiguous(), sgu[:, :n_i].contiguous(), ids,
                                  out_dtype=torch.float32, out=yp)

    outs = [o for c in cases for o in c[2:]]
    path()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        path()  # eager work between replays
        torch.cuda.synchronize()


def test_graph_replays_of_the_block_match_eager(ref, dev):
    g = wl.rng(170)
    e, n_i, hid, t = 10, 64, 256, 5
    qgu, sgu, _, _ = moe_stack(ref, dev, g, 2 * n_i, hid, e)
    qd, sd, _, _ = moe_stack(ref, dev, g, hid, n_i, e)
    logits = torch.from_numpy(wl.router_logits(g, t, routed=e - 2)).to(dev)
    x = wl.to_bf16(wl.activations(g, t, hid)).to(dev)
    wg = wl.to_bf16(wl.weight(g, 96, 512)).to(dev)
    xg = wl.to_bf16(wl.activations(g, 3, 512)).to(dev)
    ids = torch.empty((t, 6), dtype=torch.int32, device=dev)
    w = torch.empty((t, 6), dtype=torch.float32, device=dev)
    h = torch.empty((t * 6, n_i), dtype=torch.bfloat16, device=dev)
    d = torch.empty((t * 6, hid), dtype=torch.bfloat16, device=dev)
    y = torch.empty((t, hid), dtype=torch.bfloat16, device=dev)
    qg = torch.empty((96, 512), dtype=torch.int8, device=dev)
    sg = torch.empty((96, 4), dtype=torch.float32, device=dev)
    yg = torch.empty((3, 96), dtype=torch.float32, device=dev)

    def path():
        i8.moe_route_topk(logits, 4, 2, ids_out=ids, weights_out=w)
        i8.grouped_w8a16_silu_gemm(x, qgu, sgu, ids, out=h)
        i8.grouped_w8a16_gemm(h, qd, sd, ids, x_per_assignment=True, out=d)
        i8.moe_combine(d, w, out=y)
        i8.quantize_per_group_int8(wg, q_out=qg, scale_out=sg)
        i8.w8a16_gemm_g128(xg, qg, sg, out_dtype=torch.float32, out=yg)

    outs = (ids, w, h, d, y, qg, sg, yg)
    path()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        path()  # eager work between replays
        torch.cuda.synchronize()
