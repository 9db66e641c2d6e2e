"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the same seeded
inputs.  Codes, scales and int32 accumulators must be bitwise equal; float outputs follow
the rules in tests/parity.py.  Small cases span several tiles and ragged tails; the
decoder-shaped workloads run at full size, every row compared up to 4096 tokens (sampled
rows only at 16384 tokens), each shape in float32 as well as in its bf16 (and, for W8A8,
int32) output mode."""
import numpy as np
import pytest
import torch

import int8_quantized_linear_amd as i8
from int8_quantized_linear_amd import workloads as wl
from parity import check_float, host, moe_stack, quant_gpu_vs_ref, sentinel, to_np, \
    w8a16_tol, w8a8_tol

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
# quantizers

QSHAPES = [(1, 1), (3, 7), (5, 16), (37, 1001), (130, 1000), (64, 2560), (9, 12288),
           (6, 16384), (4, 24600)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", QSHAPES)
def test_quantize_rows_small(ref, dev, dtype, shape):
    g = wl.rng(100 + shape[0])
    a = g.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    if shape[0] > 2:
        a[1] = 0.0                       # all-zero channel
        a[2] *= np.float32(1e-4)         # small channel keeps its full range
    a[:, g.choice(shape[1], 1)] *= np.float32(50.0)
    t, view = host(dtype, a)
    for per_token in (False, True):
        quant_gpu_vs_ref(ref, dev, t, view, dtype, per_token)


def test_quantize_ties_and_subnormals(ref, dev):
    s = 2.0 ** -7
    halves = np.array([0.5, 1.5, 2.5, 62.5, 125.5, 126.5])
    row = (np.concatenate([[127.0], halves, -halves, np.zeros(3)]) * s).astype(np.float32)
    sub = np.array([1e-44, -5e-45, 3e-40, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0], np.float32)
    a = np.stack([row, sub, np.ldexp(row, -130).astype(np.float32)])
    for dtype in ("f32", "bf16"):
        t, view = host(dtype, a)
        quant_gpu_vs_ref(ref, dev, t, view, dtype)


def near_tie_rows(dtype, rows, k, seed):
    """Rows whose elements sit within a few ulps of half-integer multiples of the row scale
    (element 0 holds the row maximum), so that a quotient taken through a rounded reciprocal
    of the scale often rounds the other way than the correctly rounded quotient."""
    g = wl.rng(seed)
    f32 = np.float32
    out = np.empty((rows, k), np.float32)
    naive_differs = 0
    for r in range(rows):
        amax = f32(g.uniform(0.05, 50.0))
        sc = f32(amax / f32(127.0))
        if dtype == "f32":
            n = g.integers(-127, 127, size=k - 1).astype(np.float64)
            x = ((n + 0.5) * np.float64(sc)).astype(np.float32)
            for _ in range(3):
                step = g.integers(-1, 2, size=x.size)
                x = np.where(step > 0, np.nextafter(x, f32(np.inf)),
                             np.where(step < 0, np.nextafter(x, f32(-np.inf)), x))
            x = np.clip(x, -amax, amax)
        else:  # the bf16 values in [-amax, amax] whose quotients are closest to x.5
            amax = (np.array([amax], np.float32).view(np.uint32) & 0xffff0000).view(np.float32)[0]
            sc = f32(amax / f32(127.0))
            vals = (np.arange(0, 0x10000, dtype=np.uint32) << 16).view(np.float32)
            vals = vals[np.isfinite(vals) & (np.abs(vals) <= amax)]
            qv = (vals / sc).astype(np.float32)
            closest = vals[np.argsort(np.abs(np.abs(qv - np.rint(qv)) - 0.5))[:512]]
            x = g.choice(closest, size=k - 1)
        out[r, 0] = amax
        out[r, 1:] = x
        rec = f32(f32(1.0) / sc)
        naive_differs += int(np.sum(np.rint((x * rec).astype(np.float32)) !=
                                    np.rint((x / sc).astype(np.float32))))
    return out, naive_differs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,k", [(1100, 512), (8, 4096)])
def test_quantize_near_ties(ref, dev, dtype, rows, k):
    """Codes of quotients within a few ulps of x.5 (one and four wavefronts per row)."""
    a, naive_differs = near_tie_rows(dtype, rows, k, seed=rows + k)
    assert naive_differs > 0  # the data does separate a reciprocal shortcut from division
    t, view = host(dtype, a)
    for per_token in (False, True):
        quant_gpu_vs_ref(ref, dev, t, view, dtype, per_token)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_multi_matches_the_oracle_and_single_launches(ref, dev, dtype):
    """Several matrices in one launch: one and four wavefronts per row, rows up to 24 KiB
    and beyond (the streamed path), an empty matrix; codes and scales bitwise the oracle's
    and those of quantize_per_token_int8 one matrix at a time."""
    g = wl.rng(60)
    shapes = [(128, 2560), (0, 512), (2048, 9728), (1100, 4096), (3, 16384), (700, 13000),
              (2, 53248)]
    ts, views = [], []
    for (r, k) in shapes:
        a = wl.activations(g, r, k, outlier_frac=0.01)
        if r > 2:
            a[1] = 0.0                                     # an all-zero token
        t, v = host(dtype, a)
        ts.append(t.to(dev))
        views.append(v)
    got = i8.quantize_per_token_int8_multi(ts)
    for t, v, (q, s) in zip(ts, views, got):
        qr, sr = ref.quantize_rows(v, dtype) if t.shape[0] else (np.zeros(t.shape, np.int8),
                                                                np.zeros(0, np.float32))
        np.testing.assert_array_equal(q.cpu().numpy(), qr)
        np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))
        if t.shape[0]:
            q1, s1 = i8.quantize_per_token_int8(t)
            assert torch.equal(q1, q) and torch.equal(s1, s)


def test_quantize_unaligned_base_uses_the_general_path(ref, dev):
    a = wl.weight(wl.rng(5), 33, 520)
    t, view = host("bf16", a)
    big = torch.empty(t.numel() + 1, dtype=torch.bfloat16, device=dev)
    big[1:] = t.reshape(-1).to(dev)
    q, s = i8.quantize_per_channel_int8(big[1:].view(33, 520))
    qr, sr = ref.quantize_rows(view, "bf16")
    np.testing.assert_array_equal(q.cpu().numpy(), qr)
    np.testing.assert_array_equal(s.cpu().numpy(), sr)


def test_quantize_guard_bands(ref, dev):
    a = wl.weight(wl.rng(6), 45, 264)
    t, view = host("bf16", a)
    qbuf = torch.full((45 * 264 + 512,), 0x5A, dtype=torch.int8, device=dev)
    sbuf = torch.full((45 + 64,), 7.0, dtype=torch.float32, device=dev)
    q, s = i8.quantize_per_channel_int8(t.to(dev), qbuf[256:256 + 45 * 264].view(45, 264),
                                        sbuf[32:32 + 45])
    qr, sr = ref.quantize_rows(view, "bf16")
    np.testing.assert_array_equal(q.cpu().numpy(), qr)
    assert torch.all(qbuf[:256] == 0x5A) and torch.all(qbuf[256 + 45 * 264:] == 0x5A)
    assert torch.all(sbuf[:32] == 7.0) and torch.all(sbuf[32 + 45:] == 7.0)


WEIGHT_SHAPES = sorted(set(wl.DENSE_4B.values()) | set(wl.DENSE_8B.values()))


@pytest.mark.parametrize("shape", WEIGHT_SHAPES)
def test_quantize_decoder_weights_full(ref, dev, shape):
    t, view = host("bf16", wl.weight(wl.rng(shape[0] + shape[1]), *shape))
    quant_gpu_vs_ref(ref, dev, t, view, "bf16")


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_quantize_moe_expert_stack_full(ref, dev, proj):
    n, k = wl.MOE_16B[proj]
    w = wl.moe_weights(wl.rng(7), n, k).reshape(-1, k)
    t, view = host("bf16", w)
    quant_gpu_vs_ref(ref, dev, t, view, "bf16")


@pytest.mark.parametrize("m,k,frac", [(2048, 2560, 0.001), (2048, 9728, 0.001),
                                      (16384, 4096, 0.01), (16384, 12288, 0.01)])
def test_quantize_prefill_activations_full(ref, dev, m, k, frac):
    t, view = host("bf16", wl.activations(wl.rng(m + k), m, k, outlier_frac=frac))
    quant_gpu_vs_ref(ref, dev, t, view, "bf16", per_token=True)


# ---------------------------------------------------------------------------------------
# W8A8

def w8a8_case(g, m, n, k, wdtype="bf16"):
    w = wl.weight(g, n, k)
    x = wl.activations(g, m, k, outlier_frac=0.001)
    return host(wdtype, w), host(wdtype, x)


def run_w8a8(ref, dev, m, n, k, out_dtypes=(torch.int32, torch.float32, torch.bfloat16),
             seed=0, with_bias=(False, True), config=-1, splits=None, workspace=None):
    g = wl.rng(seed)
    (wt, wv), (xt, xv) = w8a8_case(g, m, n, k)
    qw, sw, qwr, swr = quant_gpu_vs_ref(ref, dev, wt, wv, "bf16")
    qx, sx, qxr, sxr = quant_gpu_vs_ref(ref, dev, xt, xv, "bf16", per_token=True)
    bias_np = (g.standard_normal(n, dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    for use_bias in with_bias:
        b_np = bias_np if use_bias else None
        acc, yref = ref.w8a8(qxr, sxr, qwr, swr, b_np)
        for od in out_dtypes:
            if od == torch.int32:
                if use_bias:
                    continue
                y = gemm(config, splits, workspace, qx, None, qw, None, None, torch.int32,
                         sentinel((m, n), torch.int32, dev))
                np.testing.assert_array_equal(y.cpu().numpy(), acc)
                continue
            b = torch.from_numpy(b_np).to(dev) if use_bias else None
            y = gemm(config, splits, workspace, qx, sx, qw, sw, b, od, sentinel((m, n), od, dev))
            check_float(y, yref, w8a8_tol(acc, sxr, swr, b_np), f"w8a8 {m}x{n}x{k} {od}")


def gemm(config, splits, workspace, qx, sx, qw, sw, b, od, out):
    """One W8A8 call: a tile configuration without a split (splits None), or a plan."""
    if splits is None:
        return i8.w8a8_gemm_with_config(config, qx, sx, qw, sw, b, out_dtype=od, out=out)
    return i8.w8a8_gemm_with_plan(config, splits, qx, sx, qw, sw, b, out_dtype=od, out=out,
                                  workspace=workspace)


# Shapes through the cost model's choice of tile configuration (ragged edges, partial last
# k steps, one to three k steps); every configuration is also run explicitly below.
@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (4, 256, 512), (3, 130, 48), (130, 200, 272),
                                   (257, 385, 1040), (128, 128, 128), (64, 700, 4096),
                                   (300, 33, 2576), (600, 1300, 768), (700, 1500, 512),
                                   (1100, 3000, 16),
                                   (1100, 3000, 144), (1100, 3000, 272), (2100, 2600, 16),
                                   (2100, 2600, 1040), (3000, 4100, 272)])
def test_w8a8_small(ref, dev, m, n, k):
    run_w8a8(ref, dev, m, n, k, seed=m * 7 + n)


@pytest.mark.parametrize("config", range(i8.W8A8_NUM_CONFIGS))
def test_w8a8_every_tile_config(ref, dev, config):
    """Each tile configuration, forced: two tiles and a ragged third in each direction with
    four k steps (the last partial) and with one partial step; then more than one group of
    eight tile rows of the workgroup-to-tile map.  k-group configurations take k in whole
    steps per group.  N a multiple of 8 takes the LDS-staged 16-byte-store epilogue, an odd N
    the per-element one."""
    bm, bn, groups, _, _ = i8.w8a8_gemm_config_info(config)
    if groups == 1:
        shapes = [(2 * bm + 37, 2 * bn + 24, 432), (2 * bm + 37, 2 * bn + 19, 16),
                  (9 * bm + 5, 3 * bn + 8, 144)]
    else:
        shapes = [(2 * bm + 37, 2 * bn + 24, 256 * groups), (9 * bm + 5, 3 * bn + 7, 128 * groups)]
    for (m, n, k) in shapes:
        print(f"w8a8 config {config} ({bm}x{bn}, {groups} k-groups): {m}x{n}x{k}", flush=True)
        run_w8a8(ref, dev, m, n, k, seed=config * 31 + m, config=config)


@pytest.mark.parametrize("m,n,k", [(2100, 8200, 272), (4100, 4104, 256), (2310, 7700, 528),
                                   (2100, 8196, 400), (2100, 8200, 384), (2310, 7700, 1280),
                                   (4353, 4360, 640)])
def test_w8a8_persistent_tiles(ref, dev, m, n, k):
    """256 x 256 tiles (configuration 0) with more tiles than compute units, which runs the
    persistent kernel (one workgroup per compute unit walking tiles, the next tile's first
    two k steps loaded during the current tile's last two): ragged edges in m and n, partial
    and whole last k steps, exactly two and three k steps, tile counts that leave some
    workgroups one tile fewer, and an N whose float32 rows are whole 16-byte chunks but whose
    bf16 rows are not (bf16 then takes the per-tile kernel)."""
    assert i8.w8a8_gemm_config_info(0)[:2] == (256, 256)
    assert ((m + 255) // 256) * ((n + 255) // 256) > 256
    print(f"w8a8 persistent 256x256: {m}x{n}x{k}", flush=True)
    run_w8a8(ref, dev, m, n, k, seed=m + n + k, config=0)


SPLITTABLE = [c for c in range(i8.W8A8_NUM_CONFIGS) if i8.w8a8_gemm_config_info(c)[3]]


@pytest.mark.parametrize("config", SPLITTABLE)
def test_w8a8_split_plans(ref, dev, config):
    """k split across 2, 3, 5 and 8 workgroups per tile with each configuration that allows
    it: ragged tiles in both directions, a partial last k step (owned by the last split),
    splits of unequal step counts, and one workspace reused by every call, whose tile
    counters must be back at zero after each."""
    bm, bn, _, _, _ = i8.w8a8_gemm_config_info(config)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    for splits, (m, n, k) in [(2, (2 * bm + 37, 2 * bn + 24, 1040)),
                              (3, (bm + 5, 3 * bn + 8, 2576)),
                              (5, (3 * bm, bn + 16, 1152)),
                              (8, (37, 2 * bn + 19, 8 * 128 + 16))]:
        print(f"w8a8 plan ({config}, {splits}) {bm}x{bn}: {m}x{n}x{k}", flush=True)
        need = i8.w8a8_gemm_workspace_size(m, n, k, 256, config, splits)
        assert 0 < need <= ws.numel()
        run_w8a8(ref, dev, m, n, k, seed=config * 17 + splits, config=config, splits=splits,
                 workspace=ws)
        torch.cuda.synchronize()
        assert torch.all(ws[:16384] == 0), "arrival counters not returned to zero"


def test_w8a8_split_plans_agree_with_unsplit(dev):
    """Every split count of every splittable configuration gives bitwise the outputs of the
    same configuration without a split, for int32, float32 and bf16 (with bias)."""
    g = wl.rng(12)
    m, n, k = 700, 900, 2048
    qx = torch.from_numpy(g.integers(-127, 128, (m, k), dtype=np.int8)).to(dev)
    qw = torch.from_numpy(g.integers(-127, 128, (n, k), dtype=np.int8)).to(dev)
    sx = torch.rand(m, device=dev) * 0.01
    sw = torch.rand(n, device=dev) * 0.01
    b = torch.randn(n, device=dev) * 0.02
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    for c in SPLITTABLE:
        # (the workspace keeps the previous configurations' partial tiles: only the counter
        # region has to be, and is, zero)
        want = {od: i8.w8a8_gemm_with_config(c, qx, sx, qw, sw, b, out_dtype=od)
                for od in (torch.float32, torch.bfloat16)}
        want_i = i8.w8a8_gemm_with_config(c, qx, None, qw, None, out_dtype=torch.int32)
        for s in range(2, i8.W8A8_MAX_SPLITS + 1):
            for od, y in want.items():
                got = i8.w8a8_gemm_with_plan(c, s, qx, sx, qw, sw, b, out_dtype=od, workspace=ws)
                assert torch.equal(got, y), (c, s, od)
            got = i8.w8a8_gemm_with_plan(c, s, qx, None, qw, None, out_dtype=torch.int32,
                                         workspace=ws)
            assert torch.equal(got, want_i), (c, s)
        assert torch.all(ws[:16384] == 0)


def test_w8a8_configs_agree_bitwise(dev):
    """All configurations give bitwise the same int32, float32 and bf16 outputs (exact int32
    accumulation, one epilogue), on a shape every configuration accepts."""
    g = wl.rng(11)
    m, n, k = 1000, 1500, 1024
    qx = torch.from_numpy(g.integers(-127, 128, (m, k), dtype=np.int8)).to(dev)
    qw = torch.from_numpy(g.integers(-127, 128, (n, k), dtype=np.int8)).to(dev)
    sx = torch.rand(m, device=dev) * 0.01
    sw = torch.rand(n, device=dev) * 0.01
    b = torch.randn(n, device=dev) * 0.02
    want = {od: i8.w8a8_gemm(qx, sx, qw, sw, b, out_dtype=od)
            for od in (torch.float32, torch.bfloat16)}
    want_i = i8.w8a8_gemm(qx, None, qw, None, out_dtype=torch.int32)
    for c in range(i8.W8A8_NUM_CONFIGS):
        for od, y in want.items():
            assert torch.equal(i8.w8a8_gemm_with_config(c, qx, sx, qw, sw, b, out_dtype=od), y), c
        assert torch.equal(i8.w8a8_gemm_with_config(c, qx, None, qw, None,
                                                    out_dtype=torch.int32), want_i), c


def test_w8a8_tiny_workload_end_to_end(ref, dev):
    """fp32 weight [256,512] with 2 zero channels and a x50 column; 4 tokens with 2 x100
    dims; per-channel + per-token int8, int32 GEMM, fp32 output; seed 0."""
    t = wl.tiny_w8a8(0)
    wt, wv = host("f32", t["w"])
    xt, xv = host("f32", t["x"])
    qw, sw, qwr, swr = quant_gpu_vs_ref(ref, dev, wt, wv, "f32")
    qx, sx, qxr, sxr = quant_gpu_vs_ref(ref, dev, xt, xv, "f32", per_token=True)
    acc, yref = ref.w8a8(qxr, sxr, qwr, swr)
    y = i8.w8a8_gemm(qx, sx, qw, sw, out_dtype=torch.float32)
    check_float(y, yref, w8a8_tol(acc, sxr, swr, None), "tiny w8a8")
    yc = y.cpu().numpy()
    for r in t["zero_rows"]:
        assert np.all(yc[:, r] == 0.0)
    np.testing.assert_array_equal(i8.w8a8_gemm(qx, None, qw, None, out_dtype=torch.int32)
                                  .cpu().numpy(), acc)


def test_w8a8_extreme_accumulator(ref, dev):
    k = 133136  # largest multiple of 16 below the int32 limit
    xq = torch.full((2, k), 127, dtype=torch.int8, device=dev)
    xq[1] = -127
    wq = torch.full((3, k), 127, dtype=torch.int8, device=dev)
    wq[2] = -127
    y = i8.w8a8_gemm(xq, None, wq, None, out_dtype=torch.int32).cpu().numpy()
    v = k * 127 * 127
    np.testing.assert_array_equal(y, [[v, v, -v], [-v, -v, v]])


def test_w8a8_deterministic_and_guarded(ref, dev):
    g = wl.rng(3)
    qx = torch.from_numpy(g.integers(-127, 128, (200, 1024), dtype=np.int8)).to(dev)
    qw = torch.from_numpy(g.integers(-127, 128, (300, 1024), dtype=np.int8)).to(dev)
    sx = torch.rand(200, device=dev) * 0.01
    sw = torch.rand(300, device=dev) * 0.01
    buf = torch.full((200 * 300 + 1024,), -7.0, dtype=torch.float32, device=dev)
    y1 = i8.w8a8_gemm(qx, sx, qw, sw, out_dtype=torch.float32, out=buf[512:512 + 60000].view(200, 300))
    y2 = i8.w8a8_gemm(qx, sx, qw, sw, out_dtype=torch.float32)
    assert torch.equal(y1, y2)
    assert torch.all(buf[:512] == -7.0) and torch.all(buf[512 + 60000:] == -7.0)
    # an output 4 bytes off 16-byte alignment takes the per-element epilogue: same values,
    # guard bands intact
    buf.fill_(-7.0)
    y3 = i8.w8a8_gemm(qx, sx, qw, sw, out_dtype=torch.float32, out=buf[513:513 + 60000].view(200, 300))
    assert torch.equal(y3, y2)
    assert torch.all(buf[:513] == -7.0) and torch.all(buf[513 + 60000:] == -7.0)
    hb = torch.zeros((200 * 304 + 64,), dtype=torch.bfloat16, device=dev)
    y4 = i8.w8a8_gemm(qx[:, :1024], sx, qw[:4].repeat(76, 1), sw[:4].repeat(76),
                      out_dtype=torch.bfloat16, out=hb[1:1 + 200 * 304].view(200, 304))
    y5 = i8.w8a8_gemm(qx[:, :1024], sx, qw[:4].repeat(76, 1), sw[:4].repeat(76),
                      out_dtype=torch.bfloat16)
    assert torch.equal(y4, y5)
    assert torch.all(hb[:1] == 0) and torch.all(hb[1 + 200 * 304:] == 0)


def sampled_rows(m, n_rand=256, seed=0):
    g = wl.rng(seed)
    rows = set(range(min(8, m))) | set(range(max(0, m - 8), m))
    rows |= set(g.choice(m, min(n_rand, m), replace=False).tolist())
    return np.array(sorted(rows))


PREFILL_4B = [(m, n, k) for m in wl.PREFILL_4B_TOKENS for (n, k) in wl.DENSE_4B.values()]
# the fused launches of the benchmark step (q/k/v and gate/up over concatenated weights)
PREFILL_4B += [(m, sum(wl.DENSE_4B[p][0] for p in parts), wl.DENSE_4B[parts[0]][1])
               for m in wl.PREFILL_4B_TOKENS for parts in wl.DENSE_4B_FUSED.values()
               if len(parts) > 1]
PREFILL_8B = [(m, n, k) for m in wl.PREFILL_8B_TOKENS
              for (n, k) in sorted(set(wl.DENSE_8B.values()))]


# Every output row is compared up to this many tokens; above it (the 16384-token shapes)
# the first and last 8 rows and 256 seeded random rows are, and every element is checked to
# have been written.
FULL_ROWS_MAX_M = 4096


def run_w8a8_full(ref, dev, m, n, k, frac, bias, seed):
    """One decoder-shaped W8A8 product at full size: codes and scales of both operands, the
    int32 accumulators, and the bf16 and float32 outputs of the fused epilogue."""
    g = wl.rng(seed)
    wt, wv = host("bf16", wl.weight(g, n, k))
    xt, xv = host("bf16", wl.activations(g, m, k, outlier_frac=frac))
    b_np = (g.standard_normal(n, dtype=np.float32) * np.float32(0.02)) if bias else None
    qw, sw = i8.quantize_per_channel_int8(wt.to(dev))
    qx, sx = i8.quantize_per_token_int8(xt.to(dev))
    b = torch.from_numpy(b_np).to(dev) if bias else None
    ys = {od: i8.w8a8_gemm(qx, sx, qw, sw, b, out_dtype=od, out=sentinel((m, n), od, dev))
          for od in (torch.bfloat16, torch.float32)}
    yi = i8.w8a8_gemm(qx, None, qw, None, out_dtype=torch.int32,
                      out=sentinel((m, n), torch.int32, dev))
    qwr, swr = ref.quantize_rows(wv, "bf16")
    np.testing.assert_array_equal(qw.cpu().numpy(), qwr)
    np.testing.assert_array_equal(sw.cpu().numpy(), swr)
    if m <= FULL_ROWS_MAX_M:
        rows = None
        qxr, sxr = ref.quantize_rows(xv, "bf16")
        np.testing.assert_array_equal(qx.cpu().numpy(), qxr)
        np.testing.assert_array_equal(sx.cpu().numpy(), sxr)
    else:
        for y in ys.values():
            assert not torch.isnan(y).any()  # every element written
        # |acc| <= k * 127^2 < 0x55555556 here, so the int32 sentinel cannot be a result
        assert k * 127 * 127 < 0x55555556 and not (yi == -0x55555556).any()
        rows = sampled_rows(m, seed=seed)
        qxr, sxr = ref.quantize_rows(xv[rows], "bf16")
        idx = torch.from_numpy(rows).to(dev)
        np.testing.assert_array_equal(qx[idx].cpu().numpy(), qxr)
        np.testing.assert_array_equal(sx[idx].cpu().numpy(), sxr)
        ys = {od: y[idx] for od, y in ys.items()}
        yi = yi[idx]
    acc, yref = ref.w8a8(qxr, sxr, qwr, swr, b_np)
    np.testing.assert_array_equal(yi.cpu().numpy(), acc)
    tol = w8a8_tol(acc, sxr, swr, b_np)
    del acc
    for od, y in ys.items():
        check_float(y, yref, tol, f"w8a8 {m}x{n}x{k} {od}")


@pytest.mark.parametrize("m,n,k", PREFILL_4B)
def test_w8a8_dense_4b_prefill_full(ref, dev, m, n, k):
    run_w8a8_full(ref, dev, m, n, k, 0.001, False, seed=m + n + k)


@pytest.mark.parametrize("m,n,k", PREFILL_8B)
def test_w8a8_dense_8b_prefill_full(ref, dev, m, n, k):
    run_w8a8_full(ref, dev, m, n, k, 0.01, True, seed=m + n + k)


# ---------------------------------------------------------------------------------------
# W8A16

def run_w8a16(ref, dev, m, n, k, bias, out_dtype, seed):
    g = wl.rng(seed)
    wt, wv = host("bf16", wl.weight(g, n, k))
    xt, xv = host("bf16", wl.activations(g, m, k))
    qw, sw, qwr, swr = quant_gpu_vs_ref(ref, dev, wt, wv, "bf16")
    b_np = (g.standard_normal(n, dtype=np.float32) * np.float32(0.02)) if bias else None
    b = torch.from_numpy(b_np).to(dev) if bias else None
    y = i8.w8a16_gemm(xt.to(dev), qw, sw, b, out_dtype=out_dtype,
                      out=sentinel((m, n), out_dtype, dev))
    yref = ref.w8a16(xv, qwr, swr, b_np)
    absdot = np.abs(xt.double().numpy()) @ (np.abs(qwr.astype(np.float64)) * swr[:, None]).T
    check_float(y, yref, w8a16_tol(yref, absdot, k, b_np), f"w8a16 {m}x{n}x{k}")
    return y


# one activation row: the one-wavefront-per-channel kernel at 4 and 8 chunks per lane (full,
# ragged, and channels not a multiple of the workgroup's 4), and past its k limit
@pytest.mark.parametrize("m,n,k", [(1, 16, 16), (1, 50, 208), (1, 7, 1040), (1, 37, 4112),
                                   (1, 1003, 8192), (1, 9, 8208), (3, 130, 1040), (8, 256, 4096),
                                   (16, 1000, 4096), (17, 100, 512), (33, 70, 272),
                                   (70, 100, 256), (130, 45, 128)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_w8a16_small(ref, dev, m, n, k, out_dtype):
    run_w8a16(ref, dev, m, n, k, bias=(m % 2 == 1), out_dtype=out_dtype, seed=m + n)


DECODE_8B = [(m, n, k) for m in wl.DECODE_8B_BATCH for (n, k) in sorted(set(wl.DENSE_8B.values()))]
# the fused launches of the benchmark's decode layer (q/k/v and gate/up concatenated)
DECODE_8B += [(m, sum(wl.DENSE_8B[p][0] for p in parts), wl.DENSE_8B[parts[0]][1])
              for m in wl.DECODE_8B_BATCH for parts in wl.DENSE_8B_FUSED.values()
              if len(parts) > 1]


@pytest.mark.parametrize("m,n,k", DECODE_8B)
def test_w8a16_dense_8b_decode_full(ref, dev, m, n, k):
    run_w8a16(ref, dev, m, n, k, bias=False, out_dtype=torch.float32, seed=m * n + k)
    y1 = run_w8a16(ref, dev, m, n, k, bias=False, out_dtype=torch.bfloat16, seed=m * n + k)
    # same inputs, same bits
    g = wl.rng(m * n + k)
    wt, _ = host("bf16", wl.weight(g, n, k))
    xt, _ = host("bf16", wl.activations(g, m, k))
    qw, sw = i8.quantize_per_channel_int8(wt.to(dev))
    assert torch.equal(i8.w8a16_gemm(xt.to(dev), qw, sw), y1)


# ---------------------------------------------------------------------------------------
# grouped W8A16 over experts

def run_grouped(ref, dev, qw, sw, qwr, swr, ids, x_rows, per_assign, out_dtype, g):
    e, n, k = qwr.shape
    xt, xv = host("bf16", wl.activations(g, x_rows, k))
    y = i8.grouped_w8a16_gemm(xt.to(dev), qw, sw, torch.from_numpy(ids).to(dev),
                              x_per_assignment=per_assign, out_dtype=out_dtype,
                              out=sentinel((ids.size, n), out_dtype, dev))
    yref = ref.grouped_w8a16(xv, per_assign, qwr, swr, ids)
    t, topk = ids.shape
    xd = np.abs(xt.double().numpy())
    absdot = np.zeros_like(yref)
    for p in range(t * topk):
        ex = ids.flat[p]
        if 0 <= ex < e:
            absdot[p] = (np.abs(qwr[ex].astype(np.float64)) * swr[ex][:, None]) @ \
                xd[p if per_assign else p // topk]
    check_float(y, yref, w8a16_tol(yref, absdot, k), f"grouped e={e} n={n} k={k} t={t}")
    yc = to_np(y)
    for p in range(t * topk):
        if not 0 <= ids.flat[p] < e:
            assert np.all(yc[p] == 0.0)
    return y


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_grouped_small_edge_cases(ref, dev, out_dtype):
    g = wl.rng(21)
    e, n, k = 7, 40, 272
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = np.stack([g.choice(e, 3, replace=False) for _ in range(11)]).astype(np.int32)
    ids[2, 1] = -1
    ids[4, 0] = e      # out of range -> zero rows
    ids[5] = 6         # one token routed three times to the same expert
    for per_assign in (False, True):
        run_grouped(ref, dev, qw, sw, qwr, swr, ids, 33 if per_assign else 11, per_assign,
                    out_dtype, g)


@pytest.mark.parametrize("e,n,k", [(5, 30, 1040), (3, 7, 16), (4, 64, 8192), (3, 9, 8208)])
def test_grouped_one_token(ref, dev, e, n, k):
    """One token: the per-assignment kernel (ragged k, one chunk, its longest k, and past
    it), with an invalid id, an out-of-range id and a repeated expert, both activation
    layouts and both output types."""
    g = wl.rng(26 + k)
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = np.array([[e - 1, -1, 0, e, 0, 1]], dtype=np.int32)
    for per_assign, out_dtype in ((False, torch.bfloat16), (True, torch.float32)):
        run_grouped(ref, dev, qw, sw, qwr, swr, ids, 6 if per_assign else 1, per_assign,
                    out_dtype, g)


@pytest.mark.parametrize("e,n,k,t,topk", [(9, 30, 1040, 3, 4), (20, 13, 8192, 4, 16),
                                          (6, 24, 512, 2, 33), (70, 40, 2048, 4, 6)])
def test_grouped_few_tokens(ref, dev, e, n, k, t, topk):
    """Two to four tokens with at most 64 assignments (the SiLU·mul form of this call takes
    the few-token kernel; the plain call keeps the tiled one): ragged k, a long k, 64
    assignments and 66; invalid and out-of-range ids, an expert repeated within a token."""
    g = wl.rng(27 + k + t)
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = np.stack([g.choice(e, topk, replace=topk > e) for _ in range(t)]).astype(np.int32)
    ids[0, 0] = -1
    ids[t - 1, topk - 1] = e
    ids[1, :2] = ids[0, 1]
    for per_assign, out_dtype in ((False, torch.bfloat16), (True, torch.float32)):
        run_grouped(ref, dev, qw, sw, qwr, swr, ids, t * topk if per_assign else t, per_assign,
                    out_dtype, g)


def test_grouped_later_passes_split(ref, dev):
    """More tokens than two passes of 8 rows: an expert's later passes go to extra rows of
    workgroups (highest expert first, at most 32 rows), the rest stay with the expert's own
    workgroup.  Every later pass taken by an extra row (6 experts, 40 tokens, some extra
    rows idle), more later passes than extra rows (one expert receives every one of 300
    tokens), later passes only on experts of two different 64-expert groups with most
    experts empty (100 experts), and all ids beyond one scan window (no split)."""
    g = wl.rng(25)
    e, n, k = 6, 40, 272
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = np.stack([g.choice(e, 3, replace=False) for _ in range(40)]).astype(np.int32)
    ids[3, 2] = -1
    ids[7, 0] = e
    for per_assign in (False, True):
        run_grouped(ref, dev, qw, sw, qwr, swr, ids, 120 if per_assign else 40, per_assign,
                    torch.bfloat16, g)
    e, n, k = 4, 24, 128
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = np.stack([np.r_[3, g.choice(3, 2, replace=False)] for _ in range(300)]).astype(np.int32)
    run_grouped(ref, dev, qw, sw, qwr, swr, ids, 300, False, torch.float32, g)
    e, n, k = 100, 20, 256
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = np.array([[99, 70, 1, g.integers(0, e)] for _ in range(40)], dtype=np.int32)
    ids[5, 3] = -1
    run_grouped(ref, dev, qw, sw, qwr, swr, ids, 40, False, torch.bfloat16, g)
    e, n, k = 3, 16, 64
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = np.stack([g.choice(e, 3, replace=False) for _ in range(400)]).astype(np.int32)
    run_grouped(ref, dev, qw, sw, qwr, swr, ids, 400, False, torch.bfloat16, g)


def test_grouped_single_token_repeated_expert(ref, dev):
    """One token routed three times to one expert: the expert's rows exceed the token count
    that sizes the staged passes, so it takes several passes."""
    g = wl.rng(24)
    e, n, k = 6, 72, 2048
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = np.array([[2, 2, 5, 2]], dtype=np.int32)
    for per_assign in (False, True):
        run_grouped(ref, dev, qw, sw, qwr, swr, ids, 4 if per_assign else 1, per_assign,
                    torch.bfloat16, g)


def test_grouped_one_expert_equals_w8a16(ref, dev):
    """One expert that every row is routed to: the grouped kernel computes the dense W8A16
    product.  Float32 outputs; the two kernels sum the k products (exact in float32) in
    different orders and then scale, each within (k + 1) * 2^-24 * s * sum|x * q| of the exact
    value, so they differ by at most twice that."""
    g = wl.rng(22)
    n, k = 100, 512
    qw, sw, _, _ = moe_stack(ref, dev, g, n, k, 1)
    x = wl.to_bf16(wl.activations(g, 19, k)).to(dev)
    yg = i8.grouped_w8a16_gemm(x, qw, sw, torch.zeros((19, 1), dtype=torch.int32, device=dev),
                               out_dtype=torch.float32)
    yd = i8.w8a16_gemm(x, qw[0], sw[0], out_dtype=torch.float32)
    xa = np.abs(to_np(x).astype(np.float64))
    qa = np.abs(to_np(qw[0]).astype(np.float64))
    bound = 2.0 * (k + 1) * 2.0**-24 * (xa @ qa.T) * to_np(sw[0]).astype(np.float64)[None, :]
    check_float(yg, to_np(yd).astype(np.float64), bound + 1e-30, "E=1")


def test_grouped_many_rows_per_expert(ref, dev):
    """More than 64 rows for one expert (several 64-row passes) and more than one 1024-entry
    scan window."""
    g = wl.rng(23)
    e, n, k = 3, 48, 256
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = g.integers(0, e, size=(700, 2), dtype=np.int32)
    ids[::97, 1] = 9
    run_grouped(ref, dev, qw, sw, qwr, swr, ids, 700, False, torch.float32, g)


def test_grouped_experts_picked_from_a_wide_bitmap(ref, dev):
    """5000 experts: the presence bitmap spans 157 words, so a workgroup's expert is found in
    the first, second or third group of 64 words; ids sit on word and group boundaries, next
    to invalid ones, and several tokens share experts (fewer distinct experts than slots)."""
    g = wl.rng(25)
    e, n, k = 5000, 24, 128
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = np.array([[4999, 0, 31, 32, 2047],
                    [2048, 4999, -3, 63, 64],
                    [1, 4096, 4095, 5000, 0],
                    [3000, 2, 4998, 1000, 31],
                    [2047, 2048, 4064, 4063, 7]], dtype=np.int32)
    for per_assign in (False, True):
        run_grouped(ref, dev, qw, sw, qwr, swr, ids, ids.size if per_assign else 5, per_assign,
                    torch.float32, g)


def test_grouped_every_slot_a_distinct_expert(ref, dev):
    """As many distinct experts as assignments (every slot of the grid has an expert) and a
    single token whose ids are all distinct."""
    g = wl.rng(26)
    e, n, k = 40, 56, 640
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    for t, topk in ((2, 6), (1, 8)):
        ids = g.choice(e, t * topk, replace=False).astype(np.int32).reshape(t, topk)
        run_grouped(ref, dev, qw, sw, qwr, swr, ids, t, False, torch.bfloat16, g)


@pytest.mark.parametrize("t", wl.MOE_TOKENS)
@pytest.mark.parametrize("proj", ["gate", "down"])
def test_grouped_moe_16b_full(ref, dev, t, proj):
    g = wl.rng(30 + t)
    n, k = wl.MOE_16B[proj]
    e = wl.MOE_ROUTED + wl.MOE_SHARED
    qw, sw, qwr, swr = moe_stack(ref, dev, g, n, k, e)
    ids = wl.moe_expert_ids(g, t)
    per_assign = proj == "down"
    for od in (torch.bfloat16, torch.float32):
        run_grouped(ref, dev, qw, sw, qwr, swr, ids, t * ids.shape[1] if per_assign else t,
                    per_assign, od, g)


# ---------------------------------------------------------------------------------------
# HIP graph capture (the benchmark replays the path from graphs)

def test_graph_replays_match_eager(ref, dev):
    g = wl.rng(40)
    w = wl.to_bf16(wl.weight(g, 320, 1024)).to(dev)
    x = wl.to_bf16(wl.activations(g, 96, 1024, 0.001)).to(dev)
    e_w = wl.to_bf16(wl.moe_weights(g, 64, 1024, experts=5).reshape(5 * 64, 1024)).to(dev)
    ids = torch.from_numpy(np.stack([g.choice(5, 2, replace=False) for _ in range(7)])
                           .astype(np.int32)).to(dev)
    xd = wl.to_bf16(wl.activations(g, 3, 1024)).to(dev)
    xg = wl.to_bf16(wl.activations(g, 7, 1024)).to(dev)

    qw, sw = i8.quantize_per_channel_int8(w)
    qe, se = i8.quantize_per_channel_int8(e_w)
    qx = torch.empty((96, 1024), dtype=torch.int8, device=dev)
    sx = torch.empty(96, dtype=torch.float32, device=dev)
    y8 = torch.empty((96, 320), dtype=torch.bfloat16, device=dev)
    y16 = torch.empty((3, 320), dtype=torch.bfloat16, device=dev)
    yg = torch.empty((14, 64), dtype=torch.float32, device=dev)

    ys = torch.empty((96, 320), dtype=torch.float32, device=dev)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    # one activation row: the one-row kernel, per-channel and group-128 scales
    qg, sg = i8.quantize_per_group_int8(w)
    y1 = torch.empty((1, 320), dtype=torch.bfloat16, device=dev)
    y1g = torch.empty((1, 320), dtype=torch.float32, device=dev)

    def path():
        i8.quantize_per_token_int8(x, qx, sx)
        i8.w8a8_gemm(qx, sx, qw, sw, out=y8)
        i8.w8a8_gemm_with_plan(6, 4, qx, sx, qw, sw, out_dtype=torch.float32, out=ys,
                               workspace=ws)
        i8.w8a16_gemm(xd, qw, sw, out=y16)
        i8.w8a16_gemm(xd[:1], qw, sw, out=y1)
        i8.w8a16_gemm_g128(xd[1:2], qg, sg, out_dtype=torch.float32, out=y1g)
        i8.grouped_w8a16_gemm(xg, qe.view(5, 64, 1024), se.view(5, 64), ids,
                              out_dtype=torch.float32, out=yg)

    path()
    torch.cuda.synchronize()
    outs = (qx, sx, y8, ys, y16, y1, y1g, yg)
    eager = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for rep in range(3):
        for t in outs:
            t.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        assert torch.all(ws[:16384] == 0)  # the arrival counters
        path()  # eager work between replays
        torch.cuda.synchronize()
