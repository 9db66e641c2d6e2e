"""The C ABI on the CPU: the library loads, exports every symbol the header declares, and
rejects bad arguments before any HIP call (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "i8ql.h")

OK, NULL, SHAPE, DTYPE, ALIGN, KBIG, ARG, WORKSPACE = 0, 1, 2, 3, 4, 5, 6, 8
F32, BF16, F16, I8, I32 = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    from int8_quantized_linear_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from int8_quantized_linear_amd import build
        build.build()
    return _binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"defined", "sizeof"})


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) >= {"quantize_per_channel_int8", "quantize_per_token_int8", "w8a8_gemm",
                          "w8a16_gemm", "grouped_w8a16_gemm", "i8ql_status_string",
                          "i8ql_last_hip_error"}
    for nm in names:
        assert hasattr(lib, nm), nm


def test_status_strings(lib):
    for code, name in enumerate(["I8QL_OK", "I8QL_ERR_NULL", "I8QL_ERR_SHAPE", "I8QL_ERR_DTYPE",
                                 "I8QL_ERR_ALIGN", "I8QL_ERR_K_TOO_LARGE", "I8QL_ERR_ARG",
                                 "I8QL_ERR_HIP", "I8QL_ERR_WORKSPACE"]):
        assert lib.i8ql_status_string(code).decode() == name
    assert lib.i8ql_last_hip_error() == 0


# Fake, never-dereferenced addresses: every call below fails validation before any HIP call.
A16 = ctypes.c_void_p(0x10000)          # 16-byte aligned
A4 = ctypes.c_void_p(0x10004)           # 4-byte aligned only
A2 = ctypes.c_void_p(0x10002)
NUL = None


@pytest.mark.parametrize("fn", ["quantize_per_channel_int8", "quantize_per_token_int8"])
def test_quantizer_validation(lib, fn):
    f = getattr(lib, fn)
    assert f(A16, I8, 4, 8, A16, A16, NUL) == DTYPE
    assert f(A16, I32, 4, 8, A16, A16, NUL) == DTYPE
    assert f(A16, 9, 4, 8, A16, A16, NUL) == DTYPE
    assert f(A16, F32, -1, 8, A16, A16, NUL) == SHAPE
    assert f(A16, F32, 4, 0, A16, A16, NUL) == SHAPE
    assert f(A16, F32, 1 << 40, 1 << 30, A16, A16, NUL) == SHAPE
    assert f(NUL, F32, 0, 8, NUL, NUL, NUL) == OK      # zero rows: no-op
    assert f(NUL, F32, 4, 8, A16, A16, NUL) == NULL
    assert f(A16, F32, 4, 8, NUL, A16, NUL) == NULL
    assert f(A16, F32, 4, 8, A16, NUL, NUL) == NULL
    assert f(A2, F32, 4, 8, A16, A16, NUL) == ALIGN
    assert f(ctypes.c_void_p(0x10001), BF16, 4, 8, A16, A16, NUL) == ALIGN
    assert f(A16, F32, 4, 8, A16, A2, NUL) == ALIGN


def test_quantizer_multi_validation(lib):
    from int8_quantized_linear_amd._binding import QuantJob
    f = lib.quantize_per_token_int8_multi

    def call(jobs, count=None, dt=BF16):
        arr = (QuantJob * max(1, len(jobs)))(*jobs)
        return f(ctypes.cast(arr, ctypes.c_void_p), len(jobs) if count is None else count, dt,
                 NUL)

    ok = QuantJob(0x10000, 4, 64, 0x20000, 0x30000)
    assert f(NUL, 1, BF16, NUL) == ARG
    assert call([ok], count=0) == ARG
    assert call([ok] * 9) == ARG
    assert call([ok], dt=I8) == DTYPE
    assert call([ok, QuantJob(0x10000, -1, 64, 0x20000, 0x30000)]) == SHAPE
    assert call([ok, QuantJob(0x10000, 4, 0, 0x20000, 0x30000)]) == SHAPE
    assert call([QuantJob(0, 0, 64, 0, 0)]) == OK                 # empty: nothing to do
    assert call([ok, QuantJob(0, 4, 64, 0x20000, 0x30000)]) == NULL
    assert call([ok, QuantJob(0x10008, 4, 64, 0x20000, 0x30000)]) == ALIGN   # x 8-aligned
    assert call([ok, QuantJob(0x10000, 4, 60, 0x20000, 0x30000)]) == ALIGN   # 120-byte rows
    assert call([ok, QuantJob(0x10000, 4, 64, 0x20004, 0x30000)]) == ALIGN   # q 4-aligned


def test_w8a8_validation(lib):
    f = lib.w8a8_gemm
    args = lambda **kw: dict(dict(xq=A16, sx=A16, wq=A16, sw=A16, b=NUL, y=A16, yt=BF16,
                                  m=4, n=8, k=64), **kw)
    call = lambda a: f(a["xq"], a["sx"], a["wq"], a["sw"], a["b"], a["y"], a["yt"], a["m"],
                       a["n"], a["k"], NUL)
    assert call(args(yt=F16)) == DTYPE
    assert call(args(yt=I8)) == DTYPE
    assert call(args(m=-1)) == SHAPE
    assert call(args(n=-2)) == SHAPE
    assert call(args(k=0)) == SHAPE
    assert call(args(m=1 << 30, n=1 << 30, k=16)) == SHAPE  # 2^49 output tiles of 64 x 32
    assert call(args(m=0, xq=NUL, y=NUL)) == OK
    assert call(args(n=0)) == OK
    assert call(args(xq=NUL)) == NULL
    assert call(args(wq=NUL)) == NULL
    assert call(args(y=NUL)) == NULL
    assert call(args(sx=NUL)) == NULL
    assert call(args(sw=NUL, yt=F32)) == NULL
    assert call(args(yt=I32, b=A16)) == ARG
    assert call(args(k=72)) == ALIGN
    assert call(args(k=8)) == ALIGN
    assert call(args(xq=A4)) == ALIGN
    assert call(args(wq=ctypes.c_void_p(0x10008))) == ALIGN
    assert call(args(y=ctypes.c_void_p(0x10001))) == ALIGN
    assert call(args(y=A2, yt=F32)) == ALIGN
    assert call(args(b=A2, yt=F32)) == ALIGN
    assert call(args(k=133152)) == KBIG


def test_w8a8_with_config_validation(lib):
    f = lib.w8a8_gemm_with_config
    call = lambda c, m=4, n=8, k=64, xq=A16, y=A16: f(c, xq, A16, A16, A16, NUL, y, BF16, m, n,
                                                      k, NUL)
    assert call(12) == ARG
    assert call(-2) == ARG
    assert call(12, m=0) == ARG             # checked before the zero-size no-op
    assert call(-1, m=0, xq=NUL, y=NUL) == OK
    assert call(0, xq=NUL) == NULL
    assert call(0, k=72) == ALIGN
    for c in range(12):
        geo = (ctypes.c_int32 * 5)()
        assert lib.w8a8_gemm_config_info(c, ctypes.cast(geo, ctypes.c_void_p)) == OK
        if geo[2] > 1:                      # k-groups need k % (128 * groups) == 0
            assert call(c, k=64) == ARG
            assert call(c, k=128 * geo[2] + 16) == ARG
            assert call(c, m=0, k=64) == ARG
    assert lib.w8a8_gemm_config_info(12, ctypes.cast((ctypes.c_int32 * 5)(), ctypes.c_void_p)) == ARG
    assert lib.w8a8_gemm_config_info(0, NUL) == NULL


def plan_ws(geo, splits, m, n):
    """Workspace of a split plan: 4096 tile counters, then one int32 partial tile per (tile,
    split)."""
    if splits == 1:
        return 0
    tiles = -(-m // geo[0]) * -(-n // geo[1])
    return (4096 + tiles * splits * geo[0] * geo[1]) * 4


def test_w8a8_with_plan_validation(lib):
    import int8_quantized_linear_amd as i8
    f = lib.w8a8_gemm_with_plan
    W = ctypes.c_void_p(0x20000)

    def call(c, s, m=300, n=200, k=1024, ws=W, wsb=1 << 30, xq=A16, y=A16, yt=BF16):
        return f(c, s, xq, A16, A16, A16, NUL, y, yt, m, n, k, ws, wsb, NUL)

    assert call(-1, 2) == ARG                 # auto plan takes no split count
    assert call(-1, 1) == ARG
    assert call(6, 0) == ARG
    assert call(6, -1) == ARG
    assert call(6, 9) == ARG                  # beyond I8QL_W8A8_MAX_SPLITS
    assert call(6, 2, wsb=-1) == ARG
    assert call(13, 1) == ARG
    assert call(6, 9, m=0) == ARG             # checked before the zero-size no-op
    assert call(6, 2, m=0, xq=NUL, y=NUL) == OK
    assert call(6, 8, k=896) == ARG           # 7 steps of 128 cannot take 8 splits
    for c in range(12):
        geo = i8.w8a8_gemm_config_info(c)
        if not geo[3]:
            assert call(c, 2) == ARG          # configurations that cannot split k
            continue
        need = plan_ws(geo, 3, 300, 200)
        assert i8.w8a8_gemm_workspace_size(300, 200, 1024, 256, c, 3) == need
        assert i8.w8a8_gemm_workspace_size(300, 200, 1024, 256, c, 1) == 0
        assert call(c, 3, ws=NUL) == NULL
        assert call(c, 3, wsb=need - 4) == WORKSPACE
        assert call(c, 3, ws=ctypes.c_void_p(0x20008)) == ALIGN
    assert call(10, 2, m=64 * 65, n=64 * 64) == SHAPE  # 4160 tiles: too many to split
    assert lib.w8a8_gemm_workspace_size(10, 2, 64 * 65, 64 * 64, 1024, 256) == -1
    assert lib.w8a8_gemm_workspace_size(10, 2, 64 * 64, 64 * 64, 1024, 256) > 0  # 4096: fine
    assert lib.w8a8_gemm_workspace_size(1, 3, 300, 200, 1024, 256) == -1  # cannot split
    assert lib.w8a8_gemm_workspace_size(6, 9, 300, 200, 1024, 256) == -1
    assert lib.w8a8_gemm_workspace_size(-1, -1, 0, 200, 1024, 256) == -1


def test_w8a8_plan_choices():
    import int8_quantized_linear_amd as i8
    geos = [i8.w8a8_gemm_config_info(c) for c in range(i8.W8A8_NUM_CONFIGS)]
    for m in (1, 16, 128, 512, 777, 2048, 16384):
        for n in (32, 1000, 2560, 6144, 19456):
            for k in (16, 272, 2560, 4096, 9728):
                # no workspace: exactly the configuration w8a8_gemm launches
                assert i8.w8a8_gemm_choose_plan(m, n, k, 256, 0) == (
                    i8.w8a8_gemm_choose_config(m, n, k, 256), 1)
                c, s = i8.w8a8_gemm_choose_plan(m, n, k, 256)
                assert 1 <= s <= i8.W8A8_MAX_SPLITS and (s == 1 or geos[c][3])
                assert s <= -(-k // 128)
                need = i8.w8a8_gemm_workspace_size(m, n, k, 256)
                assert need == plan_ws(geos[c], s, m, n)
                # given exactly that much, the same plan; any budget gives a plan that fits
                assert i8.w8a8_gemm_choose_plan(m, n, k, 256, need) == (c, s)
                c2, s2 = i8.w8a8_gemm_choose_plan(m, n, k, 256, need // 2)
                assert plan_ws(geos[c2], s2, m, n) <= need // 2


def test_w8a8_config_table_and_choices():
    import int8_quantized_linear_amd as i8
    geos = [i8.w8a8_gemm_config_info(c) for c in range(i8.W8A8_NUM_CONFIGS)]
    assert len(set(geos)) == len(geos)
    assert "#define I8QL_W8A8_NUM_CONFIGS %d" % i8.W8A8_NUM_CONFIGS in open(HEADER).read()
    # invalid sizes
    for m, n, k, cus in [(0, 8, 64, 256), (4, 0, 64, 256), (4, 8, 8, 256), (4, 8, 72, 256),
                         (4, 8, 133152, 256), (4, 8, 64, 0), (1 << 30, 1 << 30, 16, 256)]:
        assert i8.w8a8_gemm_choose_config(m, n, k, cus) == -1
    # every choice is a valid configuration; k-groups only where k splits into whole steps
    for m in (1, 16, 128, 512, 777, 2048, 4096, 16384):
        for n in (32, 1000, 2560, 6144, 19456):
            for k in (16, 272, 2560, 4096, 9728):
                c = i8.w8a8_gemm_choose_config(m, n, k, 256)
                bm, bn, g, _, _ = geos[c]
                assert g == 1 or k % (128 * g) == 0
    # the benchmark step's fused 4B projections at 2048 tokens take the 256x320, 256x192 and
    # 128x160 tiles that fill the 256 CUs in whole rounds
    pick = lambda m, n, k, cus=256: geos[i8.w8a8_gemm_choose_config(m, n, k, cus)]
    assert pick(2048, 19456, 2560)[:3] == (256, 320, 1)
    assert pick(2048, 6144, 2560)[:3] == (256, 192, 1)
    assert pick(2048, 2560, 4096)[:3] == (128, 160, 1)
    assert pick(2048, 2560, 9728)[:3] == (128, 160, 1)
    # many rounds of tiles: the 256x256 tiles, whose persistent kernel keeps each compute
    # unit's pipeline running from one tile into the next
    assert pick(16384, 12288, 4096)[:3] == (256, 256, 1)
    assert pick(16384, 24576, 4096)[:3] == (256, 256, 1)
    # few tiles and a long k: k split over k-groups inside the workgroup
    assert pick(128, 2560, 9728)[2] == 4
    assert pick(512, 2560, 9728)[2] == 2
    # fewer compute units: the same shape needs more rounds, and the choice may change
    assert all(0 <= i8.w8a8_gemm_choose_config(2048, 19456, 2560, cus) < i8.W8A8_NUM_CONFIGS
               for cus in (1, 32, 80, 304))


def test_w8a8_int32_limit_is_exactly_the_header_constant():
    # 133144 * 127 * 127 fits in int32; 133160 (next multiple of 16) would not.
    assert 133144 * 127 * 127 < 2 ** 31 <= 133160 * 127 * 127
    assert "#define I8QL_W8A8_MAX_K 133144" in open(HEADER).read()


def test_w8a16_validation(lib):
    f = lib.w8a16_gemm
    base = dict(x=A16, wq=A16, sw=A16, b=NUL, y=A16, yt=BF16, m=1, n=8, k=64)
    call = lambda **kw: (lambda a: f(a["x"], a["wq"], a["sw"], a["b"], a["y"], a["yt"], a["m"],
                                     a["n"], a["k"], NUL))(dict(base, **kw))
    assert call(yt=I32) == DTYPE
    assert call(yt=F16) == DTYPE
    assert call(m=-1) == SHAPE
    assert call(k=0) == SHAPE
    assert call(m=0, x=NUL) == OK
    assert call(x=NUL) == NULL
    assert call(sw=NUL) == NULL
    assert call(k=40) == ALIGN
    assert call(x=A4) == ALIGN
    assert call(wq=A4) == ALIGN
    assert call(b=A2) == ALIGN


def test_grouped_validation(lib):
    f = lib.grouped_w8a16_gemm
    base = dict(x=A16, pa=0, wq=A16, sw=A16, e=66, ids=A16, t=4, topk=8, y=A16, yt=BF16, n=16,
                k=64)
    call = lambda **kw: (lambda a: f(a["x"], a["pa"], a["wq"], a["sw"], a["e"], a["ids"], a["t"],
                                     a["topk"], a["y"], a["yt"], a["n"], a["k"], NUL))(dict(base, **kw))
    assert call(yt=I32) == DTYPE
    assert call(pa=2) == ARG
    assert call(topk=0) == ARG
    assert call(topk=65) == ARG
    assert call(e=0) == ARG
    assert call(e=65535) == ARG
    assert call(t=-1) == SHAPE
    assert call(t=8193, topk=8) == SHAPE
    assert call(k=0) == SHAPE
    assert call(k=32768 + 16) == SHAPE   # past I8QL_GROUPED_MAX_K: one row no longer fits LDS
    assert call(k=32768 + 16, t=0, x=NUL) == SHAPE
    assert call(t=0, x=NUL) == OK
    assert call(ids=NUL) == NULL
    assert call(x=NUL) == NULL
    assert call(k=24) == ALIGN
    assert call(x=A4) == ALIGN
    assert call(ids=A2) == ALIGN


def test_grouped_silu_validation(lib):
    f = lib.grouped_w8a16_silu_gemm
    base = dict(x=A16, pa=0, wq=A16, sw=A16, e=66, ids=A16, t=4, topk=8, h=A16, ht=BF16, n=16,
                k=64)
    call = lambda **kw: (lambda a: f(a["x"], a["pa"], a["wq"], a["sw"], a["e"], a["ids"], a["t"],
                                     a["topk"], a["h"], a["ht"], a["n"], a["k"], NUL))(dict(base, **kw))
    assert call(ht=I8) == DTYPE
    assert call(pa=3) == ARG
    assert call(topk=0) == ARG
    assert call(e=0) == ARG
    assert call(t=-1) == SHAPE
    assert call(k=32768 + 16) == SHAPE
    assert call(t=0, x=NUL) == OK
    assert call(n=0, h=NUL) == OK
    assert call(h=NUL) == NULL
    assert call(k=40) == ALIGN
    assert call(h=A2, ht=F32) == ALIGN


def test_group_scale_validation(lib):
    f = lib.quantize_per_group_int8
    assert f(A16, I8, 4, 256, A16, A16, NUL) == DTYPE
    assert f(A16, BF16, -1, 256, A16, A16, NUL) == SHAPE
    assert f(A16, BF16, 4, 200, A16, A16, NUL) == SHAPE    # not a multiple of 128
    assert f(A16, BF16, 4, 0, A16, A16, NUL) == SHAPE
    assert f(NUL, BF16, 0, 256, NUL, NUL, NUL) == OK
    assert f(NUL, BF16, 4, 256, A16, A16, NUL) == NULL
    assert f(A4, BF16, 4, 256, A16, A16, NUL) == ALIGN
    assert f(A16, BF16, 4, 256, A4, A16, NUL) == ALIGN
    assert f(A16, BF16, 4, 256, A16, A2, NUL) == ALIGN
    g = lib.w8a16_gemm_g128
    call = lambda **kw: (lambda a: g(a["x"], a["wq"], a["sw"], a["b"], a["y"], a["yt"], a["m"],
                                     a["n"], a["k"], NUL))(dict(dict(x=A16, wq=A16, sw=A16, b=NUL,
                                                                     y=A16, yt=BF16, m=1, n=16,
                                                                     k=256), **kw))
    assert call(yt=I32) == DTYPE
    assert call(k=192) == SHAPE
    assert call(m=-1) == SHAPE
    assert call(m=0, x=NUL) == OK
    assert call(sw=NUL) == NULL
    assert call(x=A4) == ALIGN
    assert call(b=A2) == ALIGN


def test_moe_route_validation(lib):
    f = lib.moe_route_topk
    base = dict(lg=A16, lt=F32, t=4, e=64, kr=6, ns=2, ids=A16, w=A16)
    call = lambda **kw: (lambda a: f(a["lg"], a["lt"], a["t"], a["e"], a["kr"], a["ns"], a["ids"],
                                     a["w"], NUL))(dict(base, **kw))
    assert call(lt=I32) == DTYPE
    assert call(lt=F16) == DTYPE
    assert call(t=-1) == SHAPE
    assert call(e=0) == ARG
    assert call(e=257) == ARG
    assert call(kr=0) == ARG
    assert call(kr=33) == ARG
    assert call(kr=7, e=6) == ARG         # more picks than experts
    assert call(ns=-1) == ARG
    assert call(ns=33) == ARG
    assert call(kr=32, ns=32, e=256, t=0) == OK   # 64 slots: the largest allowed
    assert call(t=0, lg=NUL) == OK
    assert call(lg=NUL) == NULL
    assert call(ids=NUL) == NULL
    assert call(w=NUL) == NULL
    assert call(lg=A2) == ALIGN
    assert call(lg=ctypes.c_void_p(0x10001), lt=BF16) == ALIGN
    assert call(ids=A2) == ALIGN


def test_moe_combine_validation(lib):
    f = lib.moe_combine
    base = dict(d=A16, dt=BF16, w=A16, t=4, topk=8, n=2048, y=A16, yt=BF16)
    call = lambda **kw: (lambda a: f(a["d"], a["dt"], a["w"], a["t"], a["topk"], a["n"], a["y"],
                                     a["yt"], NUL))(dict(base, **kw))
    assert call(dt=I8) == DTYPE
    assert call(yt=I32) == DTYPE
    assert call(topk=0) == ARG
    assert call(topk=65) == ARG
    assert call(t=-1) == SHAPE
    assert call(n=-1) == SHAPE
    assert call(t=0, d=NUL) == OK
    assert call(n=0, y=NUL) == OK
    assert call(d=NUL) == NULL
    assert call(w=NUL) == NULL
    assert call(y=NUL) == NULL
    assert call(d=ctypes.c_void_p(0x10001)) == ALIGN
    assert call(w=A2) == ALIGN
    assert call(y=A2, yt=F32) == ALIGN


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0  # counts devices without initializing HIP


@pytest.mark.skipif(_gpu_visible(), reason="the fake pointers below must never reach a GPU")
def test_rmsnorm_validation(lib):
    fq, fb = lib.rmsnorm_quantize_per_token_int8, lib.rmsnorm_bf16
    for f, outs in ((fq, (A16, A16)), (fb, (A16,))):
        assert f(A16, NUL, A16, 1e-6, -1, 64, *outs, NUL) == SHAPE
        assert f(A16, NUL, A16, 1e-6, 4, 0, *outs, NUL) == SHAPE
        assert f(A16, NUL, A16, 1e-6, 4, 60, *outs, NUL) == SHAPE       # k % 8
        assert f(A16, NUL, A16, 1e-6, 4, 24576 + 8, *outs, NUL) == SHAPE  # I8QL_NORM_MAX_K
        assert f(A16, NUL, A16, 0.0, 4, 64, *outs, NUL) == ARG
        assert f(A16, NUL, A16, -1e-6, 4, 64, *outs, NUL) == ARG
        assert f(A16, NUL, A16, float("inf"), 4, 64, *outs, NUL) == ARG
        assert f(A16, NUL, A16, float("nan"), 4, 64, *outs, NUL) == ARG
        assert f(NUL, NUL, NUL, 1e-6, 0, 64, *[NUL] * len(outs), NUL) == OK  # no rows: no-op
        assert f(NUL, NUL, A16, 1e-6, 4, 64, *outs, NUL) == NULL
        assert f(A16, NUL, NUL, 1e-6, 4, 64, *outs, NUL) == NULL
        assert f(A4, NUL, A16, 1e-6, 4, 64, *outs, NUL) == ALIGN
        assert f(A16, A4, A16, 1e-6, 4, 64, *outs, NUL) == ALIGN
        assert f(A16, NUL, A4, 1e-6, 4, 64, *outs, NUL) == ALIGN
    assert fq(A16, NUL, A16, 1e-6, 4, 64, NUL, A16, NUL) == NULL
    assert fq(A16, NUL, A16, 1e-6, 4, 64, A16, NUL, NUL) == NULL
    assert fq(A16, NUL, A16, 1e-6, 4, 64, A4, A16, NUL) == ALIGN      # codes: 8-byte aligned
    assert fq(A16, NUL, A16, 1e-6, 4, 64, A16, A2, NUL) == ALIGN
    assert fb(A16, NUL, A16, 1e-6, 4, 64, NUL, NUL) == NULL
    assert fb(A16, NUL, A16, 1e-6, 4, 64, A4, NUL) == ALIGN


def test_silu_mul_validation(lib):
    fq, fb = lib.silu_mul_quantize_per_token_int8, lib.silu_mul_bf16
    for f, outs in ((fq, (A16, A16)), (fb, (A16,))):
        assert f(A16, -1, 64, *outs, NUL) == SHAPE
        assert f(A16, 4, 0, *outs, NUL) == SHAPE
        assert f(A16, 4, 60, *outs, NUL) == SHAPE                 # n % 8
        assert f(A16, 4, 24576 + 8, *outs, NUL) == SHAPE          # I8QL_SILU_MAX_N
        assert f(NUL, 0, 64, *[NUL] * len(outs), NUL) == OK      # no rows: no-op
        assert f(NUL, 4, 64, *outs, NUL) == NULL
        assert f(A4, 4, 64, *outs, NUL) == ALIGN
    assert fq(A16, 4, 64, NUL, A16, NUL) == NULL
    assert fq(A16, 4, 64, A16, NUL, NUL) == NULL
    assert fq(A16, 4, 64, A4, A16, NUL) == ALIGN
    assert fq(A16, 4, 64, A16, A2, NUL) == ALIGN
    assert fb(A16, 4, 64, NUL, NUL) == NULL
    assert fb(A16, 4, 64, A4, NUL) == ALIGN


def test_valid_calls_without_a_device_report_hip_errors(lib):
    """With no device, a call that passes validation fails at its first HIP call with
    I8QL_ERR_HIP (and a recorded hipError), instead of crashing."""
    HIP = 7
    from int8_quantized_linear_amd._binding import QuantJob as QJ
    calls = [
        lambda: lib.quantize_per_channel_int8(A16, BF16, 4, 64, A16, A16, NUL),
        lambda: lib.quantize_per_token_int8(A16, F32, 4, 64, A16, A16, NUL),
        lambda: lib.quantize_per_token_int8_multi(
            ctypes.cast((QJ * 1)(QJ(0x10000, 4, 64, 0x20000, 0x30000)), ctypes.c_void_p), 1,
            BF16, NUL),
        lambda: lib.w8a8_gemm(A16, A16, A16, A16, NUL, A16, BF16, 4, 8, 64, NUL),
        lambda: lib.w8a8_gemm_with_config(0, A16, A16, A16, A16, NUL, A16, F32, 4, 8, 64, NUL),
        lambda: lib.w8a8_gemm_with_plan(6, 2, A16, A16, A16, A16, NUL, A16, F32, 4, 8, 256,
                                        ctypes.c_void_p(0x20000), 1 << 20, NUL),
        lambda: lib.w8a16_gemm(A16, A16, A16, NUL, A16, BF16, 1, 16, 64, NUL),
        lambda: lib.grouped_w8a16_gemm(A16, 0, A16, A16, 66, A16, 4, 8, A16, BF16, 16, 64, NUL),
        lambda: lib.grouped_w8a16_silu_gemm(A16, 0, A16, A16, 66, A16, 4, 8, A16, BF16, 16, 64,
                                            NUL),
        lambda: lib.moe_route_topk(A16, F32, 4, 64, 6, 2, A16, A16, NUL),
        lambda: lib.quantize_per_group_int8(A16, BF16, 4, 256, A16, A16, NUL),
        lambda: lib.w8a16_gemm_g128(A16, A16, A16, NUL, A16, BF16, 1, 16, 256, NUL),
        lambda: lib.moe_combine(A16, BF16, A16, 4, 8, 2048, A16, BF16, NUL),
        lambda: lib.rmsnorm_quantize_per_token_int8(A16, A16, A16, 1e-6, 4, 64, A16, A16, NUL),
        lambda: lib.rmsnorm_bf16(A16, NUL, A16, 1e-6, 4, 64, A16, NUL),
        lambda: lib.silu_mul_quantize_per_token_int8(A16, 4, 64, A16, A16, NUL),
        lambda: lib.silu_mul_bf16(A16, 4, 64, A16, NUL),
    ]
    for call in calls:
        assert call() == HIP
        assert lib.i8ql_last_hip_error() != 0


def test_binding_fails_loudly_without_a_gpu_tensor():
    import torch
    import int8_quantized_linear_amd as i8
    with pytest.raises(ValueError, match="GPU"):
        i8.quantize_per_channel_int8(torch.zeros(4, 8))
