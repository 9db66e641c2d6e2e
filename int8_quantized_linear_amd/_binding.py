"""ctypes binding of ``libi8ql.so``: argument marshalling only.

Every function takes torch tensors on the GPU, checks that they are dense and of the dtype
the C entry point expects, allocates outputs with torch when the caller passes none, and
forwards raw device pointers plus ``torch.cuda.current_stream().cuda_stream`` to the C ABI
of ``include/i8ql.h``.  All arithmetic happens in the HIP kernels.  There is no fallback:
a missing library or a non-OK status raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libi8ql.so")

I8QL_F32, I8QL_BF16, I8QL_F16, I8QL_I8, I8QL_I32 = 0, 1, 2, 3, 4
_DTYPE = {torch.float32: I8QL_F32, torch.bfloat16: I8QL_BF16, torch.float16: I8QL_F16,
          torch.int8: I8QL_I8, torch.int32: I8QL_I32}
EXPORTS = ("quantize_per_channel_int8", "quantize_per_token_int8",
           "quantize_per_token_int8_multi", "w8a8_gemm", "w8a16_gemm",
           "grouped_w8a16_gemm", "w8a8_gemm_config_info", "w8a8_gemm_choose_config",
           "w8a8_gemm_with_config", "w8a8_gemm_choose_plan", "w8a8_gemm_workspace_size",
           "w8a8_gemm_with_plan", "w8a8_gemm_noalloc", "w8a8_gemm_g128",
           "w8a8_gemm_g128_with_config", "grouped_w8a16_silu_gemm", "moe_route_topk",
           "moe_combine", "quantize_per_group_int8", "w8a16_gemm_g128",
           "rmsnorm_quantize_per_token_int8", "rmsnorm_bf16",
           "silu_mul_quantize_per_token_int8", "silu_mul_bf16", "i8ql_status_string",
           "i8ql_last_hip_error")
GROUP_SIZE = 128  # I8QL_GROUP_SIZE
ROUTE_MAX_EXPERTS, ROUTE_MAX_K = 256, 32  # I8QL_ROUTE_MAX_EXPERTS, I8QL_ROUTE_MAX_K
W8A8_NUM_CONFIGS = 12  # I8QL_W8A8_NUM_CONFIGS
W8A8_MAX_SPLITS = 8  # I8QL_W8A8_MAX_SPLITS
W8A8_SPLIT_MAX_TILES = 4096  # I8QL_W8A8_SPLIT_MAX_TILES
W8A8_SCRATCH_BYTES = 32 << 20  # I8QL_W8A8_SCRATCH_BYTES
QUANT_MAX_JOBS = 8  # I8QL_QUANT_MAX_JOBS
NORM_MAX_K = 24576  # I8QL_NORM_MAX_K
SILU_MAX_N = 24576  # I8QL_SILU_MAX_N


class QuantJob(ctypes.Structure):
    """i8ql_quant_job."""
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("k", ctypes.c_int64),
                ("q_out", ctypes.c_void_p), ("scale_out", ctypes.c_void_p)]


class I8qlError(RuntimeError):
    def __init__(self, fn: str, status: int, lib):
        name = lib.i8ql_status_string(status).decode()
        hip = lib.i8ql_last_hip_error() if name == "I8QL_ERR_HIP" else 0
        super().__init__(f"{fn} failed: {name}" + (f" (hipError {hip})" if hip else ""))
        self.status = status
        self.name = name


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libi8ql.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python __graft_entry__.py build` "
                               "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        for fn in ("quantize_per_channel_int8", "quantize_per_token_int8"):
            getattr(lib, fn).argtypes = [P, I, I64, I64, P, P, P]
            getattr(lib, fn).restype = I
        lib.quantize_per_token_int8_multi.argtypes = [P, I, I, P]
        lib.quantize_per_token_int8_multi.restype = I
        lib.w8a8_gemm.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, P]
        lib.w8a8_gemm.restype = I
        lib.w8a8_gemm_with_config.argtypes = [I, P, P, P, P, P, P, I, I64, I64, I64, P]
        lib.w8a8_gemm_with_config.restype = I
        lib.w8a8_gemm_config_info.argtypes = [I, P]
        lib.w8a8_gemm_config_info.restype = I
        lib.w8a8_gemm_choose_config.argtypes = [I64, I64, I64, I]
        lib.w8a8_gemm_choose_config.restype = I
        lib.w8a8_gemm_choose_plan.argtypes = [I64, I64, I64, I, I64, P]
        lib.w8a8_gemm_choose_plan.restype = I
        lib.w8a8_gemm_workspace_size.argtypes = [I, I, I64, I64, I64, I]
        lib.w8a8_gemm_workspace_size.restype = I64
        lib.w8a8_gemm_with_plan.argtypes = [I, I, P, P, P, P, P, P, I, I64, I64, I64, P, I64, P]
        lib.w8a8_gemm_with_plan.restype = I
        lib.w8a8_gemm_noalloc.argtypes = [I, I, P, P, P, P, P, P, I, I64, I64, I64, P]
        lib.w8a8_gemm_noalloc.restype = I
        lib.w8a8_gemm_g128_with_config.argtypes = [I, P, P, P, P, P, P, I, I64, I64, I64, P]
        lib.w8a8_gemm_g128_with_config.restype = I
        lib.w8a8_gemm_g128.argtypes = [P, P, P, P, P, P, I, I64, I64, I64, P]
        lib.w8a8_gemm_g128.restype = I
        lib.w8a16_gemm.argtypes = [P, P, P, P, P, I, I64, I64, I64, P]
        lib.w8a16_gemm.restype = I
        lib.grouped_w8a16_gemm.argtypes = [P, I, P, P, I64, P, I64, I64, P, I, I64, I64, P]
        lib.grouped_w8a16_gemm.restype = I
        lib.grouped_w8a16_silu_gemm.argtypes = [P, I, P, P, I64, P, I64, I64, P, I, I64, I64,
                                                P]
        lib.grouped_w8a16_silu_gemm.restype = I
        lib.quantize_per_group_int8.argtypes = [P, I, I64, I64, P, P, P]
        lib.quantize_per_group_int8.restype = I
        lib.w8a16_gemm_g128.argtypes = [P, P, P, P, P, I, I64, I64, I64, P]
        lib.w8a16_gemm_g128.restype = I
        lib.moe_route_topk.argtypes = [P, I, I64, I64, I64, I64, P, P, P]
        lib.moe_route_topk.restype = I
        lib.moe_combine.argtypes = [P, I, P, I64, I64, I64, P, I, P]
        lib.moe_combine.restype = I
        lib.rmsnorm_quantize_per_token_int8.argtypes = [P, P, P, ctypes.c_float, I64, I64, P,
                                                         P, P]
        lib.rmsnorm_quantize_per_token_int8.restype = I
        lib.rmsnorm_bf16.argtypes = [P, P, P, ctypes.c_float, I64, I64, P, P]
        lib.rmsnorm_bf16.restype = I
        lib.silu_mul_quantize_per_token_int8.argtypes = [P, I64, I64, P, P, P]
        lib.silu_mul_quantize_per_token_int8.restype = I
        lib.silu_mul_bf16.argtypes = [P, I64, I64, P, P]
        lib.silu_mul_bf16.restype = I
        lib.i8ql_status_string.argtypes = [I]
        lib.i8ql_status_string.restype = ctypes.c_char_p
        lib.i8ql_last_hip_error.argtypes = []
        lib.i8ql_last_hip_error.restype = I
        _lib = lib
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(t: torch.Tensor, name: str, dtypes, dim: int | None = None, dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _call(fn: str, *args):
    lib = load_library()
    st = getattr(lib, fn)(*args)
    if st != 0:
        raise I8qlError(fn, st, lib)


def _quantize(fn: str, a: torch.Tensor, q_out=None, scale_out=None):
    _check(a, "input", (torch.float32, torch.bfloat16, torch.float16), 2)
    r, k = a.shape
    q = q_out if q_out is not None else torch.empty((r, k), dtype=torch.int8, device=a.device)
    s = scale_out if scale_out is not None else torch.empty((r,), dtype=torch.float32,
                                                            device=a.device)
    _check(q, "q_out", (torch.int8,), 2, a.device)
    _check(s, "scale_out", (torch.float32,), 1, a.device)
    if tuple(q.shape) != (r, k) or tuple(s.shape) != (r,):
        raise ValueError("output shapes do not match the input")
    with torch.cuda.device(a.device):
        _call(fn, _ptr(a), _DTYPE[a.dtype], r, k, _ptr(q), _ptr(s), _stream(a.device))
    return q, s


def quantize_per_channel_int8(w: torch.Tensor, q_out=None, scale_out=None):
    """Per-output-channel symmetric int8: ``w`` [N, K] fp32/bf16/fp16 -> (q int8 [N, K],
    scale fp32 [N])."""
    return _quantize("quantize_per_channel_int8", w, q_out, scale_out)


def quantize_per_token_int8(x: torch.Tensor, q_out=None, scale_out=None):
    """Dynamic per-token symmetric int8: ``x`` [M, K] -> (q int8 [M, K], scale fp32 [M])."""
    return _quantize("quantize_per_token_int8", x, q_out, scale_out)


def _norm_args(x, gamma, residual):
    _check(x, "x", (torch.bfloat16,), 2)
    m, k = x.shape
    _check(gamma, "gamma", (torch.bfloat16,), 1, x.device)
    if gamma.shape[0] != k:
        raise ValueError(f"gamma has {gamma.shape[0]} elements, x has {k} columns")
    if residual is not None:
        _check(residual, "residual", (torch.bfloat16,), 2, x.device)
        if tuple(residual.shape) != (m, k):
            raise ValueError("residual must have the shape of x")
    return m, k


def rmsnorm_quantize_per_token_int8(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
                                    residual: torch.Tensor | None = None, q_out=None,
                                    scale_out=None):
    """RMS norm of bf16 rows ``x`` [M, K] with weights ``gamma`` [K] (after adding
    ``residual`` in place, if given) fused with the per-token int8 quantization of the
    result: (q int8 [M, K], scale fp32 [M]).  ``residual`` is overwritten with x + residual."""
    m, k = _norm_args(x, gamma, residual)
    q = q_out if q_out is not None else torch.empty((m, k), dtype=torch.int8, device=x.device)
    s = scale_out if scale_out is not None else torch.empty((m,), dtype=torch.float32,
                                                            device=x.device)
    _check(q, "q_out", (torch.int8,), 2, x.device)
    _check(s, "scale_out", (torch.float32,), 1, x.device)
    if tuple(q.shape) != (m, k) or tuple(s.shape) != (m,):
        raise ValueError("output shapes do not match the input")
    with torch.cuda.device(x.device):
        _call("rmsnorm_quantize_per_token_int8", _ptr(x), _ptr(residual), _ptr(gamma),
              float(eps), m, k, _ptr(q), _ptr(s), _stream(x.device))
    return q, s


def rmsnorm_bf16(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
                 residual: torch.Tensor | None = None, y_out=None):
    """The same RMS norm written as bf16 [M, K] (the unfused producer)."""
    m, k = _norm_args(x, gamma, residual)
    y = y_out if y_out is not None else torch.empty((m, k), dtype=torch.bfloat16, device=x.device)
    _check(y, "y_out", (torch.bfloat16,), 2, x.device)
    if tuple(y.shape) != (m, k):
        raise ValueError("y_out must have the shape of x")
    with torch.cuda.device(x.device):
        _call("rmsnorm_bf16", _ptr(x), _ptr(residual), _ptr(gamma), float(eps), m, k, _ptr(y),
              _stream(x.device))
    return y


def silu_mul_quantize_per_token_int8(gu: torch.Tensor, q_out=None, scale_out=None):
    """SiLU·mul of a gate/up product ``gu`` [M, 2N] bf16 (gate columns first) fused with the
    per-token int8 quantization of the result: (q int8 [M, N], scale fp32 [M])."""
    _check(gu, "gu", (torch.bfloat16,), 2)
    m, n2 = gu.shape
    if n2 % 2:
        raise ValueError("gu must hold gate and up halves of equal width")
    n = n2 // 2
    q = q_out if q_out is not None else torch.empty((m, n), dtype=torch.int8, device=gu.device)
    s = scale_out if scale_out is not None else torch.empty((m,), dtype=torch.float32,
                                                            device=gu.device)
    _check(q, "q_out", (torch.int8,), 2, gu.device)
    _check(s, "scale_out", (torch.float32,), 1, gu.device)
    if tuple(q.shape) != (m, n) or tuple(s.shape) != (m,):
        raise ValueError("output shapes do not match the input")
    with torch.cuda.device(gu.device):
        _call("silu_mul_quantize_per_token_int8", _ptr(gu), m, n, _ptr(q), _ptr(s),
              _stream(gu.device))
    return q, s


def silu_mul_bf16(gu: torch.Tensor, h_out=None):
    """The same SiLU·mul written as bf16 [M, N] (the unfused producer)."""
    _check(gu, "gu", (torch.bfloat16,), 2)
    m, n2 = gu.shape
    if n2 % 2:
        raise ValueError("gu must hold gate and up halves of equal width")
    n = n2 // 2
    h = h_out if h_out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=gu.device)
    _check(h, "h_out", (torch.bfloat16,), 2, gu.device)
    if tuple(h.shape) != (m, n):
        raise ValueError("h_out must be [M, N]")
    with torch.cuda.device(gu.device):
        _call("silu_mul_bf16", _ptr(gu), m, n, _ptr(h), _stream(gu.device))
    return h


def quantize_per_token_int8_multi(xs, outs=None):
    """``quantize_per_token_int8`` of several activation matrices (one dtype, up to
    QUANT_MAX_JOBS) in one launch: a list of (q int8 [M, K], scale fp32 [M]), bitwise those
    of the separate calls.  ``outs``: optional list of (q, scale) to write into."""
    if not 1 <= len(xs) <= QUANT_MAX_JOBS:
        raise ValueError(f"1 to {QUANT_MAX_JOBS} matrices per launch")
    dev, dt = xs[0].device, xs[0].dtype
    res, jobs = [], (QuantJob * len(xs))()
    for i, x in enumerate(xs):
        _check(x, f"xs[{i}]", (dt,), 2, dev)
        r, k = x.shape
        q, s = outs[i] if outs is not None else (
            torch.empty((r, k), dtype=torch.int8, device=dev),
            torch.empty((r,), dtype=torch.float32, device=dev))
        _check(q, "q_out", (torch.int8,), 2, dev)
        _check(s, "scale_out", (torch.float32,), 1, dev)
        if tuple(q.shape) != (r, k) or tuple(s.shape) != (r,):
            raise ValueError("output shapes do not match the input")
        jobs[i] = QuantJob(x.data_ptr(), r, k, q.data_ptr(), s.data_ptr())
        res.append((q, s))
    with torch.cuda.device(dev):
        _call("quantize_per_token_int8_multi", ctypes.cast(jobs, ctypes.c_void_p), len(xs),
              _DTYPE[dt], _stream(dev))
    return res


def _out(out, shape, dtype, dev):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _check(out, "out", (dtype,), len(shape), dev)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    return out


def _cus(dev) -> int:
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if idx not in _CUS:
        _CUS[idx] = torch.cuda.get_device_properties(idx).multi_processor_count
    return _CUS[idx]


_CUS: dict = {}
_WORKSPACE: dict = {}


def w8a8_workspace(dev, nbytes: int) -> torch.Tensor:
    """The W8A8 workspace this binding keeps for ``dev``: a zero-filled uint8 tensor of at
    least ``nbytes``, grown (never inside a graph capture) when a call needs more.  The
    kernels leave its counters at zero after every call, so it is reused without clearing.
    Calls on several streams that may overlap must each pass a workspace of their own."""
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    ws = _WORKSPACE.get(idx)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("w8a8_gemm needs a larger workspace during a graph capture: run "
                               "the same call once before capturing it")
        nbytes = max(int(nbytes), 1 << 20)
        ws = torch.zeros(-(-nbytes // (1 << 20)) << 20, dtype=torch.uint8,
                         device=torch.device("cuda", idx))
        _WORKSPACE[idx] = ws
    return ws


def w8a8_gemm(xq, x_scale, wq, w_scale, bias=None, out_dtype=torch.bfloat16, out=None,
              workspace=None):
    """``y = (xq @ wq.T) * x_scale[:, None] * w_scale[None, :] (+ bias)``; int32 when
    ``out_dtype`` is torch.int32 (then scales may be None and bias must be None).  Launches
    the cost model's best plan, which may split k across workgroups through ``workspace``
    (a zero-filled uint8 CUDA tensor) or, when None, the workspace kept per device."""
    return w8a8_gemm_with_plan(-1, -1, xq, x_scale, wq, w_scale, bias, out_dtype, out,
                               workspace)


def w8a8_gemm_with_config(config, xq, x_scale, wq, w_scale, bias=None,
                          out_dtype=torch.bfloat16, out=None):
    """``w8a8_gemm`` with tile configuration ``config`` and no split (-1: the cost model's
    choice among plans without a split)."""
    m, n, k, y, dev = _w8a8_args(xq, x_scale, wq, w_scale, bias, out_dtype, out)
    with torch.cuda.device(dev):
        _call("w8a8_gemm_with_config", int(config), _ptr(xq), _ptr(x_scale), _ptr(wq),
              _ptr(w_scale), _ptr(bias), _ptr(y), _DTYPE[out_dtype], m, n, k, _stream(dev))
    return y


def w8a8_gemm_with_plan(config, splits, xq, x_scale, wq, w_scale, bias=None,
                        out_dtype=torch.bfloat16, out=None, workspace=None):
    """``w8a8_gemm`` with plan (``config``, ``splits``): k split across ``splits`` workgroups
    per output tile; (-1, -1) is the cost model's best plan.  ``workspace``: a zero-filled
    uint8 CUDA tensor, or None for the one kept per device."""
    m, n, k, y, dev = _w8a8_args(xq, x_scale, wq, w_scale, bias, out_dtype, out)
    need = w8a8_gemm_workspace_size(m, n, k, _cus(dev), config, splits) if m and n else 0
    if workspace is None:
        workspace = w8a8_workspace(dev, need) if need > 0 else None
    else:
        _check(workspace, "workspace", (torch.uint8,), 1, dev)
    nbytes = 0 if workspace is None else workspace.numel()
    with torch.cuda.device(dev):
        _call("w8a8_gemm_with_plan", int(config), int(splits), _ptr(xq), _ptr(x_scale),
              _ptr(wq), _ptr(w_scale), _ptr(bias), _ptr(y), _DTYPE[out_dtype], m, n, k,
              _ptr(workspace), nbytes, _stream(dev))
    return y


def w8a8_gemm_noalloc(xq, x_scale, wq, w_scale, bias=None, out_dtype=torch.bfloat16,
                      out=None, config=-1, splits=-1):
    """``w8a8_gemm_with_plan`` with the library's static scratch array as the workspace (the
    C entry point allocates nothing; pass ``out`` to keep this wrapper from allocating the
    output).  Calls that overlap in time on one GPU race on the scratch."""
    m, n, k, y, dev = _w8a8_args(xq, x_scale, wq, w_scale, bias, out_dtype, out)
    with torch.cuda.device(dev):
        _call("w8a8_gemm_noalloc", int(config), int(splits), _ptr(xq), _ptr(x_scale),
              _ptr(wq), _ptr(w_scale), _ptr(bias), _ptr(y), _DTYPE[out_dtype], m, n, k,
              _stream(dev))
    return y


def w8a8_gemm_g128(xq, x_scale, wq, w_scale, bias=None, out_dtype=torch.bfloat16, out=None,
                   config=-1):
    """W8A8 with weight scales per group of 128 input channels: ``w_scale`` [N, K/128]
    (from ``quantize_per_group_int8``); ``y = x_scale[:, None] * sum_g w_scale[:, g] *
    (xq_g @ wq_g.T) (+ bias)``, bf16 or float32."""
    _check(xq, "xq", (torch.int8,), 2)
    dev = xq.device
    _check(wq, "wq", (torch.int8,), 2, dev)
    _check(x_scale, "x_scale", (torch.float32,), 1, dev)
    _check(w_scale, "w_scale", (torch.float32,), 2, dev)
    m, k = xq.shape
    n = wq.shape[0]
    if wq.shape[1] != k or x_scale.shape[0] != m or k % GROUP_SIZE or \
            tuple(w_scale.shape) != (n, k // GROUP_SIZE):
        raise ValueError("xq, x_scale, wq and w_scale disagree")
    if bias is not None:
        _check(bias, "bias", (torch.float32,), 1, dev)
        if bias.shape[0] != n:
            raise ValueError("bias must have N entries")
    y = _out(out, (m, n), out_dtype, dev)
    with torch.cuda.device(dev):
        _call("w8a8_gemm_g128_with_config", int(config), _ptr(xq), _ptr(x_scale), _ptr(wq),
              _ptr(w_scale), _ptr(bias), _ptr(y), _DTYPE[out_dtype], m, n, k, _stream(dev))
    return y


def _w8a8_args(xq, x_scale, wq, w_scale, bias, out_dtype, out):
    _check(xq, "xq", (torch.int8,), 2)
    dev = xq.device
    _check(wq, "wq", (torch.int8,), 2, dev)
    m, k = xq.shape
    n = wq.shape[0]
    if wq.shape[1] != k:
        raise ValueError("xq and wq disagree on K")
    for t, nm, ln in ((x_scale, "x_scale", m), (w_scale, "w_scale", n), (bias, "bias", n)):
        if t is not None:
            _check(t, nm, (torch.float32,), 1, dev)
            if t.shape[0] != ln:
                raise ValueError(f"{nm} must have {ln} entries")
    return m, n, k, _out(out, (m, n), out_dtype, dev), dev


def w8a8_gemm_config_info(config: int):
    """(tile rows, tile columns, k-groups, splittable, runs group scales) of W8A8 tile
    configuration ``config``."""
    lib = load_library()
    out = (ctypes.c_int32 * 5)()
    st = lib.w8a8_gemm_config_info(int(config), ctypes.cast(out, ctypes.c_void_p))
    if st != 0:
        raise I8qlError("w8a8_gemm_config_info", st, lib)
    return tuple(out)


def w8a8_gemm_choose_config(m: int, n: int, k: int, cus: int = 256) -> int:
    """The configuration ``w8a8_gemm`` launches without a workspace for an m x n x k product
    on ``cus`` compute units (-1 for sizes ``w8a8_gemm`` rejects); host arithmetic only."""
    return load_library().w8a8_gemm_choose_config(m, n, k, cus)


def w8a8_gemm_choose_plan(m: int, n: int, k: int, cus: int = 256,
                          workspace_bytes: int = 1 << 62):
    """(config, splits) the cost model launches with a workspace of ``workspace_bytes``."""
    lib = load_library()
    out = (ctypes.c_int32 * 2)()
    st = lib.w8a8_gemm_choose_plan(m, n, k, cus, workspace_bytes,
                                   ctypes.cast(out, ctypes.c_void_p))
    if st != 0:
        raise I8qlError("w8a8_gemm_choose_plan", st, lib)
    return tuple(out)


def w8a8_gemm_workspace_size(m: int, n: int, k: int, cus: int = 256, config: int = -1,
                             splits: int = -1) -> int:
    """Workspace bytes of plan (config, splits), or of the cost model's preferred plan."""
    nb = load_library().w8a8_gemm_workspace_size(int(config), int(splits), m, n, k, cus)
    if nb < 0:
        raise ValueError(f"no valid W8A8 plan ({config}, {splits}) for {m}x{n}x{k}")
    return nb


def w8a16_gemm(x, wq, w_scale, bias=None, out_dtype=torch.bfloat16, out=None):
    """``y = x @ (w_scale[:, None] * wq).T (+ bias)`` with bf16 ``x`` [M, K]."""
    _check(x, "x", (torch.bfloat16,), 2)
    dev = x.device
    _check(wq, "wq", (torch.int8,), 2, dev)
    _check(w_scale, "w_scale", (torch.float32,), 1, dev)
    m, k = x.shape
    n = wq.shape[0]
    if wq.shape[1] != k or w_scale.shape[0] != n:
        raise ValueError("x, wq and w_scale disagree")
    if bias is not None:
        _check(bias, "bias", (torch.float32,), 1, dev)
        if bias.shape[0] != n:
            raise ValueError("bias must have N entries")
    y = _out(out, (m, n), out_dtype, dev)
    with torch.cuda.device(dev):
        _call("w8a16_gemm", _ptr(x), _ptr(wq), _ptr(w_scale), _ptr(bias), _ptr(y),
              _DTYPE[out_dtype], m, n, k, _stream(dev))
    return y


def grouped_w8a16_gemm(x, wq, w_scale, expert_ids, x_per_assignment=False,
                       out_dtype=torch.bfloat16, out=None):
    """Grouped weight-only GEMM over experts: ``wq`` [E, N, K], ``w_scale`` [E, N],
    ``expert_ids`` [T, topk] int32, ``x`` [T, K] (or [T*topk, K] when
    ``x_per_assignment``) -> [T*topk, N]."""
    _check(x, "x", (torch.bfloat16,), 2)
    dev = x.device
    _check(wq, "wq", (torch.int8,), 3, dev)
    _check(w_scale, "w_scale", (torch.float32,), 2, dev)
    _check(expert_ids, "expert_ids", (torch.int32,), 2, dev)
    e, n, k = wq.shape
    t, topk = expert_ids.shape
    if tuple(w_scale.shape) != (e, n) or x.shape[1] != k:
        raise ValueError("x, wq and w_scale disagree")
    if x.shape[0] != (t * topk if x_per_assignment else t):
        raise ValueError("x has the wrong number of rows for x_per_assignment")
    y = _out(out, (t * topk, n), out_dtype, dev)
    with torch.cuda.device(dev):
        _call("grouped_w8a16_gemm", _ptr(x), int(bool(x_per_assignment)), _ptr(wq),
              _ptr(w_scale), e, _ptr(expert_ids), t, topk, _ptr(y), _DTYPE[out_dtype], n, k,
              _stream(dev))
    return y


def grouped_w8a16_silu_gemm(x, wq, w_scale, expert_ids, x_per_assignment=False,
                            out_dtype=torch.bfloat16, out=None):
    """Gate and up projections of the experts with SiLU·mul fused: ``wq`` [E, 2N, K] (gate
    rows, then up rows, per expert), ``w_scale`` [E, 2N] -> ``silu(gate) * up`` [T*topk, N]."""
    _check(x, "x", (torch.bfloat16,), 2)
    dev = x.device
    _check(wq, "wq", (torch.int8,), 3, dev)
    _check(w_scale, "w_scale", (torch.float32,), 2, dev)
    _check(expert_ids, "expert_ids", (torch.int32,), 2, dev)
    e, n2, k = wq.shape
    if n2 % 2:
        raise ValueError("wq must stack gate and up rows: an even number of rows per expert")
    n = n2 // 2
    t, topk = expert_ids.shape
    if tuple(w_scale.shape) != (e, n2) or x.shape[1] != k:
        raise ValueError("x, wq and w_scale disagree")
    if x.shape[0] != (t * topk if x_per_assignment else t):
        raise ValueError("x has the wrong number of rows for x_per_assignment")
    h = _out(out, (t * topk, n), out_dtype, dev)
    with torch.cuda.device(dev):
        _call("grouped_w8a16_silu_gemm", _ptr(x), int(bool(x_per_assignment)), _ptr(wq),
              _ptr(w_scale), e, _ptr(expert_ids), t, topk, _ptr(h), _DTYPE[out_dtype], n, k,
              _stream(dev))
    return h


def moe_route_topk(logits, k_routed, n_shared=0, ids_out=None, weights_out=None):
    """Top-k routing: ``logits`` [T, E] fp32/bf16 -> (ids int32 [T, k+shared], weights fp32
    [T, k+shared]); softmax weights of the k largest logits, shared experts E.. appended with
    weight 1."""
    _check(logits, "logits", (torch.float32, torch.bfloat16), 2)
    dev = logits.device
    t, e = logits.shape
    kk = k_routed + n_shared
    ids = _out(ids_out, (t, kk), torch.int32, dev)
    w = _out(weights_out, (t, kk), torch.float32, dev)
    with torch.cuda.device(dev):
        _call("moe_route_topk", _ptr(logits), _DTYPE[logits.dtype], t, e, k_routed, n_shared,
              _ptr(ids), _ptr(w), _stream(dev))
    return ids, w


def moe_combine(d, weights, out_dtype=torch.bfloat16, out=None):
    """Routing-weighted combine: ``d`` [T*topk, N] bf16/fp32, ``weights`` [T, topk] fp32 ->
    ``y[i] = sum_j weights[i, j] * d[i*topk + j]`` [T, N]."""
    _check(d, "d", (torch.bfloat16, torch.float32), 2)
    dev = d.device
    _check(weights, "weights", (torch.float32,), 2, dev)
    t, topk = weights.shape
    if d.shape[0] != t * topk:
        raise ValueError("d must have t * topk rows")
    n = d.shape[1]
    y = _out(out, (t, n), out_dtype, dev)
    with torch.cuda.device(dev):
        _call("moe_combine", _ptr(d), _DTYPE[d.dtype], _ptr(weights), t, topk, n, _ptr(y),
              _DTYPE[out_dtype], _stream(dev))
    return y


def quantize_per_group_int8(w: torch.Tensor, q_out=None, scale_out=None):
    """One int8 scale per group of 128 input channels: ``w`` [N, K] fp32/bf16/fp16 (K a
    multiple of 128) -> (q int8 [N, K], scale fp32 [N, K/128])."""
    _check(w, "w", (torch.float32, torch.bfloat16, torch.float16), 2)
    n, k = w.shape
    q = q_out if q_out is not None else torch.empty((n, k), dtype=torch.int8, device=w.device)
    s = scale_out if scale_out is not None else torch.empty(
        (n, k // GROUP_SIZE), dtype=torch.float32, device=w.device)
    _check(q, "q_out", (torch.int8,), 2, w.device)
    _check(s, "scale_out", (torch.float32,), 2, w.device)
    if tuple(q.shape) != (n, k) or tuple(s.shape) != (n, k // GROUP_SIZE):
        raise ValueError("output shapes do not match the input")
    with torch.cuda.device(w.device):
        _call("quantize_per_group_int8", _ptr(w), _DTYPE[w.dtype], n, k, _ptr(q), _ptr(s),
              _stream(w.device))
    return q, s


def w8a16_gemm_g128(x, wq, w_scale, bias=None, out_dtype=torch.bfloat16, out=None):
    """Weight-only GEMM with group scales: ``x`` [M, K] bf16, ``wq`` [N, K] int8,
    ``w_scale`` [N, K/128] fp32 -> [M, N]."""
    _check(x, "x", (torch.bfloat16,), 2)
    dev = x.device
    _check(wq, "wq", (torch.int8,), 2, dev)
    _check(w_scale, "w_scale", (torch.float32,), 2, dev)
    m, k = x.shape
    n = wq.shape[0]
    if wq.shape[1] != k or tuple(w_scale.shape) != (n, k // GROUP_SIZE):
        raise ValueError("x, wq and w_scale disagree")
    if bias is not None:
        _check(bias, "bias", (torch.float32,), 1, dev)
        if bias.shape[0] != n:
            raise ValueError("bias must have N entries")
    y = _out(out, (m, n), out_dtype, dev)
    with torch.cuda.device(dev):
        _call("w8a16_gemm_g128", _ptr(x), _ptr(wq), _ptr(w_scale), _ptr(bias), _ptr(y),
              _DTYPE[out_dtype], m, n, k, _stream(dev))
    return y
