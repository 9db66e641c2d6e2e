"""CPU oracle of the int8 quantized linear layer (ctypes wrapper over ``ref.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the HIP library never does, and this package imports nothing from
the library.  Every function here marshals numpy arrays into the plain C loops of ``ref.c``,
which follow the pages:

* "Day 6 — Quantize It Yourself", The mechanism, block 1 (absmax scale, clamp(round(w/s)))
  and block 5 (W8A8 vs weight-only W8A16);
* "Phase 5a: int8 weight-only quantization", Summary (float32 quantizer arithmetic, the
  all-zero-channel guard, the grouped expert GEMM);
* "feat(quantization): support compressed-tensors W8A8 and mixed modules", Design and
  Supported Execution Scheme (per-channel weights, dynamic per-token activations);
* the mixture-of-experts block around the grouped GEMM (routing, SiLU·mul, combine), which
  "Phase 5a" measures but no page spells out: readings stated in ``ref.c``.

Parity pins: every function is pinned by ``tests/test_oracle_pins.py``; none is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libi8ql_oracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra"]

REF_F32, REF_BF16, REF_F16 = 0, 1, 2


def build(out_path: str = LIB_PATH, defines: tuple[str, ...] = ()) -> str:
    """Compile ``ref.c`` with gcc into ``out_path`` (``defines`` e.g. ``("REF_MUTANT_BF16_ARITH",)``)."""
    cmd = ["gcc", *CFLAGS, *[f"-D{d}" for d in defines], os.path.join(_HERE, "ref.c"),
           "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class Oracle:
    """One loaded build of the oracle (the normal one, or a mutant for teeth tests)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library {path} is not built (run oracle.build())")
        lib = ctypes.CDLL(path)
        lib.ref_quantize_rows.argtypes = [_P, ctypes.c_int, _I64, _I64, _P, _P]
        lib.ref_quantize_rows.restype = ctypes.c_int
        lib.ref_w8a8.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
        lib.ref_w8a8.restype = ctypes.c_int
        lib.ref_w8a16.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P]
        lib.ref_w8a16.restype = None
        lib.ref_grouped_w8a16.argtypes = [_P, ctypes.c_int, _P, _P, _I64, _P, _I64, _I64,
                                          _I64, _I64, _P]
        lib.ref_grouped_w8a16.restype = None
        lib.ref_moe_route_topk.argtypes = [_P, _I64, _I64, _I64, _I64, _P, _P]
        lib.ref_moe_route_topk.restype = None
        lib.ref_grouped_w8a16_silu.argtypes = [_P, ctypes.c_int, _P, _P, _I64, _P, _I64, _I64,
                                               _I64, _I64, _P]
        lib.ref_grouped_w8a16_silu.restype = None
        lib.ref_moe_combine.argtypes = [_P, _P, _I64, _I64, _I64, _P]
        lib.ref_moe_combine.restype = None
        lib.ref_quantize_groups.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P]
        lib.ref_quantize_groups.restype = ctypes.c_int
        lib.ref_w8a16_grouped_scales.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
        lib.ref_w8a16_grouped_scales.restype = None
        lib.ref_w8a8_grouped_scales.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
        lib.ref_w8a8_grouped_scales.restype = None
        lib.ref_rmsnorm.argtypes = [_P, _P, _P, ctypes.c_float, _I64, _I64, _P, _P]
        lib.ref_rmsnorm.restype = None
        lib.ref_silu_mul.argtypes = [_P, _I64, _I64, ctypes.c_double, _P, _P, _P]
        lib.ref_silu_mul.restype = None
        lib.ref_codes_with_scale.argtypes = [_P, _P, _I64, _I64, _P]
        lib.ref_codes_with_scale.restype = None
        lib.ref_set_threads.argtypes = [ctypes.c_int]
        lib.ref_get_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # -- helpers ---------------------------------------------------------------------------
    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    def set_threads(self, n: int) -> None:
        self.lib.ref_set_threads(int(n))

    def threads(self) -> int:
        return int(self.lib.ref_get_threads())

    # -- the method -----------------------------------------------------------------------
    def quantize_rows(self, a: np.ndarray, dtype: str):
        """Row-wise symmetric int8 quantization of ``a`` ([r, k]).

        ``dtype`` names how ``a`` is stored: "f32" (float32 array), "bf16" or "f16"
        (uint16 bit patterns).  Returns ``(q int8 [r, k], scale float32 [r])``.
        """
        code = {"f32": REF_F32, "bf16": REF_BF16, "f16": REF_F16}[dtype]
        want = np.float32 if code == REF_F32 else np.uint16
        a = np.ascontiguousarray(a, dtype=want)
        r, k = a.shape
        q = np.empty((r, k), np.int8)
        s = np.empty((r,), np.float32)
        rc = self.lib.ref_quantize_rows(self._ptr(a), code, r, k, self._ptr(q), self._ptr(s))
        if rc != 0:
            raise ValueError("bad dtype")
        return q, s

    def w8a8(self, xq, x_scale, wq, w_scale, bias=None, want_y=True):
        """Exact int32 accumulators and the float64 epilogue value ``acc*sx*sw (+bias)``."""
        xq = np.ascontiguousarray(xq, np.int8)
        wq = np.ascontiguousarray(wq, np.int8)
        m, k = xq.shape
        n, k2 = wq.shape
        assert k == k2
        sx = None if x_scale is None else np.ascontiguousarray(x_scale, np.float32)
        sw = None if w_scale is None else np.ascontiguousarray(w_scale, np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, np.float32)
        acc = np.empty((m, n), np.int32)
        y = np.empty((m, n), np.float64) if want_y else None
        rc = self.lib.ref_w8a8(self._ptr(xq), self._ptr(sx), self._ptr(wq), self._ptr(sw),
                               self._ptr(b), m, n, k, self._ptr(acc), self._ptr(y))
        if rc != 0:
            raise OverflowError("int32 accumulator overflow")
        return acc, y

    def w8a16(self, x_bf16_bits, wq, w_scale, bias=None):
        """float64 ``w_scale[j] * sum_c x[i,c]*wq[j,c] (+bias[j])``; x as bf16 bit patterns."""
        x = np.ascontiguousarray(x_bf16_bits, np.uint16)
        wq = np.ascontiguousarray(wq, np.int8)
        sw = np.ascontiguousarray(w_scale, np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, np.float32)
        m, k = x.shape
        n, k2 = wq.shape
        assert k == k2
        y = np.empty((m, n), np.float64)
        self.lib.ref_w8a16(self._ptr(x), self._ptr(wq), self._ptr(sw), self._ptr(b), m, n, k,
                           self._ptr(y))
        return y

    def grouped_w8a16(self, x_bf16_bits, x_per_assignment, wq, w_scale, expert_ids):
        """float64 grouped weight-only product, one output row per (token, slot)."""
        x = np.ascontiguousarray(x_bf16_bits, np.uint16)
        wq = np.ascontiguousarray(wq, np.int8)
        sw = np.ascontiguousarray(w_scale, np.float32)
        ids = np.ascontiguousarray(expert_ids, np.int32)
        e, n, k = wq.shape
        t, topk = ids.shape
        assert x.shape[1] == k
        assert x.shape[0] == (t * topk if x_per_assignment else t)
        y = np.empty((t * topk, n), np.float64)
        self.lib.ref_grouped_w8a16(self._ptr(x), int(bool(x_per_assignment)), self._ptr(wq),
                                   self._ptr(sw), e, self._ptr(ids), t, topk, n, k,
                                   self._ptr(y))
        return y


    # -- one scale per group of input channels ("Day 6", The mechanism, block 1) ---------
    def quantize_groups(self, a: np.ndarray, dtype: str, group: int = 128):
        """Per-group symmetric int8 of ``a`` [r, k] (k % group == 0): ``(q int8 [r, k],
        scale float32 [r, k // group])``, the row rule applied to every group."""
        code = {"f32": REF_F32, "bf16": REF_BF16, "f16": REF_F16}[dtype]
        want = np.float32 if code == REF_F32 else np.uint16
        a = np.ascontiguousarray(a, dtype=want)
        r, k = a.shape
        q = np.empty((r, k), np.int8)
        s = np.empty((r, k // group), np.float32)
        rc = self.lib.ref_quantize_groups(self._ptr(a), code, r, k, group, self._ptr(q),
                                          self._ptr(s))
        if rc != 0:
            raise ValueError("bad dtype or k not a multiple of the group")
        return q, s

    def w8a16_grouped_scales(self, x_bf16_bits, wq, w_scale, group: int = 128, bias=None):
        """float64 ``sum_g w_scale[j, g] * sum_{c in g} x[i, c] * wq[j, c] (+ bias[j])``."""
        x = np.ascontiguousarray(x_bf16_bits, np.uint16)
        wq = np.ascontiguousarray(wq, np.int8)
        sw = np.ascontiguousarray(w_scale, np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, np.float32)
        m, k = x.shape
        n, k2 = wq.shape
        assert k == k2 and k % group == 0 and sw.shape == (n, k // group)
        y = np.empty((m, n), np.float64)
        self.lib.ref_w8a16_grouped_scales(self._ptr(x), self._ptr(wq), self._ptr(sw),
                                          self._ptr(b), m, n, k, group, self._ptr(y))
        return y

    def w8a8_grouped_scales(self, xq, x_scale, wq, w_scale, group: int = 128, bias=None):
        """float64 ``x_scale[i] * sum_g w_scale[j, g] * sum_{c in g} xq[i,c]*wq[j,c] (+ bias)``
        with each group's code products summed exactly."""
        xq = np.ascontiguousarray(xq, np.int8)
        wq = np.ascontiguousarray(wq, np.int8)
        sx = np.ascontiguousarray(x_scale, np.float32)
        sw = np.ascontiguousarray(w_scale, np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, np.float32)
        m, k = xq.shape
        n, k2 = wq.shape
        assert k == k2 and k % group == 0 and sw.shape == (n, k // group) and sx.shape == (m,)
        y = np.empty((m, n), np.float64)
        self.lib.ref_w8a8_grouped_scales(self._ptr(xq), self._ptr(sx), self._ptr(wq),
                                         self._ptr(sw), self._ptr(b), m, n, k, group,
                                         self._ptr(y))
        return y

    # -- mixture-of-experts steps around the grouped GEMM (readings stated in ref.c) -----
    def moe_route_topk(self, logits, k_routed: int, n_shared: int):
        """``(ids int32 [t, k_routed + n_shared], weights float64 [t, ...])`` from float32
        router logits ``[t, e_routed]``: softmax, the k_routed largest kept by decreasing
        logit (lower index first on ties), shared experts appended with weight 1."""
        lg = np.ascontiguousarray(logits, np.float32)
        t, e_routed = lg.shape
        kk = k_routed + n_shared
        ids = np.empty((t, kk), np.int32)
        w = np.empty((t, kk), np.float64)
        self.lib.ref_moe_route_topk(self._ptr(lg), t, e_routed, k_routed, n_shared,
                                    self._ptr(ids), self._ptr(w))
        return ids, w

    def grouped_w8a16_silu(self, x_bf16_bits, x_per_assignment, wq, w_scale, expert_ids):
        """float64 ``silu(gate) * up`` per assignment; ``wq`` is ``[e, 2n, k]`` with each
        expert's gate rows before its up rows."""
        x = np.ascontiguousarray(x_bf16_bits, np.uint16)
        wq = np.ascontiguousarray(wq, np.int8)
        sw = np.ascontiguousarray(w_scale, np.float32)
        ids = np.ascontiguousarray(expert_ids, np.int32)
        e, n2, k = wq.shape
        assert n2 % 2 == 0
        n = n2 // 2
        t, topk = ids.shape
        assert x.shape[1] == k
        assert x.shape[0] == (t * topk if x_per_assignment else t)
        h = np.empty((t * topk, n), np.float64)
        self.lib.ref_grouped_w8a16_silu(self._ptr(x), int(bool(x_per_assignment)),
                                        self._ptr(wq), self._ptr(sw), e, self._ptr(ids), t,
                                        topk, n, k, self._ptr(h))
        return h

    def moe_combine(self, d, weights):
        """float64 ``y[i] = sum_j weights[i, j] * d[i * topk + j]`` (``d`` float32 values)."""
        dd = np.ascontiguousarray(d, np.float32)
        w = np.ascontiguousarray(weights, np.float32)
        t, topk = w.shape
        assert dd.shape[0] == t * topk
        n = dd.shape[1]
        y = np.empty((t, n), np.float64)
        self.lib.ref_moe_combine(self._ptr(dd), self._ptr(w), t, topk, n, self._ptr(y))
        return y

    def rmsnorm(self, x_bf16_bits, gamma_bf16_bits, eps: float, residual_bf16_bits=None):
        """RMS normalization of bf16 rows (reading in ``ref.c``).

        Returns ``h`` (uint16 bf16 bits, [m, k]) and, with a residual, the updated residual
        ``bf16(x + residual)`` as well: ``(h, res_out)``; ``res_out`` is None without one.
        """
        x = np.ascontiguousarray(x_bf16_bits, np.uint16)
        g = np.ascontiguousarray(gamma_bf16_bits, np.uint16)
        m, k = x.shape
        assert g.shape == (k,)
        res = None if residual_bf16_bits is None else np.ascontiguousarray(residual_bf16_bits,
                                                                           np.uint16)
        assert res is None or res.shape == (m, k)
        h = np.empty((m, k), np.uint16)
        res_out = None if res is None else np.empty((m, k), np.uint16)
        self.lib.ref_rmsnorm(self._ptr(x), self._ptr(res), self._ptr(g), float(eps), m, k,
                             self._ptr(res_out), self._ptr(h))
        return h, res_out

    def rmsnorm_quantize(self, x_bf16_bits, gamma_bf16_bits, eps: float,
                         residual_bf16_bits=None):
        """Per-token int8 quantization of the RMS-normalized rows: the row quantizer applied
        to ``rmsnorm``'s bf16 output.  Returns ``(q, scale, res_out)``."""
        h, res_out = self.rmsnorm(x_bf16_bits, gamma_bf16_bits, eps, residual_bf16_bits)
        q, s = self.quantize_rows(h, "bf16")
        return q, s, res_out

    def silu_mul(self, gu_bf16_bits, rel: float = 0.0):
        """SiLU·mul of a gate/up product ``gu`` [m, 2i] (bf16 bits, gate columns first):
        returns ``(h, other, amb)``: h [m, i] the bf16 nearest to g / (1 + e^-g) * u (double),
        other the bf16 on the other side of the exact value, amb where the exact value is
        within ``rel`` of the halfway point between them."""
        gu = np.ascontiguousarray(gu_bf16_bits, np.uint16)
        m, i2 = gu.shape
        assert i2 % 2 == 0
        i = i2 // 2
        h = np.empty((m, i), np.uint16)
        other = np.empty((m, i), np.uint16)
        amb = np.empty((m, i), np.uint8)
        self.lib.ref_silu_mul(self._ptr(gu), m, i, float(rel), self._ptr(h), self._ptr(other),
                              self._ptr(amb))
        return h, other, amb.astype(bool)

    def codes_with_scale(self, a_bf16_bits, scale):
        """The row quantizer's code step with given per-row scales (bf16 rows)."""
        a = np.ascontiguousarray(a_bf16_bits, np.uint16)
        s = np.ascontiguousarray(scale, np.float32)
        r, k = a.shape
        q = np.empty((r, k), np.int8)
        self.lib.ref_codes_with_scale(self._ptr(a), self._ptr(s), r, k, self._ptr(q))
        return q


_DEFAULT: Oracle | None = None


def load(build_if_missing: bool = True) -> Oracle:
    """The normal oracle build, compiled first if it is missing."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIB_PATH) and build_if_missing:
            build()
        _DEFAULT = Oracle(LIB_PATH)
    return _DEFAULT
