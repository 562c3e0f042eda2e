"""Float64 CPU oracle for RMSNorm, its fused residual pre-norm form and its
backward pass (plain C in rmsnorm_oracle.c, loaded with ctypes).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  The GPU library never imports, links or calls it,
and this package imports nothing from the GPU library.

Every function takes stored bits (numpy arrays: float32, float16, or uint16
bit patterns for bfloat16, or float64 for finite-difference checks) and
returns float64 results computed from their exact values.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rmsnorm_oracle.c")
_LIB = os.path.join(_HERE, "_liboracle.so")

CODES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "f64": np.float64}

_lock = threading.Lock()
_default = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (IEEE float64, no contraction, no fast-math)."""
    if force or not os.path.exists(out):
        tmp = f"{out}.{os.getpid()}.tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-Werror", src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data


def _rows(a, dtype):
    """(array, row stride in elements) for a 2-D array with unit column stride."""
    a = np.asarray(a)
    if a.dtype != np.dtype(_NP[dtype]):
        raise TypeError(f"expected {_NP[dtype]} storage for {dtype}, got {a.dtype}")
    if a.ndim != 2:
        raise ValueError("expected a 2-D (rows, H) array")
    if a.strides[1] != a.itemsize or a.strides[0] % a.itemsize or a.strides[0] < a.shape[1] * a.itemsize:
        a = np.ascontiguousarray(a)
    return a, (a.strides[0] // a.itemsize if a.shape[0] > 1 else a.shape[1])


def _vec(a, dtype):
    a = np.ascontiguousarray(np.asarray(a))
    if a.dtype != np.dtype(_NP[dtype]):
        raise TypeError(f"expected {_NP[dtype]} storage for {dtype}, got {a.dtype}")
    return a


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, lib_path: str = _LIB):
        lib = ctypes.CDLL(lib_path)
        vp, i64, i32, dp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.orc_decode.argtypes = [vp, i32, i64, vp]
        lib.orc_encode.argtypes = [vp, i64, i32, vp]
        lib.orc_fwd.argtypes = [vp, i64, vp, i32, i32, i64, i64, dp, vp, vp]
        lib.orc_fwd_residual.argtypes = [vp, i64, vp, i64, vp, i32, i32, i64, i64, dp, vp, vp, vp]
        lib.orc_bwd.argtypes = [vp, i64, vp, i64, vp, vp, i32, i32, i64, i64, vp, vp, vp]
        lib.orc_adaln_fwd.argtypes = [vp, i64, vp, vp, vp, i64, i64, i32, i32, i32, i64, i64, dp, vp, vp]
        lib.orc_bwd_residual.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, i32, i32, i64, i64, vp, vp, vp]
        lib.orc_rope.argtypes = [vp, i64, i64, vp, vp, i64, i32, i32, i64, i64, i64, i64, i32, vp]
        lib.orc_layernorm.argtypes = [vp, i64, vp, i64, vp, vp, i32, i32, i64, i64, dp, vp, vp, vp, vp]
        for f in (lib.orc_decode, lib.orc_encode, lib.orc_fwd, lib.orc_fwd_residual, lib.orc_bwd,
                  lib.orc_adaln_fwd, lib.orc_bwd_residual, lib.orc_rope, lib.orc_layernorm):
            f.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def decode(self, bits, dtype: str) -> np.ndarray:
        a = np.ascontiguousarray(np.asarray(bits, dtype=_NP[dtype]))
        out = np.empty(a.shape, dtype=np.float64)
        if self.lib.orc_decode(_ptr(a), CODES[dtype], a.size, _ptr(out)) != 0:
            raise ValueError("orc_decode rejected its arguments")
        return out

    def encode(self, values, dtype: str) -> np.ndarray:
        """Round-to-nearest-even of float64 values into the storage format."""
        v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
        out = np.empty(v.shape, dtype=_NP[dtype])
        if self.lib.orc_encode(_ptr(v), v.size, CODES[dtype], _ptr(out)) != 0:
            raise ValueError("orc_encode rejected its arguments")
        return out

    def fwd(self, x, w, eps: float, dtype: str, wdtype: str | None = None):
        """-> (y float64 (M, H), rrms float64 (M,)).  w=None means weightless."""
        x, xs = _rows(x, dtype)
        M, H = x.shape
        wv = None if w is None else _vec(w, wdtype or dtype)
        y = np.empty((M, H), dtype=np.float64)
        r = np.empty(M, dtype=np.float64)
        rc = self.lib.orc_fwd(_ptr(x), xs, _ptr(wv), CODES[dtype], CODES[wdtype or dtype],
                              M, H, float(eps), _ptr(y), _ptr(r))
        if rc != 0:
            raise ValueError("orc_fwd rejected its arguments")
        return y, r

    def fwd_residual(self, x, res, w, eps: float, dtype: str, wdtype: str | None = None):
        """-> (y float64, h float64 = x + res unrounded, rrms float64)."""
        x, xs = _rows(x, dtype)
        res, rs = _rows(res, dtype)
        if x.shape != res.shape:
            raise ValueError("x and residual shapes differ")
        M, H = x.shape
        wv = None if w is None else _vec(w, wdtype or dtype)
        y = np.empty((M, H), dtype=np.float64)
        h = np.empty((M, H), dtype=np.float64)
        r = np.empty(M, dtype=np.float64)
        rc = self.lib.orc_fwd_residual(_ptr(x), xs, _ptr(res), rs, _ptr(wv), CODES[dtype],
                                       CODES[wdtype or dtype], M, H, float(eps),
                                       _ptr(y), _ptr(h), _ptr(r))
        if rc != 0:
            raise ValueError("orc_fwd_residual rejected its arguments")
        return y, h, r

    def bwd(self, dy, x, w, rrms, dtype: str, wdtype: str | None = None, want_dw: bool = True):
        """-> (dx float64 (M, H), dw float64 (H,) or None, dx_terms float64 (M, H)).

        rrms is the saved per-row statistic (any float array, converted exactly
        to float64).  dx_terms holds |rrms*g| + |xn*rrms*c/H| per element."""
        x, xs = _rows(x, dtype)
        dy, dys = _rows(dy, dtype)
        if x.shape != dy.shape:
            raise ValueError("x and dy shapes differ")
        M, H = x.shape
        wv = None if w is None else _vec(w, wdtype or dtype)
        r = np.ascontiguousarray(np.asarray(rrms).astype(np.float64))
        if r.shape != (M,):
            raise ValueError("rrms must have shape (M,)")
        dx = np.empty((M, H), dtype=np.float64)
        terms = np.empty((M, H), dtype=np.float64)
        dw = np.empty(H, dtype=np.float64) if (want_dw and w is not None) else None
        rc = self.lib.orc_bwd(_ptr(dy), dys, _ptr(x), xs, _ptr(wv), _ptr(r), CODES[dtype],
                              CODES[wdtype or dtype], M, H, _ptr(dx), _ptr(dw), _ptr(terms))
        if rc != 0:
            raise ValueError("orc_bwd rejected its arguments")
        return dx, dw, terms


    def adaln_fwd(self, x, w, scale, shift, rows_per_cond: int, eps: float, dtype: str,
                  wdtype: str | None = None, cdtype: str | None = None):
        """-> (y float64 (M, H), rrms float64 (M,)).  scale and shift are
        (ceil(M / rows_per_cond), H); row i uses conditioning row i // rows_per_cond."""
        x, xs = _rows(x, dtype)
        sc, css = _rows(scale, cdtype or dtype)
        sh, chs = _rows(shift, cdtype or dtype)
        M, H = x.shape
        if sc.shape != sh.shape or sc.shape[1] != H or sc.shape[0] * rows_per_cond < M:
            raise ValueError("scale/shift must be (ceil(M / rows_per_cond), H)")
        if css != chs:
            sc, sh = np.ascontiguousarray(sc), np.ascontiguousarray(sh)
            css = H
        wv = None if w is None else _vec(w, wdtype or dtype)
        y = np.empty((M, H), dtype=np.float64)
        r = np.empty(M, dtype=np.float64)
        rc = self.lib.orc_adaln_fwd(_ptr(x), xs, _ptr(wv), _ptr(sc), _ptr(sh), css, int(rows_per_cond),
                                    CODES[dtype], CODES[wdtype or dtype], CODES[cdtype or dtype], M, H, float(eps),
                                    _ptr(y), _ptr(r))
        if rc != 0:
            raise ValueError("orc_adaln_fwd rejected its arguments")
        return y, r


    def bwd_residual(self, dy, h, dres, w, rrms, dtype: str, wdtype: str | None = None, want_dw: bool = True):
        """-> (dh float64 (M, H), dw or None, dh_terms): gradient reaching both
        inputs of the fused residual add; dres (gradient on residual_out) may be
        None.  dh_terms adds |dres| to the norm's two terms."""
        h, hs = _rows(h, dtype)
        dy, dys = _rows(dy, dtype)
        M, H = h.shape
        if dres is not None:
            dres, drs = _rows(dres, dtype)
            if dres.shape != h.shape:
                raise ValueError("dres shape differs")
        else:
            drs = H
        wv = None if w is None else _vec(w, wdtype or dtype)
        r = np.ascontiguousarray(np.asarray(rrms).astype(np.float64))
        dh = np.empty((M, H), dtype=np.float64)
        terms = np.empty((M, H), dtype=np.float64)
        dw = np.empty(H, dtype=np.float64) if (want_dw and w is not None) else None
        rc = self.lib.orc_bwd_residual(_ptr(dy), dys, _ptr(h), hs, _ptr(dres), drs, _ptr(wv), _ptr(r),
                                       CODES[dtype], CODES[wdtype or dtype], M, H, _ptr(dh), _ptr(dw), _ptr(terms))
        if rc != 0:
            raise ValueError("orc_bwd_residual rejected its arguments")
        return dh, dw, terms


    def rope(self, x, cos, sin, dtype: str, tdtype: str | None = None, transpose: bool = False):
        """Rotate-half RoPE of x (batch, seq_len, heads, head_dim) with
        (seq_len, >= head_dim/2) cos and sin tables -> float64 array of x's
        shape.  x may be any view whose last axis is contiguous and whose
        (heads, head_dim) block of a token row has one head stride."""
        x = np.asarray(x)
        if x.dtype != np.dtype(_NP[dtype]):
            raise TypeError(f"expected {_NP[dtype]} storage for {dtype}, got {x.dtype}")
        if x.ndim != 4:
            raise ValueError("x must be (batch, seq_len, heads, head_dim)")
        B, S, NH, D = x.shape
        it = x.itemsize
        if (x.strides[3] != it or x.strides[2] % it or x.strides[1] % it or x.strides[0] != S * x.strides[1]
                or x.strides[2] < D * it or x.strides[1] < NH * x.strides[2]):
            x = np.ascontiguousarray(x)
        hs, rs = x.strides[2] // it, x.strides[1] // it
        td = tdtype or dtype
        cos, sin = np.asarray(cos), np.asarray(sin)
        for t in (cos, sin):
            if t.dtype != np.dtype(_NP[td]):
                raise TypeError(f"expected {_NP[td]} table storage for {td}, got {t.dtype}")
        if cos.shape != sin.shape or cos.ndim != 2 or cos.shape[0] != S:
            raise ValueError("cos and sin must both be (seq_len, >= head_dim/2)")
        cos, sin = np.ascontiguousarray(cos), np.ascontiguousarray(sin)
        out = np.empty((B, S, NH, D), dtype=np.float64)
        rc = self.lib.orc_rope(_ptr(x), rs, hs, _ptr(cos), _ptr(sin), cos.shape[1], CODES[dtype], CODES[td], B, S,
                               NH, D, 1 if transpose else 0, _ptr(out))
        if rc != 0:
            raise ValueError("orc_rope rejected its arguments")
        return out


    def layernorm(self, x, residual, w, b, eps, dtype: str, wdtype: str | None = None):
        """Residual + LayerNorm: -> (y, h, mean, rstd), float64.  residual, w
        and b may each be None.  h is the exact sum x + residual (x when there
        is no residual)."""
        x, xs = _rows(x, dtype)
        M, H = x.shape
        rs = H
        if residual is not None:
            residual, rs = _rows(residual, dtype)
            if residual.shape != x.shape:
                raise ValueError("residual shape differs")
        wd = wdtype or dtype
        wv = None if w is None else _vec(w, wd)
        bv = None if b is None else _vec(b, wd)
        y = np.empty((M, H), dtype=np.float64)
        h = np.empty((M, H), dtype=np.float64)
        mean = np.empty(M, dtype=np.float64)
        rstd = np.empty(M, dtype=np.float64)
        rc = self.lib.orc_layernorm(_ptr(x), xs, _ptr(residual), rs, _ptr(wv), _ptr(bv), CODES[dtype], CODES[wd], M,
                                    H, float(eps), _ptr(y), _ptr(h), _ptr(mean), _ptr(rstd))
        if rc != 0:
            raise ValueError("orc_layernorm rejected its arguments")
        return y, h, mean, rstd


def default() -> Oracle:
    """The oracle built from rmsnorm_oracle.c (rebuilt when the source is newer)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            _default = Oracle(_LIB)
    return _default


def decode(bits, dtype):
    return default().decode(bits, dtype)


def encode(values, dtype):
    return default().encode(values, dtype)


def fwd(x, w, eps, dtype, wdtype=None):
    return default().fwd(x, w, eps, dtype, wdtype)


def fwd_residual(x, res, w, eps, dtype, wdtype=None):
    return default().fwd_residual(x, res, w, eps, dtype, wdtype)


def bwd(dy, x, w, rrms, dtype, wdtype=None, want_dw=True):
    return default().bwd(dy, x, w, rrms, dtype, wdtype, want_dw)


def adaln_fwd(x, w, scale, shift, rows_per_cond, eps, dtype, wdtype=None, cdtype=None):
    return default().adaln_fwd(x, w, scale, shift, rows_per_cond, eps, dtype, wdtype, cdtype)


def bwd_residual(dy, h, dres, w, rrms, dtype, wdtype=None, want_dw=True):
    return default().bwd_residual(dy, h, dres, w, rrms, dtype, wdtype, want_dw)


def rope(x, cos, sin, dtype, tdtype=None, transpose=False):
    return default().rope(x, cos, sin, dtype, tdtype, transpose)


def layernorm(x, residual, w, b, eps, dtype, wdtype=None):
    return default().layernorm(x, residual, w, b, eps, dtype, wdtype)
