"""Seeded synthetic inputs shared by the oracle-side tests and the GPU-side tests.

This module draws numbers and encodes them into storage formats. It holds none
of the methods' arithmetic: no squares, no means, no reciprocal roots, no
rotation.  RoPE's cos/sin tables are inputs to the rotation (a position
embedding prepares them); here they are the cosines and sines of uniformly
drawn angles.

Generator (a reading: the pages name no seeds and no generator), in _gen.c:
  * SplitMix64 in counter form.  The stream for (seed, stream id) starts from
    key = mix64(seed * GOLDEN + stream + 1); its i-th output is
    mix64(key + (i + 1) * GOLDEN), where mix64 is Steele, Lea and Flood's
    SplitMix64 finaliser (OOPSLA 2014) and GOLDEN = 0x9E3779B97F4A7C15.
  * Uniforms use the top 53 bits: u = (bits >> 11) * 2**-53 in [0, 1).
  * Normals use Box-Muller in float64 on outputs (2k, 2k+1) of the stream:
    rad = sqrt(-2 ln(1 - u0)), theta = 2 pi u1; element 2k takes rad*cos(theta),
    element 2k+1 takes rad*sin(theta).
  * A float64 draw is stored with one round-to-nearest-even into the target
    format.  bfloat16 goes through float32 first; that double rounding is
    harmless because float32 keeps 24 >= 2*8 + 2 significand bits.

Stream ids: x = 0, weight = 1, residual = 2, upstream gradient = 3,
outlier mask = 4, outlier value = 5, AdaLN scale = 6, AdaLN shift = 7,
RoPE angle = 8, LayerNorm bias = 9.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

STREAM_X = 0
STREAM_W = 1
STREAM_RESIDUAL = 2
STREAM_DY = 3
STREAM_OUTLIER_MASK = 4
STREAM_OUTLIER_VALUE = 5
STREAM_SCALE = 6
STREAM_SHIFT = 7
STREAM_ANGLE = 8
STREAM_BIAS = 9

# Storage formats, by name.  "bf16" arrays are returned as uint16 bit patterns.
DTYPES = ("f32", "f16", "bf16")

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "_gen.c")
_LIB = os.path.join(_HERE, "_libgen.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the generator (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = f"{_LIB}.{os.getpid()}.tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                        "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _gen():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            u64, i32, i64, dp, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
            lib.syn_uniform.argtypes = [u64, i32, i64, i64, vp]
            lib.syn_normal.argtypes = [u64, i32, i64, i64, dp, dp, vp]
            lib.syn_outliers.argtypes = [u64, i32, i32, i64, i64, dp, dp, dp, vp]
            _lib = lib
    return _lib


def uniform(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """n float64 uniforms in [0, 1): positions start .. start+n-1 of the stream."""
    out = np.empty(n, dtype=np.float64)
    _gen().syn_uniform(seed, stream, start, n, out.ctypes.data)
    return out


def normal(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0, start: int = 0) -> np.ndarray:
    """n float64 draws from N(mean, std**2) (std is the standard deviation)."""
    out = np.empty(n, dtype=np.float64)
    _gen().syn_normal(seed, stream, start, n, float(mean), float(std), out.ctypes.data)
    return out


def encode(values: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage format (round to nearest even).

    f32 -> float32 array, f16 -> float16 array, bf16 -> uint16 bit patterns.
    """
    v = np.asarray(values, dtype=np.float64)
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "f16":
        return v.astype(np.float16)
    if dtype == "bf16":
        f = v.astype(np.float32)
        u = f.view(np.uint32)
        nan = np.isnan(f)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        with np.errstate(over="ignore"):
            r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
        if nan.any():
            r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
        return r
    raise ValueError(f"unknown dtype {dtype!r}")


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored elements."""
    if dtype in ("f32", "f16"):
        return np.asarray(bits).astype(np.float64)
    if dtype == "bf16":
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def element_size(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def normal_tensor(seed: int, stream: int, shape, dtype: str, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return encode(normal(seed, stream, n, mean, std), dtype).reshape(shape)


def rope_tables(seed: int, seq_len: int, head_dim: int, dtype: str):
    """(cos, sin) tables [seq_len, head_dim] of angles drawn uniformly in
    [0, 2 pi), one per (position, pair), repeated in both halves of a row as
    in the rotate-half layout; each value rounded once to dtype."""
    half = head_dim // 2
    ang = 2.0 * np.pi * uniform(seed, STREAM_ANGLE, seq_len * half).reshape(seq_len, half)
    ang = np.concatenate([ang, ang], axis=1)
    return encode(np.cos(ang), dtype), encode(np.sin(ang), dtype)


def with_outliers(seed: int, shape, dtype: str, mean: float, std: float,
                  frac: float, lo: float, hi: float) -> np.ndarray:
    """N(mean, std) draws where each element independently (probability frac)
    is replaced by sign * U(lo, hi), the sign +1 or -1 with equal odds."""
    n = int(np.prod(shape))
    v = normal(seed, STREAM_X, n, mean, std)
    _gen().syn_outliers(seed, STREAM_OUTLIER_MASK, STREAM_OUTLIER_VALUE, 0, n, float(frac), float(lo), float(hi),
                        v.ctypes.data)
    return encode(v, dtype).reshape(shape)


# ---------------------------------------------------------------------------
# Named workloads.  Shapes, distributions and eps follow the five RMSNorm
# workloads this library is measured on; seeds are fixed per workload.
# ---------------------------------------------------------------------------

WORKLOADS = {
    "fwd_f32_64x512": dict(kind="fwd", M=64, H=512, dtype="f32", wdtype="f32",
                           x=(0.0, 1.0), w=(1.0, 0.1), eps=1e-6, seed=1001),
    "fwd_bf16_8192x4096": dict(kind="fwd", M=8192, H=4096, dtype="bf16", wdtype="bf16",
                               x=(0.0, 1.0), w=(1.0, 0.1), eps=1e-5, seed=1002),
    "fwd_bf16_32768x2048": dict(kind="fwd", M=32768, H=2048, dtype="bf16", wdtype="bf16",
                                x=(0.0, 2.0), w=(1.0, 0.1), eps=1e-6, seed=1003),
    "fwd_f16_32768x2048_outliers": dict(kind="fwd", M=32768, H=2048, dtype="f16", wdtype="f16",
                                        x=(0.0, 2.0), w=(1.0, 0.1), eps=1e-6, seed=1013,
                                        outliers=(0.01, 200.0, 300.0)),
    # a ragged row length: rows of 8194 bytes leave the 16-byte grid
    "fwd_bf16_8192x4097": dict(kind="fwd", M=8192, H=4097, dtype="bf16", wdtype="bf16",
                               x=(0.0, 1.0), w=(1.0, 0.1), eps=1e-5, seed=1014),
    "fwd_residual_bf16_16384x8192": dict(kind="fwd_residual", M=16384, H=8192, dtype="bf16", wdtype="bf16",
                                         x=(0.0, 1.0), r=(0.0, 1.0), w=(1.0, 0.1), eps=1e-5, seed=1004),
    "bwd_bf16_8192x6144": dict(kind="bwd", M=8192, H=6144, dtype="bf16", wdtype="bf16",
                               x=(0.0, 1.0), w=(1.0, 0.1), dy=(0.0, 1.0), eps=1e-6, seed=1005),
    # the backward on the ragged row length above (rows off the 16-byte grid)
    "bwd_bf16_8192x4097": dict(kind="bwd", M=8192, H=4097, dtype="bf16", wdtype="bf16",
                               x=(0.0, 1.0), w=(1.0, 0.1), dy=(0.0, 1.0), eps=1e-6, seed=1015),
    # backward of the residual pre-norm above: h is the stored post-add
    # stream (x + r of two N(0, 1) draws has std sqrt(2)); dres is the
    # gradient arriving on it, drawn from the residual stream
    "bwd_residual_bf16_16384x8192": dict(kind="bwd_residual", M=16384, H=8192, dtype="bf16", wdtype="bf16",
                                         x=(0.0, 2.0 ** 0.5), w=(1.0, 0.1), dy=(0.0, 1.0), dres=(0.0, 1.0),
                                         eps=1e-5, seed=1008),
    # RoPE apply on video tokens: 2 clips of 21 x 16 x 24 latent patches
    # (8064 positions), 32 heads of 64 (hidden 2048), float32 tables
    "rope_bf16_2x8064x32x64": dict(kind="rope", B=2, S=8064, NH=32, D=64, dtype="bf16", tdtype="f32",
                                   x=(0.0, 1.0), seed=1009),
    # head_dim 128 (32 heads of a 4096-wide model), tables in bfloat16
    "rope_bf16_2x4096x32x128": dict(kind="rope", B=2, S=4096, NH=32, D=128, dtype="bf16", tdtype="bf16",
                                    x=(0.0, 1.0), seed=1010),
    # residual + LayerNorm of a pre-LayerNorm transformer in float32 at
    # d_model 1024 (the width of the largest published rows), 16384 tokens
    "ln_residual_f32_16384x1024": dict(kind="ln_residual", M=16384, H=1024, dtype="f32", wdtype="f32",
                                       x=(0.0, 1.0), r=(0.0, 1.0), w=(1.0, 0.1), b=(0.0, 0.1), eps=1e-5,
                                       seed=1011),
    # DiT-style AdaLN on 2 x 4096 tokens of width 2048 (LTX-Video's hidden
    # size); scale/shift per batch ([B, 1, H]) and per token ([B, S, H])
    "adaln_bf16_2x4096x2048_batchcond": dict(kind="adaln", M=8192, H=2048, dtype="bf16", wdtype="bf16",
                                             x=(0.0, 1.0), w=(1.0, 0.1), cond=(0.0, 0.5), rows_per_cond=4096,
                                             eps=1e-6, seed=1006),
    "adaln_bf16_2x4096x2048_tokencond": dict(kind="adaln", M=8192, H=2048, dtype="bf16", wdtype="bf16",
                                             x=(0.0, 1.0), w=(1.0, 0.1), cond=(0.0, 0.5), rows_per_cond=1,
                                             eps=1e-6, seed=1007),
}


def make_inputs(name: str, rows: int | None = None) -> dict:
    """Host arrays for a named workload.  rows, if given, keeps the first rows
    rows of every (M, H) tensor (the draws of those rows are unchanged)."""
    spec = dict(WORKLOADS[name])
    if spec["kind"] == "rope":
        return _rope_inputs(spec, rows)
    M, H, dt, wdt, seed = spec["M"], spec["H"], spec["dtype"], spec["wdtype"], spec["seed"]
    m = M if rows is None else min(rows, M)
    out = dict(spec)
    out["M"] = m
    n = m * H
    if "outliers" in spec:
        # every draw is keyed by its position, so the first m rows equal the
        # first m rows of the full tensor
        out["x"] = with_outliers(seed, (m, H), dt, *spec["x"], *spec["outliers"])
    else:
        out["x"] = encode(normal(seed, STREAM_X, n, *spec["x"]), dt).reshape(m, H)
    out["w"] = encode(normal(seed, STREAM_W, H, *spec["w"]), wdt)
    if "r" in spec:
        out["r"] = encode(normal(seed, STREAM_RESIDUAL, n, *spec["r"]), dt).reshape(m, H)
    if "b" in spec:
        out["b"] = encode(normal(seed, STREAM_BIAS, H, *spec["b"]), wdt)
    if "dres" in spec:
        out["dres"] = encode(normal(seed, STREAM_RESIDUAL, n, *spec["dres"]), dt).reshape(m, H)
    if "dy" in spec:
        out["dy"] = encode(normal(seed, STREAM_DY, n, *spec["dy"]), dt).reshape(m, H)
    if "cond" in spec:
        rpc = spec["rows_per_cond"]
        C = (M + rpc - 1) // rpc if rows is None else (m + rpc - 1) // rpc
        out["scale"] = encode(normal(seed, STREAM_SCALE, C * H, *spec["cond"]), wdt).reshape(C, H)
        out["shift"] = encode(normal(seed, STREAM_SHIFT, C * H, *spec["cond"]), wdt).reshape(C, H)
    return out



def _rope_inputs(spec: dict, positions: int | None) -> dict:
    """x [B, S, NH, D] and its tables; positions, if given, keeps the first
    positions of every batch (their draws are unchanged)."""
    B, S, NH, D, seed = spec["B"], spec["S"], spec["NH"], spec["D"], spec["seed"]
    m = S if positions is None else min(positions, S)
    out = dict(spec)
    out["S"] = m
    per = NH * D
    x = np.empty((B, m, NH, D), dtype=np.dtype({"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[spec["dtype"]]))
    for b in range(B):
        v = normal(seed, STREAM_X, m * per, *spec["x"], start=b * S * per)
        x[b] = encode(v, spec["dtype"]).reshape(m, NH, D)
    out["x"] = x
    cos, sin = rope_tables(seed, S, D, spec["tdtype"])
    out["cos"], out["sin"] = cos[:m], sin[:m]
    return out
