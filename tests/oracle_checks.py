"""Checks that pin the float64 oracle to facts other than its own code.

Each check takes an oracle.Oracle and raises AssertionError when a fact fails.
The facts come from the definition of RMSNorm on the page "Skill: Write a
Triton RMSNorm Kernel" (ahel.ai; "Purpose", "Required reasoning process"
steps 5-12, "Correctness requirements") and from mathematics:

  * exact cases worked out with rational arithmetic (Fraction), where
    mean(x^2) + eps is the square of a dyadic rational;
  * closed forms (constant rows, zero rows, H = 1);
  * invariants (weightless mean square, column-indexed weight, scaling,
    permutation, strided rows, x/residual symmetry);
  * central finite differences of L = sum(dy * y) for the backward pass, and
    identities that follow from differentiating the forward definition;
  * library routines for the storage formats (numpy float16/float32, torch
    bfloat16) and Python's decimal module for high-precision brute force.

test_oracle_pins.py runs every check on the oracle; test_oracle_mutants.py
runs them on copies of the oracle with planted mistakes and requires each copy
to fail at least one check.
"""

from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

RNG_SEED = 12345


def _rng(k=0):
    return np.random.default_rng(RNG_SEED + k)


def _bf16_bits_from_f32(f32):
    """bfloat16 bits via torch's float32 -> bfloat16 conversion (a library routine)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_values(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def _storage(values, dtype):
    """Store float64 values that are already exact in the format."""
    v = np.asarray(values, dtype=np.float64)
    if dtype == "f32":
        out = v.astype(np.float32)
    elif dtype == "f16":
        out = v.astype(np.float16)
    elif dtype == "bf16":
        out = _bf16_bits_from_f32(v.astype(np.float32))
    elif dtype == "f64":
        out = v.copy()
    else:
        raise ValueError(dtype)
    back = v if dtype == "f64" else (_bf16_values(out) if dtype == "bf16" else out.astype(np.float64))
    assert np.array_equal(back, v), "test input not exact in its format"
    return out


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def check_decode_all_16bit_patterns(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got16 = o.decode(bits.view(np.float16), "f16")
    ref16 = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref16)
    assert np.array_equal(np.isnan(got16), nan)
    assert np.array_equal(got16[~nan], ref16[~nan])
    assert np.array_equal(np.signbit(got16[~nan]), np.signbit(ref16[~nan]))
    gotb = o.decode(bits, "bf16")
    refb = _bf16_values(bits)
    nan = np.isnan(refb)
    assert np.array_equal(np.isnan(gotb), nan)
    assert np.array_equal(gotb[~nan], refb[~nan])
    assert np.array_equal(np.signbit(gotb[~nan]), np.signbit(refb[~nan]))


def _encode_probe_values():
    rng = _rng(1)
    parts = [
        rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000)),
        rng.standard_normal(5000) * 1e-6,                 # fp16 subnormal range
        rng.standard_normal(5000) * 1e-39,                # fp32/bf16 subnormal range
        rng.uniform(65000, 66000, 2000) * rng.choice([-1, 1], 2000),   # fp16 overflow edge
        np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 3.4e38, 3.5e38]),
    ]
    # exact midpoints between neighbouring representable values (ties)
    for p in (11, 8, 24):
        m = rng.integers(1 << (p - 1), 1 << p, 2000).astype(np.float64)
        e = rng.integers(-10, 10, 2000)
        parts.append((m + 0.5) * np.exp2(e - (p - 1)))
    return np.concatenate(parts)


def check_encode_matches_libraries(o):
    v = _encode_probe_values()
    # float16: numpy rounds float64 -> float16 directly, to nearest even
    got = o.encode(v, "f16")
    ref = v.astype(np.float16)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    # float32: the C/numpy float64 -> float32 conversion
    got = o.encode(v, "f32")
    ref = v.astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # bfloat16: torch float32 -> bfloat16 after numpy float64 -> float32; the
    # two roundings equal one because float32 keeps >= 2*8+2 significand bits
    got = o.encode(v, "bf16")
    ref = _bf16_bits_from_f32(v.astype(np.float32))
    assert np.array_equal(got, ref)


def check_encode_ties_by_hand(o):
    # 1 + 2^-8 lies half way between bf16 neighbours 1 and 1 + 2^-7: ties go to
    # the even significand (1.0); 1 + 3*2^-8 goes up to 1 + 2^-6.
    got = o.encode(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]), "bf16")
    assert list(got) == [0x3F80, 0x3F82, 0xBF80]
    # fp16: 1 + 2^-11 ties to 1.0 (0x3C00), 1 + 3*2^-11 to 1 + 2^-9 (0x3C02);
    # 2^-25 ties to 0, 3*2^-25 rounds to 2*2^-24 (0x0002)
    got = o.encode(np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -25]), "f16")
    assert list(got.view(np.uint16)) == [0x3C00, 0x3C02, 0x0000, 0x0002]


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

# rows whose mean square plus eps is a perfect square of a dyadic rational
_EXACT_FWD = [
    # (row, eps, expected rrms)
    ([6, 8], 14, Fraction(1, 8)),                 # ms = 50, 50 + 14 = 64
    ([2, 0, 0, 0], 3, Fraction(1, 2)),            # ms = 1
    ([3, -3, 3, -3], 7, Fraction(1, 4)),          # ms = 9
    ([1, 2, 2], 1, Fraction(1, 2)),               # ms = 3
    ([0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5], 0.75, Fraction(1, 1)),  # ms = 1/4
]


def check_exact_rational_rows(o):
    for row, eps, rr in _EXACT_FWD:
        H = len(row)
        ms = sum(Fraction(v) ** 2 for v in row) / H
        assert (ms + Fraction(eps)) * rr * rr == 1  # the case really is exact
        w = [1.5, -2.0, 0.25, 4.0, 1.0, 0.5, 2.0, -1.0][:H]
        for dt in ("f32", "f16", "bf16"):
            x = _storage(np.array([row], dtype=np.float64), dt)
            wv = _storage(np.array(w), dt)
            y, r = o.fwd(x, wv, eps, dt)
            assert r[0] == float(rr), (row, dt, r[0])
            exp = np.array([float(Fraction(v) * rr * Fraction(wj)) for v, wj in zip(row, w)])
            assert np.array_equal(y[0], exp), (row, dt, y[0], exp)
            y0, _ = o.fwd(x, None, eps, dt)
            exp0 = np.array([float(Fraction(v) * rr) for v in row])
            assert np.array_equal(y0[0], exp0)


def check_constant_and_zero_rows(o):
    rng = _rng(2)
    for H in (1, 3, 64, 257, 4096):
        for eps in (1e-6, 1e-5, 0.5):
            c = float(np.float32(rng.uniform(-4, 4)))
            x = np.full((2, H), c, dtype=np.float32)
            x[1] = 0.0
            w = rng.uniform(0.5, 1.5, H).astype(np.float32)
            y, r = o.fwd(x, w, eps, "f32")
            r_exp = 1.0 / np.sqrt(c * c + eps)
            # a float64 sum of H terms is within (H-1) units of 2^-53 of exact
            tol = 4 * H * 2.0 ** -53 + 1e-15
            assert abs(r[0] - r_exp) <= tol * r_exp
            assert np.allclose(y[0], c * r_exp * w.astype(np.float64), rtol=tol, atol=0)
            assert abs(r[1] - eps ** -0.5) <= 1e-15 * eps ** -0.5
            assert np.all(y[1] == 0.0)


def check_h1_closed_form(o):
    # H = 1: y = x / sqrt(x^2 + eps) * w, so y^2 + eps * rrms^2 = w^2 and
    # sign(y) = sign(x * w), over every finite bfloat16 value below 2^63
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = _bf16_values(bits)
    keep = np.isfinite(vals) & (np.abs(vals) < 2.0 ** 63)
    x = bits[keep].reshape(-1, 1)
    eps = 1e-6
    y, r = o.fwd(x, None, eps, "bf16")
    xv = vals[keep]
    assert np.allclose(y[:, 0] ** 2 + eps * r ** 2, 1.0, rtol=0, atol=1e-14)
    nz = xv != 0
    assert np.array_equal(np.sign(y[nz, 0]), np.sign(xv[nz]))
    assert np.all(y[~nz, 0] == 0)


def check_weightless_mean_square(o):
    # mean_j(y_ij^2) = ms/(ms+eps), i.e. mean(y^2) + eps*rrms^2 = 1 per row
    rng = _rng(3)
    for dt in ("f32", "f16", "bf16"):
        for H in (1, 7, 512, 2049):
            xv = rng.standard_normal((5, H)) * np.array([[1e-3], [1.0], [30.0], [0.01], [2.0]])
            x = _storage(_round_like(xv, dt), dt)
            for eps in (1e-6, 1e-2):
                y, r = o.fwd(x, None, eps, dt)
                lhs = (y ** 2).mean(axis=1) + eps * r ** 2
                assert np.allclose(lhs, 1.0, rtol=0, atol=1e-13), (dt, H, lhs)


def _round_like(v, dt):
    if dt == "f32":
        return v.astype(np.float32).astype(np.float64)
    if dt == "f16":
        return v.astype(np.float16).astype(np.float64)
    if dt == "bf16":
        return _bf16_values(_bf16_bits_from_f32(v.astype(np.float32)))
    return v


def check_weight_indexed_by_column(o):
    # y(w)_ij = y(None)_ij * w_j for every row: the weight broadcasts over rows
    rng = _rng(4)
    for dt in ("f32", "bf16"):
        H = 33
        x = _storage(_round_like(rng.standard_normal((6, H)), dt), dt)
        w = _storage(_round_like(rng.uniform(0.5, 2.0, H) * rng.choice([-1, 1], H), dt), dt)
        y, _ = o.fwd(x, w, 1e-5, dt)
        y0, _ = o.fwd(x, None, 1e-5, dt)
        wd = w.astype(np.float64) if dt != "bf16" else _bf16_values(w)
        assert np.allclose(y, y0 * wd[None, :], rtol=1e-15, atol=0)
    # fp32 weight with 16-bit x gives the same numbers as the same weight values
    x = _storage(_round_like(rng.standard_normal((3, 16)), "bf16"), "bf16")
    w16 = _storage(_round_like(rng.uniform(0.5, 2, 16), "bf16"), "bf16")
    w32 = _bf16_values(w16).astype(np.float32)
    a, _ = o.fwd(x, w16, 1e-5, "bf16", "bf16")
    b, _ = o.fwd(x, w32, 1e-5, "bf16", "f32")
    assert np.array_equal(a, b)


def check_scale_law(o):
    # y(2^k x) / y(x) = sqrt((ms + eps) / (ms + eps * 4^-k)) with ms = ms(x)
    rng = _rng(5)
    H = 300
    xv = rng.standard_normal((4, H))
    x = xv.copy()
    eps = 1e-3
    _, r1 = o.fwd(x, None, eps, "f64")
    ms = (xv ** 2).mean(axis=1)
    for k in (-3, 1, 5):
        y2, _ = o.fwd(x * 2.0 ** k, None, eps, "f64")
        y1, _ = o.fwd(x, None, eps, "f64")
        ratio = np.sqrt((ms + eps) / (ms + eps * 4.0 ** (-k)))
        assert np.allclose(y2, y1 * ratio[:, None], rtol=1e-13, atol=0)


def check_permutation_and_strides(o):
    rng = _rng(6)
    H = 97
    xv = _round_like(rng.standard_normal((8, H)), "bf16")
    x = _storage(xv, "bf16")
    w = _storage(_round_like(rng.uniform(0.5, 1.5, H), "bf16"), "bf16")
    y, r = o.fwd(x, w, 1e-5, "bf16")
    perm = rng.permutation(H)
    yp, rp = o.fwd(np.ascontiguousarray(x[:, perm]), np.ascontiguousarray(w[perm]), 1e-5, "bf16")
    assert np.allclose(yp, y[:, perm], rtol=1e-15, atol=0)
    assert np.allclose(rp, r, rtol=1e-15, atol=0)
    # rows taken from a padded buffer (row stride > H) give the same numbers
    pad = np.zeros((8, H + 11), dtype=np.uint16)
    pad[:, :H] = x
    pad[:, H:] = 0x7F80  # +inf in the padding must never be read
    ys, rs = o.fwd(pad[:, :H], w, 1e-5, "bf16")
    assert np.array_equal(ys, y) and np.array_equal(rs, r)
    # each row alone equals the same row within the batch
    for i in (0, 5):
        y1, r1 = o.fwd(x[i:i + 1], w, 1e-5, "bf16")
        assert np.array_equal(y1[0], y[i]) and r1[0] == r[i]


def check_fp16_large_values(o):
    # 256^2 = 65536 is above the largest float16 (65504); the definition
    # squares exactly, so a row of +-256 is a constant-magnitude row
    x = np.array([[256.0, -256.0, 256.0, -256.0], [300.0, 0, 0, 0]], dtype=np.float16)
    y, r = o.fwd(x, None, 1e-6, "f16")
    assert np.all(np.isfinite(y))
    assert np.allclose(np.abs(y[0]), 256.0 / np.sqrt(65536.0 + 1e-6), rtol=1e-15)
    assert abs(y[1, 0] - 300.0 / np.sqrt(300.0 ** 2 / 4 + 1e-6)) < 1e-14


def check_decimal_bruteforce(o):
    getcontext().prec = 60
    rng = _rng(7)
    for dt in ("f32", "f16", "bf16"):
        for H in (1, 2, 3, 5):
            xv = _round_like(rng.standard_normal((3, H)) * rng.choice([1e-2, 1.0, 100.0], (3, 1)), dt)
            wv = _round_like(rng.uniform(0.5, 1.5, H), dt)
            eps = 1e-5
            y, r = o.fwd(_storage(xv, dt), _storage(wv, dt), eps, dt)
            for i in range(3):
                ss = sum(Decimal(float(v)) ** 2 for v in xv[i])
                rd = 1 / (ss / H + Decimal(eps)).sqrt()
                assert abs(Decimal(float(r[i])) - rd) <= rd * Decimal("1e-15")
                for j in range(H):
                    yd = Decimal(float(xv[i, j])) * rd * Decimal(float(wv[j]))
                    assert abs(Decimal(float(y[i, j])) - yd) <= abs(yd) * Decimal("1e-15") + Decimal("1e-300")


# ---------------------------------------------------------------------------
# fused residual
# ---------------------------------------------------------------------------

def check_residual_identities(o):
    import torch
    rng = _rng(8)
    for dt in ("bf16", "f16", "f32"):
        H = 130
        xv = _round_like(rng.standard_normal((6, H)), dt)
        rv = _round_like(rng.standard_normal((6, H)) * 3, dt)
        x, res = _storage(xv, dt), _storage(rv, dt)
        w = _storage(_round_like(rng.uniform(0.5, 1.5, H), dt), dt)
        y, h, r = o.fwd_residual(x, res, w, 1e-5, dt)
        # the sum is exact in float64 for these formats
        assert np.array_equal(h, xv + rv)
        # rounding the sum: torch adds in float32 and rounds to the format;
        # the float32 step is harmless (24 >= 2p+2 for p = 8 and 11)
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
        ref = (torch.from_numpy(xv.astype(np.float32)) + torch.from_numpy(rv.astype(np.float32))).to(tdt)
        enc = o.encode(h, dt)
        if dt == "bf16":
            assert np.array_equal(enc, ref.view(torch.int16).numpy().view(np.uint16))
        elif dt == "f16":
            assert np.array_equal(enc.view(np.uint16), ref.view(torch.int16).numpy().view(np.uint16))
        # y is the plain forward applied to the unrounded sum
        wd = _bf16_values(w) if dt == "bf16" else w.astype(np.float64)
        y2, r2 = o.fwd(h, wd, 1e-5, "f64")
        assert np.array_equal(y, y2) and np.array_equal(r, r2)
        # x and residual play symmetric roles
        ys, hs, rs = o.fwd_residual(res, x, w, 1e-5, dt)
        assert np.array_equal(ys, y) and np.array_equal(hs, h) and np.array_equal(rs, r)
        # a zero residual reduces to the plain forward
        yz, hz, rz = o.fwd_residual(x, _storage(np.zeros_like(xv), dt), w, 1e-5, dt)
        yp, rp = o.fwd(x, w, 1e-5, dt)
        assert np.array_equal(yz, yp) and np.array_equal(rz, rp) and np.array_equal(hz, xv)


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def check_bwd_exact_case(o):
    # x = [6, 8], eps = 14 -> rrms = 1/8 exactly; w = 1, dy = [1, 0].
    # Differentiating y_1 = x_1 * (ms + eps)^-1/2 with ms = (x_1^2 + x_2^2)/2:
    #   dy_1/dx_1 = r (1 - x_1^2 r^2 / 2) = 23/256,  dy_1/dx_2 = -x_1 x_2 r^3 / 2 = -3/64
    # and dw_j = dy_j * x_j * r = [3/4, 0].
    x = np.array([[6.0, 8.0]], dtype=np.float32)
    dy = np.array([[1.0, 0.0]], dtype=np.float32)
    w = np.array([1.0, 1.0], dtype=np.float32)
    _, r = o.fwd(x, w, 14.0, "f32")
    dx, dw, _ = o.bwd(dy, x, w, r, "f32")
    assert np.array_equal(dx[0], np.array([23 / 256, -3 / 64]))
    assert np.array_equal(dw, np.array([0.75, 0.0]))


def _loss(o, xv, wv, dyv, eps):
    y, _ = o.fwd(xv, wv, eps, "f64")
    return float((dyv * y).sum())


def check_bwd_finite_differences(o):
    rng = _rng(9)
    for (M, H) in ((1, 1), (2, 2), (3, 3), (2, 16), (4, 257)):
        eps = 1e-2
        xv = rng.standard_normal((M, H))
        wv = rng.uniform(0.5, 1.5, H)
        dyv = rng.standard_normal((M, H))
        _, r = o.fwd(xv, wv, eps, "f64")
        dx, dw, _ = o.bwd(dyv, xv, wv, r, "f64")
        hstep = 1e-5
        cols = range(H) if H <= 16 else rng.choice(H, 12, replace=False)
        fdx = np.zeros((M, H))
        for i in range(M):
            for j in cols:
                xp = xv.copy(); xp[i, j] += hstep
                xm = xv.copy(); xm[i, j] -= hstep
                fdx[i, j] = (_loss(o, xp, wv, dyv, eps) - _loss(o, xm, wv, dyv, eps)) / (2 * hstep)
        sel = np.zeros((M, H), dtype=bool)
        sel[:, list(cols)] = True
        scale = np.abs(dx).max()
        assert np.all(np.abs(fdx[sel] - dx[sel]) <= 1e-7 * scale + 1e-9), (M, H)
        for j in cols:
            wp = wv.copy(); wp[j] += hstep
            wm = wv.copy(); wm[j] -= hstep
            fdw = (_loss(o, xv, wp, dyv, eps) - _loss(o, xv, wm, dyv, eps)) / (2 * hstep)
            assert abs(fdw - dw[j]) <= 1e-7 * np.abs(dw).max() + 1e-9, (M, H, j)
        # weightless backward is the w = 1 backward
        _, r0 = o.fwd(xv, None, eps, "f64")
        dx0, dw0, _ = o.bwd(dyv, xv, None, r0, "f64")
        dx1, _, _ = o.bwd(dyv, xv, np.ones(H), r0, "f64")
        assert dw0 is None and np.array_equal(dx0, dx1)


def check_bwd_identities(o):
    # with c_i = sum_j dy_ij w_j x_ij r_i:
    #   sum_j x_ij dx_ij = c_i * eps / (ms_i + eps)   (dx is orthogonal to x as eps -> 0)
    #   sum_j w_j dw_j   = sum_i c_i
    rng = _rng(10)
    M, H = 7, 300
    eps = 1e-3
    xv = rng.standard_normal((M, H)) * rng.uniform(0.1, 3, (M, 1))
    wv = rng.uniform(0.5, 1.5, H)
    dyv = rng.standard_normal((M, H))
    _, r = o.fwd(xv, wv, eps, "f64")
    dx, dw, _ = o.bwd(dyv, xv, wv, r, "f64")
    ms = (xv ** 2).mean(axis=1)
    c = (dyv * wv[None, :] * xv * r[:, None]).sum(axis=1)
    assert np.allclose((xv * dx).sum(axis=1), c * eps / (ms + eps), rtol=1e-10, atol=1e-12)
    assert abs((wv * dw).sum() - c.sum()) <= 1e-11 * np.abs(c).sum()


def check_bwd_special_cases(o):
    rng = _rng(11)
    H, eps = 64, 1e-2
    # one row: dw is dy * xn elementwise
    xv = rng.standard_normal((1, H))
    wv = rng.uniform(0.5, 1.5, H)
    dyv = rng.standard_normal((1, H))
    _, r = o.fwd(xv, wv, eps, "f64")
    _, dw, _ = o.bwd(dyv, xv, wv, r, "f64")
    assert np.allclose(dw, dyv[0] * xv[0] * r[0], rtol=1e-15, atol=0)
    # weightless with dy = y: dx = x * r^2 * eps / (ms + eps)
    xv = rng.standard_normal((3, H))
    y, r = o.fwd(xv, None, eps, "f64")
    dx, _, _ = o.bwd(y, xv, None, r, "f64")
    ms = (xv ** 2).mean(axis=1)
    exp = xv * (r ** 2 * eps / (ms + eps))[:, None]
    assert np.allclose(dx, exp, rtol=1e-11, atol=1e-15)
    # the saved rrms is used as given, not recomputed from x
    dxa, _, _ = o.bwd(y, xv, None, r, "f64")
    dxb, _, _ = o.bwd(y, xv, None, r * 2.0, "f64")
    assert not np.allclose(dxa, dxb)


def check_bwd_linearity_and_rows(o):
    rng = _rng(12)
    M, H = 5, 40
    xv = rng.standard_normal((M, H))
    wv = rng.uniform(0.5, 1.5, H)
    d1, d2 = rng.standard_normal((M, H)), rng.standard_normal((M, H))
    _, r = o.fwd(xv, wv, 1e-5, "f64")
    a1, w1, _ = o.bwd(d1, xv, wv, r, "f64")
    a2, w2, _ = o.bwd(d2, xv, wv, r, "f64")
    a3, w3, _ = o.bwd(2 * d1 - 3 * d2, xv, wv, r, "f64")
    assert np.allclose(a3, 2 * a1 - 3 * a2, rtol=1e-12, atol=1e-13)
    assert np.allclose(w3, 2 * w1 - 3 * w2, rtol=1e-12, atol=1e-13)
    # dw sums over rows: the rows' separate dw add up to the batch's
    parts = sum(o.bwd(d1[i:i + 1], xv[i:i + 1], wv, r[i:i + 1], "f64")[1] for i in range(M))
    assert np.allclose(parts, w1, rtol=1e-13, atol=1e-14)
    # dx of one row does not depend on the other rows
    a_row, _, _ = o.bwd(d1[2:3], xv[2:3], wv, r[2:3], "f64")
    assert np.array_equal(a_row[0], a1[2])


# ---------------------------------------------------------------------------
# AdaLN
# ---------------------------------------------------------------------------

def check_adaln_exact_case(o):
    # x = [6, 8], eps = 14 -> rrms = 1/8, xn = [3/4, 1]; w = 1;
    # y = xn * (1 + scale) + shift with scale = [1, -1/2], shift = [1/4, 2]
    x = np.array([[6.0, 8.0]], dtype=np.float32)
    sc = np.array([[1.0, -0.5]], dtype=np.float32)
    sh = np.array([[0.25, 2.0]], dtype=np.float32)
    y, r = o.adaln_fwd(x, np.ones(2, np.float32), sc, sh, 1, 14.0, "f32")
    assert r[0] == 0.125 and np.array_equal(y[0], np.array([1.75, 2.5]))


def check_adaln_reduces_to_rmsnorm(o):
    rng = _rng(20)
    M, H = 6, 40
    for dt in ("bf16", "f16", "f32"):
        x = _storage(_round_like(rng.standard_normal((M, H)), dt), dt)
        w = _storage(_round_like(rng.uniform(0.5, 1.5, H), dt), dt)
        zeros = _storage(np.zeros((M, H)), dt)
        y0, r0 = o.fwd(x, w, 1e-5, dt)
        # zero conditioning is the plain norm, exactly
        y, r = o.adaln_fwd(x, w, zeros, zeros, 1, 1e-5, dt)
        assert np.array_equal(y, y0) and np.array_equal(r, r0)
        # scale = -1 leaves the shift alone, exactly
        sh = _storage(_round_like(rng.standard_normal((M, H)), dt), dt)
        minus1 = _storage(-np.ones((M, H)), dt)
        y, _ = o.adaln_fwd(x, w, minus1, sh, 1, 1e-5, dt)
        shv = _bf16_values(sh) if dt == "bf16" else sh.astype(np.float64)
        assert np.array_equal(y, shv)
        # y - shift = (plain norm) * (1 + scale)
        sc = _storage(_round_like(rng.standard_normal((M, H)) * 0.3, dt), dt)
        scv = _bf16_values(sc) if dt == "bf16" else sc.astype(np.float64)
        y, _ = o.adaln_fwd(x, w, sc, sh, 1, 1e-5, dt)
        assert np.allclose(y - shv, y0 * (1.0 + scv), rtol=1e-12, atol=1e-14)


def check_adaln_broadcast_rows(o):
    # one conditioning row per batch of S rows equals that row repeated S times
    rng = _rng(21)
    B, S, H = 3, 5, 24
    x = _storage(_round_like(rng.standard_normal((B * S, H)), "bf16"), "bf16")
    w = _storage(_round_like(rng.uniform(0.5, 1.5, H), "bf16"), "bf16")
    sc = _storage(_round_like(rng.standard_normal((B, H)) * 0.2, "bf16"), "bf16")
    sh = _storage(_round_like(rng.standard_normal((B, H)) * 0.2, "bf16"), "bf16")
    yb, rb = o.adaln_fwd(x, w, sc, sh, S, 1e-6, "bf16")
    yf, rf = o.adaln_fwd(x, w, np.repeat(sc, S, axis=0), np.repeat(sh, S, axis=0), 1, 1e-6, "bf16")
    assert np.array_equal(yb, yf) and np.array_equal(rb, rf)
    # the conditioning row is chosen by batch: a change in batch 1's row moves
    # only rows S..2S-1
    sc2 = sc.copy()
    sc2[1] = _storage(_round_like(rng.standard_normal(H), "bf16"), "bf16")
    y2, _ = o.adaln_fwd(x, w, sc2, sh, S, 1e-6, "bf16")
    changed = np.any(y2 != yb, axis=1)
    assert np.array_equal(changed, np.repeat([False, True, False], S))


def check_adaln_decimal(o):
    getcontext().prec = 60
    rng = _rng(22)
    H = 3
    x = _round_like(rng.standard_normal((2, H)), "f32")
    w = _round_like(rng.uniform(0.5, 1.5, H), "f32")
    sc = _round_like(rng.standard_normal((2, H)), "f32")
    sh = _round_like(rng.standard_normal((2, H)), "f32")
    y, _ = o.adaln_fwd(x.astype(np.float32), w.astype(np.float32), sc.astype(np.float32), sh.astype(np.float32),
                       1, 1e-5, "f32")
    for i in range(2):
        ss = sum(Decimal(float(v)) ** 2 for v in x[i])
        r = 1 / (ss / H + Decimal(1e-5)).sqrt()  # the oracle was given the float64 1e-5
        for j in range(H):
            t = Decimal(float(x[i, j])) * r * Decimal(float(w[j])) * (1 + Decimal(float(sc[i, j])))
            e = t + Decimal(float(sh[i, j]))
            # float64 rounding is relative to the terms, which may cancel
            assert abs(Decimal(float(y[i, j])) - e) <= (abs(t) + abs(Decimal(float(sh[i, j])))) * Decimal("1e-15")


# ---------------------------------------------------------------------------
# backward of the fused residual pre-norm
# ---------------------------------------------------------------------------

def check_bwd_residual_finite_differences(o):
    # L(x, r, w) = sum(dy * y) + sum(g * h) with h = x + r, y = RMSNorm(h):
    # dL/dx = dL/dr = dh, dL/dw = dw
    rng = _rng(30)
    for (M, H) in ((1, 1), (2, 3), (3, 16), (2, 64)):
        eps = 1e-2
        xv, rv = rng.standard_normal((M, H)), rng.standard_normal((M, H))
        wv = rng.uniform(0.5, 1.5, H)
        dyv, gv = rng.standard_normal((M, H)), rng.standard_normal((M, H))

        def loss(x, r, w):
            y, h, _ = o.fwd_residual(x, r, w, eps, "f64")
            return float((dyv * y).sum() + (gv * h).sum())

        _, hh, rr = o.fwd_residual(xv, rv, wv, eps, "f64")
        dh, dw, _ = o.bwd_residual(dyv, hh, gv, wv, rr, "f64")
        step = 1e-5
        scale = np.abs(dh).max()
        for i in range(M):
            for j in range(H):
                for which in (0, 1):
                    a = [xv.copy(), rv.copy()]
                    b = [xv.copy(), rv.copy()]
                    a[which][i, j] += step
                    b[which][i, j] -= step
                    fd = (loss(a[0], a[1], wv) - loss(b[0], b[1], wv)) / (2 * step)
                    assert abs(fd - dh[i, j]) <= 1e-7 * scale + 1e-9, (M, H, i, j, which)
        for j in range(H):
            wp, wm = wv.copy(), wv.copy()
            wp[j] += step
            wm[j] -= step
            fd = (loss(xv, rv, wp) - loss(xv, rv, wm)) / (2 * step)
            assert abs(fd - dw[j]) <= 1e-7 * np.abs(dw).max() + 1e-9


def check_bwd_residual_reduces_to_bwd(o):
    rng = _rng(31)
    M, H = 4, 50
    h = rng.standard_normal((M, H))
    w = rng.uniform(0.5, 1.5, H)
    dy, g = rng.standard_normal((M, H)), rng.standard_normal((M, H))
    _, r = o.fwd(h, w, 1e-5, "f64")
    dx, dw, _ = o.bwd(dy, h, w, r, "f64")
    dh0, dw0, _ = o.bwd_residual(dy, h, None, w, r, "f64")
    assert np.array_equal(dh0, dx) and np.array_equal(dw0, dw)
    dh1, dw1, _ = o.bwd_residual(dy, h, g, w, r, "f64")
    assert np.allclose(dh1 - g, dx, rtol=1e-14, atol=1e-15) and np.array_equal(dw1, dw)


# ---------------------------------------------------------------------------
# RoPE apply ("rocm-kernels", Core Kernel Implementations 2 and Template 2)
# ---------------------------------------------------------------------------

def check_rope_hand_example(o):
    # head_dim 4: pairs (0, 2) and (1, 3); the table's last two columns are
    # never read (filled with 9)
    x = np.array([1.0, 3.0, 2.0, 5.0]).reshape(1, 1, 1, 4)
    c = np.array([[0.5, 0.25, 9.0, 9.0]])
    sn = np.array([[0.75, -1.0, 9.0, 9.0]])
    # out0 = x0*c - x1*s, out1 = x0*s + x1*c, worked by hand
    assert np.array_equal(o.rope(x, c, sn, "f64")[0, 0, 0], [-1.0, 5.75, 1.75, -1.75])
    # transposed: s -> -s
    assert np.array_equal(o.rope(x, c, sn, "f64", transpose=True)[0, 0, 0], [2.0, -4.25, 0.25, 4.25])
    # half-width tables give the same result
    assert np.array_equal(o.rope(x, c[:, :2], sn[:, :2], "f64")[0, 0, 0], [-1.0, 5.75, 1.75, -1.75])


def check_rope_quarter_turns_by_position(o):
    # token s of every batch turns by s quarter turns: cos/sin in {0, +-1}, so
    # each output is exactly +-x0 or +-x1; this fixes which table row each
    # flat row (b * S + s) reads
    B, S, NH, D = 3, 5, 2, 6
    rng = _rng(40)
    x = rng.standard_normal((B, S, NH, D))
    ang = np.arange(S)
    c = np.repeat(np.array([1.0, 0.0, -1.0, 0.0])[ang % 4][:, None], D, axis=1)
    sn = np.repeat(np.array([0.0, 1.0, 0.0, -1.0])[ang % 4][:, None], D, axis=1)
    out = o.rope(x, c, sn, "f64")
    h = D // 2
    x0, x1 = x[..., :h], x[..., h:]
    for s in range(S):
        q = s % 4
        want0 = [x0, -x1, -x0, x1][q][:, s]
        want1 = [x1, x0, -x1, -x0][q][:, s]
        assert np.array_equal(out[:, s, :, :h], want0) and np.array_equal(out[:, s, :, h:], want1), s


def check_rope_rotation_invariants(o):
    # each (j, j + D/2) pair is rotated by its angle: the pair's norm is kept,
    # two rotations compose to the rotation by the summed angle, and the
    # transposed rotation undoes the rotation
    rng = _rng(41)
    B, S, NH, D = 2, 7, 3, 16
    x = rng.standard_normal((B, S, NH, D))
    t1, t2 = rng.uniform(-np.pi, np.pi, (S, D // 2)), rng.uniform(-np.pi, np.pi, (S, D // 2))
    y = o.rope(x, np.cos(t1), np.sin(t1), "f64")
    h = D // 2
    n_in = x[..., :h] ** 2 + x[..., h:] ** 2
    n_out = y[..., :h] ** 2 + y[..., h:] ** 2
    assert np.allclose(n_out, n_in, rtol=1e-14, atol=0)
    z = o.rope(y, np.cos(t2), np.sin(t2), "f64")
    z2 = o.rope(x, np.cos(t1 + t2), np.sin(t1 + t2), "f64")
    assert np.allclose(z, z2, rtol=0, atol=1e-13)
    back = o.rope(y, np.cos(t1), np.sin(t1), "f64", transpose=True)
    assert np.allclose(back, x, rtol=0, atol=1e-14)
    # the angle's complex form: (x0 + i x1) * exp(i t)
    zc = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * t1)[None, :, None, :]
    assert np.allclose(y[..., :h], zc.real, rtol=0, atol=1e-14) and np.allclose(y[..., h:], zc.imag, rtol=0,
                                                                                 atol=1e-14)


def check_rope_batches_and_strides(o):
    # batches are independent and read the same table rows; a padded view
    # (head and row strides) gives the same values as its contiguous copy
    rng = _rng(42)
    B, S, NH, D = 3, 4, 2, 8
    x = rng.standard_normal((B, S, NH, D))
    t = rng.uniform(-np.pi, np.pi, (S, D))
    c, sn = np.cos(t), np.sin(t)
    full = o.rope(x, c, sn, "f64")
    for b in range(B):
        assert np.array_equal(full[b], o.rope(x[b:b + 1], c, sn, "f64")[0])
    big = np.zeros((B, S, NH + 1, D + 3))
    big[:, :, :NH, :D] = x
    assert np.array_equal(o.rope(big[:, :, :NH, :D], c, sn, "f64"), full)
    # bf16 storage: decode is exact, the result is the float64 rotation of
    # the decoded values
    xb = o.encode(x, "bf16")
    cb, sb = o.encode(c, "bf16"), o.encode(sn, "bf16")
    got = o.rope(xb, cb, sb, "bf16")
    want = o.rope(o.decode(xb, "bf16"), o.decode(cb, "bf16"), o.decode(sb, "bf16"), "f64")
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# residual + LayerNorm ("SpeedROCm", item 4; torch.nn's LayerNorm)
# ---------------------------------------------------------------------------

def check_layernorm_hand_example(o):
    # row 1 2 3 4: mean 2.5, population variance 1.25; eps 2.75 makes
    # var + eps = 4, so rstd = 1/2 and (h - mean) * rstd = -0.75 -0.25 0.25 0.75
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    w = np.array([1.0, 2.0, -1.0, 0.5])
    b = np.array([0.5, 0.0, 1.0, -1.0])
    y, h, mean, rstd = o.layernorm(x, None, w, b, 2.75, "f64")
    assert np.array_equal(y[0], [-0.25, -0.5, 0.75, -0.625])
    assert mean[0] == 2.5 and rstd[0] == 0.5 and np.array_equal(h, x)
    # the same row split as x + residual
    y2, h2, _, _ = o.layernorm(np.array([[0.5, 4.0, 3.0, -1.0]]), np.array([[0.5, -2.0, 0.0, 5.0]]), w, b, 2.75,
                               "f64")
    assert np.array_equal(y2, y) and np.array_equal(h2, x)


def check_layernorm_matches_torch_float64(o):
    torch = __import__("torch")
    rng = _rng(50)
    for (M, H, mu) in ((3, 1, 0.0), (4, 7, 0.0), (5, 64, 3.0), (2, 1000, -50.0)):
        x = rng.standard_normal((M, H)) + mu
        r = rng.standard_normal((M, H))
        w, b = rng.uniform(0.5, 1.5, H), rng.standard_normal(H)
        y, h, mean, rstd = o.layernorm(x, r, w, b, 1e-5, "f64")
        t = torch.nn.functional.layer_norm(torch.from_numpy(x + r), (H,), torch.from_numpy(w), torch.from_numpy(b),
                                           1e-5).numpy()
        assert np.allclose(y, t, rtol=1e-12, atol=1e-12), (M, H)
        t0 = torch.nn.functional.layer_norm(torch.from_numpy(x), (H,), None, None, 1e-5).numpy()
        assert np.allclose(o.layernorm(x, None, None, None, 1e-5, "f64")[0], t0, rtol=1e-12, atol=1e-12)


def check_layernorm_is_rmsnorm_of_centred_row(o):
    # LayerNorm(h) = RMSNorm(h - mean(h)) with the same eps; mean(y) = 0 and
    # mean(y^2) = var / (var + eps) without the affine part
    rng = _rng(51)
    M, H, eps = 6, 48, 1e-3
    x = rng.standard_normal((M, H)) * 3 + 1
    y, h, mean, rstd = o.layernorm(x, None, None, None, eps, "f64")
    centred = x - x.mean(axis=1, keepdims=True)
    yr, rr = o.fwd(centred, None, eps, "f64")
    assert np.allclose(y, yr, rtol=1e-13, atol=1e-13) and np.allclose(rstd, rr, rtol=1e-13)
    assert np.allclose(mean, x.mean(axis=1), rtol=1e-14, atol=1e-14)
    assert np.all(np.abs(y.mean(axis=1)) < 1e-14)
    var = 1.0 / rstd ** 2 - eps
    assert np.allclose((y ** 2).mean(axis=1), var / (var + eps), rtol=1e-13)


def check_layernorm_shift_and_scale(o):
    # a constant added to a row changes nothing; scaling a row by k with eps
    # scaled by k^2 changes nothing; a constant row gives exactly the bias
    rng = _rng(52)
    M, H = 4, 32
    x = rng.standard_normal((M, H))
    b = rng.standard_normal(H)
    y0 = o.layernorm(x, None, None, b, 1e-4, "f64")[0]
    assert np.allclose(o.layernorm(x + 1000.0, None, None, b, 1e-4, "f64")[0], y0, rtol=0, atol=1e-9)
    assert np.allclose(o.layernorm(x * 8.0, None, None, b, 64e-4, "f64")[0], y0, rtol=0, atol=1e-12)
    c = np.full((2, 64), 0.75)
    assert np.array_equal(o.layernorm(c, None, np.full(64, 3.0), b[:1].repeat(64), 1e-5, "f64")[0],
                          np.tile(b[:1].repeat(64), (2, 1)))


ALL_CHECKS = [
    check_decode_all_16bit_patterns,
    check_encode_matches_libraries,
    check_encode_ties_by_hand,
    check_exact_rational_rows,
    check_constant_and_zero_rows,
    check_h1_closed_form,
    check_weightless_mean_square,
    check_weight_indexed_by_column,
    check_scale_law,
    check_permutation_and_strides,
    check_fp16_large_values,
    check_decimal_bruteforce,
    check_residual_identities,
    check_bwd_exact_case,
    check_bwd_finite_differences,
    check_bwd_identities,
    check_bwd_special_cases,
    check_bwd_linearity_and_rows,
    check_adaln_exact_case,
    check_adaln_reduces_to_rmsnorm,
    check_adaln_broadcast_rows,
    check_adaln_decimal,
    check_bwd_residual_finite_differences,
    check_bwd_residual_reduces_to_bwd,
    check_rope_hand_example,
    check_rope_quarter_turns_by_position,
    check_rope_rotation_invariants,
    check_rope_batches_and_strides,
    check_layernorm_hand_example,
    check_layernorm_matches_torch_float64,
    check_layernorm_is_rmsnorm_of_centred_row,
    check_layernorm_shift_and_scale,
]
