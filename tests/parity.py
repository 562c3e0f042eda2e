"""Comparison rules between the GPU library's outputs and the float64 oracle.

  * float32 outputs (y, dx in float32, rrms): |got - ref| <= 1e-5*|ref| + 1e-6.
  * 16-bit outputs: the stored bits are at most one unit in the last place
    away from the oracle's value rounded to nearest even (distance between
    the two bit patterns on the ordered integer line; +0 and -0 are equal).
  * residual write-back: bit-exact.
  * dx (16-bit): one ulp as above, where an element whose two terms
    rrms*g and xn*rrms*c/H nearly cancel may instead be within one ulp taken
    at 2^-10 * (|rrms*g| + |xn*rrms*c/H|): no float32 evaluation can do better
    on such elements.  The number of elements judged by that floor is reported.
  * dx (float32): |got - ref| <= 1e-5*max(|ref|, 2^-4 * terms) + 1e-6, with
    terms = |rrms*g| + |xn*rrms*c/H|.  Evaluating the difference of two terms
    of size T in float32 costs about 4 * 2^-24 * T (2.4e-7 T); the floor
    1e-5 * 2^-4 * T (6.25e-7 T) is about 2.6 times that.  (Rows with H = 1
    cancel to dx = rrms*g*eps/(x^2+eps).)
  * AdaLN output y = a + shift (a = norm * w * (1 + scale)) is judged like
    dx, with terms = |a| + |shift|: the final addition can cancel.
  * dw: |got - ref| <= 1e-3*|ref| + 1e-5 * sum_i |dy*xn| for each column (a
    pure relative bound is ill-posed for columns whose sum crosses zero).
    Reported besides: the normwise error ||got - ref||_2 / ||ref||_2, and the
    largest pure relative error over the well-conditioned columns, those
    whose sum keeps at least 1 % of sum_i |dy*xn| (cancellation of at most
    100x); there it must be <= 1e-3 as well.

Every comparison reports the elements compared, the failed count, the
largest ulp distance (16-bit outputs) or relative error, and how many
elements the cancellation floor judged.  The named full-size workloads
record their reports (record()); the test session prints them at its end
and, with TN_PARITY_DIR set, writes one text file per workload there.
"""

from __future__ import annotations

import numpy as np

PREC = {"bf16": 8, "f16": 11}
MIN_QUANTUM = {"bf16": 2.0 ** -133, "f16": 2.0 ** -24}


def ordered16(bits):
    b = np.asarray(bits).view(np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_distance16(a_bits, b_bits):
    return np.abs(ordered16(a_bits) - ordered16(b_bits))


def ulp_at(mag, dtype):
    """One unit in the last place of the format at magnitude mag (>= 0)."""
    p = PREC[dtype]
    m = np.maximum(np.asarray(mag, dtype=np.float64), 1e-300)
    return np.maximum(np.exp2(np.floor(np.log2(m)) - (p - 1)), MIN_QUANTUM[dtype])


class Report:
    def __init__(self, name):
        self.name = name
        self.n = 0
        self.failed = 0
        self.max_ulp = 0
        self.floor_used = 0
        self.max_rel = 0.0
        self.first_bad = None
        # float32 outputs and dw: the largest error as a fraction of the
        # element's allowed error (<= 1 passes)
        self.max_tol = 0.0
        # dw only: normwise error and well-conditioned columns
        self.err2 = 0.0
        self.ref2 = 0.0
        self.wc_cols = 0
        self.wc_max_rel = 0.0

    def merge_bad(self, bad_mask, offset=0):
        nb = int(np.count_nonzero(bad_mask))
        if nb and self.first_bad is None:
            self.first_bad = offset + int(np.flatnonzero(bad_mask.ravel())[0])
        self.failed += nb

    def ok(self):
        return self.failed == 0

    def normwise(self):
        return (self.err2 / self.ref2) ** 0.5 if self.ref2 > 0 else 0.0

    def __str__(self):
        s = (f"{self.name}: {self.n} elements, {self.failed} failed, max ulp {self.max_ulp}, "
             f"floor-judged {self.floor_used}, max rel {self.max_rel:.3g}, "
             f"max fraction of tolerance {self.max_tol:.3g}, first bad {self.first_bad}")
        if self.ref2 > 0:
            s += (f", normwise {self.normwise():.3g}, max rel over {self.wc_cols} well-conditioned columns "
                  f"{self.wc_max_rel:.3g}")
        return s


# reports of the named full-size workloads, in the order they were recorded
RECORDS: list[tuple[str, list[Report]]] = []


def record(workload: str, *reports: Report) -> None:
    RECORDS.append((workload, list(reports)))


def compact(r: Report) -> str:
    """One short line: elements, failed, max ulp, floor-judged, max relative
    error, and for dw the normwise and well-conditioned relative errors."""
    s = f"{r.name}: n={r.n} fail={r.failed} ulp={r.max_ulp} floor={r.floor_used} rel={r.max_rel:.2g} tol={r.max_tol:.2g}"
    if r.ref2 > 0:
        s += f" norm={r.normwise():.2g} wc={r.wc_cols}:{r.wc_max_rel:.2g}"
    return s


def format_records() -> list[str]:
    return [compact(r) for _, reps in RECORDS for r in reps if r.n]


def check16(report, got_bits, ref64, dtype, encode, offset=0):
    ref_bits = encode(ref64, dtype)
    d = ulp_distance16(got_bits, ref_bits)
    # NaN in the reference must be NaN on the GPU too
    report.n += d.size
    report.max_ulp = max(report.max_ulp, int(d.max()) if d.size else 0)
    report.merge_bad(d > 1, offset)
    return report


def check_f32(report, got, ref64, offset=0):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref64)
    allowed = 1e-5 * np.abs(ref64) + 1e-6
    bad = ~(err <= allowed)
    report.n += got.size
    if got.size:
        report.max_rel = max(report.max_rel, float((err / np.maximum(np.abs(ref64), 1e-30)).max()))
        report.max_tol = max(report.max_tol, float(np.nanmax(err / allowed)))
    report.merge_bad(bad, offset)
    return report


def check_dx16(report, got_bits, ref64, terms, dtype, encode, decode, offset=0):
    ref_bits = encode(ref64, dtype)
    d = ulp_distance16(got_bits, ref_bits)
    within = d <= 1
    got = decode(got_bits, dtype)
    floor_ok = np.abs(got - ref64) <= ulp_at(2.0 ** -10 * terms, dtype)
    report.n += d.size
    report.max_ulp = max(report.max_ulp, int(d.max()) if d.size else 0)
    report.floor_used += int(np.count_nonzero(~within & floor_ok))
    report.merge_bad(~(within | floor_ok), offset)
    return report


def check_dx_f32(report, got, ref64, terms, offset=0):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref64)
    strict = err <= 1e-5 * np.abs(ref64) + 1e-6
    relaxed = err <= 1e-5 * np.maximum(np.abs(ref64), 2.0 ** -4 * terms) + 1e-6
    # relative error where the relative bound governs: terms that do not
    # cancel, and |ref| >= 0.1 (below it the 1e-6 absolute term dominates)
    plain = (np.abs(ref64) >= 2.0 ** -4 * terms) & (np.abs(ref64) >= 0.1)
    if np.any(plain):
        report.max_rel = max(report.max_rel, float((err[plain] / np.abs(ref64[plain])).max()))
    if got.size:
        allowed = 1e-5 * np.maximum(np.abs(ref64), 2.0 ** -4 * terms) + 1e-6
        report.max_tol = max(report.max_tol, float(np.nanmax(err / allowed)))
    report.n += got.size
    report.floor_used += int(np.count_nonzero(~strict & relaxed))
    report.merge_bad(~relaxed, offset)
    return report


def check_dw(report, got, ref64, colscale):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref64)
    bad = ~(err <= 1e-3 * np.abs(ref64) + 1e-5 * colscale)
    rel = err / np.maximum(np.abs(ref64), 1e-30)
    report.n += got.size
    report.max_rel = max(report.max_rel, float(rel.max()))
    report.max_tol = max(report.max_tol, float(np.nanmax(err / (1e-3 * np.abs(ref64) + 1e-5 * colscale))))
    report.err2 += float(np.sum(err * err))
    report.ref2 += float(np.sum(ref64 * ref64))
    wc = np.abs(ref64) >= 0.01 * colscale
    report.wc_cols += int(np.count_nonzero(wc))
    if wc.any():
        report.wc_max_rel = max(report.wc_max_rel, float(rel[wc].max()))
    report.merge_bad(bad | (wc & (rel > 1e-3)))
    return report
