"""Helpers for GPU tests: host <-> device transfers of stored bits and
chunked comparison of library outputs against the float64 oracle."""

from __future__ import annotations

import numpy as np

import oracle
import synthetic
from tests import parity

DEV = "cuda:0"


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_dev(a, dtype):
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t, dtype):
    import torch
    t = t.detach()
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def check_out(rep, got, ref64, dtype, offset=0):
    if dtype == "f32":
        parity.check_f32(rep, got, ref64, offset)
    else:
        parity.check16(rep, got, ref64, dtype, oracle.encode, offset)
    return rep


def eps32(eps):
    """The float32 value the library receives; the oracle uses the same."""
    return float(np.float32(eps))


def fwd_vs_oracle(x, w, y_host, rrms_host, eps, dtype, wdtype=None, chunk=2048, name="fwd"):
    M, H = x.shape
    rep_y, rep_r = parity.Report(f"{name} y"), parity.Report(f"{name} rrms")
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        yref, rref = oracle.fwd(x[r0:r1], w, eps32(eps), dtype, wdtype)
        check_out(rep_y, y_host[r0:r1], yref, dtype, r0 * H)
        if rrms_host is not None:
            parity.check_f32(rep_r, rrms_host[r0:r1], rref, r0)
    return rep_y, rep_r


def residual_vs_oracle(x, r, w, y_host, ro_host, rrms_host, eps, dtype, wdtype=None, chunk=1024, name="residual"):
    M, H = x.shape
    rep_y, rep_ro, rep_r = (parity.Report(f"{name} y"), parity.Report(f"{name} residual_out"),
                            parity.Report(f"{name} rrms"))
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        yref, href, rref = oracle.fwd_residual(x[r0:r1], r[r0:r1], w, eps32(eps), dtype, wdtype)
        check_out(rep_y, y_host[r0:r1], yref, dtype, r0 * H)
        if ro_host is not None:
            hb = oracle.encode(href, dtype)
            bad = (ro_host[r0:r1].view(np.uint16 if dtype != "f32" else np.uint32)
                   != hb.view(np.uint16 if dtype != "f32" else np.uint32))
            rep_ro.n += bad.size
            rep_ro.merge_bad(bad, r0 * H)
        if rrms_host is not None:
            parity.check_f32(rep_r, rrms_host[r0:r1], rref, r0)
    return rep_y, rep_ro, rep_r


def bwd_vs_oracle(dy, x, w, rrms32, dx_host, dw_host, dtype, wdtype=None, chunk=1024, name="bwd"):
    M, H = x.shape
    rep_dx, rep_dw = parity.Report(f"{name} dx"), parity.Report(f"{name} dw")
    dw_ref = np.zeros(H) if w is not None else None
    colscale = np.zeros(H)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        dxref, dwref, terms = oracle.bwd(dy[r0:r1], x[r0:r1], w, rrms32[r0:r1], dtype, wdtype)
        if dtype == "f32":
            parity.check_dx_f32(rep_dx, dx_host[r0:r1], dxref, terms, r0 * H)
        else:
            parity.check_dx16(rep_dx, dx_host[r0:r1], dxref, terms, dtype, oracle.encode, oracle.decode, r0 * H)
        if w is not None:
            dw_ref += dwref
            xn = oracle.decode(x[r0:r1], dtype) * rrms32[r0:r1].astype(np.float64)[:, None]
            colscale += np.abs(oracle.decode(dy[r0:r1], dtype) * xn).sum(axis=0)
    if w is not None and dw_host is not None:
        parity.check_dw(rep_dw, dw_host, dw_ref, colscale)
    return rep_dx, rep_dw


def bwd_residual_vs_oracle(dy, h, dres, w, rrms32, dh_host, dw_host, dtype, wdtype=None, chunk=1024,
                          name="bwd_residual"):
    """dh = norm backward through h + dres: dres joins the terms that set the
    cancellation floor (dh may cancel between the norm's gradient and dres)."""
    M, H = h.shape
    rep_dh, rep_dw = parity.Report(f"{name} dh"), parity.Report(f"{name} dw")
    dw_ref = np.zeros(H) if w is not None else None
    colscale = np.zeros(H)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        g = None if dres is None else dres[r0:r1]
        dhref, dwref, terms = oracle.bwd_residual(dy[r0:r1], h[r0:r1], g, w, rrms32[r0:r1], dtype, wdtype)
        if dtype == "f32":
            parity.check_dx_f32(rep_dh, dh_host[r0:r1], dhref, terms, r0 * H)
        else:
            parity.check_dx16(rep_dh, dh_host[r0:r1], dhref, terms, dtype, oracle.encode, oracle.decode, r0 * H)
        if w is not None:
            dw_ref += dwref
            xn = oracle.decode(h[r0:r1], dtype) * rrms32[r0:r1].astype(np.float64)[:, None]
            colscale += np.abs(oracle.decode(dy[r0:r1], dtype) * xn).sum(axis=0)
    if w is not None and dw_host is not None:
        parity.check_dw(rep_dw, dw_host, dw_ref, colscale)
    return rep_dh, rep_dw


def ln_vs_oracle(x, r, w, b, y_host, ro_host, mean_host, rstd_host, eps, dtype, wdtype=None, chunk=2048,
                 name="layernorm"):
    """Residual + LayerNorm against the oracle.  y = (h - mean) * rstd * w + b
    cancels twice (h - mean, and the bias), so its ulp floor is taken at the
    size of the terms, (|h| + |mean|) * rstd * |w| + |b|.  residual_out is
    bit-exact; mean within 1e-5 of mean(|h|) (a float32 sum of the row) and
    rstd within 1e-5 relative."""
    M, H = x.shape
    reps = {k: parity.Report(f"{name} {k}") for k in ("y", "residual_out", "mean", "rstd")}
    wd = wdtype or dtype
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        rr = None if r is None else r[r0:r1]
        yref, href, mref, sref = oracle.layernorm(x[r0:r1], rr, w, b, eps32(eps), dtype, wdtype)
        wv = np.ones(H) if w is None else oracle.decode(w, wd)
        bv = np.zeros(H) if b is None else oracle.decode(b, wd)
        terms = (np.abs(href) + np.abs(mref)[:, None]) * sref[:, None] * np.abs(wv)[None, :] + np.abs(bv)[None, :]
        if dtype == "f32":
            parity.check_dx_f32(reps["y"], y_host[r0:r1], yref, terms, r0 * H)
        else:
            parity.check_dx16(reps["y"], y_host[r0:r1], yref, terms, dtype, oracle.encode, oracle.decode, r0 * H)
        if ro_host is not None:
            hb = oracle.encode(href, dtype)
            view = np.uint16 if dtype != "f32" else np.uint32
            bad = ro_host[r0:r1].view(view) != hb.view(view)
            reps["residual_out"].n += bad.size
            reps["residual_out"].merge_bad(bad, r0 * H)
        if mean_host is not None:
            scale = np.abs(href).mean(axis=1)
            bad = np.abs(mean_host[r0:r1].astype(np.float64) - mref) > 1e-5 * scale + 1e-30
            reps["mean"].n += bad.size
            reps["mean"].merge_bad(bad, r0)
        if rstd_host is not None:
            parity.check_f32(reps["rstd"], rstd_host[r0:r1], sref, r0)
    return tuple(reps.values())


def assert_ok(*reports, record=None):
    """Fail on any failed element; `record` names a full-size workload whose
    reports the session lists at its end."""
    for r in reports:
        print(r, flush=True)
    if record is not None:
        parity.record(record, *reports)
    bad = [str(r) for r in reports if not r.ok()]
    assert not bad, "; ".join(bad)


def inputs(seed, M, H, dtype, wdtype=None, xdist=(0.0, 1.0), weight=True, residual=False, dy=False):
    """Seeded host arrays: x, w (or None), and optionally r (the residual
    stream, which the backward tests also use as dres) and dy."""
    d = {"x": synthetic.normal_tensor(seed, synthetic.STREAM_X, (M, H), dtype, *xdist)}
    d["w"] = synthetic.normal_tensor(seed, synthetic.STREAM_W, (H,), wdtype or dtype, 1.0, 0.1) if weight else None
    if residual:
        d["r"] = synthetic.normal_tensor(seed, synthetic.STREAM_RESIDUAL, (M, H), dtype)
    if dy:
        d["dy"] = synthetic.normal_tensor(seed, synthetic.STREAM_DY, (M, H), dtype)
    return d


def adaln_vs_oracle(x, w, scale, shift, rows_per_cond, y_host, rrms_host, eps, dtype, pdtype=None, chunk=2048,
                    name="adaln"):
    M, H = x.shape
    rep_y, rep_r = parity.Report(f"{name} y"), parity.Report(f"{name} rrms")
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        # conditioning rows of this chunk, re-based so that row r0 maps to 0
        c0 = r0 // rows_per_cond
        c1 = (r1 - 1) // rows_per_cond + 1
        if rows_per_cond > 1 and r0 % rows_per_cond:
            raise ValueError("chunk must start at a conditioning boundary")
        yref, rref = oracle.adaln_fwd(x[r0:r1], w, scale[c0:c1], shift[c0:c1], rows_per_cond, eps32(eps), dtype,
                                      pdtype, pdtype)
        # y = a + shift may cancel: judge against the size of its two terms,
        # as for dx (a = norm * w * (1 + scale))
        shv = oracle.decode(np.repeat(shift[c0:c1], rows_per_cond, axis=0)[: r1 - r0], pdtype or dtype)
        terms = np.abs(yref - shv) + np.abs(shv)
        if dtype == "f32":
            parity.check_dx_f32(rep_y, y_host[r0:r1], yref, terms, r0 * H)
        else:
            parity.check_dx16(rep_y, y_host[r0:r1], yref, terms, dtype, oracle.encode, oracle.decode, r0 * H)
        parity.check_f32(rep_r, rrms_host[r0:r1], rref, r0)
    return rep_y, rep_r


def sentinel_view(M, H, pad, offset, dtype, fill):
    """(M, H) view at element `offset` of a buffer with rows of H + pad,
    every element first set to `fill`."""
    import torch

    buf = torch.full((offset + M * (H + pad) + 16,), fill, dtype=torch_dtype(dtype), device=DEV)
    return buf, buf[offset:offset + M * (H + pad)].view(M, H + pad)[:, :H]


def untouched(buf, view, fill):
    """Every element of buf outside `view` still holds `fill`."""
    import torch

    mask = torch.ones(buf.numel(), dtype=torch.bool, device=buf.device)
    off = view.storage_offset() - buf.storage_offset()
    rows = torch.arange(view.shape[0], device=buf.device)[:, None] * view.stride(0)
    cols = torch.arange(view.shape[1], device=buf.device)[None, :]
    mask[(off + rows + cols).reshape(-1)] = False
    return bool(torch.all(buf[mask] == fill))
