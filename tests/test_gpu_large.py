"""Calls past 2^31 elements: the kernels' 64-bit row offsets, and grids of
hundreds of thousands of workgroups, at the largest sizes a test can afford.

The inputs are a seeded synthetic block of rows repeated on the device
(row i holds block row i mod R), so the oracle's result for any row is its
block row's, and sums over all rows are the block's sums weighted by how
often each block row occurs.  Outputs are checked on rows sampled at the
start, around the 2^31-element boundary and at the end.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import gpu_util as G
from tests import parity

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import transformer_normalization_amd as tn  # noqa: E402

H = 4096
R = 1024                        # block rows
M = (1 << 31) // H + 5          # 524293 rows: 2^31 + 5*4096 elements
BOUNDARY = (1 << 31) // H       # first row past 2^31 elements


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def repeated(block, dtype, m=M):
    """(m, H') device tensor whose row i is block row i mod R (H' = the block's width)."""
    b = G.to_dev(block, dtype)
    h = b.shape[1]
    out = torch.empty((m, h), dtype=b.dtype, device=G.DEV)
    full = m // R
    out[: full * R].view(full, R, h).copy_(b.unsqueeze(0).expand(full, R, h))
    out[full * R:] = b[: m - full * R]
    return out


def sample_rows(m=M, boundary=BOUNDARY):
    rows = list(range(0, 3)) + list(range(boundary - 3, boundary + 3)) + list(range(m - 3, m))
    return np.array(sorted(set(rows)))


# Rows off the 16-byte grid (8194 bytes each) take the kernels for such rows; the
# row that holds element 2^31 starts below it and ends above it.
HS = 4097
MS = (1 << 31) // HS + 5        # 524165 rows
BOUNDARY_S = (1 << 31) // HS    # the row that crosses 2^31 elements


@pytest.mark.parametrize("op", ["fwd", "residual", "layernorm"])
def test_off_grid_rows_past_2_31_elements(op):
    import synthetic
    d = G.inputs(7007, R, HS, "bf16", residual=True)
    x, w = repeated(d["x"], "bf16", MS), G.to_dev(d["w"], "bf16")
    rows = sample_rows(MS, BOUNDARY_S)
    idx = torch.from_numpy(rows).to(G.DEV)
    rep = parity.Report(f"off-grid {op} y past 2^31")
    if op == "fwd":
        y, rr = tn.rmsnorm_fwd(x, w, 1e-5, return_rrms=True)
        del x
        torch.cuda.synchronize()
        yref, rref = oracle.fwd(d["x"], d["w"], G.eps32(1e-5), "bf16")
        rep_r = parity.Report("off-grid fwd rrms past 2^31")
        parity.check_f32(rep_r, rr.cpu().numpy()[rows], rref[rows % R])
        G.assert_ok(rep_r)
    else:
        r = repeated(d["r"], "bf16", MS)
        if op == "residual":
            y, ro = tn.rmsnorm_fwd_residual(x, r, w, 1e-5)
            yref, href, _ = oracle.fwd_residual(d["x"], d["r"], d["w"], G.eps32(1e-5), "bf16")
        else:
            b = synthetic.normal_tensor(7007, synthetic.STREAM_BIAS, (HS,), "bf16", 0.0, 0.1)
            y, ro = tn.layernorm_fwd_residual(x, r, w, G.to_dev(b, "bf16"), 1e-5)
            del x, r
            torch.cuda.synchronize()
            # LayerNorm's rule: y cancels in h - mean and in the bias, so the
            # ulp floor is taken at the size of the terms; residual_out exact
            G.assert_ok(*G.ln_vs_oracle(d["x"][rows % R], d["r"][rows % R], d["w"], b, G.to_host(y[idx], "bf16"),
                                        G.to_host(ro[idx], "bf16"), None, None, 1e-5, "bf16",
                                        name="off-grid layernorm past 2^31"))
            return
        del x, r
        torch.cuda.synchronize()
        assert np.array_equal(G.to_host(ro[idx], "bf16"), oracle.encode(href[rows % R], "bf16"))
    parity.check16(rep, G.to_host(y[idx], "bf16"), yref[rows % R], "bf16", oracle.encode)
    G.assert_ok(rep)


def test_forward_past_2_31_elements():
    d = G.inputs(7000, R, H, "bf16")
    x = repeated(d["x"], "bf16")
    w = G.to_dev(d["w"], "bf16")
    y, rr = tn.rmsnorm_fwd(x, w, 1e-5, return_rrms=True)
    torch.cuda.synchronize()
    rows = sample_rows()
    yref, rref = oracle.fwd(d["x"], d["w"], G.eps32(1e-5), "bf16")
    got = G.to_host(y[torch.from_numpy(rows).to(G.DEV)], "bf16")
    rep_y, rep_r = parity.Report("fwd y past 2^31"), parity.Report("fwd rrms past 2^31")
    parity.check16(rep_y, got, yref[rows % R], "bf16", oracle.encode)
    parity.check_f32(rep_r, rr.cpu().numpy()[rows], rref[rows % R])
    G.assert_ok(rep_y, rep_r)


def test_backward_past_2_31_elements():
    d = G.inputs(7001, R, H, "bf16", dy=True)
    x, dy = repeated(d["x"], "bf16"), repeated(d["dy"], "bf16")
    w = G.to_dev(d["w"], "bf16")
    _, r = oracle.fwd(d["x"], d["w"], G.eps32(1e-5), "bf16")
    r32 = r.astype(np.float32)
    rr = torch.from_numpy(np.resize(r32, M)).to(G.DEV)
    dx, dw = tn.rmsnorm_bwd(dy, x, w, rr)
    torch.cuda.synchronize()
    rows = sample_rows()
    dxref, _, terms = oracle.bwd(d["dy"], d["x"], d["w"], r32, "bf16")
    rep_dx = parity.Report("bwd dx past 2^31")
    parity.check_dx16(rep_dx, G.to_host(dx[torch.from_numpy(rows).to(G.DEV)], "bf16"), dxref[rows % R],
                      terms[rows % R], "bf16", oracle.encode, oracle.decode)
    # dw over all M rows: block row k occurs full + (k < rest) times
    full, rest = divmod(M, R)
    _, dw_all, _ = oracle.bwd(d["dy"], d["x"], d["w"], r32, "bf16")
    _, dw_rest, _ = oracle.bwd(d["dy"][:rest], d["x"][:rest], d["w"], r32[:rest], "bf16")
    dw_ref = full * dw_all + dw_rest
    xn = oracle.decode(d["x"], "bf16") * r32.astype(np.float64)[:, None]
    per_row = np.abs(oracle.decode(d["dy"], "bf16") * xn)
    colscale = full * per_row.sum(axis=0) + per_row[:rest].sum(axis=0)
    rep_dw = parity.Report("bwd dw past 2^31")
    parity.check_dw(rep_dw, dw.cpu().numpy(), dw_ref, colscale)
    G.assert_ok(rep_dx, rep_dw)


def test_rope_past_2_31_elements():
    NH, D = 32, 128
    S = (1 << 31) // (2 * NH * D) + 3          # two batches of S positions
    Sb = 512                                   # block positions
    q_block = G.inputs(7002, Sb, NH * D, "bf16")["x"].reshape(Sb, NH, D)
    import synthetic
    c, s = synthetic.rope_tables(7002, Sb, D, "bf16")
    qb = G.to_dev(np.ascontiguousarray(q_block), "bf16")
    q = torch.empty((2, S, NH, D), dtype=torch.bfloat16, device=G.DEV)
    full = S // Sb
    for b in range(2):
        q[b, : full * Sb].view(full, Sb, NH, D).copy_(qb.unsqueeze(0).expand(full, Sb, NH, D))
        q[b, full * Sb:] = qb[: S - full * Sb]
    ct = G.to_dev(c, "bf16").repeat(full + 1, 1)[:S].contiguous()
    st = G.to_dev(s, "bf16").repeat(full + 1, 1)[:S].contiguous()
    out = tn.rope_apply(q, ct, st)
    torch.cuda.synchronize()
    ref = oracle.rope(q_block[None], c, s, "bf16")[0]  # (Sb, NH, D)
    pos = np.array([0, 1, S // 2, S - 2, S - 1])
    for b in range(2):
        got = G.to_host(out[b, torch.from_numpy(pos).to(G.DEV)], "bf16").reshape(len(pos), NH * D)
        want = ref[pos % Sb].reshape(len(pos), NH * D)
        rep = parity.Report(f"rope past 2^31 batch {b}")
        # the table rows repeat with the positions, so the block's values apply
        xv = oracle.decode(q_block[pos % Sb], "bf16")
        h = D // 2
        cv = oracle.decode(c[pos % Sb, :h], "bf16")[:, None, :]
        sv = oracle.decode(s[pos % Sb, :h], "bf16")[:, None, :]
        terms = np.concatenate([np.abs(xv[..., :h] * cv) + np.abs(xv[..., h:] * sv),
                                np.abs(xv[..., :h] * sv) + np.abs(xv[..., h:] * cv)], axis=-1)
        parity.check_dx16(rep, got, want, terms.reshape(len(pos), NH * D), "bf16", oracle.encode, oracle.decode)
        G.assert_ok(rep)


def test_fused_residual_past_2_31_elements():
    d = G.inputs(7003, R, H, "bf16", residual=True)
    x, r = repeated(d["x"], "bf16"), repeated(d["r"], "bf16")
    w = G.to_dev(d["w"], "bf16")
    y, ro = tn.rmsnorm_fwd_residual(x, r, w, 1e-5)
    del x, r
    torch.cuda.synchronize()
    rows = sample_rows()
    idx = torch.from_numpy(rows).to(G.DEV)
    yref, href, _ = oracle.fwd_residual(d["x"], d["r"], d["w"], G.eps32(1e-5), "bf16")
    rep = parity.Report("fused residual y past 2^31")
    parity.check16(rep, G.to_host(y[idx], "bf16"), yref[rows % R], "bf16", oracle.encode)
    assert np.array_equal(G.to_host(ro[idx], "bf16"), oracle.encode(href[rows % R], "bf16"))
    G.assert_ok(rep)


def test_layernorm_residual_past_2_31_elements():
    import synthetic
    d = G.inputs(7004, R, H, "bf16", residual=True)
    b = synthetic.normal_tensor(7004, synthetic.STREAM_BIAS, (H,), "bf16", 0.0, 0.1)
    x, r = repeated(d["x"], "bf16"), repeated(d["r"], "bf16")
    y, ro = tn.layernorm_fwd_residual(x, r, G.to_dev(d["w"], "bf16"), G.to_dev(b, "bf16"), 1e-5)
    del x, r
    torch.cuda.synchronize()
    rows = sample_rows()
    idx = torch.from_numpy(rows).to(G.DEV)
    # LayerNorm's rule (y's ulp floor at the size of its terms; residual_out exact)
    G.assert_ok(*G.ln_vs_oracle(d["x"][rows % R], d["r"][rows % R], d["w"], b, G.to_host(y[idx], "bf16"),
                                G.to_host(ro[idx], "bf16"), None, None, 1e-5, "bf16", name="layernorm past 2^31"))


def test_adaln_past_2_31_elements():
    """Per-token conditioning rows repeated like x, so conditioning row i is
    block row i mod R as well (64-bit offsets in the conditioning rows too)."""
    import synthetic
    d = G.inputs(7005, R, H, "bf16")
    sc = synthetic.normal_tensor(7005, synthetic.STREAM_SCALE, (R, H), "bf16", 0.0, 0.5)
    sh = synthetic.normal_tensor(7005, synthetic.STREAM_SHIFT, (R, H), "bf16", 0.0, 0.5)
    x, scd, shd = repeated(d["x"], "bf16"), repeated(sc, "bf16"), repeated(sh, "bf16")
    y = tn.rmsnorm_adaln_fwd(x.view(1, M, H), G.to_dev(d["w"], "bf16"), scd.view(1, M, H), shd.view(1, M, H), 1e-6)
    del x, scd, shd
    torch.cuda.synchronize()
    rows = sample_rows()
    idx = torch.from_numpy(rows).to(G.DEV)
    yref, _ = oracle.adaln_fwd(d["x"], d["w"], sc, sh, 1, G.eps32(1e-6), "bf16")
    rep = parity.Report("adaln y past 2^31")
    parity.check16(rep, G.to_host(y.view(M, H)[idx], "bf16"), yref[rows % R], "bf16", oracle.encode)
    G.assert_ok(rep)


def test_backward_residual_past_2_31_elements():
    d = G.inputs(7006, R, H, "bf16", residual=True, dy=True)
    dy, h, dres = repeated(d["dy"], "bf16"), repeated(d["x"], "bf16"), repeated(d["r"], "bf16")
    w = G.to_dev(d["w"], "bf16")
    _, r = oracle.fwd(d["x"], d["w"], G.eps32(1e-5), "bf16")
    r32 = r.astype(np.float32)
    rr = torch.from_numpy(np.resize(r32, M)).to(G.DEV)
    dh, dw = tn.rmsnorm_bwd_residual(dy, h, dres, w, rr)
    del dy, h, dres
    torch.cuda.synchronize()
    rows = sample_rows()
    dhref, dwref1, terms = oracle.bwd_residual(d["dy"], d["x"], d["r"], d["w"], r32, "bf16")
    rep_dh = parity.Report("residual bwd dh past 2^31")
    parity.check_dx16(rep_dh, G.to_host(dh[torch.from_numpy(rows).to(G.DEV)], "bf16"), dhref[rows % R],
                      terms[rows % R], "bf16", oracle.encode, oracle.decode)
    # dw over all M rows: block row k occurs full + (k < rest) times
    full, rest = divmod(M, R)
    _, dw_rest, _ = oracle.bwd_residual(d["dy"][:rest], d["x"][:rest], d["r"][:rest], d["w"], r32[:rest], "bf16")
    xn = oracle.decode(d["x"], "bf16") * r32.astype(np.float64)[:, None]
    per_row = np.abs(oracle.decode(d["dy"], "bf16") * xn)
    rep_dw = parity.Report("residual bwd dw past 2^31")
    parity.check_dw(rep_dw, dw.cpu().numpy(), full * dwref1 + dw_rest, full * per_row.sum(axis=0) + per_row[:rest].sum(axis=0))
    G.assert_ok(rep_dh, rep_dw)
