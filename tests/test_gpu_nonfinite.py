"""Non-finite inputs: NaN and infinities planted in a few rows.

Their values are out of contract (float32 sums of such rows are not
meaningful), but a call must never crash, and a non-finite row must never
leak into another row.  The reference classification follows from IEEE
arithmetic and is the oracle's own: in float64 a NaN in a row makes the
row's sum of squares NaN, so every output of the row is NaN; an infinity
makes the sum infinite and rrms = 1/sqrt(inf) = 0, so the row's finite
elements become +-0 and the infinite ones NaN (inf * 0).  Each test checks
that the GPU's NaN and infinity positions are exactly the oracle's, that the
other special-row outputs are equal to the oracle's rounded values, and that
every row without a planted value still matches the oracle to the usual
tolerance.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic
from tests import gpu_util as G
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import transformer_normalization_amd as tn  # noqa: E402

# (row, column, value) planted; rows 1, 4 and 9 are special, the rest normal
PLANTS = [(1, 5, np.nan), (4, 0, np.inf), (9, -1, -np.inf), (9, 7, np.inf)]
SPECIAL = sorted({r for r, _, _ in PLANTS})


def plant(a, dtype, plants=PLANTS):
    a = np.array(a, copy=True)
    for r, c, v in plants:
        enc = oracle.encode(np.array([v]), dtype)
        a[r, c] = enc.view(a.dtype)[0]
    return a


def normal_rows(M):
    return np.array([i for i in range(M) if i not in SPECIAL])


def rounded(ref64, dtype):
    """The oracle's values rounded to the output format, as float64."""
    return oracle.decode(oracle.encode(ref64, dtype), dtype)


def same_classes(got64, ref64, what):
    """NaN and infinity positions identical; every other value equal."""
    assert np.array_equal(np.isnan(got64), np.isnan(ref64)), f"{what}: NaN positions differ"
    assert np.array_equal(np.isposinf(got64), np.isposinf(ref64)), f"{what}: +inf positions differ"
    assert np.array_equal(np.isneginf(got64), np.isneginf(ref64)), f"{what}: -inf positions differ"
    fin = np.isfinite(ref64)
    assert np.array_equal(got64[fin], ref64[fin]), f"{what}: finite values differ"


@pytest.mark.parametrize("H", [4096, 4097], ids=["aligned", "off_grid"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_forward(dtype, H):
    M = 16
    d = G.inputs(501, M, H, dtype)
    x = plant(d["x"], dtype)
    y, rr = tn.rmsnorm_fwd(G.to_dev(x, dtype), G.to_dev(d["w"], dtype), 1e-5, return_rrms=True)
    torch.cuda.synchronize()
    got, rrg = G.to_host(y, dtype), rr.cpu().numpy()
    yref, rref = oracle.fwd(x, d["w"], G.eps32(1e-5), dtype)
    rows = normal_rows(M)
    G.assert_ok(*G.fwd_vs_oracle(x[rows], d["w"], got[rows], rrg[rows], 1e-5, dtype, name=f"fwd {dtype} normal rows"))
    same_classes(oracle.decode(got[SPECIAL], dtype), rounded(yref[SPECIAL], dtype), f"fwd {dtype} y")
    same_classes(rrg[SPECIAL].astype(np.float64), rref[SPECIAL].astype(np.float32).astype(np.float64),
                 f"fwd {dtype} rrms")
    assert np.isnan(rrg[1]) and rrg[4] == 0.0 and rrg[9] == 0.0


@pytest.mark.parametrize("H", [2048, 2049], ids=["aligned", "off_grid"])
def test_fused_residual_nan_in_residual(H):
    M, dt = 16, "bf16"
    d = G.inputs(502, M, H, dt, residual=True)
    r = plant(d["r"], dt)
    y, ro, rr = tn.rmsnorm_fwd_residual(G.to_dev(d["x"], dt), G.to_dev(r, dt), G.to_dev(d["w"], dt), 1e-5,
                                        return_rrms=True)
    torch.cuda.synchronize()
    got, rog, rrg = G.to_host(y, dt), G.to_host(ro, dt), rr.cpu().numpy()
    yref, href, _ = oracle.fwd_residual(d["x"], r, d["w"], G.eps32(1e-5), dt)
    rows = normal_rows(M)
    G.assert_ok(*G.residual_vs_oracle(d["x"][rows], r[rows], d["w"], got[rows], rog[rows], rrg[rows], 1e-5, dt))
    same_classes(oracle.decode(got[SPECIAL], dt), rounded(yref[SPECIAL], dt), "residual y")
    same_classes(oracle.decode(rog[SPECIAL], dt), rounded(href[SPECIAL], dt), "residual_out")


def test_backward_nan_in_dy():
    """A NaN in dy makes its row of dx NaN (through the row sum) and its
    column of dw NaN; every other row of dx and column of dw is normal."""
    M, H, dt = 64, 1024, "bf16"
    d = G.inputs(503, M, H, dt, dy=True)
    dy = plant(d["dy"], dt, [(1, 5, np.nan)])
    _, r = oracle.fwd(d["x"], d["w"], G.eps32(1e-5), dt)
    r32 = r.astype(np.float32)
    dx, dw = tn.rmsnorm_bwd(G.to_dev(dy, dt), G.to_dev(d["x"], dt), G.to_dev(d["w"], dt), torch.from_numpy(r32).to(G.DEV))
    torch.cuda.synchronize()
    dxg, dwg = G.to_host(dx, dt), dw.cpu().numpy().astype(np.float64)
    dxref, dwref, _ = oracle.bwd(dy, d["x"], d["w"], r32, dt)
    assert np.isnan(oracle.decode(dxg[1], dt)).all() and np.isnan(dxref[1]).all()
    rows = np.array([i for i in range(M) if i != 1])
    G.assert_ok(*G.bwd_vs_oracle(dy[rows], d["x"][rows], d["w"], r32[rows], dxg[rows], None, dt))
    assert np.array_equal(np.isnan(dwg), np.isnan(dwref)) and np.isnan(dwg[5])
    cols = np.array([j for j in range(H) if j != 5])
    xn = oracle.decode(d["x"], dt) * r32.astype(np.float64)[:, None]
    colscale = np.abs(np.where(np.isnan(oracle.decode(dy, dt)), 0, oracle.decode(dy, dt)) * xn).sum(axis=0)
    rep = parity.Report("bwd dw, other columns")
    parity.check_dw(rep, dwg[cols], dwref[cols], colscale[cols])
    G.assert_ok(rep)


@pytest.mark.parametrize("H", [2048, 2049], ids=["aligned", "off_grid"])
def test_layernorm(H):
    M, dt = 16, "bf16"
    d = G.inputs(504, M, H, dt, residual=True)
    x = plant(d["x"], dt)
    b = synthetic.normal_tensor(504, synthetic.STREAM_BIAS, (H,), dt, 0.0, 0.1)
    y, ro = tn.layernorm_fwd_residual(G.to_dev(x, dt), G.to_dev(d["r"], dt), G.to_dev(d["w"], dt), G.to_dev(b, dt),
                                      1e-5)
    torch.cuda.synchronize()
    got = G.to_host(y, dt)
    yref, _, _, _ = oracle.layernorm(x, d["r"], d["w"], b, G.eps32(1e-5), dt)
    same_classes(oracle.decode(got[SPECIAL], dt), rounded(yref[SPECIAL], dt), "layernorm y")
    rows = normal_rows(M)
    rep = parity.Report("layernorm normal rows")
    G.check_out(rep, got[rows], yref[rows], dt)
    G.assert_ok(rep)


def test_adaln():
    B, S, H, dt = 2, 8, 2048, "bf16"
    M = B * S
    d = G.inputs(505, M, H, dt)
    x = plant(d["x"], dt)
    sc = synthetic.normal_tensor(505, synthetic.STREAM_SCALE, (B, H), dt, 0.0, 0.5)
    sh = synthetic.normal_tensor(505, synthetic.STREAM_SHIFT, (B, H), dt, 0.0, 0.5)
    y = tn.rmsnorm_adaln_fwd(G.to_dev(x, dt).view(B, S, H), G.to_dev(d["w"], dt), G.to_dev(sc, dt).view(B, 1, H),
                             G.to_dev(sh, dt).view(B, 1, H), 1e-6)
    torch.cuda.synchronize()
    got = G.to_host(y, dt).reshape(M, H)
    yref, _ = oracle.adaln_fwd(x, d["w"], sc, sh, S, G.eps32(1e-6), dt)
    same_classes(oracle.decode(got[SPECIAL], dt), rounded(yref[SPECIAL], dt), "adaln y")
    rows = normal_rows(M)
    rep = parity.Report("adaln normal rows")
    G.check_out(rep, got[rows], yref[rows], dt)
    G.assert_ok(rep)


def test_rope():
    """RoPE is elementwise per pair: only the pair (j, j + D/2) holding a
    planted value is affected, in the oracle's classes; every other output
    has the bits of a run on the clean input, which matches the oracle."""
    from tests.test_gpu_rope import rope_vs_oracle

    B, S, NH, D, dt = 2, 12, 4, 128, "bf16"
    clean = synthetic.normal_tensor(506, synthetic.STREAM_X, (B * S, NH * D), dt)
    xq = plant(clean, dt, [(1, 5, np.nan), (4, 0, np.inf), (9, 3 * D + 70, -np.inf)]).reshape(B, S, NH, D)
    clean = clean.reshape(B, S, NH, D)
    c, s = synthetic.rope_tables(506, S, D, "f32")
    cd, sd = G.to_dev(c, "f32"), G.to_dev(s, "f32")
    got_bits = G.to_host(tn.rope_apply(G.to_dev(xq, dt), cd, sd), dt).reshape(B * S, NH * D)
    clean_bits = G.to_host(tn.rope_apply(G.to_dev(clean, dt), cd, sd), dt)
    torch.cuda.synchronize()
    G.assert_ok(rope_vs_oracle(clean, c, s, clean_bits, dt, "f32", name="rope clean run"))
    ref = rounded(oracle.rope(xq, c, s, dt, "f32"), dt).reshape(B * S, NH * D)
    same_classes(oracle.decode(got_bits, dt)[SPECIAL], ref[SPECIAL], "rope special rows")
    # pairs without a planted value are the clean run's bits, in every row
    touched = np.zeros((B * S, NH * D), dtype=bool)
    for r, col in ((1, 5), (4, 0), (9, 3 * D + 70)):
        h, j = divmod(col, D)
        j0 = j % (D // 2)
        touched[r, h * D + j0] = touched[r, h * D + j0 + D // 2] = True
    clean_bits = clean_bits.reshape(B * S, NH * D)
    assert np.array_equal(got_bits[~touched], clean_bits[~touched])
    assert np.isnan(oracle.decode(got_bits, dt)[touched]).sum() + np.isinf(oracle.decode(got_bits, dt)[touched]).sum() \
        == touched.sum()
