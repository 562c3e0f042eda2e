"""GPU parity of the LayerNorm forward (layernorm_fwd, layernorm_fwd_residual)
against the float64 oracle.

y is judged within 1 ulp of the oracle rounded to the output format, the ulp
taken at no less than 2^-10 of the size of its terms ((|h| + |mean|) * rstd *
|w| + |b|; float32: 1e-5 relative above a floor of 2^-4 of that size), since
h - mean and the bias may cancel; residual_out is bit-exact; the per-row mean
is within 1e-5 of the row's mean |h| and rstd within 1e-5 relative.
"""

from __future__ import annotations

import numpy as np
import pytest

import synthetic
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import transformer_normalization_amd as tn  # noqa: E402


@pytest.fixture(autouse=True)
def _default_geometry():
    tn.set_geometry("fwd")
    tn.set_streaming(-1)
    yield
    tn.set_geometry("fwd")
    tn.set_streaming(-1)


def bias_of(seed, H, dtype, std=0.1):
    return synthetic.normal_tensor(seed, synthetic.STREAM_BIAS, (H,), dtype, 0.0, std)


def run_ln(x, r, w, b, eps, dtype, wdtype=None):
    wd = wdtype or dtype
    xd = G.to_dev(x, dtype)
    wt = None if w is None else G.to_dev(w, wd)
    bt = None if b is None else G.to_dev(b, wd)
    if r is None:
        y, mean, rstd = tn.layernorm_fwd(xd, wt, bt, eps, return_stats=True)
        ro = None
    else:
        y, ro, mean, rstd = tn.layernorm_fwd_residual(xd, G.to_dev(r, dtype), wt, bt, eps, return_stats=True)
    torch.cuda.synchronize()
    return (G.to_host(y, dtype), None if ro is None else G.to_host(ro, dtype), mean.cpu().numpy(),
            rstd.cpu().numpy())


def check(x, r, w, b, eps, dtype, wdtype=None, name="ln", record=None):
    y, ro, mean, rstd = run_ln(x, r, w, b, eps, dtype, wdtype)
    G.assert_ok(*G.ln_vs_oracle(x, r, w, b, y, ro, mean, rstd, eps, dtype, wdtype, name=name), record=record)
    return y, ro


def test_workload_ln_residual():
    name = "ln_residual_f32_16384x1024"
    d = synthetic.make_inputs(name)
    print(f"[gpu] {name}", flush=True)
    check(d["x"], d["r"], d["w"], d["b"], d["eps"], d["dtype"], d["wdtype"], name=name, record=name)


# 12288 and 16384 (16-bit) and 8192 (float32) take tiles capped at 4 waves per
# row; 24576 is the longest 16-bit row held in registers; 16-bit rows of 6152
# to 8192 take two waves of 8 vectors per thread without the residual add
# (6152: 769 of 1024 vector slots used)
LN_H = [1, 3, 8, 64, 65, 512, 1000, 1024, 2049, 2056, 3584, 4096, 6144, 6152, 7168, 8191, 8192, 12288, 16384,
        16385, 24576, 24577, 65536]


@pytest.mark.parametrize("resid", [True, False], ids=["residual", "plain"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("H", LN_H)
def test_ln_shapes(H, dtype, resid):
    M = 257 if H <= 8192 else 5
    print(f"[gpu] ln {dtype} M={M} H={H} resid={resid}", flush=True)
    d = G.inputs(4000 + H, M, H, dtype, residual=resid)
    b = bias_of(4000 + H, H, dtype)
    check(d["x"], d.get("r"), d["w"], b, 1e-5, dtype, name=f"ln {dtype} H={H}")


@pytest.mark.parametrize("affine", ["none", "weight", "bias", "f32params"])
def test_ln_optional_weight_and_bias(affine):
    M, H = 300, 2048
    d = G.inputs(41, M, H, "bf16", residual=True)
    w, b, wd = d["w"], bias_of(41, H, "bf16"), None
    if affine == "none":
        w = b = None
    elif affine == "weight":
        b = None
    elif affine == "bias":
        w = None
    else:
        wd = "f32"
        w = synthetic.normal_tensor(41, synthetic.STREAM_W, (H,), "f32", 1.0, 0.1)
        b = bias_of(41, H, "f32")
    check(d["x"], d["r"], w, b, 1e-5, "bf16", wd, name=f"ln affine {affine}")


def test_ln_large_mean_offset():
    """Rows whose mean is far larger than their spread: the centred second
    reduction keeps the variance accurate."""
    M, H = 256, 1024
    x = synthetic.normal_tensor(42, synthetic.STREAM_X, (M, H), "f32", 100.0, 1.0)
    y, _ = check(x, None, None, None, 1e-5, "f32", name="ln offset 100")
    # the output has unit spread, not the offset's
    assert abs(float(np.std(y)) - 1.0) < 1e-3


def test_ln_constant_rows_give_the_bias():
    M, H = 64, 1024
    x = np.full((M, H), 0.75, dtype=np.float32)
    w = synthetic.normal_tensor(43, synthetic.STREAM_W, (H,), "f32", 1.0, 0.1)
    b = bias_of(43, H, "f32")
    y, _, mean, rstd = run_ln(x, None, w, b, 1e-5, "f32")
    assert np.array_equal(y, np.tile(b, (M, 1)))
    assert np.all(mean == 0.75)


# (vpt, wpr, rpw, grid): row tiles (exact, and with idle slots), several rows
# per workgroup, and capped grids walking the rows grid-stride (long rows'
# three-pass path is reached by the H = 65536 shapes)
LN_GEOMS = [(1, 4, 1, 0), (2, 2, 2, 0), (4, 1, 4, 0), (2, 2, 1, 7), (4, 1, 1, 0), (8, 1, 1, 0), (4, 2, 2, 5)]


@pytest.mark.parametrize("stream", [0, 1], ids=["cached", "streaming"])
@pytest.mark.parametrize("geom", LN_GEOMS, ids=[str(g) for g in LN_GEOMS])
def test_ln_forced_geometry(geom, stream):
    M, H = 300, 2048
    d = G.inputs(44, M, H, "bf16", residual=True)
    b = bias_of(44, H, "bf16")
    tn.set_geometry("fwd", *geom)
    tn.set_streaming(stream)
    check(d["x"], d["r"], d["w"], b, 1e-5, "bf16", name=f"ln geom {geom}")


def test_ln_streaming_and_determinism():
    d = G.inputs(45, 1000, 4096, "bf16", residual=True)
    b = bias_of(45, 4096, "bf16")
    runs = []
    for mode in (0, 1, -1, -1):
        tn.set_streaming(mode)
        runs.append(run_ln(d["x"], d["r"], d["w"], b, 1e-5, "bf16"))
    for r in runs[1:]:
        for a, c in zip(runs[0], r):
            assert np.array_equal(a, c)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_misaligned_and_strided_rows(dtype):
    """Odd H, and a residual one element into its buffer, leave the
    16-byte grid (another tile and reduction order: within tolerance of the
    oracle); row strides padded by whole 16-byte vectors give the same bits
    as contiguous rows."""
    M, H = 129, 1023
    d = G.inputs(46, M, H, dtype, residual=True)
    b = bias_of(46, H, dtype)
    check(d["x"], d["r"], d["w"], b, 1e-5, dtype, name=f"ln odd H {dtype}")
    H = 1024
    d = G.inputs(47, M, H, dtype, residual=True)
    b = bias_of(47, H, dtype)
    ref = run_ln(d["x"], d["r"], d["w"], b, 1e-5, dtype)
    td = G.torch_dtype(dtype)
    wt, bt = G.to_dev(d["w"], dtype), G.to_dev(b, dtype)
    xb = torch.zeros((M, H + 8), dtype=td, device=G.DEV)
    xb[:, :H] = G.to_dev(d["x"], dtype)
    rb = torch.zeros((M, H + 16), dtype=td, device=G.DEV)
    rb[:, :H] = G.to_dev(d["r"], dtype)
    y, ro = tn.layernorm_fwd_residual(xb[:, :H], rb[:, :H], wt, bt, 1e-5)
    torch.cuda.synchronize()
    assert np.array_equal(G.to_host(y, dtype), ref[0]) and np.array_equal(G.to_host(ro, dtype), ref[1])
    flat = torch.zeros(M * H + 1, dtype=td, device=G.DEV)
    rv = flat[1:].view(M, H)
    rv.copy_(G.to_dev(d["r"], dtype))
    y, ro, mean, rstd = tn.layernorm_fwd_residual(xb[:, :H], rv, wt, bt, 1e-5, return_stats=True)
    torch.cuda.synchronize()
    G.assert_ok(*G.ln_vs_oracle(d["x"], d["r"], d["w"], b, G.to_host(y, dtype), G.to_host(ro, dtype),
                                mean.cpu().numpy(), rstd.cpu().numpy(), 1e-5, dtype, name=f"ln misaligned {dtype}"))


@pytest.mark.parametrize("dtype,wdtype", [("bf16", "bf16"), ("f16", "f32"), ("f32", "f32")])
@pytest.mark.parametrize("H", [600, 2049, 4096, 6143, 16385, 24577, 70001])
def test_ln_rows_off_the_grid(dtype, wdtype, H):
    """Rows off the 16-byte grid (ragged H, or views at element offsets)
    are read and written in 16-byte vectors at each row's byte offset, on a
    tile that depends on H only: every layout gives the same bits, at parity
    with the oracle, and nothing around the output rows is written; the
    forced element-wise tile is at parity too.  16-bit rows with 16-bit
    parameters stay in registers to 24575 columns; 16385 in float32 or with
    float32 parameters, and 24577 and 70001 everywhere, take the passes over
    the row."""
    M = 67 if H <= 8192 else 9
    d = G.inputs(5100 + H, M, H, dtype, wdtype=wdtype, residual=True)
    b = bias_of(5100 + H, H, wdtype)
    wt, bt = G.to_dev(d["w"], wdtype), G.to_dev(b, wdtype)
    first = None
    for pad, xoff, yoff in ((1, 1, 0), (0, 3, 1), (5, 0, 7), (8, 1, 1)):
        print(f"[gpu] ln off the grid {dtype}/{wdtype} H={H} pad={pad} xoff={xoff} yoff={yoff}", flush=True)
        _, xv = G.sentinel_view(M, H, pad, xoff, dtype, 0.0)
        _, rv = G.sentinel_view(M, H, pad + 1, xoff + 2, dtype, 0.0)
        xv.copy_(G.to_dev(d["x"], dtype))
        rv.copy_(G.to_dev(d["r"], dtype))
        ybuf, yv = G.sentinel_view(M, H, pad + 3, yoff, dtype, -77.0)
        robuf, rov = G.sentinel_view(M, H, pad, yoff + 1, dtype, -77.0)
        _, _, mean, rstd = tn.layernorm_fwd_residual(xv, rv, wt, bt, 1e-5, out=yv, residual_out=rov,
                                                     return_stats=True)
        y2 = tn.layernorm_fwd(xv, wt, bt, 1e-5)
        torch.cuda.synchronize()
        assert G.untouched(ybuf, yv, -77.0) and G.untouched(robuf, rov, -77.0), (pad, xoff, yoff)
        got = [G.to_host(yv.contiguous(), dtype), G.to_host(rov.contiguous(), dtype), mean.cpu().numpy(),
               rstd.cpu().numpy(), G.to_host(y2, dtype)]
        if first is None:
            first = got
            G.assert_ok(*G.ln_vs_oracle(d["x"], d["r"], d["w"], b, got[0], got[1], got[2], got[3], 1e-5, dtype,
                                        wdtype, name=f"ln off the grid {dtype} H={H}"))
            G.assert_ok(*G.ln_vs_oracle(d["x"], None, d["w"], b, got[4], None, None, None, 1e-5, dtype, wdtype,
                                        name=f"ln off the grid plain {dtype} H={H}"))
        else:
            for a, c in zip(got, first):
                assert np.array_equal(a, c), (pad, xoff, yoff)
    # ragged H: the contiguous call leaves the grid too, and a forced tile
    # keeps it on single elements
    vpt = 8
    wpr = -(-H // (64 * vpt))
    if (H * (4 if dtype == "f32" else 2)) % 16 and 64 * wpr <= 512:
        tn.set_geometry("fwd", vpt, wpr, 1, 0)
        try:
            y3, ro3, m3, r3 = run_ln(d["x"], d["r"], d["w"], b, 1e-5, dtype, wdtype)
        finally:
            tn.set_geometry("fwd")
        G.assert_ok(*G.ln_vs_oracle(d["x"], d["r"], d["w"], b, y3, ro3, m3, r3, 1e-5, dtype, wdtype,
                                    name=f"ln element tile {dtype} H={H}"))


# 4097: rows off the 16-byte grid; 70001: off the grid and longer than a tile
@pytest.mark.parametrize("H", [4096, 65536, 4097, 70001])
def test_ln_in_place(H):
    M = 64 if H <= 8192 else 4
    d = G.inputs(48, M, H, "bf16", residual=True)
    b = bias_of(48, H, "bf16")
    ref = run_ln(d["x"], d["r"], d["w"], b, 1e-5, "bf16")
    x, r = G.to_dev(d["x"], "bf16"), G.to_dev(d["r"], "bf16")
    w, bt = G.to_dev(d["w"], "bf16"), G.to_dev(b, "bf16")
    # y over x, residual_out over residual: the usual in-place update
    y, ro = tn.layernorm_fwd_residual(x, r, w, bt, 1e-5, out=x, residual_out=r)
    torch.cuda.synchronize()
    assert y.data_ptr() == x.data_ptr() and ro.data_ptr() == r.data_ptr()
    assert np.array_equal(G.to_host(x, "bf16"), ref[0]) and np.array_equal(G.to_host(r, "bf16"), ref[1])


def test_ln_rejects_bad_arguments():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=G.DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=G.DEV)
    with pytest.raises(tn.RMSNormError):
        tn.layernorm_fwd(x, w, None, 0.0)  # eps must be positive
    with pytest.raises(tn.RMSNormError):
        tn.layernorm_fwd(x, w.half(), None, 1e-5)  # float16 parameters for bfloat16 x
    with pytest.raises(ValueError):
        tn.layernorm_fwd(x, w, w.float(), 1e-5)  # weight and bias formats differ
    buf = torch.zeros(4 * 64 + 8, dtype=torch.bfloat16, device=G.DEV)
    with pytest.raises(tn.RMSNormError):
        tn.layernorm_fwd(buf[:256].view(4, 64), w, None, 1e-5, out=buf[8:264].view(4, 64))


def test_ln_empty_batch():
    x = torch.empty((0, 512), dtype=torch.float32, device=G.DEV)
    y = tn.layernorm_fwd(x, None, None, 1e-5)
    torch.cuda.synchronize()
    assert y.shape == (0, 512)


def test_ln_guard_regions_untouched():
    M, H = 33, 1000
    d = G.inputs(49, M, H, "f32", residual=True)
    n = M * H
    yb = torch.full((n + 128,), 7.0, dtype=torch.float32, device=G.DEV)
    rb = torch.full((n + 128,), 7.0, dtype=torch.float32, device=G.DEV)
    tn.layernorm_fwd_residual(G.to_dev(d["x"], "f32"), G.to_dev(d["r"], "f32"), G.to_dev(d["w"], "f32"), None, 1e-5,
                              out=yb[64:64 + n].view(M, H), residual_out=rb[64:64 + n].view(M, H))
    torch.cuda.synchronize()
    for t in (yb, rb):
        assert torch.all(t[:64] == 7.0) and torch.all(t[64 + n:] == 7.0)


@pytest.mark.parametrize("dtype,H,M", [("bf16", 4096, 8195), ("f32", 4096, 8195), ("bf16", 4097, 16389)])
def test_ln_rows_walked_in_pairs(dtype, H, M):
    """LayerNorm without the residual whose weight and bias take 16 KiB or
    more, on at least 32 row groups per CU, has each row group walk 2 rows
    (an odd number of row groups leaves the last workgroup one row): parity
    with the oracle over the whole call and, on the 16-byte grid, the same
    bits as the same tile on one row per row group (a forced geometry never
    walks)."""
    print(f"[gpu] ln walked {dtype} M={M} H={H}", flush=True)
    d = G.inputs(6100 + H, M, H, dtype)
    b = bias_of(6100 + H, H, dtype)
    y, _, mean, rstd = run_ln(d["x"], None, d["w"], b, 1e-5, dtype)
    G.assert_ok(*G.ln_vs_oracle(d["x"], None, d["w"], b, y, None, mean, rstd, 1e-5, dtype,
                                name=f"ln walked {dtype} H={H}"))
    if H % 8 == 0:
        t = tn.tile("layernorm", H, dtype, off_grid=False)
        tn.set_geometry("fwd", t["vpt"], t["wpr"], t["rpw"], 0)
        try:
            y1, _, mean1, rstd1 = run_ln(d["x"], None, d["w"], b, 1e-5, dtype)
        finally:
            tn.set_geometry("fwd")
        assert np.array_equal(y, y1) and np.array_equal(mean, mean1) and np.array_equal(rstd, rstd1)
