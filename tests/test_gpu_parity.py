"""GPU parity: the HIP library, called through its C ABI (via the Python
binding), against the float64 oracle on the same seeded inputs.

Full-size workloads are compared element by element (the oracle handles them
in row chunks).  Smaller cases cover the kernels' other paths: ragged and
tiny H, unaligned rows (16-byte vectors at the row offset, or single elements when forced),
strided rows, the two-pass path and the grid-stride loop (forced through the
tuning hook), aliasing of outputs with inputs, guard regions around outputs,
determinism and the method's exact invariants.
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


@pytest.fixture(autouse=True)
def _default_geometry():
    tn.set_geometry("fwd")
    tn.set_geometry("bwd")
    tn.set_streaming(-1)
    yield
    tn.set_geometry("fwd")
    tn.set_geometry("bwd")
    tn.set_streaming(-1)


def run_fwd(x, w, eps, dtype, wdtype=None):
    xd = G.to_dev(x, dtype)
    wd = None if w is None else G.to_dev(w, wdtype or dtype)
    y, rr = tn.rmsnorm_fwd(xd, wd, eps, return_rrms=True)
    torch.cuda.synchronize()
    return G.to_host(y, dtype), rr.cpu().numpy()


def run_residual(x, r, w, eps, dtype, wdtype=None):
    xd, rd = G.to_dev(x, dtype), G.to_dev(r, dtype)
    wd = None if w is None else G.to_dev(w, wdtype or dtype)
    y, ro, rr = tn.rmsnorm_fwd_residual(xd, rd, wd, eps, return_rrms=True)
    torch.cuda.synchronize()
    return G.to_host(y, dtype), G.to_host(ro, dtype), rr.cpu().numpy()


def run_bwd(dy, x, w, rrms32, dtype, wdtype=None):
    dyd, xd = G.to_dev(dy, dtype), G.to_dev(x, dtype)
    wd = None if w is None else G.to_dev(w, wdtype or dtype)
    dx, dw = tn.rmsnorm_bwd(dyd, xd, wd, torch.from_numpy(rrms32).to(G.DEV))
    torch.cuda.synchronize()
    return G.to_host(dx, dtype), (None if dw is None else dw.cpu().numpy())


def oracle_rrms32(x, w, eps, dtype, wdtype=None, chunk=2048):
    """Per-row rrms from the oracle, rounded to float32 (the saved statistic)."""
    out = np.empty(x.shape[0], dtype=np.float32)
    for r0 in range(0, x.shape[0], chunk):
        _, r = oracle.fwd(x[r0:r0 + chunk], w, G.eps32(eps), dtype, wdtype)
        out[r0:r0 + chunk] = r.astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# the named workloads, full size
# ---------------------------------------------------------------------------

# fwd_bf16_8192x4097: rows of 8194 bytes, the forward for rows off the grid at full
# size (with streaming accesses, as bench.py times it)
@pytest.mark.parametrize("name", ["fwd_f32_64x512", "fwd_bf16_8192x4096", "fwd_bf16_8192x4097"])
def test_workload_fwd(name):
    d = synthetic.make_inputs(name)
    print(f"[gpu] {name}", flush=True)
    y, rr = run_fwd(d["x"], d["w"], d["eps"], d["dtype"], d["wdtype"])
    G.assert_ok(*G.fwd_vs_oracle(d["x"], d["w"], y, rr, d["eps"], d["dtype"], d["wdtype"], name=name), record=name)


@pytest.mark.parametrize("name", ["fwd_bf16_32768x2048", "fwd_f16_32768x2048_outliers"])
@pytest.mark.parametrize("weighted", [True, False], ids=["weight", "weightless"])
def test_workload_fwd_mix(name, weighted):
    d = synthetic.make_inputs(name)
    w = d["w"] if weighted else None
    print(f"[gpu] {name} weighted={weighted}", flush=True)
    y, rr = run_fwd(d["x"], w, d["eps"], d["dtype"], d["wdtype"])
    tag = name if weighted else name + "_noweight"
    G.assert_ok(*G.fwd_vs_oracle(d["x"], w, y, rr, d["eps"], d["dtype"], d["wdtype"], name=tag), record=tag)
    if d["dtype"] == "f16":
        # squares of the +-200..300 outliers exceed the float16 range; the
        # outputs stay finite because the sums are float32
        assert np.isfinite(y.astype(np.float32)).all()


def test_workload_fwd_residual():
    name = "fwd_residual_bf16_16384x8192"
    d = synthetic.make_inputs(name)
    print(f"[gpu] {name}", flush=True)
    y, ro, rr = run_residual(d["x"], d["r"], d["w"], d["eps"], d["dtype"], d["wdtype"])
    G.assert_ok(*G.residual_vs_oracle(d["x"], d["r"], d["w"], y, ro, rr, d["eps"], d["dtype"], d["wdtype"],
                                      name=name), record=name)


# bwd_bf16_8192x4097: the backward on rows off the 16-byte grid at full size
@pytest.mark.parametrize("name", ["bwd_bf16_8192x6144", "bwd_bf16_8192x4097"])
def test_workload_bwd(name):
    d = synthetic.make_inputs(name)
    print(f"[gpu] {name}", flush=True)
    rr = oracle_rrms32(d["x"], d["w"], d["eps"], d["dtype"])
    dx, dw = run_bwd(d["dy"], d["x"], d["w"], rr, d["dtype"])
    rep_dx, rep_dw = G.bwd_vs_oracle(d["dy"], d["x"], d["w"], rr, dx, dw, d["dtype"], name=name)
    G.assert_ok(rep_dx, rep_dw, record=name)
    # the cancellation floor judges only the few elements whose two terms
    # nearly cancel: at most 1e-4 of them (a rough count from the size of
    # float32 rounding against the terms gives 10-100 of the 5e7)
    assert rep_dx.floor_used <= 1e-4 * rep_dx.n, rep_dx
    # columns whose sum does not cancel meet the pure relative bound
    assert rep_dw.wc_cols > 0 and rep_dw.wc_max_rel <= 1e-3, rep_dw
    if name == "bwd_bf16_8192x6144":
        # here every column, cancelling or not, meets it too (max 1.6e-4);
        # at H = 4097 one strongly cancelling column is 1.2e-3 off, inside
        # the cancellation floor
        assert rep_dw.max_rel <= 1e-3, rep_dw


def test_workload_bwd_chained_with_gpu_rrms():
    """The GPU forward's own rrms feeds the GPU backward; the oracle backward
    gets the oracle forward's rrms rounded to float32 (the two differ by at
    most a float32 rounding, far below the outputs' tolerance)."""
    name = "bwd_bf16_8192x6144"
    d = synthetic.make_inputs(name, rows=2048)
    _, rr = run_fwd(d["x"], d["w"], d["eps"], d["dtype"])
    dx, dw = run_bwd(d["dy"], d["x"], d["w"], rr.astype(np.float32), d["dtype"])
    ro = oracle_rrms32(d["x"], d["w"], d["eps"], d["dtype"])
    G.assert_ok(*G.bwd_vs_oracle(d["dy"], d["x"], d["w"], ro, dx, dw, d["dtype"], name=name + " chained"))


# ---------------------------------------------------------------------------
# shapes: ragged, tiny and long rows, every format
# ---------------------------------------------------------------------------

# 16384 takes a tile capped below 16 waves per row (3 x 11 in 16 bits, 6 x 11
# for the plain float32 forward), and so does 8192 in float32 (3 x 11);
# 32768 and 65536 (32767 and 65535 off the grid) are the longest 16-bit rows
# the fused residual and the plain forward hold in registers
EDGE_H = [1, 3, 7, 8, 63, 64, 65, 127, 511, 512, 513, 1000, 2047, 2049, 2056, 3072, 3584, 4097, 4104, 5120, 6144,
          8191, 8192, 12288,
          16384, 16385, 32767, 32768, 65535, 65536]


def _rows_for(H):
    return 257 if H <= 8192 else 5


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("H", EDGE_H)
def test_edge_shapes_all_paths(dtype, H):
    M = _rows_for(H)
    d = G.inputs(1000 + H, M, H, dtype, residual=True, dy=True)
    x, w, r, dy = d["x"], d["w"], d["r"], d["dy"]
    print(f"[gpu] edge {dtype} M={M} H={H}", flush=True)
    y, rr = run_fwd(x, w, 1e-5, dtype)
    reps = list(G.fwd_vs_oracle(x, w, y, rr, 1e-5, dtype, name=f"fwd {dtype} H={H}"))
    y2, ro, rr2 = run_residual(x, r, w, 1e-6, dtype)
    reps += list(G.residual_vs_oracle(x, r, w, y2, ro, rr2, 1e-6, dtype, name=f"res {dtype} H={H}"))
    r32 = oracle_rrms32(x, w, 1e-5, dtype)
    dx, dw = run_bwd(dy, x, w, r32, dtype)
    reps += list(G.bwd_vs_oracle(dy, x, w, r32, dx, dw, dtype, name=f"bwd {dtype} H={H}"))
    G.assert_ok(*reps)


@pytest.mark.parametrize("M", [1, 2, 255, 257])
def test_row_counts(M):
    H = 4096
    d = G.inputs(7 + M, M, H, "bf16", residual=True, dy=True)
    y, rr = run_fwd(d["x"], d["w"], 1e-5, "bf16")
    reps = list(G.fwd_vs_oracle(d["x"], d["w"], y, rr, 1e-5, "bf16"))
    r32 = oracle_rrms32(d["x"], d["w"], 1e-5, "bf16")
    dx, dw = run_bwd(d["dy"], d["x"], d["w"], r32, "bf16")
    reps += list(G.bwd_vs_oracle(d["dy"], d["x"], d["w"], r32, dx, dw, "bf16"))
    G.assert_ok(*reps)


def test_page_test_shapes():
    """Shapes the pages test with: (1,1024,2048), (2,1024,2048), (2,4096,3072)
    in float16 with a weight of ones, and (4,4096,4096) in bfloat16."""
    import json
    import os
    spec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_cases.json")))
    for case in spec["fwd_cases"]:
        shape, dtype = tuple(case["shape"]), case["dtype"]
        M, H = int(np.prod(shape[:-1])), shape[-1]
        x = synthetic.normal_tensor(case["seed"], synthetic.STREAM_X, (M, H), dtype)
        w = synthetic.encode(np.ones(H), dtype) if case["weight"] == "ones" else \
            synthetic.normal_tensor(case["seed"], synthetic.STREAM_W, (H,), dtype, 1.0, 0.1)
        y, rr = run_fwd(x, w, case["eps"], dtype)
        G.assert_ok(*G.fwd_vs_oracle(x, w, y, rr, case["eps"], dtype, name=f"page {shape} {dtype}"))


def test_float32_weight_with_16bit_x():
    for dtype in ("bf16", "f16"):
        d = G.inputs(31, 300, 4096, dtype, wdtype="f32", residual=True, dy=True)
        y, rr = run_fwd(d["x"], d["w"], 1e-5, dtype, "f32")
        reps = list(G.fwd_vs_oracle(d["x"], d["w"], y, rr, 1e-5, dtype, "f32"))
        y2, ro, rr2 = run_residual(d["x"], d["r"], d["w"], 1e-5, dtype, "f32")
        reps += list(G.residual_vs_oracle(d["x"], d["r"], d["w"], y2, ro, rr2, 1e-5, dtype, "f32"))
        r32 = oracle_rrms32(d["x"], d["w"], 1e-5, dtype, "f32")
        dx, dw = run_bwd(d["dy"], d["x"], d["w"], r32, dtype, "f32")
        reps += list(G.bwd_vs_oracle(d["dy"], d["x"], d["w"], r32, dx, dw, dtype, "f32"))
        G.assert_ok(*reps)


# ---------------------------------------------------------------------------
# forced geometries: multi-row workgroups, grid-stride loop, two passes
# ---------------------------------------------------------------------------

FWD_GEOMS = [
    (1, 8, 1, 0), (2, 4, 1, 0), (4, 2, 2, 0), (8, 1, 4, 0), (8, 1, 2, 0), (2, 4, 2, 0),
    (2, 4, 1, 7),      # 7 workgroups walk 300 rows grid-stride (LDS parity reuse)
    (8, 1, 4, 5),      # one wave per row, 4 rows per workgroup, grid-stride
    (4, 1, 1, 0),      # 256 vectors per chunk < 512: two passes
    (4, 1, 2, 3),      # two passes inside a grid-stride loop
]


@pytest.mark.parametrize("stream", [0, 1], ids=["cached", "streaming"])
@pytest.mark.parametrize("geom", FWD_GEOMS, ids=[str(g) for g in FWD_GEOMS])
def test_forced_fwd_geometry(geom, stream):
    M, H = 300, 4096
    d = G.inputs(55, M, H, "bf16", residual=True)
    tn.set_geometry("fwd", *geom)
    tn.set_streaming(stream)
    y, rr = run_fwd(d["x"], d["w"], 1e-5, "bf16")
    reps = list(G.fwd_vs_oracle(d["x"], d["w"], y, rr, 1e-5, "bf16", name=f"fwd {geom}"))
    y2, ro, rr2 = run_residual(d["x"], d["r"], d["w"], 1e-5, "bf16")
    reps += list(G.residual_vs_oracle(d["x"], d["r"], d["w"], y2, ro, rr2, 1e-5, "bf16", name=f"res {geom}"))
    G.assert_ok(*reps)


# (vpt, wpr, P, row order: 0 default, 1 interleaved, 2 contiguous blocks)
BWD_GEOMS = [(1, 8, 0, 0), (2, 4, 0, 0), (4, 2, 0, 0), (2, 4, 1, 0), (2, 4, 7, 1), (2, 4, 7, 2), (2, 4, 300, 0),
             (1, 8, 37, 2), (4, 1, 16, 1), (4, 1, 16, 2), (4, 2, 3, 2), (1, 8, 1000, 1)]


@pytest.mark.parametrize("stream", [0, 1], ids=["cached", "streaming"])
@pytest.mark.parametrize("geom", BWD_GEOMS, ids=[str(g) for g in BWD_GEOMS])
def test_forced_bwd_geometry(geom, stream):
    M, H = 300, 4096
    d = G.inputs(56, M, H, "bf16", dy=True)
    r32 = oracle_rrms32(d["x"], d["w"], 1e-6, "bf16")
    tn.set_geometry("bwd", geom[0], geom[1], geom[2], geom[3])
    tn.set_streaming(stream)
    dx, dw = run_bwd(d["dy"], d["x"], d["w"], r32, "bf16")
    G.assert_ok(*G.bwd_vs_oracle(d["dy"], d["x"], d["w"], r32, dx, dw, "bf16", name=f"bwd {geom}"))


def test_forced_geometry_rejected_when_it_cannot_fit():
    tn.set_geometry("fwd", 3, 1, 1, 0)  # 192 vectors < 512 and vpt != 4: no two-pass tile
    d = G.inputs(57, 4, 4096, "bf16")
    with pytest.raises(tn.RMSNormError) as e:
        run_fwd(d["x"], d["w"], 1e-5, "bf16")
    assert e.value.status == 1


# ---------------------------------------------------------------------------
# layout: strides, alignment, aliasing, guard regions
# ---------------------------------------------------------------------------

def test_aligned_padding_is_bit_identical():
    M, H, pad = 64, 4096, 64  # pad keeps 16-byte alignment of every row
    d = G.inputs(61, M, H, "bf16", residual=True, dy=True)
    base = G.to_dev(d["x"], "bf16")
    wide = torch.zeros((M, H + pad), dtype=torch.bfloat16, device=G.DEV)
    wide[:, :H] = base
    y1 = tn.rmsnorm_fwd(base, G.to_dev(d["w"], "bf16"), 1e-5)
    y2 = tn.rmsnorm_fwd(wide[:, :H], G.to_dev(d["w"], "bf16"), 1e-5)
    out_wide = torch.zeros_like(wide)
    y3 = tn.rmsnorm_fwd(base, G.to_dev(d["w"], "bf16"), 1e-5, out=out_wide[:, :H])
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    assert torch.count_nonzero(out_wide[:, H:].view(torch.int16)) == 0


@pytest.mark.parametrize("stream", [0, 1], ids=["cached", "streaming"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_misaligned_rows(dtype, stream):
    tn.set_streaming(stream)
    M, H = 33, 4096
    d = G.inputs(62, M, H, dtype, residual=True, dy=True)
    for pad, offset in ((1, 0), (0, 1), (3, 1)):
        buf = torch.zeros(offset + M * (H + pad), dtype=G.torch_dtype(dtype), device=G.DEV)
        view = buf[offset:].view(M, H + pad)[:, :H]
        view.copy_(G.to_dev(d["x"], dtype))
        wd = G.to_dev(d["w"], dtype)
        y, rr = tn.rmsnorm_fwd(view, wd, 1e-5, return_rrms=True)
        rview = torch.zeros_like(buf)[offset:].view(M, H + pad)[:, :H]
        rview.copy_(G.to_dev(d["r"], dtype))
        y2, ro, rr2 = tn.rmsnorm_fwd_residual(view, rview, wd, 1e-5, return_rrms=True)
        dyv = torch.zeros_like(buf)[offset:].view(M, H + pad)[:, :H]
        dyv.copy_(G.to_dev(d["dy"], dtype))
        r32 = oracle_rrms32(d["x"], d["w"], 1e-5, dtype)
        dx, dw = tn.rmsnorm_bwd(dyv, view, wd, torch.from_numpy(r32).to(G.DEV))
        torch.cuda.synchronize()
        reps = list(G.fwd_vs_oracle(d["x"], d["w"], G.to_host(y, dtype), rr.cpu().numpy(), 1e-5, dtype,
                                    name=f"fwd pad={pad} off={offset}"))
        reps += list(G.residual_vs_oracle(d["x"], d["r"], d["w"], G.to_host(y2, dtype), G.to_host(ro, dtype),
                                          rr2.cpu().numpy(), 1e-5, dtype, name=f"res pad={pad} off={offset}"))
        reps += list(G.bwd_vs_oracle(d["dy"], d["x"], d["w"], r32, G.to_host(dx, dtype), dw.cpu().numpy(), dtype,
                                     name=f"bwd pad={pad} off={offset}"))
        G.assert_ok(*reps)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_misaligned_views_same_bits_at_any_offset(dtype):
    """Rows off the 16-byte grid take 16-byte vectors at each row's byte
    offset on a vector tile that depends on H only, so every layout of the same rows -- any element offset of x,
    the residual and the outputs, any row pitch -- gives the same bits, at
    parity with the oracle, for the plain and the fused residual forward;
    the elements around the output rows (pads, the buffer's head and tail)
    are never written."""
    M, H = 37, 4096
    d = G.inputs(66, M, H, dtype, residual=True)
    xd, rd, wd = G.to_dev(d["x"], dtype), G.to_dev(d["r"], dtype), G.to_dev(d["w"], dtype)
    bits = (lambda t: t.view(torch.int32)) if dtype == "f32" else (lambda t: t.view(torch.int16))
    first = None
    for pad, xoff, yoff in ((1, 0, 1), (0, 1, 3), (3, 1, 0), (5, 7, 2), (8, 3, 5)):
        print(f"[gpu] off-grid views {dtype} pad={pad} xoff={xoff} yoff={yoff}", flush=True)
        _, xv = G.sentinel_view(M, H, pad, xoff, dtype, 0.0)
        _, rv = G.sentinel_view(M, H, pad, xoff + 1, dtype, 0.0)
        xv.copy_(xd)
        rv.copy_(rd)
        ybuf, yv = G.sentinel_view(M, H, pad + 2, yoff, dtype, -77.0)
        robuf, rov = G.sentinel_view(M, H, pad, yoff + 1, dtype, -77.0)
        _, rr = tn.rmsnorm_fwd(xv, wd, 1e-5, out=yv, return_rrms=True)
        y2, _, rr2 = tn.rmsnorm_fwd_residual(xv, rv, wd, 1e-6, residual_out=rov, return_rrms=True)
        torch.cuda.synchronize()
        got = (bits(yv.contiguous()), rr, bits(y2), bits(rov.contiguous()), rr2)
        assert G.untouched(ybuf, yv, -77.0) and G.untouched(robuf, rov, -77.0), (pad, xoff, yoff)
        if first is None:
            first = got
            reps = list(G.fwd_vs_oracle(d["x"], d["w"], G.to_host(yv.contiguous(), dtype), rr.cpu().numpy(), 1e-5,
                                        dtype, name=f"fwd {dtype} off-grid view"))
            reps += list(G.residual_vs_oracle(d["x"], d["r"], d["w"], G.to_host(y2, dtype),
                                              G.to_host(rov.contiguous(), dtype), rr2.cpu().numpy(), 1e-6, dtype,
                                              name=f"res {dtype} off-grid view"))
            G.assert_ok(*reps)
        else:
            for a, b in zip(got, first):
                assert torch.equal(a, b), (pad, xoff, yoff)


@pytest.mark.parametrize("dtype,wdtype", [("bf16", "bf16"), ("f16", "f32"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("H", [5, 13, 63, 129, 1001, 4097, 6143, 8190, 12289, 16385, 30001, 32769, 70001])
def test_ragged_rows_parity_and_pads(dtype, wdtype, H):
    """Ragged H (rows off the 16-byte grid by their length) in padded
    layouts: parity with the oracle for the plain and fused residual forward,
    and the pads between output rows never written; the forced element-wise
    tile gives results at parity too.  16-bit rows with a 16-bit weight stay
    in registers to 32767 columns (fused residual) and 65535 (plain); in
    float32 or with a float32 weight the fused residual takes two passes from
    16385 and the plain forward from 32769."""
    M = 41 if H <= 8192 else 9
    d = G.inputs(67 + H, M, H, dtype, wdtype=wdtype, residual=True)
    wd = G.to_dev(d["w"], wdtype)
    xd, rd = G.to_dev(d["x"], dtype), G.to_dev(d["r"], dtype)
    print(f"[gpu] ragged {dtype}/{wdtype} H={H}", flush=True)
    ybuf, yv = G.sentinel_view(M, H, 3, 1, dtype, -77.0)
    robuf, rov = G.sentinel_view(M, H, 1, 2, dtype, -77.0)
    _, rr = tn.rmsnorm_fwd(xd, wd, 1e-5, out=yv, return_rrms=True)
    y2, _, rr2 = tn.rmsnorm_fwd_residual(xd, rd, wd, 1e-6, residual_out=rov, return_rrms=True)
    torch.cuda.synchronize()
    reps = list(G.fwd_vs_oracle(d["x"], d["w"], G.to_host(yv.contiguous(), dtype), rr.cpu().numpy(), 1e-5, dtype,
                                wdtype=wdtype, name=f"fwd {dtype} H={H}"))
    reps += list(G.residual_vs_oracle(d["x"], d["r"], d["w"], G.to_host(y2, dtype), G.to_host(rov.contiguous(), dtype),
                                      rr2.cpu().numpy(), 1e-6, dtype, wdtype=wdtype, name=f"res {dtype} H={H}"))
    G.assert_ok(*reps)
    assert G.untouched(ybuf, yv, -77.0) and G.untouched(robuf, rov, -77.0)
    # the element-wise tile, forced: a resident tile of single elements
    vpt = 8
    wpr = max(1, -(-H // (64 * vpt)))
    if wpr <= 16:
        tn.set_geometry("fwd", vpt, wpr, 1, 0)
        try:
            y3, rr3 = tn.rmsnorm_fwd(xd, wd, 1e-5, return_rrms=True)
            torch.cuda.synchronize()
        finally:
            tn.set_geometry("fwd", 0, 0, 0, 0)
        G.assert_ok(*G.fwd_vs_oracle(d["x"], d["w"], G.to_host(y3, dtype), rr3.cpu().numpy(), 1e-5, dtype,
                                     wdtype=wdtype, name=f"fwd element tile {dtype} H={H}"))


@pytest.mark.parametrize("H", [6144, 4097, 70001], ids=["aligned", "off_grid", "off_grid_two_pass"])
def test_in_place_outputs(H):
    """y written over x, residual_out over the residual, dx over dy.  At
    H = 4097 (bf16) the rows are off the 16-byte grid and take 16-byte
    vectors at the row's byte offset on a 2-wave row (6 vectors per thread):
    the row's last vector, 512, is a window over the row's last 16 bytes,
    held by thread 0 (wave 0), and its leading 7 columns are also vector
    511's, held by thread 127 (wave 1).  Only the order of every aligned-away
    store after all of the row's loads keeps the in-place result equal to
    the out-of-place one there.  At H = 70001 every call takes two passes
    over rows off the grid, where the lane of the last partial vector writes
    only its own columns."""
    M = 200 if H <= 8192 else 24
    d = G.inputs(63, M, H, "bf16", residual=True, dy=True)
    wd = G.to_dev(d["w"], "bf16")
    ref_y = tn.rmsnorm_fwd(G.to_dev(d["x"], "bf16"), wd, 1e-5)
    x = G.to_dev(d["x"], "bf16")
    tn.rmsnorm_fwd(x, wd, 1e-5, out=x)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), ref_y.view(torch.int16))
    # residual stream updated in place, y written over x
    ref = tn.rmsnorm_fwd_residual(G.to_dev(d["x"], "bf16"), G.to_dev(d["r"], "bf16"), wd, 1e-5)
    x, r = G.to_dev(d["x"], "bf16"), G.to_dev(d["r"], "bf16")
    tn.rmsnorm_fwd_residual(x, r, wd, 1e-5, out=x, residual_out=r)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), ref[0].view(torch.int16))
    assert torch.equal(r.view(torch.int16), ref[1].view(torch.int16))
    # dx written over dy
    r32 = torch.from_numpy(oracle_rrms32(d["x"], d["w"], 1e-5, "bf16")).to(G.DEV)
    dref, wref = tn.rmsnorm_bwd(G.to_dev(d["dy"], "bf16"), G.to_dev(d["x"], "bf16"), wd, r32)
    dy = G.to_dev(d["dy"], "bf16")
    _, dw = tn.rmsnorm_bwd(dy, G.to_dev(d["x"], "bf16"), wd, r32, dx=dy)
    torch.cuda.synchronize()
    assert torch.equal(dy.view(torch.int16), dref.view(torch.int16))
    assert torch.equal(dw, wref)


def test_in_place_two_pass():
    M, H = 40, 4096
    d = G.inputs(64, M, H, "bf16", residual=True)
    wd = G.to_dev(d["w"], "bf16")
    tn.set_geometry("fwd", 4, 1, 1, 0)  # two passes over 256-vector chunks
    ref = tn.rmsnorm_fwd_residual(G.to_dev(d["x"], "bf16"), G.to_dev(d["r"], "bf16"), wd, 1e-5)
    x, r = G.to_dev(d["x"], "bf16"), G.to_dev(d["r"], "bf16")
    tn.rmsnorm_fwd_residual(x, r, wd, 1e-5, out=x, residual_out=r)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), ref[0].view(torch.int16))
    assert torch.equal(r.view(torch.int16), ref[1].view(torch.int16))


GUARD = 4096


def _guarded(shape, dtype, fill):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), fill, dtype=dtype, device=G.DEV)
    return buf, buf[GUARD:GUARD + n].view(*shape)


def test_guard_regions_untouched():
    for (M, H) in ((17, 4097), (33, 4096), (9, 65536), (5, 3)):
        d = G.inputs(65 + H, M, H, "bf16", residual=True, dy=True)
        xd, rd, dyd, wd = (G.to_dev(d["x"], "bf16"), G.to_dev(d["r"], "bf16"), G.to_dev(d["dy"], "bf16"),
                           G.to_dev(d["w"], "bf16"))
        sentinel = -1234.0
        ybuf, y = _guarded((M, H), torch.bfloat16, sentinel)
        robuf, ro = _guarded((M, H), torch.bfloat16, sentinel)
        rrbuf, rr = _guarded((M,), torch.float32, sentinel)
        dxbuf, dx = _guarded((M, H), torch.bfloat16, sentinel)
        dwbuf, dw = _guarded((H,), torch.float32, sentinel)
        tn.rmsnorm_fwd(xd, wd, 1e-5, out=y, rrms=rr)
        tn.rmsnorm_fwd_residual(xd, rd, wd, 1e-5, out=torch.empty_like(xd), residual_out=ro)
        tn.rmsnorm_bwd(dyd, xd, wd, rr, dx=dx, dw=dw)
        torch.cuda.synchronize()
        for buf in (ybuf, robuf, rrbuf, dxbuf, dwbuf):
            head, tail = buf[:GUARD], buf[-GUARD:]
            assert torch.all(head == sentinel) and torch.all(tail == sentinel), (M, H)


# ---------------------------------------------------------------------------
# determinism and exact invariants
# ---------------------------------------------------------------------------

def test_streaming_does_not_change_bits():
    d = synthetic.make_inputs("bwd_bf16_8192x6144", rows=2048)
    xd, dyd, wd = G.to_dev(d["x"], "bf16"), G.to_dev(d["dy"], "bf16"), G.to_dev(d["w"], "bf16")
    outs = []
    for mode in (0, 1):
        tn.set_streaming(mode)
        y, rr = tn.rmsnorm_fwd(xd, wd, 1e-6, return_rrms=True)
        y2, ro = tn.rmsnorm_fwd_residual(xd, dyd, wd, 1e-6)
        dx, dw = tn.rmsnorm_bwd(dyd, xd, wd, rr)
        torch.cuda.synchronize()
        outs.append([t.view(-1).view(torch.uint8).clone() for t in (y, rr, y2, ro, dx, dw)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_determinism():
    d = synthetic.make_inputs("bwd_bf16_8192x6144", rows=1024)
    xd, dyd, wd = G.to_dev(d["x"], "bf16"), G.to_dev(d["dy"], "bf16"), G.to_dev(d["w"], "bf16")
    a = tn.rmsnorm_fwd(xd, wd, 1e-6, return_rrms=True)
    b = tn.rmsnorm_fwd(xd, wd, 1e-6, return_rrms=True)
    c = tn.rmsnorm_bwd(dyd, xd, wd, a[1])
    e = tn.rmsnorm_bwd(dyd, xd, wd, a[1])
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])
    assert torch.equal(c[0].view(torch.int16), e[0].view(torch.int16)) and torch.equal(c[1], e[1])


@pytest.mark.parametrize("H,groups", [(512, 4), (3072, 1)])
def test_bwd_deep_prefetch_same_bits(H, groups):
    """bf16 rows on the grid whose one-vector tile leaves at most 6 waves per
    CU (H = 512: one wave per row, 4 workgroups per CU; H = 3072: 6 waves,
    one workgroup) keep three rows in flight per wave.  The same tile forced
    through the tuning hook, with the same number of workgroups, runs the
    kernel with two rows in flight: dx and dw keep their bits, and both are
    at parity with the oracle."""
    M = 4096
    d = G.inputs(73 + H, M, H, "bf16", dy=True)
    r32 = oracle_rrms32(d["x"], d["w"], 1e-5, "bf16")
    rr = torch.from_numpy(r32).to(G.DEV)
    xd, dyd, wd = G.to_dev(d["x"], "bf16"), G.to_dev(d["dy"], "bf16"), G.to_dev(d["w"], "bf16")
    t = tn.tile("bwd", H, "bf16", off_grid=False)
    assert (t["vec"], t["vpt"], t["mis"], t["multi_pass"]) == (8, 1, False, False)
    assert groups * t["wpr"] <= 6
    print(f"[gpu] deep prefetch bf16 H={H}", flush=True)
    dx, dw = tn.rmsnorm_bwd(dyd, xd, wd, rr)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tn.set_geometry("bwd", 1, t["wpr"], groups * cus, 1)
    try:
        dx2, dw2 = tn.rmsnorm_bwd(dyd, xd, wd, rr)
        torch.cuda.synchronize()
    finally:
        tn.set_geometry("bwd")
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16)) and torch.equal(dw, dw2)
    G.assert_ok(*G.bwd_vs_oracle(d["dy"], d["x"], d["w"], r32, G.to_host(dx, "bf16"), dw.cpu().numpy(), "bf16",
                                 name=f"bwd deep bf16 H={H}"))


def test_weightless_equals_weight_of_ones():
    for dtype in ("bf16", "f16", "f32"):
        d = G.inputs(71, 128, 2048, dtype, xdist=(0.0, 2.0), residual=True)
        xd = G.to_dev(d["x"], dtype)
        ones = torch.ones(2048, dtype=G.torch_dtype(dtype), device=G.DEV)
        a = tn.rmsnorm_fwd(xd, None, 1e-6)
        b = tn.rmsnorm_fwd(xd, ones, 1e-6)
        torch.cuda.synchronize()
        assert torch.equal(a.view(-1).view(torch.uint8), b.view(-1).view(torch.uint8))


def test_zero_residual_equals_plain_forward():
    for dtype in ("bf16", "f16", "f32"):
        d = G.inputs(72, 100, 4096, dtype)
        xd, wd = G.to_dev(d["x"], dtype), G.to_dev(d["w"], dtype)
        y, rr = tn.rmsnorm_fwd(xd, wd, 1e-5, return_rrms=True)
        y2, ro, rr2 = tn.rmsnorm_fwd_residual(xd, torch.zeros_like(xd), wd, 1e-5, return_rrms=True)
        torch.cuda.synchronize()
        assert torch.equal(y.view(-1).view(torch.uint8), y2.view(-1).view(torch.uint8))
        assert torch.equal(ro.view(-1).view(torch.uint8), xd.view(-1).view(torch.uint8))
        assert torch.equal(rr, rr2)


def test_residual_symmetric_in_x_and_r():
    d = G.inputs(73, 64, 8192, "bf16", residual=True)
    xd, rd, wd = G.to_dev(d["x"], "bf16"), G.to_dev(d["r"], "bf16"), G.to_dev(d["w"], "bf16")
    a = tn.rmsnorm_fwd_residual(xd, rd, wd, 1e-5)
    b = tn.rmsnorm_fwd_residual(rd, xd, wd, 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))


def test_unit_rows_give_weight_exactly():
    # rows of +-1 with eps = 1e-5: y = +-w * 0.999995..., which rounds back to w in bf16
    H = 4096
    rng = np.random.default_rng(5)
    x = synthetic.encode(rng.choice([-1.0, 1.0], (16, H)), "bf16")
    w = synthetic.normal_tensor(74, synthetic.STREAM_W, (H,), "bf16", 1.0, 0.1)
    y, _ = run_fwd(x, w, 1e-5, "bf16")
    expect = synthetic.encode(synthetic.decode(x, "bf16") * synthetic.decode(w, "bf16")[None, :], "bf16")
    assert np.array_equal(y, expect)


def test_scale_law_with_tiny_eps():
    # eps = 1e-30 vanishes next to mean(x^2) in float32, so y(2^k x) = y(x)
    d = G.inputs(75, 64, 4096, "bf16")
    x = synthetic.decode(d["x"], "bf16")
    y1, _ = run_fwd(d["x"], d["w"], 1e-30, "bf16")
    for k in (-8, 3):
        y2, _ = run_fwd(synthetic.encode(x * 2.0 ** k, "bf16"), d["w"], 1e-30, "bf16")
        assert parity.ulp_distance16(y1, y2).max() <= 1


def test_weightless_mean_square():
    d = G.inputs(76, 256, 2048, "bf16", xdist=(0.0, 2.0))
    y, rr = run_fwd(d["x"], None, 1e-6, "bf16")
    yv = synthetic.decode(y, "bf16")
    ms = (yv ** 2).mean(axis=1) + 1e-6 * rr.astype(np.float64) ** 2
    assert np.all(np.abs(ms - 1.0) <= 2.0 ** -7)


def test_constant_and_zero_rows():
    H = 4096
    x = np.zeros((3, H), dtype=np.float32)
    x[0] = 0.75
    x[1] = -3.0
    y, rr = run_fwd(x, None, 1e-6, "f32")
    assert np.all(y[2] == 0.0)
    assert abs(rr[2] - 1000.0) <= 1e-5 * 1000.0
    for i, c in ((0, 0.75), (1, -3.0)):
        exp = c / np.sqrt(c * c + float(np.float32(1e-6)))
        assert np.all(np.abs(y[i] - exp) <= 1e-5 * abs(exp) + 1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_exhaustive_h1(dtype):
    """H = 1 over every finite value of the format: y = x / sqrt(x^2 + eps)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = synthetic.decode(bits if dtype == "bf16" else bits.view(np.float16), dtype)
    keep = np.isfinite(vals) & (np.abs(vals) < 2.0 ** 63)
    x = (bits[keep] if dtype == "bf16" else bits[keep].view(np.float16)).reshape(-1, 1)
    y, rr = run_fwd(x, None, 1e-6, dtype)
    G.assert_ok(*G.fwd_vs_oracle(x, None, y, rr, 1e-6, dtype, name=f"H=1 {dtype}"))


def test_empty_batch_is_a_no_op():
    xd = torch.empty((0, 4096), dtype=torch.bfloat16, device=G.DEV)
    y = tn.rmsnorm_fwd(xd, None, 1e-5)
    assert y.shape == (0, 4096)
    wd = torch.ones(4096, dtype=torch.bfloat16, device=G.DEV)
    dx, dw = tn.rmsnorm_bwd(xd, xd, wd, torch.empty(0, dtype=torch.float32, device=G.DEV))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw) == 0  # dw over zero rows is zero


@pytest.mark.parametrize("dtype,wdtype", [("bf16", "bf16"), ("f16", "f32"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("H", [1, 5, 13, 63, 129, 1001, 4096, 4097, 6143, 8190, 12289, 16385, 30001, 70001])
def test_bwd_rows_off_the_grid_views_and_pads(dtype, wdtype, H):
    """The backward on rows off the 16-byte grid (16-byte vectors read and
    written at each row's byte offset): dy, x, dres and dx each at their own
    element offset in padded buffers, so the four tensors' rows sit at
    different offsets within their 16-byte blocks.  Parity with the oracle for
    the plain and the residual backward, the pads and the buffers' heads and
    tails never written, dx written in place over dy and dh over dres with the
    same bits, and, for an H of whole vectors, the bits of the contiguous
    (aligned) run; the forced single-element tile is at parity too.  Rows
    longer than one tile (plain from 16385; residual from 16385 at 16 bits,
    from 8193 in float32) take two passes; beyond
    65536 columns their later chunks add into the workspace row at each row,
    and at 70001 the row's last partial vector lies in such a chunk."""
    M = 41 if H <= 8192 else 9
    d = G.inputs(68 + H, M, H, dtype, wdtype=wdtype, residual=True, dy=True)
    r32 = oracle_rrms32(d["x"], d["w"], 1e-5, dtype, wdtype)
    rr = torch.from_numpy(r32).to(G.DEV)
    wd = G.to_dev(d["w"], wdtype)
    print(f"[gpu] bwd off the grid {dtype}/{wdtype} H={H}", flush=True)
    _, dyv = G.sentinel_view(M, H, 1, 1, dtype, 0.0)
    _, xv = G.sentinel_view(M, H, 3, 2, dtype, 0.0)
    _, gv = G.sentinel_view(M, H, 2, 3, dtype, 0.0)
    dyv.copy_(G.to_dev(d["dy"], dtype))
    xv.copy_(G.to_dev(d["x"], dtype))
    gv.copy_(G.to_dev(d["r"], dtype))
    dxbuf, dxv = G.sentinel_view(M, H, 5, 5, dtype, -77.0)
    dhbuf, dhv = G.sentinel_view(M, H, 1, 0, dtype, -77.0)
    _, dw = tn.rmsnorm_bwd(dyv, xv, wd, rr, dx=dxv)
    _, dw2 = tn.rmsnorm_bwd_residual(dyv, xv, gv, wd, rr, dh=dhv)
    torch.cuda.synchronize()
    assert G.untouched(dxbuf, dxv, -77.0) and G.untouched(dhbuf, dhv, -77.0)
    reps = list(G.bwd_vs_oracle(d["dy"], d["x"], d["w"], r32, G.to_host(dxv.contiguous(), dtype), dw.cpu().numpy(),
                                dtype, wdtype=wdtype, name=f"bwd {dtype}/{wdtype} H={H}"))
    reps += list(G.bwd_residual_vs_oracle(d["dy"], d["x"], d["r"], d["w"], r32, G.to_host(dhv.contiguous(), dtype),
                                          dw2.cpu().numpy(), dtype, wdtype=wdtype, name=f"bwd_res {dtype} H={H}"))
    G.assert_ok(*reps)
    bits = (lambda t: t.contiguous().view(torch.int32)) if dtype == "f32" else \
        (lambda t: t.contiguous().view(torch.int16))
    if (H * (4 if dtype == "f32" else 2)) % 16 == 0:
        # whole vectors: the views run the aligned path's tile, so the bits
        # of the contiguous (aligned) run
        dxa, dwa = tn.rmsnorm_bwd(G.to_dev(d["dy"], dtype), G.to_dev(d["x"], dtype), wd, rr)
        torch.cuda.synchronize()
        assert torch.equal(bits(dxv), bits(dxa)) and torch.equal(dw, dwa)
    # in place over dy, and dh over dres: the same bits
    dh_in, _ = tn.rmsnorm_bwd_residual(dyv, xv, gv, wd, rr, dh=gv)
    dx_in, _ = tn.rmsnorm_bwd(dyv, xv, wd, rr, dx=dyv)
    torch.cuda.synchronize()
    assert dh_in.data_ptr() == gv.data_ptr() and torch.equal(bits(gv), bits(dhv))
    assert dx_in.data_ptr() == dyv.data_ptr() and torch.equal(bits(dyv), bits(dxv))
    # the single-element tile, forced (contiguous rows of a ragged H only:
    # rows on the grid keep the vector tile)
    wpr = max(1, -(-H // (64 * 8)))
    if wpr <= 16 and (H * (4 if dtype == "f32" else 2)) % 16:
        tn.set_geometry("bwd", 8, wpr, 0, 0)
        try:
            dx3, dw3 = tn.rmsnorm_bwd(G.to_dev(d["dy"], dtype), G.to_dev(d["x"], dtype), wd, rr)
            torch.cuda.synchronize()
        finally:
            tn.set_geometry("bwd")
        G.assert_ok(*G.bwd_vs_oracle(d["dy"], d["x"], d["w"], r32, G.to_host(dx3, dtype), dw3.cpu().numpy(), dtype,
                                     wdtype=wdtype, name=f"bwd element tile {dtype} H={H}"))


@pytest.mark.parametrize("dtype,wdtype", [("bf16", "bf16"), ("f16", "f32"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("H,M,off,pad", [(4097, 300, 1, 0), (4095, 41, 3, 0), (2049, 263, 1, 6), (1001, 5, 2, 1),
                                         (8, 64, 1, 0), (12, 33, 1, 3), (6143, 17, 1, 0), (4096, 90, 1, 0),
                                         (12289, 9, 1, 0)])
def test_bwd_rows_off_the_grid_shared_offset(dtype, wdtype, H, M, off, pad):
    """dy, x, dres and dx rows at one shared offset within their 16-byte
    chunks (the same element offset and row stride in every buffer), so the
    backward sets its vectors on memory's 16-byte grid: the row's first
    vector at the row start, the chunks in between aligned, the last one the
    window over the row's last 16 bytes.  Row lengths that touch one more
    chunk than vectors at the row offset (4095, 2049 + 6 pad, 12), rows of
    one vector (8), several hundred rows whose workgroup count is rounded down
    so that every row of a workgroup keeps one offset (300 rows of 4097).
    Parity with the oracle for the plain and the residual backward, pads and
    buffer ends never written; dx written over dy and over x, and dh over
    dres, give the same bits; and dx at another offset (vectors at the row
    offset) is at parity too."""
    d = G.inputs(91 + H + off, M, H, dtype, wdtype=wdtype, residual=True, dy=True)
    r32 = oracle_rrms32(d["x"], d["w"], 1e-5, dtype, wdtype)
    rr = torch.from_numpy(r32).to(G.DEV)
    wd = G.to_dev(d["w"], wdtype)
    es = 4 if dtype == "f32" else 2
    print(f"[gpu] bwd shared offset {dtype}/{wdtype} H={H} M={M} off={off} pad={pad}", flush=True)
    assert tn.tile("bwd", H, dtype, off_grid=True, shared_offset=True)["frame"] == \
        (not tn.tile("bwd", H, dtype, off_grid=True)["multi_pass"]
         and not tn.tile("bwd", H + (16 - es) // es, dtype, off_grid=True)["multi_pass"])

    def views():
        out = {}
        for key in ("dy", "x", "r"):
            _, v = G.sentinel_view(M, H, pad, off, dtype, 0.0)
            v.copy_(G.to_dev(d[key], dtype))
            out[key] = v
        return out

    v = views()
    dxbuf, dxv = G.sentinel_view(M, H, pad, off, dtype, -77.0)
    dhbuf, dhv = G.sentinel_view(M, H, pad, off, dtype, -77.0)
    _, dw = tn.rmsnorm_bwd(v["dy"], v["x"], wd, rr, dx=dxv)
    _, dw2 = tn.rmsnorm_bwd_residual(v["dy"], v["x"], v["r"], wd, rr, dh=dhv)
    torch.cuda.synchronize()
    assert G.untouched(dxbuf, dxv, -77.0) and G.untouched(dhbuf, dhv, -77.0)
    reps = list(G.bwd_vs_oracle(d["dy"], d["x"], d["w"], r32, G.to_host(dxv, dtype), dw.cpu().numpy(), dtype,
                                wdtype=wdtype, name=f"bwd frame {dtype}/{wdtype} H={H}"))
    reps += list(G.bwd_residual_vs_oracle(d["dy"], d["x"], d["r"], d["w"], r32, G.to_host(dhv, dtype),
                                          dw2.cpu().numpy(), dtype, wdtype=wdtype, name=f"bwd_res frame {dtype} H={H}"))
    G.assert_ok(*reps)
    bits = (lambda t: t.contiguous().view(torch.int32)) if dtype == "f32" else \
        (lambda t: t.contiguous().view(torch.int16))
    # in place (fresh inputs for each call): the same tile, the same bits
    _, dw_a = tn.rmsnorm_bwd(v["dy"], v["x"], wd, rr, dx=v["dy"])
    torch.cuda.synchronize()
    assert torch.equal(bits(v["dy"]), bits(dxv)) and torch.equal(dw_a, dw)
    v = views()
    _, dw_b = tn.rmsnorm_bwd_residual(v["dy"], v["x"], v["r"], wd, rr, dh=v["r"])
    torch.cuda.synchronize()
    assert torch.equal(bits(v["r"]), bits(dhv)) and torch.equal(dw_b, dw2)
    v = views()
    _, dw_c = tn.rmsnorm_bwd(v["dy"], v["x"], wd, rr, dx=v["x"])
    torch.cuda.synchronize()
    assert torch.equal(bits(v["x"]), bits(dxv)) and torch.equal(dw_c, dw)
    # dx one element further on: its rows sit at another offset, so the
    # vectors go to each row's offset instead
    v = views()
    _, dxo = G.sentinel_view(M, H, pad, off + 1, dtype, -77.0)
    _, dw_o = tn.rmsnorm_bwd(v["dy"], v["x"], wd, rr, dx=dxo)
    torch.cuda.synchronize()
    G.assert_ok(*G.bwd_vs_oracle(d["dy"], d["x"], d["w"], r32, G.to_host(dxo, dtype), dw_o.cpu().numpy(), dtype,
                                 wdtype=wdtype, name=f"bwd row offset {dtype}/{wdtype} H={H}"))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("H", [8, 15, 63, 64, 128, 255, 256, 257, 384, 511])
def test_fwd_short_rows_off_the_grid(dtype, H):
    """Rows under 1 KiB off the 16-byte grid (from 512 bytes: 16-byte vectors
    at each row's byte offset; shorter rows: the element-wise tile): x, the
    residual and the outputs at different element offsets in padded buffers,
    for the plain and fused residual forward -- parity with the oracle, the
    pads never written, in place over x and over the residual with the same
    bits, and, for an H of whole vectors from 512 bytes, the bits of the
    contiguous (aligned) run."""
    M = 300
    d = G.inputs(90 + H, M, H, dtype, residual=True)
    wd = G.to_dev(d["w"], dtype)
    print(f"[gpu] short rows off the grid {dtype} H={H}", flush=True)
    _, xv = G.sentinel_view(M, H, 1, 1, dtype, 0.0)
    _, rv = G.sentinel_view(M, H, 2, 3, dtype, 0.0)
    xv.copy_(G.to_dev(d["x"], dtype))
    rv.copy_(G.to_dev(d["r"], dtype))
    ybuf, yv = G.sentinel_view(M, H, 3, 2, dtype, -77.0)
    robuf, rov = G.sentinel_view(M, H, 1, 5, dtype, -77.0)
    _, rr = tn.rmsnorm_fwd(xv, wd, 1e-5, out=yv, return_rrms=True)
    y2, _, rr2 = tn.rmsnorm_fwd_residual(xv, rv, wd, 1e-6, residual_out=rov, return_rrms=True)
    torch.cuda.synchronize()
    assert G.untouched(ybuf, yv, -77.0) and G.untouched(robuf, rov, -77.0)
    reps = list(G.fwd_vs_oracle(d["x"], d["w"], G.to_host(yv.contiguous(), dtype), rr.cpu().numpy(), 1e-5, dtype,
                                name=f"fwd {dtype} H={H}"))
    reps += list(G.residual_vs_oracle(d["x"], d["r"], d["w"], G.to_host(y2, dtype), G.to_host(rov.contiguous(), dtype),
                                      rr2.cpu().numpy(), 1e-6, dtype, name=f"res {dtype} H={H}"))
    G.assert_ok(*reps)
    bits = (lambda t: t.contiguous().view(torch.int32)) if dtype == "f32" else \
        (lambda t: t.contiguous().view(torch.int16))
    row_bytes = H * (4 if dtype == "f32" else 2)
    if row_bytes % 16 == 0 and 512 <= row_bytes < 1024:
        ya = tn.rmsnorm_fwd(G.to_dev(d["x"], dtype), wd, 1e-5)
        torch.cuda.synchronize()
        assert torch.equal(bits(yv), bits(ya))
    # in place: y over x, residual_out over the residual
    y_first, ro_first = bits(yv).clone(), bits(rov).clone()
    y3, _ = tn.rmsnorm_fwd_residual(xv, rv, wd, 1e-6, residual_out=rv)
    torch.cuda.synchronize()
    assert torch.equal(bits(rv), ro_first) and torch.equal(bits(y3), bits(y2))
    tn.rmsnorm_fwd(xv, wd, 1e-5, out=xv)
    torch.cuda.synchronize()
    assert torch.equal(bits(xv), y_first)
