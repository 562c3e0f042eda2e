"""GPU parity of the AdaLN-RMSNorm entry point against the float64 oracle:
full-size DiT-style workloads with per-batch and per-token conditioning,
ragged shapes in every format, float32 parameters, forced kernel paths, and
the exact special cases (zero conditioning, scale = -1)."""

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


def run(x, w, sc, sh, B, S, eps, dtype, pdtype=None, per_batch=True):
    """x (B*S, H) host storage; sc/sh (B, H) when per_batch else (B*S, H)."""
    H = x.shape[1]
    xd = G.to_dev(x, dtype).view(B, S, H)
    pd = pdtype or dtype
    wd = None if w is None else G.to_dev(w, pd)
    scd = G.to_dev(sc, pd).view(B, 1 if per_batch else S, H)
    shd = G.to_dev(sh, pd).view(B, 1 if per_batch else S, H)
    y, rr = tn.rmsnorm_adaln_fwd(xd, wd, scd, shd, eps, return_rrms=True)
    torch.cuda.synchronize()
    return G.to_host(y.view(B * S, H), dtype), rr.view(-1).cpu().numpy()


@pytest.mark.parametrize("name", ["adaln_bf16_2x4096x2048_batchcond", "adaln_bf16_2x4096x2048_tokencond"])
def test_workload_adaln(name):
    d = synthetic.make_inputs(name)
    rpc = d["rows_per_cond"]
    B, S = (d["M"] // rpc, rpc) if rpc > 1 else (2, d["M"] // 2)
    print(f"[gpu] {name}", flush=True)
    y, rr = run(d["x"], d["w"], d["scale"], d["shift"], B, S, d["eps"], d["dtype"], per_batch=rpc > 1)
    G.assert_ok(*G.adaln_vs_oracle(d["x"], d["w"], d["scale"], d["shift"], rpc, y, rr, d["eps"], d["dtype"],
                                   chunk=4096, name=name), record=name)


@pytest.mark.parametrize("B,S,H,dt", [(2, 6000, 2048, "bf16"), (2, 9001, 2048, "bf16"), (2, 9001, 4104, "bf16"),
                                      (3, 6001, 2048, "f32"), (16, 1100, 2048, "f32"), (3, 6001, 2048, "bf16"),
                                      (16, 1100, 2048, "bf16"), (2, 4501, 4096, "bf16"), (2, 4501, 2048, "f32")])
def test_per_batch_rows_walked_by_each_row_group(B, S, H, dt):
    """Per-batch conditioning on a large grid: each row group walks 4 rows
    a quarter of the call apart (16-bit rows with at most two conditioning
    rows, float32 rows with any number; rows of 8 KiB or more with at most
    two conditioning rows walk 8), so its rows cross batch boundaries
    (the conditioning rows are reloaded there) and the last iteration runs
    past M (ragged: 2 x 9001 rows is an odd number of two-row groups);
    16-bit calls of more batches take one row per row group.  Parity with
    the oracle and the same bits as the one-row-per-row-group grid of the
    same tile (H = 4104: the two-wave tile of 513 vectors)."""
    M = B * S
    d = G.inputs(470 + S, M, H, dt)
    sc = synthetic.normal_tensor(470 + S, synthetic.STREAM_SCALE, (B, H), dt, 0.0, 0.5)
    sh = synthetic.normal_tensor(470 + S, synthetic.STREAM_SHIFT, (B, H), dt, 0.0, 0.5)
    print(f"[gpu] adaln per-batch walk {dt} B={B} S={S} H={H}", flush=True)
    y, rr = run(d["x"], d["w"], sc, sh, B, S, 1e-6, dt)
    G.assert_ok(*G.adaln_vs_oracle(d["x"], d["w"], sc, sh, S, y, rr, 1e-6, dt, chunk=S * max(1, 4096 // S),
                                   name=f"adaln walk {B}x{S}"))
    t = tn.tile("adaln", H, dt, off_grid=False)
    tn.set_geometry("fwd", t["vpt"], t["wpr"], t["rpw"], 0)  # the same tile, one row per row group
    y1, rr1 = run(d["x"], d["w"], sc, sh, B, S, 1e-6, dt)
    assert np.array_equal(y, y1) and np.array_equal(rr, rr1)


@pytest.mark.parametrize("pdtype", ["same", "f32"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
# 10240 and 16384: capped tiles (16-bit rows at most 8 waves); 32768: the
# longest 16-bit row held in registers with 16-bit parameters (two passes with
# float32 ones)
@pytest.mark.parametrize("H", [1, 7, 64, 1000, 2048, 2056, 3072, 3584, 4097, 4104, 6144, 8192, 10240, 16384, 20000,
                               32768])
def test_adaln_shapes(dtype, pdtype, H):
    pd = dtype if pdtype == "same" else "f32"
    B, S = 3, 7
    M = B * S
    seed = 3000 + H
    x = synthetic.normal_tensor(seed, synthetic.STREAM_X, (M, H), dtype)
    w = synthetic.normal_tensor(seed, synthetic.STREAM_W, (H,), pd, 1.0, 0.1)
    for per_batch in (True, False):
        C = B if per_batch else M
        sc = synthetic.normal_tensor(seed, synthetic.STREAM_SCALE, (C, H), pd, 0.0, 0.5)
        sh = synthetic.normal_tensor(seed, synthetic.STREAM_SHIFT, (C, H), pd, 0.0, 0.5)
        for weight in (w, None):
            y, rr = run(x, weight, sc, sh, B, S, 1e-6, dtype, pd, per_batch)
            G.assert_ok(*G.adaln_vs_oracle(x, weight, sc, sh, S if per_batch else 1, y, rr, 1e-6, dtype, pd,
                                           chunk=M, name=f"adaln {dtype}/{pd} H={H} batch={per_batch} w={weight is not None}"))


# H = 4096 bf16 is 512 vectors: resident tiles (1,8), (2,4), (4,2), (8,1);
# (4,1) tiles of 256 vectors take two passes; grid > 0 walks rows grid-stride
GEOMS = [(1, 8, 1, 0), (2, 4, 1, 0), (4, 2, 2, 0), (8, 1, 2, 0), (2, 4, 1, 5), (4, 1, 1, 0), (4, 1, 2, 3)]


@pytest.mark.parametrize("stream", [0, 1])
@pytest.mark.parametrize("geom", GEOMS, ids=[str(g) for g in GEOMS])
def test_adaln_forced_geometry(geom, stream):
    H = 4096
    B, S = 4, 75
    M = B * S
    d = G.inputs(91, M, H, "bf16")
    sc = synthetic.normal_tensor(91, synthetic.STREAM_SCALE, (B, H), "bf16", 0.0, 0.5)
    sh = synthetic.normal_tensor(91, synthetic.STREAM_SHIFT, (B, H), "bf16", 0.0, 0.5)
    tn.set_geometry("fwd", *geom)
    tn.set_streaming(stream)
    y, rr = run(d["x"], d["w"], sc, sh, B, S, 1e-5, "bf16")
    G.assert_ok(*G.adaln_vs_oracle(d["x"], d["w"], sc, sh, S, y, rr, 1e-5, "bf16", chunk=M, name=f"adaln {geom}"))


def test_adaln_special_cases():
    H, B, S = 2048, 2, 64
    d = G.inputs(92, B * S, H, "bf16")
    xd, wd = G.to_dev(d["x"], "bf16").view(B, S, H), G.to_dev(d["w"], "bf16")
    zero = torch.zeros(B, 1, H, dtype=torch.bfloat16, device=G.DEV)
    y0 = tn.rmsnorm_fwd(xd, wd, 1e-6)
    y = tn.rmsnorm_adaln_fwd(xd, wd, zero, zero, 1e-6)
    # scale = -1: (1 + scale) is exactly 0, so y is the shift exactly
    sh = torch.randn(B, 1, H, device=G.DEV).to(torch.bfloat16)
    y2 = tn.rmsnorm_adaln_fwd(xd, wd, -torch.ones_like(sh), sh, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
    assert torch.equal(y2.view(torch.int16), sh.expand(B, S, H).contiguous().view(torch.int16))


def test_adaln_misaligned_rows():
    H, B, S = 2047, 2, 33
    M = B * S
    d = G.inputs(93, M, H, "bf16")
    sc = synthetic.normal_tensor(93, synthetic.STREAM_SCALE, (M, H), "bf16", 0.0, 0.5)
    sh = synthetic.normal_tensor(93, synthetic.STREAM_SHIFT, (M, H), "bf16", 0.0, 0.5)
    y, rr = run(d["x"], d["w"], sc, sh, B, S, 1e-6, "bf16", per_batch=False)
    G.assert_ok(*G.adaln_vs_oracle(d["x"], d["w"], sc, sh, 1, y, rr, 1e-6, "bf16", chunk=M, name="adaln H=2047"))


@pytest.mark.parametrize("per_batch", [True, False], ids=["per_batch", "per_token"])
@pytest.mark.parametrize("dtype,pdtype", [("bf16", "bf16"), ("f16", "f32"), ("f32", "f32")])
@pytest.mark.parametrize("H", [2049, 4096, 16385, 32767, 40001])
def test_adaln_rows_off_the_grid(H, dtype, pdtype, per_batch):
    """Rows off the 16-byte grid (ragged H, x and the modulation at element
    offsets; scale and shift as column slices of one modulation tensor, per
    batch as [B, 1, H] views): the tile depends on H only, so every layout
    gives the same bits, at parity with the oracle, and nothing around the
    output rows is written.  16-bit rows with 16-bit parameters stay in
    registers to 32767 columns; 16385 and 32767 with float32 parameters, and
    40001 everywhere, take two passes."""
    B, S = 3, 11
    M = B * S
    C = B if per_batch else M
    d = G.inputs(5200 + H, M, H, dtype, wdtype=pdtype)
    sc = synthetic.normal_tensor(5200 + H, synthetic.STREAM_SCALE, (C, H), pdtype, 0.0, 0.5)
    sh = synthetic.normal_tensor(5200 + H, synthetic.STREAM_SHIFT, (C, H), pdtype, 0.0, 0.5)
    wd = G.to_dev(d["w"], pdtype)
    first = None
    for pad, xoff, moff, yoff in ((1, 1, 0, 0), (0, 3, 1, 1), (5, 0, 3, 7), (8, 1, 2, 1)):
        print(f"[gpu] adaln off-grid {dtype}/{pdtype} H={H} per_batch={per_batch} layout {pad},{xoff},{moff},{yoff}",
              flush=True)
        _, xv = G.sentinel_view(M, H, pad, xoff, dtype, 0.0)
        xv.copy_(G.to_dev(d["x"], dtype))
        # scale and shift: two column slices of one modulation tensor
        _, mv = G.sentinel_view(C, 2 * H, pad, moff, pdtype, 0.0)
        mv[:, :H].copy_(G.to_dev(sc, pdtype))
        mv[:, H:].copy_(G.to_dev(sh, pdtype))
        scv, shv = mv[:, :H], mv[:, H:]
        if per_batch:
            scv, shv = scv.unsqueeze(1), shv.unsqueeze(1)
        else:
            scv, shv = scv.view(B, S, H), shv.view(B, S, H)
        ybuf, yv = G.sentinel_view(M, H, pad + 2, yoff, dtype, -77.0)
        _, rr = tn.rmsnorm_adaln_fwd(xv.view(B, S, H), wd, scv, shv, 1e-6, out=yv.view(B, S, H),
                                     return_rrms=True)
        torch.cuda.synchronize()
        assert G.untouched(ybuf, yv, -77.0)
        got = (G.to_host(yv.contiguous(), dtype), rr.view(-1).cpu().numpy())
        if first is None:
            first = got
            rpc = S if per_batch else 1
            G.assert_ok(*G.adaln_vs_oracle(d["x"], d["w"], sc, sh, rpc, got[0], got[1], 1e-6, dtype, pdtype,
                                           chunk=M, name=f"adaln off-grid {dtype} H={H}"))
        else:
            assert np.array_equal(got[0], first[0]) and np.array_equal(got[1], first[1])


def test_adaln_modulation_slices():
    """scale and shift as two column slices of one [B, 1, 6H] modulation tensor
    (DiT's six values per block), sharing its row stride."""
    H, B, S = 1024, 2, 16
    d = G.inputs(94, B * S, H, "bf16")
    mod = synthetic.normal_tensor(94, synthetic.STREAM_SCALE, (B, 6 * H), "bf16", 0.0, 0.5)
    modd = G.to_dev(mod, "bf16").view(B, 1, 6 * H)
    sc, sh = modd[..., 0:H], modd[..., H:2 * H]
    xd, wd = G.to_dev(d["x"], "bf16").view(B, S, H), G.to_dev(d["w"], "bf16")
    y, rr = tn.rmsnorm_adaln_fwd(xd, wd, sc, sh, 1e-6, return_rrms=True)
    torch.cuda.synchronize()
    G.assert_ok(*G.adaln_vs_oracle(d["x"], d["w"], np.ascontiguousarray(mod[:, 0:H]),
                                   np.ascontiguousarray(mod[:, H:2 * H]), S, G.to_host(y.view(B * S, H), "bf16"),
                                   rr.view(-1).cpu().numpy(), 1e-6, "bf16", chunk=B * S, name="adaln slices"))
