"""Every entry point captured in a HIP graph (torch.cuda.graph) gives, on each
of several replays, the same bits as the same calls launched eagerly.  The
library enqueues only kernel launches (no memset, no allocation), so its
calls can be captured; replays are separated by unrelated eager work and
synchronisations, and each replay is checked, not only the first.
"""

from __future__ import annotations

import pytest

import synthetic
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import transformer_normalization_amd as tn  # noqa: E402


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def test_graph_replays_match_eager():
    M, H, eps = 300, 4096, 1e-5
    d = G.inputs(90, M, H, "bf16", residual=True, dy=True)
    x, w, r, dy = (G.to_dev(d[k], "bf16") for k in ("x", "w", "r", "dy"))
    sc = G.to_dev(synthetic.normal_tensor(90, synthetic.STREAM_SCALE, (M, H), "bf16", 0.0, 0.5), "bf16")
    sh = G.to_dev(synthetic.normal_tensor(90, synthetic.STREAM_SHIFT, (M, H), "bf16", 0.0, 0.5), "bf16")
    B, S, NH, D = 2, 150, 8, 64
    q = G.to_dev(synthetic.normal_tensor(91, synthetic.STREAM_X, (B, S, NH, D), "bf16"), "bf16")
    ct, st = synthetic.rope_tables(91, S, D, "f32")
    cos, sin = G.to_dev(ct, "f32"), G.to_dev(st, "f32")

    outs = {k: torch.empty_like(x) for k in ("y", "y2", "ro", "dx", "dh", "ya", "dx3")}
    outs["q"] = torch.empty_like(q)
    rr = torch.empty(M, dtype=torch.float32, device=G.DEV)
    rr2 = torch.empty(M, dtype=torch.float32, device=G.DEV)
    dw = torch.empty(H, dtype=torch.float32, device=G.DEV)
    dw2 = torch.empty(H, dtype=torch.float32, device=G.DEV)
    dw3 = torch.empty(H, dtype=torch.float32, device=G.DEV)
    ws = torch.empty(tn.rmsnorm_bwd_workspace_bytes(M, H), dtype=torch.uint8, device=G.DEV)
    ws2 = torch.empty_like(ws)

    def calls():
        tn.rmsnorm_fwd(x, w, eps, out=outs["y"], rrms=rr)
        tn.rmsnorm_fwd_residual(x, r, w, eps, out=outs["y2"], residual_out=outs["ro"], rrms=rr2)
        tn.rmsnorm_bwd(dy, x, w, rr, dx=outs["dx"], dw=dw, workspace=ws)
        tn.rmsnorm_bwd_residual(dy, outs["ro"], r, w, rr2, dh=outs["dh"], dw=dw2, workspace=ws2)
        tn.rmsnorm_adaln_fwd(x, w, sc, sh, eps, out=outs["ya"])
        tn.rope_apply(q, cos, sin, out=outs["q"])
        # the backward with its partial rows in the library's static scratch:
        # nothing to allocate or clear inside the capture
        tn.rmsnorm_bwd_noalloc(dy, x, w, rr, outs["dx3"], dw3)

    calls()  # eager, also caches the device facts before capture
    torch.cuda.synchronize()
    want = {k: _bits(v).clone() for k, v in outs.items()}
    want.update(rr=_bits(rr).clone(), rr2=_bits(rr2).clone(), dw=_bits(dw).clone(), dw2=_bits(dw2).clone(),
                dw3=_bits(dw3).clone())
    assert torch.equal(want["dx3"], want["dx"]) and torch.equal(want["dw3"], want["dw"])

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(G.DEV)
    for t in list(outs.values()) + [rr, rr2, dw, dw2, dw3]:
        t.fill_(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        calls()
    for rep in range(3):
        for t in list(outs.values()) + [rr, rr2, dw, dw2, dw3]:
            t.fill_(0)
        # unrelated eager work between replays
        _ = (x.float() * 2).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: _bits(v) for k, v in outs.items()}
        got.update(rr=_bits(rr), rr2=_bits(rr2), dw=_bits(dw), dw2=_bits(dw2), dw3=_bits(dw3))
        for k in want:
            assert torch.equal(got[k], want[k]), f"replay {rep}: {k}"


def test_calls_run_on_the_current_stream():
    """The binding hands the library the current stream of the tensor's
    device, also inside `with torch.cuda.stream(...)`."""
    x = torch.ones((64, 512), dtype=torch.bfloat16, device=G.DEV)
    # (ctypes shows the null stream, handle 0, as None)
    assert (tn._stream(x).value or 0) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream(G.DEV)
    with torch.cuda.stream(side):
        assert (tn._stream(x).value or 0) == side.cuda_stream
        y = tn.rmsnorm_fwd(x, None, 1e-6)
    side.synchronize()
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))  # rows of ones normalise to ones
