"""The torch custom operators (transformer_normalization_amd.ops): the same
bits as the direct binding and the autograd Functions, torch.library's own
consistency checks (opcheck), and a compiled graph (torch.compile with the
aot_eager backend, fullgraph: no graph break at the library calls) that
gives the eager bits for outputs and gradients."""

from __future__ import annotations

import pytest

import synthetic
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import transformer_normalization_amd as tn  # noqa: E402
from transformer_normalization_amd import autograd as ag  # noqa: E402
from transformer_normalization_amd import ops  # noqa: E402


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def _leaf(a, dtype, grad=True):
    return G.to_dev(a, dtype).requires_grad_(grad)


def test_ops_match_the_autograd_functions():
    M, H = 130, 2048
    d = G.inputs(95, M, H, "bf16", residual=True, dy=True)
    gy = G.to_dev(d["dy"], "bf16")
    gh = G.to_dev(synthetic.normal_tensor(95, synthetic.STREAM_SHIFT, (M, H), "bf16"), "bf16")
    results = []
    for impl in (ag, ops):
        x, r, w = _leaf(d["x"], "bf16"), _leaf(d["r"], "bf16"), _leaf(d["w"], "bf16")
        y1 = impl.rms_norm(x, w, 1e-5)
        y2, h = impl.fused_add_rms_norm(x, r, w, 1e-5)
        loss = (y1.float() * gy.float()).sum() + (y2.float() * gy.float()).sum() + (h.float() * gh.float()).sum()
        loss.backward()
        results.append([y1.detach(), y2.detach(), h.detach(), x.grad, r.grad, w.grad])
    for a, b in zip(*results):
        assert torch.equal(_bits(a), _bits(b))


def test_rope_op_matches_and_differentiates():
    B, S, NH, D = 2, 33, 4, 64
    q_h = synthetic.normal_tensor(96, synthetic.STREAM_X, (B, S, NH, D), "bf16")
    g = G.to_dev(synthetic.normal_tensor(96, synthetic.STREAM_DY, (B, S, NH, D), "bf16"), "bf16")
    c, s = synthetic.rope_tables(96, S, D, "f32")
    cd, sd = G.to_dev(c, "f32"), G.to_dev(s, "f32")
    outs = []
    for f in (lambda q: ag.rope_3d(q, cd, sd), lambda q: ops.rope(q, cd, sd)):
        q = _leaf(q_h, "bf16")
        y = f(q)
        (y.float() * g.float()).sum().backward()
        outs.append((y.detach(), q.grad))
    assert torch.equal(_bits(outs[0][0]), _bits(outs[1][0])) and torch.equal(_bits(outs[0][1]), _bits(outs[1][1]))


def test_forward_only_ops_match_the_binding():
    M, H = 64, 1024
    d = G.inputs(97, M, H, "f32", residual=True)
    x, r, w = (G.to_dev(d[k], "f32") for k in ("x", "r", "w"))
    b = G.to_dev(synthetic.normal_tensor(97, synthetic.STREAM_BIAS, (H,), "f32", 0.0, 0.1), "f32")
    y, h = ops.layer_norm_residual(x, r, w, b, 1e-5)
    y2, h2 = tn.layernorm_fwd_residual(x, r, w, b, 1e-5)
    assert torch.equal(y, y2) and torch.equal(h, h2)
    sc = torch.randn(1, M, H, device=G.DEV) * 0.5
    ya = ops.adaln_rms_norm(x.view(1, M, H), w, sc, sc, 1e-6)
    assert torch.equal(ya, tn.rmsnorm_adaln_fwd(x.view(1, M, H), w, sc, sc, 1e-6))


def test_opcheck():
    M, H = 16, 512
    x = torch.randn(M, H, device=G.DEV, dtype=torch.bfloat16)
    r = torch.randn_like(x)
    w = torch.rand(H, device=G.DEV, dtype=torch.bfloat16) + 0.5
    torch.library.opcheck(ops._rms_norm_fwd, (x.requires_grad_(), w.requires_grad_(), 1e-5))
    torch.library.opcheck(ops._fused_fwd, (x.detach().requires_grad_(), r.requires_grad_(), w, 1e-5))
    q = torch.randn(2, 8, 2, 64, device=G.DEV, dtype=torch.bfloat16, requires_grad=True)
    c = torch.rand(8, 64, device=G.DEV)
    torch.library.opcheck(ops._rope, (q, c, c, False))


def test_compiled_block_gives_the_eager_bits():
    """A pre-norm block fragment -- fused add + norm, then RoPE of a head
    view -- compiled whole (fullgraph) with the aot_eager backend."""
    B, S, NH, D = 2, 16, 4, 64
    H = NH * D
    d = G.inputs(98, B * S, H, "bf16", residual=True, dy=True)
    c, s = synthetic.rope_tables(98, S, D, "f32")
    cd, sd = G.to_dev(c, "f32"), G.to_dev(s, "f32")

    def block(x, r, w):
        y, h = ops.fused_add_rms_norm(x, r, w, 1e-5)
        q = ops.rope(y.view(B, S, NH, D), cd, sd)
        return q.float().square().sum() + h.float().sum()

    compiled = torch.compile(block, backend="aot_eager", fullgraph=True)
    res = []
    for f in (block, compiled):
        x, r, w = _leaf(d["x"], "bf16"), _leaf(d["r"], "bf16"), _leaf(d["w"], "bf16")
        loss = f(x, r, w)
        loss.backward()
        res.append((loss.detach(), x.grad, r.grad, w.grad))
    for a, b in zip(*res):
        assert torch.equal(_bits(a), _bits(b))
