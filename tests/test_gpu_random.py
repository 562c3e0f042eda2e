"""Randomised GPU parity: seeded random shapes, formats, row paddings
(aligned and misaligned) and optional parameters for every entry point,
against the float64 oracle with each operation's stated tolerance; and
concurrent calls from several host threads on their own streams.

The cases are drawn once from a fixed seed, so a failure names a case that
reproduces exactly (its id lists op, format, shape and padding).
"""

from __future__ import annotations

import random
import threading

import numpy as np
import pytest

import oracle
import synthetic
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import transformer_normalization_amd as tn  # noqa: E402


def _draw_cases(n=60, seed=20261202):
    rng = random.Random(seed)
    ops = ["fwd", "fwd_residual", "adaln", "bwd", "bwd_residual", "layernorm", "layernorm_residual", "rope"]
    cases = []
    for i in range(n):
        op = ops[i % len(ops)]
        dtype = rng.choice(["bf16", "f16", "f32"])
        if op == "rope":
            D = 2 * rng.choice([1, 4, 7, 16, 32, 48, 64, 100])
            shape = (rng.randint(1, 3), rng.randint(1, 40), rng.randint(1, 9), D)
        else:
            H = int(round(2 ** rng.uniform(0, 14)))
            shape = (rng.randint(1, 200 if H <= 4096 else 20), H)
        pad = rng.choice([0, 0, 8, 1])
        weighted = rng.random() < 0.8
        cases.append((i, op, dtype, shape, pad, weighted))
    return cases


CASES = _draw_cases()


def _padded(a, dtype, pad):
    """Device view of the host (M, H) rows a inside rows padded by `pad`
    elements; pad 1 also starts the view one element into its buffer
    (misaligned)."""
    t = G.to_dev(a, dtype)
    if pad == 0:
        return t
    M, H = t.shape
    buf = torch.zeros(M * (H + pad) + 1, dtype=t.dtype, device=G.DEV)
    off = 1 if pad == 1 else 0
    view = buf[off:off + M * (H + pad)].view(M, H + pad)[:, :H]
    view.copy_(t)
    return view


def _rrms32(x, w, eps, dtype):
    _, r = oracle.fwd(x, w, G.eps32(eps), dtype)
    return r.astype(np.float32)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}-{'x'.join(map(str, c[3]))}-pad{c[4]}"
                                             for c in CASES])
def test_random_case(case):
    i, op, dtype, shape, pad, weighted = case
    print(f"[gpu] random case {case}", flush=True)
    seed = 9000 + i
    eps = 1e-5
    if op == "rope":
        B, S, NH, D = shape
        x = synthetic.normal_tensor(seed, synthetic.STREAM_X, shape, dtype)
        tdt = "f32" if dtype != "f32" and i % 2 else dtype
        c, s = synthetic.rope_tables(seed, S, D, tdt)
        xd = G.to_dev(x, dtype)
        if pad:
            big = torch.zeros((B, S, NH, D + 2 * pad), dtype=xd.dtype, device=G.DEV)
            big[..., :D] = xd
            xd = big[..., :D]
        out = tn.rope_apply(xd, G.to_dev(c, tdt), G.to_dev(s, tdt), transpose=bool(i % 3 == 0))
        torch.cuda.synchronize()
        ref = oracle.rope(x, c, s, dtype, tdt, transpose=bool(i % 3 == 0))
        h = D // 2
        xv = oracle.decode(x, dtype)
        cv = oracle.decode(np.ascontiguousarray(c[:, :h]), tdt)[None, :, None, :]
        sv = oracle.decode(np.ascontiguousarray(s[:, :h]), tdt)[None, :, None, :]
        terms = np.concatenate([np.abs(xv[..., :h] * cv) + np.abs(xv[..., h:] * sv),
                                np.abs(xv[..., :h] * sv) + np.abs(xv[..., h:] * cv)], axis=-1)
        rep = G.parity.Report(f"rope {case}")
        n = NH * D
        got = G.to_host(out, dtype).reshape(-1, n)
        if dtype == "f32":
            G.parity.check_dx_f32(rep, got, ref.reshape(-1, n), terms.reshape(-1, n))
        else:
            G.parity.check_dx16(rep, got, ref.reshape(-1, n), terms.reshape(-1, n), dtype, oracle.encode,
                                oracle.decode)
        G.assert_ok(rep)
        return

    M, H = shape
    d = G.inputs(seed, M, H, dtype, residual=True, dy=True)
    x, w, r, dy = d["x"], (d["w"] if weighted else None), d["r"], d["dy"]
    xd, rd, dyd = _padded(x, dtype, pad), _padded(r, dtype, pad), _padded(dy, dtype, pad)
    wd = None if w is None else G.to_dev(w, dtype)
    if op == "fwd":
        y, rr = tn.rmsnorm_fwd(xd, wd, eps, return_rrms=True)
        torch.cuda.synchronize()
        G.assert_ok(*G.fwd_vs_oracle(x, w, G.to_host(y, dtype), rr.cpu().numpy(), eps, dtype, name=str(case)))
    elif op == "fwd_residual":
        y, ro, rr = tn.rmsnorm_fwd_residual(xd, rd, wd, eps, return_rrms=True)
        torch.cuda.synchronize()
        G.assert_ok(*G.residual_vs_oracle(x, r, w, G.to_host(y, dtype), G.to_host(ro, dtype), rr.cpu().numpy(), eps,
                                          dtype, name=str(case)))
    elif op == "adaln":
        sc = synthetic.normal_tensor(seed, synthetic.STREAM_SCALE, (M, H), dtype, 0.0, 0.5)
        sh = synthetic.normal_tensor(seed, synthetic.STREAM_SHIFT, (M, H), dtype, 0.0, 0.5)
        y, rr = tn.rmsnorm_adaln_fwd(xd, wd, G.to_dev(sc, dtype), G.to_dev(sh, dtype), eps, return_rrms=True)
        torch.cuda.synchronize()
        G.assert_ok(*G.adaln_vs_oracle(x, w, sc, sh, 1, G.to_host(y, dtype), rr.cpu().numpy(), eps, dtype,
                                       name=str(case)))
    elif op in ("bwd", "bwd_residual"):
        rr = _rrms32(x, w, eps, dtype)
        rrd = torch.from_numpy(rr).to(G.DEV)
        if op == "bwd":
            dx, dw = tn.rmsnorm_bwd(dyd, xd, wd, rrd)
            torch.cuda.synchronize()
            G.assert_ok(*G.bwd_vs_oracle(dy, x, w, rr, G.to_host(dx, dtype), None if dw is None else dw.cpu().numpy(),
                                         dtype, name=str(case)))
        else:
            dh, dw = tn.rmsnorm_bwd_residual(dyd, xd, rd, wd, rrd)
            torch.cuda.synchronize()
            G.assert_ok(*G.bwd_residual_vs_oracle(dy, x, r, w, rr, G.to_host(dh, dtype),
                                                  None if dw is None else dw.cpu().numpy(), dtype, name=str(case)))
    else:
        b = synthetic.normal_tensor(seed, synthetic.STREAM_BIAS, (H,), dtype, 0.0, 0.1) if weighted else None
        bd = None if b is None else G.to_dev(b, dtype)
        if op == "layernorm":
            y, mean, rstd = tn.layernorm_fwd(xd, wd, bd, eps, return_stats=True)
            ro_h, rr_in = None, None
        else:
            y, ro, mean, rstd = tn.layernorm_fwd_residual(xd, rd, wd, bd, eps, return_stats=True)
            ro_h, rr_in = G.to_host(ro, dtype), r
        torch.cuda.synchronize()
        G.assert_ok(*G.ln_vs_oracle(x, rr_in, w, b, G.to_host(y, dtype), ro_h, mean.cpu().numpy(), rstd.cpu().numpy(),
                                    eps, dtype, name=str(case)))


def test_concurrent_calls_from_threads_on_their_own_streams():
    """Several host threads call the library at once, each on its own stream
    with its own inputs; every result equals the same call made alone."""
    M, H = 512, 4096
    jobs = []
    for k in range(6):
        d = G.inputs(9500 + k, M, H, "bf16", residual=True, dy=True)
        jobs.append(tuple(G.to_dev(d[n], "bf16") for n in ("x", "w", "r", "dy")))

    def run(x, w, r, dy):
        y, ro, rr = tn.rmsnorm_fwd_residual(x, r, w, 1e-5, return_rrms=True)
        dh, dw = tn.rmsnorm_bwd_residual(dy, ro, r, w, rr)
        return y, ro, dh, dw

    want = [run(*j) for j in jobs]
    torch.cuda.synchronize()
    got = [None] * len(jobs)
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream(G.DEV)
            with torch.cuda.stream(s):
                for _ in range(20):
                    res = run(*jobs[k])
            s.synchronize()
            got[k] = res
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for k in range(len(jobs)):
        for a, b in zip(got[k], want[k]):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), k
