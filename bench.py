"""Throughput of the gfx950 RMSNorm library on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--graph]

A step is one library call (the whole hot path of the workload: the forward
kernel, or the backward kernel and its dw finalize, or the RoPE kernel) on
one batch of seeded synthetic input already resident in HBM.  Batches rotate
over enough buffer sets (>= 1 GiB per cycle) that no step finds its data in
the last-level cache.  W untimed steps, then exactly K steps between two
synchronisations, timed with HIP events on the stream the kernels are
launched on.  One JSON line is printed.

Workloads (default: the forward at bf16 M=8192 H=4096):
  fwd_bf16_8192x4096, fwd_f32_64x512, fwd_bf16_32768x2048, fwd_bf16_32768x2048_noweight,
  fwd_f16_32768x2048_outliers, fwd_residual_bf16_16384x8192, bwd_bf16_8192x6144, bwd_bf16_8192x4097,
  bwd_residual_bf16_16384x8192, adaln_bf16_2x4096x2048_batchcond, adaln_bf16_2x4096x2048_tokencond,
  rope_bf16_2x8064x32x64, rope_bf16_2x4096x32x128, ln_residual_f32_16384x1024

--graph captures the timed steps in HIP graphs (blocks of steps, replayed) so
that host launch overhead cannot leave the GPU idle between short kernels;
the kernels and their arguments are the same as in eager launches.  Without
it, `value` is the eager figure and `graph_launch` gives the same steps timed
again from captured graphs (--no-graph-leg skips that).

copy_ceiling times rmsnorm_tuning_copy moving the same bytes per step (half
read, half written) with the kernels' access pattern and no arithmetic: the
practical HBM ceiling of a transfer of that size, beside the 8 TB/s peak.

The CPU baseline is the float64 oracle run on the host over a sample of the
same workload, at one thread and at every thread the process may use (up to
16), each the median of three runs (reported beside the GPU figure, never a
target).  `spread` gives the per-step minimum, median, maximum and standard
deviation from a second pass with an event after every step, and `device`
what ran it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak
METRIC = "RMSNorm fwd achieved HBM GB/s (% of peak) + rows/s, bf16 M=8192 H=4096"
PROFILE_DIR = os.path.join(ROOT, "profiles")
ROTATION_BYTES = 1 << 30
GRAPH_BLOCK = 100  # steps per captured graph
SPREAD_BLOCK = 20  # steps per timed block of the spread pass

_FWD = ("numerics.hpp", "fwd_kernels.hpp", "fwd_table.hpp", "kernel_tables.hpp")
_BWD = ("numerics.hpp", "bwd_kernels.hpp", "bwd_table.hpp", "kernel_tables.hpp", "kernels_bwd.hip")
KERNEL_SOURCES = {
    "fwd": _FWD + ("kernels_fwd.hip", "rmsnorm_api.hip"),
    "fwd_residual": _FWD + ("kernels_fwd_residual.hip", "rmsnorm_api.hip"),
    "bwd": _BWD + ("rmsnorm_api.hip",),
    "bwd_residual": _BWD + ("kernels_bwd_residual.hip", "rmsnorm_api.hip"),
    "adaln": _FWD + ("kernels_adaln.hip", "rmsnorm_api.hip"),
    "rope": ("numerics.hpp", "rope_kernels.hpp", "kernel_tables.hpp", "kernels_rope.hip", "rope_api.hip"),
    "ln_residual": ("numerics.hpp", "ln_kernels.hpp", "kernel_tables.hpp", "kernels_ln.hip", "rmsnorm_api.hip"),
    "fwd_offgrid": _FWD + ("kernels_fwd_mis.hip", "rmsnorm_api.hip"),
    "bwd_offgrid": _BWD + ("kernels_bwd_mis.hip", "rmsnorm_api.hip"),
}
# the kernel whose launches the counters describe
KERNEL_KEY = {"fwd": "rmsnorm_fwd_kernel", "fwd_residual": "rmsnorm_fwd_kernel", "adaln": "rmsnorm_fwd_kernel",
              "bwd": "rmsnorm_bwd_kernel", "bwd_residual": "rmsnorm_bwd_kernel", "rope": "rope_apply_kernel",
              "ln_residual": "layernorm_fwd_kernel", "fwd_offgrid": "rmsnorm_fwd_kernel",
              "bwd_offgrid": "rmsnorm_bwd_kernel"}


def kernel_kind(spec) -> str:
    """The kernel family a workload's calls run: its kind, except that a
    forward or backward on contiguous rows whose byte length is not a
    multiple of 16 (so that rows leave the 16-byte grid) runs the
    instantiations for rows off the grid (16-byte vectors at each row's byte
    offset)."""
    if spec["kind"] in ("fwd", "bwd") and (spec["H"] * _size(spec["dtype"])) % 16:
        return spec["kind"] + "_offgrid"
    return spec["kind"]

WORKLOADS = {
    "fwd_bf16_8192x4096": ("fwd_bf16_8192x4096", True),
    "fwd_f32_64x512": ("fwd_f32_64x512", True),
    "fwd_bf16_32768x2048": ("fwd_bf16_32768x2048", True),
    "fwd_bf16_32768x2048_noweight": ("fwd_bf16_32768x2048", False),
    "fwd_f16_32768x2048_outliers": ("fwd_f16_32768x2048_outliers", True),
    "fwd_residual_bf16_16384x8192": ("fwd_residual_bf16_16384x8192", True),
    "bwd_bf16_8192x6144": ("bwd_bf16_8192x6144", True),
    "bwd_residual_bf16_16384x8192": ("bwd_residual_bf16_16384x8192", True),
    "adaln_bf16_2x4096x2048_batchcond": ("adaln_bf16_2x4096x2048_batchcond", True),
    "adaln_bf16_2x4096x2048_tokencond": ("adaln_bf16_2x4096x2048_tokencond", True),
    "rope_bf16_2x8064x32x64": ("rope_bf16_2x8064x32x64", True),
    "rope_bf16_2x4096x32x128": ("rope_bf16_2x4096x32x128", True),
    "fwd_bf16_8192x4097": ("fwd_bf16_8192x4097", True),
    "bwd_bf16_8192x4097": ("bwd_bf16_8192x4097", True),
    "ln_residual_f32_16384x1024": ("ln_residual_f32_16384x1024", True),
}


def kernel_source_digest(kind: str) -> str:
    """Digest of the HIP sources a kind of call runs (kernels and the host code
    that picks their launch geometry); a stored traffic measurement applies
    only to the sources it was taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transformer_normalization_amd", "csrc")
    for name in KERNEL_SOURCES[kind]:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary of this
    workload, or None when absent or taken on other kernel sources."""
    path = os.path.join(PROFILE_DIR, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    name, _ = WORKLOADS[workload]
    import synthetic
    if fields.get("kernel_source_digest") != kernel_source_digest(kernel_kind(synthetic.WORKLOADS[name])):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _size(fmt):
    return 4 if fmt == "f32" else 2


def algorithmic_bytes(spec, weighted, rows=None):
    """Bytes the method must move once per step: inputs, weight, outputs,
    rrms if used; for RoPE, x and out plus the first half of each table row.
    rows (positions, for RoPE) restricts the count to a leading sample."""
    kind = spec["kind"]
    if kind == "rope":
        B, NH, D = spec["B"], spec["NH"], spec["D"]
        S = spec["S"] if rows is None else rows
        return 2 * B * S * NH * D * _size(spec["dtype"]) + 2 * S * (D // 2) * _size(spec["tdtype"])
    M = spec["M"] if rows is None else rows
    H = spec["H"]
    mat = M * H * _size(spec["dtype"])
    wsz = _size(spec["wdtype"])
    w = H * wsz if weighted else 0
    if kind == "fwd":
        return 2 * mat + w
    if kind == "fwd_residual":
        return 4 * mat + w
    if kind == "ln_residual":
        # x, r read; y, residual_out written; weight and bias read once
        return 4 * mat + 2 * w
    if kind == "bwd":
        # x, dy read; dx written; rrms read; w read; dw written (float32)
        return 3 * mat + M * 4 + w + H * 4
    if kind == "bwd_residual":
        # as bwd, plus the residual-stream gradient read
        return 4 * mat + M * 4 + w + H * 4
    if kind == "adaln":
        # x read, y written, w and the scale/shift rows read once
        cond_rows = -(-M // spec["rows_per_cond"])
        return 2 * mat + w + 2 * cond_rows * H * wsz
    raise ValueError(kind)


def x_bytes(spec):
    """Size of the x tensor (the device copy of known size)."""
    if spec["kind"] == "rope":
        return spec["B"] * spec["S"] * spec["NH"] * spec["D"] * _size(spec["dtype"])
    return spec["M"] * spec["H"] * _size(spec["dtype"])


def step_rows(spec):
    """Rows (token rows for RoPE) one step processes."""
    return spec["B"] * spec["S"] if spec["kind"] == "rope" else spec["M"]


def host_threads() -> int:
    """Threads the oracle may use: the CPUs this process may run on, capped
    at 16 (one GPU's share of its host's cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:
        return "unknown"


def cpu_baseline(spec, weighted, seconds, runs=3):
    """The oracle as it stands (float64 C through ctypes, which releases the
    GIL), over a leading sample of the workload, at one thread and at
    host_threads() threads; each thread takes a contiguous block of the
    sample's rows (positions, for RoPE) per pass.  Each figure is the median
    of `runs` independent runs, each repeating passes for about
    seconds / (2 * runs); reported in GB/s of the same algorithmic bytes."""
    import statistics
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synthetic

    kind = spec["kind"]
    if kind == "rope":
        n = min(spec["S"], 512)
        d = synthetic.make_inputs(spec["name"], rows=n)
        sample = f"first {n} of {spec['S']} positions of each of {spec['B']} batches"
        rows = spec["B"] * n
    else:
        n = min(spec["M"], 2048)
        d = synthetic.make_inputs(spec["name"], rows=n)
        sample = f"first {n} of {spec['M']} rows"
        rows = n
        w = d["w"] if weighted else None
        eps = float(np.float32(spec["eps"]))
        if kind in ("bwd", "bwd_residual"):
            _, r = oracle.fwd(d["x"], w, eps, d["dtype"], d["wdtype"])
            r32 = r.astype(np.float32)

    def block(a, b):
        """The oracle over sample rows [a, b) (positions, for RoPE)."""
        if kind == "rope":
            oracle.rope(np.ascontiguousarray(d["x"][:, a:b]), d["cos"][a:b], d["sin"][a:b], d["dtype"], d["tdtype"])
        elif kind == "fwd":
            oracle.fwd(d["x"][a:b], w, eps, d["dtype"], d["wdtype"])
        elif kind == "adaln":
            # row i reads conditioning row i // rpc: blocks are cut at the
            # conditioning rows' boundaries so each call keeps that map
            rpc = d["rows_per_cond"]
            if rpc == 1:
                oracle.adaln_fwd(d["x"][a:b], w, d["scale"][a:b], d["shift"][a:b], 1, eps, d["dtype"], d["wdtype"],
                                 d["wdtype"])
            else:
                i = a
                while i < b:
                    c = i // rpc
                    e = min(b, (c + 1) * rpc)
                    oracle.adaln_fwd(d["x"][i:e], w, d["scale"][c:c + 1], d["shift"][c:c + 1], e - i, eps,
                                     d["dtype"], d["wdtype"], d["wdtype"])
                    i = e
        elif kind == "fwd_residual":
            oracle.fwd_residual(d["x"][a:b], d["r"][a:b], w, eps, d["dtype"], d["wdtype"])
        elif kind == "ln_residual":
            oracle.layernorm(d["x"][a:b], d["r"][a:b], w, d["b"] if weighted else None, eps, d["dtype"],
                             d["wdtype"])
        elif kind == "bwd_residual":
            return oracle.bwd_residual(d["dy"][a:b], d["x"][a:b], d["dres"][a:b], w, r32[a:b], d["dtype"],
                                       d["wdtype"])[1]
        else:
            return oracle.bwd(d["dy"][a:b], d["x"][a:b], w, r32[a:b], d["dtype"], d["wdtype"])[1]
        return None

    nthreads = host_threads()
    run_s = max(seconds, 0.0) / (2 * runs)
    nbytes = algorithmic_bytes(spec, weighted, n)

    def measure(threads):
        bounds = [(n * i // threads, n * (i + 1) // threads) for i in range(threads)]
        bounds = [(a, b) for a, b in bounds if b > a]
        rates = []
        with ThreadPoolExecutor(max_workers=threads) as pool:
            for _ in range(runs):
                passes = 0
                t0 = time.perf_counter()
                while True:
                    parts = list(pool.map(lambda ab: block(*ab), bounds))
                    if parts and parts[0] is not None:  # the backward's dw: the blocks' column sums added
                        sum(parts[1:], parts[0].copy())
                    passes += 1
                    el = time.perf_counter() - t0
                    if el >= run_s:
                        break
                rates.append((nbytes * passes / el, rows * passes / el, passes, el))
        return rates

    one = measure(1)
    many = measure(nthreads) if nthreads > 1 else one
    med = lambda rs, i: statistics.median(r[i] for r in rs)
    return {
        "value": round(med(many, 0) / 1e9, 4),
        "unit": "GB/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": (f"{sample}; median of {runs} runs of about {run_s:.1f} s each, float64; "
                   f"{nthreads} threads, each a contiguous block of the sample per pass"),
        "rows_per_s": round(med(many, 1), 1),
        "runs_gbs": [round(r[0] / 1e9, 4) for r in many],
        "single_thread": {"value": round(med(one, 0) / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "rows_per_s": round(med(one, 1), 1), "runs_gbs": [round(r[0] / 1e9, 4) for r in one]},
        "cpu": cpu_model(),
        "nproc": os.cpu_count(),
        "threads_available": nthreads,
    }


def summarize_pmc(fetch_csv, write_csv, workload):
    """Text summary of HBM traffic per launch of the workload's dominant
    kernel from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch), each scaled by what the same counter reads for the plain
    device copies of the x tensor (known size) in the same run."""
    import csv
    import statistics

    import synthetic

    name, weighted = WORKLOADS[workload]
    spec = synthetic.WORKLOADS[name]
    known_kib = x_bytes(spec) / 1024.0
    kernel_key = KERNEL_KEY[kernel_kind(spec)]

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        kern = [float(r["Counter_Value"]) for r in rows if kernel_key in r["Kernel_Name"]]
        copies = [(int(r["Grid_Size"]), float(r["Counter_Value"])) for r in rows
                  if "copyBuffer" in r["Kernel_Name"]]
        big = max(g for g, _ in copies)
        ref = [v for g, v in copies if g == big]
        kname = next(r["Kernel_Name"] for r in rows if kernel_key in r["Kernel_Name"])
        return statistics.mean(kern), len(kern), statistics.mean(ref), len(ref), kname

    f_k, f_n, f_ref, f_rn, kname = read(fetch_csv, "FETCH_SIZE")
    w_k, w_n, w_ref, w_rn, _ = read(write_csv, "WRITE_SIZE")
    f_scale, w_scale = known_kib / f_ref, known_kib / w_ref
    hbm = (f_k * f_scale + w_k * w_scale) * 1024.0
    alg = algorithmic_bytes(spec, weighted)
    shape = (f"B={spec['B']} S={spec['S']} heads={spec['NH']} head_dim={spec['D']}" if spec["kind"] == "rope"
             else f"M={spec['M']} H={spec['H']}")
    lines = [
        f"# HBM traffic per launch of {kname}",
        f"# workload {workload}: {shape} {spec['dtype']}",
        "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 --pmc runs of",
        f"#   python3 bench.py --workload {workload} --cpu-seconds 0 --no-ceiling --steps 20 --warmup 10 --copy-reference",
        "# each scaled by the same counter's reading for device copies of the x tensor",
        f"# ({known_kib:.0f} KiB read and written per copy) in the same run; summary made by",
        f"#   python3 bench.py --workload {workload} --summarize-pmc <fetch csv> <write csv>",
        f"kernel_source_digest: {kernel_source_digest(kernel_kind(spec))}",
        f"kernel_dispatches: {f_n} (fetch run), {w_n} (write run)",
        f"fetch_size_kib_per_launch: {f_k:.2f}",
        f"write_size_kib_per_launch: {w_k:.2f}",
        f"copy_fetch_size_kib: {f_ref:.2f} over {f_rn} copies",
        f"copy_write_size_kib: {w_ref:.2f} over {w_rn} copies",
        f"fetch_scale: {f_scale:.5f}",
        f"write_scale: {w_scale:.5f}",
        f"hbm_bytes_per_launch: {hbm:.0f}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {hbm / alg:.4f}",
    ]
    return "\n".join(lines) + "\n"


def setup_steps(spec, weighted, dev, per_step):
    """Device buffers for the workload, rotated over >= ROTATION_BYTES, and
    step(i), which launches step i on the current stream and allocates
    nothing.  Returns (step, number of buffer sets, x of set 0, and a buffer
    of x's size to copy it into for the copy reference)."""
    import numpy as np
    import torch

    import synthetic
    import transformer_normalization_amd as tn

    kind = spec["kind"]
    d = synthetic.make_inputs(spec["name"])
    dt = d["dtype"]

    def up(a, fmt):
        a = np.ascontiguousarray(a)
        if fmt == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    nsets = max(2, -(-ROTATION_BYTES // per_step))
    x0 = up(d["x"], dt)
    sets = []
    for i in range(nsets):
        s = {"x": x0 if i == 0 else x0.clone(), "y": torch.empty_like(x0)}
        for key in {"fwd_residual": ("r",), "ln_residual": ("r",), "bwd": ("dy",),
                    "bwd_residual": ("dy", "dres")}.get(kind, ()):
            s[key] = up(d[key], dt) if i == 0 else sets[0][key].clone()
        if kind in ("fwd_residual", "ln_residual"):
            s["ro"] = torch.empty_like(x0)
        sets.append(s)
    copy_src, copy_dst = sets[0]["x"], sets[1]["y"]

    if kind == "rope":
        cos, sin = up(d["cos"], d["tdtype"]), up(d["sin"], d["tdtype"])

        def step(i):
            s = sets[i % nsets]
            tn.rope_apply(s["x"], cos, sin, out=s["y"])
        return step, nsets, copy_src, copy_dst

    eps = spec["eps"]
    M, H = spec["M"], spec["H"]
    w = up(d["w"], d["wdtype"]) if weighted else None
    bias = up(d["b"], d["wdtype"]) if weighted and "b" in d else None
    if kind == "adaln":
        rpc = spec["rows_per_cond"]
        shape = (M // rpc, 1, H) if rpc > 1 else (1, M, H)
        sc, sh = up(d["scale"], d["wdtype"]).view(*shape), up(d["shift"], d["wdtype"]).view(*shape)
        for i, s in enumerate(sets):
            s.update(scale=sc if i == 0 else sc.clone(), shift=sh if i == 0 else sh.clone(),
                     x=s["x"].view(shape[0], -1, H), y=s["y"].view(shape[0], -1, H))
    if kind in ("bwd", "bwd_residual"):
        rr = torch.empty(M, dtype=torch.float32, device=dev)
        tn.rmsnorm_fwd(sets[0]["x"], w, eps, rrms=rr)
        dw = torch.empty(H, dtype=torch.float32, device=dev)
        wsp = torch.empty(tn.rmsnorm_bwd_workspace_bytes(M, H), dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % nsets]
        if kind == "fwd":
            tn.rmsnorm_fwd(s["x"], w, eps, out=s["y"])
        elif kind == "fwd_residual":
            tn.rmsnorm_fwd_residual(s["x"], s["r"], w, eps, out=s["y"], residual_out=s["ro"])
        elif kind == "ln_residual":
            tn.layernorm_fwd_residual(s["x"], s["r"], w, bias, eps, out=s["y"], residual_out=s["ro"])
        elif kind == "adaln":
            tn.rmsnorm_adaln_fwd(s["x"], w, s["scale"], s["shift"], eps, out=s["y"])
        elif kind == "bwd_residual":
            tn.rmsnorm_bwd_residual(s["dy"], s["x"], s["dres"], w, rr, dh=s["y"], dw=dw, workspace=wsp)
        else:
            tn.rmsnorm_bwd(s["dy"], s["x"], w, rr, dx=s["y"], dw=dw, workspace=wsp)
    return step, nsets, copy_src, copy_dst


def copy_ceiling(per_step, dev, steps, offset=0):
    """The speed-of-light reference: rmsnorm_tuning_copy moving per_step
    bytes (half read, half written) with the forward kernels' access pattern
    and no arithmetic, over buffers rotated like the steps', timed the same
    way.  offset > 0 starts both buffers that many bytes off the 16-byte
    grid, so every access is an unaligned 16-byte one, as for rows off the
    grid."""
    import torch

    import transformer_normalization_amd as tn

    half = max(16, (per_step // 2) // 16 * 16)
    nsets = max(2, -(-ROTATION_BYTES // (2 * half)))
    src = [torch.empty(half + 16, dtype=torch.uint8, device=dev).fill_(1)[offset:offset + half] for _ in range(nsets)]
    dst = [torch.empty(half + 16, dtype=torch.uint8, device=dev)[offset:offset + half] for _ in range(nsets)]
    for i in range(50):
        tn.copy_reference(src[i % nsets], dst[i % nsets])
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        tn.copy_reference(src[i % nsets], dst[i % nsets])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    gbs = 2 * half / (ms * 1e-3) / 1e9
    return {"value": round(gbs, 2), "unit": "GB/s", "ms_per_step": round(ms, 6), "bytes": 2 * half,
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "kind": ("16-byte non-temporal copy, 256-thread workgroups of 8 KiB (rmsnorm_tuning_copy)"
                     + (f", both buffers {offset} bytes off the 16-byte grid" if offset else ""))}


def device_provenance(dev) -> dict:
    """What ran the step: the device's architecture name and compute-unit
    count as the runtime reports them, the HIP version torch was built
    against, the installed ROCm release and the host's CPU count."""
    import torch
    props = torch.cuda.get_device_properties(dev)
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                rocm = f.read().strip()
            break
        except OSError:
            pass
    return {"name": props.name, "gcnArchName": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "wave_size": getattr(props, "warp_size", None),
            "hbm_bytes": props.total_memory,
            "hip": torch.version.hip, "rocm": rocm, "torch": torch.__version__, "host_nproc": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="fwd_bf16_8192x4096", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=18.0, help="oracle time budget, both thread counts together (0 skips it)")
    ap.add_argument("--graph", action="store_true", help="launch the timed steps from captured HIP graphs")
    ap.add_argument("--no-graph-leg", action="store_true",
                    help="skip the second timing of the same steps launched from captured HIP graphs")
    ap.add_argument("--geom", default="",
                    help="development: forced launch geometry, four integers as rmsnorm_tuning_set_geometry takes")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip timing the speed-of-light copy of the same bytes")
    ap.add_argument("--copy-reference", action="store_true",
                    help="also run a plain device copy of known size (for scaling HBM counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc counter_collection.csv files")
    args = ap.parse_args()

    if args.summarize_pmc:
        sys.stdout.write(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (rows shard across GPUs with no "
              "communication, so per-GPU throughput is the one-GPU figure)", file=sys.stderr)
        sys.exit(2)
    if args.graph and args.steps % GRAPH_BLOCK:
        print(f"--graph times whole blocks of {GRAPH_BLOCK} steps: --steps must be a multiple", file=sys.stderr)
        sys.exit(2)

    import torch

    import synthetic
    import transformer_normalization_amd as tn

    if not os.path.exists(tn.LIB_PATH):
        from transformer_normalization_amd import build as hipbuild
        hipbuild.build()
    tn.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    name, weighted = WORKLOADS[args.workload]
    spec = dict(synthetic.WORKLOADS[name])
    spec["name"] = name
    kind = spec["kind"]
    if args.geom:
        parts = [int(v) for v in args.geom.split(",")]
        tn.set_geometry("bwd" if kind.startswith("bwd") else "rope" if kind == "rope" else "fwd", *parts)

    dev = torch.device("cuda:0")
    per_step = algorithmic_bytes(spec, weighted)
    step, nsets, copy_src, copy_dst = setup_steps(spec, weighted, dev, per_step)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        step(i)
    if args.copy_reference:
        for _ in range(5):
            copy_dst.copy_(copy_src)
    torch.cuda.synchronize()

    def capture_graphs():
        # block b holds steps b*GRAPH_BLOCK .. (b+1)*GRAPH_BLOCK-1, so the
        # buffer rotation is that of eager launches; blocks whose first step
        # falls on the same buffer set share one graph
        distinct = nsets // math.gcd(nsets, GRAPH_BLOCK)
        distinct = min(distinct, args.steps // GRAPH_BLOCK)
        cap = torch.cuda.Stream(dev)
        out = []
        for b in range(distinct):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for i in range(b * GRAPH_BLOCK, (b + 1) * GRAPH_BLOCK):
                    step(i)
            out.append(g)
        for g in out:  # one untimed replay of each
            g.replay()
        torch.cuda.synchronize()
        return out

    stream = torch.cuda.current_stream(dev)

    def timed(graphs):
        """ms per step over exactly args.steps steps, HIP events on `stream`
        after a synchronisation on both sides."""
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        if graphs:
            for b in range(args.steps // GRAPH_BLOCK):
                graphs[b % len(graphs)].replay()
        else:
            for i in range(args.steps):
                step(i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    graphs = capture_graphs() if args.graph else []
    ms = timed(graphs)
    gbs = per_step / (ms * 1e-3) / 1e9
    rows = step_rows(spec)

    # Spread: a second pass timed in blocks of SPREAD_BLOCK steps, an event
    # at each block boundary (an event after every step adds its own cost to
    # the step it follows: about 2.5 us on a 23 us forward), so each block
    # gives one per-step time.
    spread = None
    n_blocks = min(args.steps // SPREAD_BLOCK, 50)
    if not graphs and n_blocks >= 2:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_blocks + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for b in range(n_blocks):
            for i in range(b * SPREAD_BLOCK, (b + 1) * SPREAD_BLOCK):
                step(i)
            evs[b + 1].record(stream)
        torch.cuda.synchronize()
        per = sorted(evs[b].elapsed_time(evs[b + 1]) / SPREAD_BLOCK for b in range(n_blocks))
        mean = sum(per) / n_blocks
        sd = (sum((v - mean) ** 2 for v in per) / (n_blocks - 1)) ** 0.5
        med = per[n_blocks // 2] if n_blocks % 2 else 0.5 * (per[n_blocks // 2 - 1] + per[n_blocks // 2])
        spread = {"blocks": n_blocks, "steps_per_block": SPREAD_BLOCK, "ms_min": round(per[0], 6),
                  "ms_median": round(med, 6), "ms_max": round(per[-1], 6), "ms_mean": round(mean, 6),
                  "ms_stddev": round(sd, 6), "gbs_at_median": round(per_step / (med * 1e-3) / 1e9, 2),
                  "how": "per-step time of each block of a second eager pass, HIP events at block boundaries"}

    traffic = stored_traffic(args.workload)
    if kind == "rope":
        config = {"workload": args.workload, "batch": spec["B"], "seq_len": spec["S"], "heads": spec["NH"],
                  "head_dim": spec["D"], "table_dtype": spec["tdtype"]}
    else:
        config = {"workload": args.workload, "M": spec["M"], "H": spec["H"], "eps": spec["eps"],
                  "weight": spec["wdtype"] if weighted else None}
    config.update(buffer_sets=nsets, bytes_per_step=per_step, launch="graph" if graphs else "eager")
    if args.geom:
        config["geom"] = args.geom
    result = {
        "metric": METRIC if args.workload == "fwd_bf16_8192x4096" else f"{args.workload} achieved HBM GB/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec["dtype"],
        "data": "synthetic",
        "config": config,
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "rows_per_s": round(rows / (ms * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
    }
    if spread is not None:
        result["spread"] = spread
    if not graphs and not args.no_graph_leg and args.steps % GRAPH_BLOCK == 0:
        # the same steps launched from captured HIP graphs, as a serving loop
        # or a captured training step launches them: no host launch gap
        # between consecutive kernels
        gms = timed(capture_graphs())
        ggbs = per_step / (gms * 1e-3) / 1e9
        result["graph_launch"] = {"ms_per_step": round(gms, 6), "value": round(ggbs, 2), "unit": "GB/s",
                                  "frac": round(ggbs / PEAK_HBM_GBS, 4), "steps_per_graph": GRAPH_BLOCK,
                                  "how": "the same steps replayed from captured HIP graphs, HIP events around the "
                                         "replays; value above stays the eager figure"}
    result["device"] = device_provenance(dev)
    if not args.no_ceiling:
        result["copy_ceiling"] = copy_ceiling(per_step, dev, min(args.steps, 1000))
        result["copy_ceiling"]["step_over_copy"] = round(gbs / result["copy_ceiling"]["value"], 4)
        if kernel_kind(spec).endswith("_offgrid"):
            # rows off the grid make unaligned 16-byte accesses: the copy
            # that makes the same ones
            un = copy_ceiling(per_step, dev, min(args.steps, 1000), offset=2)
            un["step_over_copy"] = round(gbs / un["value"], 4)
            result["copy_ceiling_unaligned"] = un
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(spec, weighted, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
