"""Throughput of the gfx950 RMSNorm library on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one launch of the library on one batch of seeded synthetic input
already resident in HBM.  Batches rotate over enough buffer sets (>= 1 GiB per
cycle) that no step finds its data in the last-level cache.  W untimed steps,
then exactly K steps between two synchronisations, timed with HIP events on
the stream the kernels are launched on.  One JSON line is printed.

Workloads (default: the forward at bf16 M=8192 H=4096):
  fwd_bf16_8192x4096, fwd_f32_64x512, fwd_bf16_32768x2048, fwd_bf16_32768x2048_noweight,
  fwd_f16_32768x2048_outliers, fwd_residual_bf16_16384x8192, bwd_bf16_8192x6144,
  bwd_residual_bf16_16384x8192, adaln_bf16_2x4096x2048_batchcond, adaln_bf16_2x4096x2048_tokencond

The CPU baseline is the float64 oracle run on the host over a sample of the
same workload (reported beside the GPU figure, never a target).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak
METRIC = "RMSNorm fwd achieved HBM GB/s (% of peak) + rows/s, bf16 M=8192 H=4096"
PROFILE_DIR = os.path.join(ROOT, "profiles")
ROTATION_BYTES = 1 << 30


_FWD = ("numerics.hpp", "fwd_kernels.hpp", "fwd_table.hpp", "kernel_tables.hpp")
_BWD = ("numerics.hpp", "bwd_kernels.hpp", "bwd_table.hpp", "kernel_tables.hpp", "kernels_bwd.hip")
KERNEL_SOURCES = {
    "fwd": _FWD + ("kernels_fwd.hip", "rmsnorm_api.hip"),
    "fwd_residual": _FWD + ("kernels_fwd_residual.hip", "rmsnorm_api.hip"),
    "bwd": _BWD + ("rmsnorm_api.hip",),
    "bwd_residual": _BWD + ("kernels_bwd_residual.hip", "rmsnorm_api.hip"),
    "adaln": _FWD + ("kernels_adaln.hip", "rmsnorm_api.hip"),
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
    if fields.get("kernel_source_digest") != kernel_source_digest(synthetic.WORKLOADS[name]["kind"]):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(kind, M, H, esize, wsize, weighted, cond_rows=0):
    """Bytes the method must move once: inputs, weight, outputs, rrms if used."""
    mat = M * H * esize
    w = H * wsize if weighted else 0
    if kind == "fwd":
        return 2 * mat + w
    if kind == "fwd_residual":
        return 4 * mat + w
    if kind == "bwd":
        # x, dy read; dx written; rrms read; w read; dw written (float32)
        return 3 * mat + M * 4 + w + H * 4
    if kind == "bwd_residual":
        # as bwd, plus the residual-stream gradient read
        return 4 * mat + M * 4 + w + H * 4
    if kind == "adaln":
        # x read, y written, w and the scale/shift rows read once
        return 2 * mat + w + 2 * cond_rows * H * wsize
    raise ValueError(kind)


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
}


def cpu_baseline(spec, kind, weighted, seconds):
    """The oracle as it stands, single-threaded, over the workload's rows
    repeated until `seconds` have passed; reported in GB/s of the same
    algorithmic bytes."""
    import numpy as np

    import oracle
    import synthetic

    rows = min(spec["M"], 1024)
    d = synthetic.make_inputs(spec["name"], rows=rows)
    w = d["w"] if weighted else None
    eps = float(np.float32(spec["eps"]))
    if kind in ("bwd", "bwd_residual"):
        _, r = oracle.fwd(d["x"], w, eps, d["dtype"], d["wdtype"])
        r32 = r.astype(np.float32)
    t0 = time.perf_counter()
    passes = 0
    while True:
        if kind == "fwd":
            oracle.fwd(d["x"], w, eps, d["dtype"], d["wdtype"])
        elif kind == "adaln":
            oracle.adaln_fwd(d["x"], w, d["scale"], d["shift"], d["rows_per_cond"], eps, d["dtype"], d["wdtype"],
                             d["wdtype"])
        elif kind == "fwd_residual":
            oracle.fwd_residual(d["x"], d["r"], w, eps, d["dtype"], d["wdtype"])
        elif kind == "bwd_residual":
            oracle.bwd_residual(d["dy"], d["x"], d["dres"], w, r32, d["dtype"], d["wdtype"])
        else:
            oracle.bwd(d["dy"], d["x"], w, r32, d["dtype"], d["wdtype"])
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    es = synthetic.element_size(d["dtype"])
    ws = synthetic.element_size(d["wdtype"])
    crows = d["scale"].shape[0] if kind == "adaln" else 0
    nbytes = algorithmic_bytes(kind, rows, spec["H"], es, ws, weighted, crows) * passes
    return {
        "value": round(nbytes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {rows} of {spec['M']} rows, {passes} passes in {el:.1f} s, float64, one thread",
        "rows_per_s": round(rows * passes / el, 1),
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
    es = synthetic.element_size(spec["dtype"])
    ws = synthetic.element_size(spec["wdtype"])
    known_kib = spec["M"] * spec["H"] * es / 1024.0
    kernel_key = {"fwd": "rmsnorm_fwd_kernel", "fwd_residual": "rmsnorm_fwd_kernel", "adaln": "rmsnorm_fwd_kernel",
                  "bwd": "rmsnorm_bwd_kernel", "bwd_residual": "rmsnorm_bwd_kernel"}[spec["kind"]]

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
    crows = -(-spec["M"] // spec.get("rows_per_cond", 1)) if spec["kind"] == "adaln" else 0
    alg = algorithmic_bytes(spec["kind"], spec["M"], spec["H"], es, ws, weighted, crows)
    lines = [
        f"# HBM traffic per launch of {kname}",
        f"# workload {workload}: M={spec['M']} H={spec['H']} {spec['dtype']}",
        "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 --pmc runs of",
        f"#   python3 bench.py --workload {workload} --cpu-seconds 0 --steps 20 --warmup 10 --copy-reference",
        "# each scaled by the same counter's reading for device copies of the x tensor",
        f"# ({known_kib:.0f} KiB read and written per copy) in the same run; summary made by",
        f"#   python3 bench.py --workload {workload} --summarize-pmc <fetch csv> <write csv>",
        f"kernel_source_digest: {kernel_source_digest(spec['kind'])}",
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="fwd_bf16_8192x4096", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget (0 skips it)")
    ap.add_argument("--geom", default="", help="development: forced launch geometry 'vpt,wpr,rpw,grid'")
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

    import numpy as np
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
        tn.set_geometry("bwd" if kind.startswith("bwd") else "fwd", *parts)

    dev = torch.device("cuda:0")
    d = synthetic.make_inputs(name)
    dt = d["dtype"]
    M, H = spec["M"], spec["H"]
    es, ws = synthetic.element_size(dt), synthetic.element_size(d["wdtype"])

    def up(a, fmt):
        a = np.ascontiguousarray(a)
        if fmt == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    crows = d["scale"].shape[0] if kind == "adaln" else 0
    per_set = algorithmic_bytes(kind, M, H, es, ws, weighted, crows)
    nsets = max(2, -(-ROTATION_BYTES // per_set))
    x0 = up(d["x"], dt)
    w = up(d["w"], d["wdtype"]) if weighted else None
    sets = []
    for i in range(nsets):
        s = {"x": x0 if i == 0 else x0.clone(), "y": torch.empty_like(x0)}
        if kind == "fwd_residual":
            r0 = up(d["r"], dt) if i == 0 else sets[0]["r"].clone()
            s.update(r=r0, ro=torch.empty_like(x0))
        if kind in ("bwd", "bwd_residual"):
            dy0 = up(d["dy"], dt) if i == 0 else sets[0]["dy"].clone()
            s.update(dy=dy0)
        if kind == "bwd_residual":
            g0 = up(d["dres"], dt) if i == 0 else sets[0]["dres"].clone()
            s.update(dres=g0)
        if kind == "adaln":
            rpc = spec["rows_per_cond"]
            shape = (M // rpc, 1, H) if rpc > 1 else (1, M, H)
            sc0 = up(d["scale"], d["wdtype"]).view(*shape) if i == 0 else sets[0]["scale"].clone()
            sh0 = up(d["shift"], d["wdtype"]).view(*shape) if i == 0 else sets[0]["shift"].clone()
            s.update(scale=sc0, shift=sh0, x=s["x"].view(shape[0], -1, H), y=s["y"].view(shape[0], -1, H))
        sets.append(s)
    del d
    eps = spec["eps"]
    if kind in ("bwd", "bwd_residual"):
        rr = torch.empty(M, dtype=torch.float32, device=dev)
        tn.rmsnorm_fwd(sets[0]["x"], w, eps, rrms=rr)
        dw = torch.empty(H, dtype=torch.float32, device=dev)
        wsp = torch.empty(tn.rmsnorm_bwd_workspace_bytes(M, H), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        s = sets[i % nsets]
        if kind == "fwd":
            tn.rmsnorm_fwd(s["x"], w, eps, out=s["y"])
        elif kind == "fwd_residual":
            tn.rmsnorm_fwd_residual(s["x"], s["r"], w, eps, out=s["y"], residual_out=s["ro"])
        elif kind == "adaln":
            tn.rmsnorm_adaln_fwd(s["x"], w, s["scale"], s["shift"], eps, out=s["y"])
        elif kind == "bwd_residual":
            tn.rmsnorm_bwd_residual(s["dy"], s["x"], s["dres"], w, rr, dh=s["y"], dw=dw, workspace=wsp)
        else:
            tn.rmsnorm_bwd(s["dy"], s["x"], w, rr, dx=s["y"], dw=dw, workspace=wsp)

    for i in range(args.warmup):
        step(i)
    if args.copy_reference:
        for _ in range(5):
            sets[1]["y"].copy_(sets[0]["x"])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps
    gbs = per_set / (ms * 1e-3) / 1e9

    traffic = stored_traffic(args.workload)
    result = {
        "metric": METRIC if args.workload == "fwd_bf16_8192x4096" else f"RMSNorm {args.workload} achieved HBM GB/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "H": H, "eps": eps,
                   "weight": spec["wdtype"] if weighted else None, "buffer_sets": nsets,
                   "bytes_per_step": per_set},
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "rows_per_s": round(M / (ms * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
    }
    if args.geom:
        result["config"]["geom"] = args.geom
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(spec, kind, weighted, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
