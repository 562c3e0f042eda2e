"""Host-side logic of bench.py (no GPU): algorithmic bytes per step, the
one-GPU guard, and the HBM-traffic summary built from counter CSV files."""

from __future__ import annotations

import csv
import os
import subprocess
import sys

import pytest

import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def spec(name):
    return dict(synthetic.WORKLOADS[name])


def test_algorithmic_bytes_of_the_named_workloads():
    # x read + y written (2 bytes each) + the weight once
    assert bench.algorithmic_bytes(spec("fwd_bf16_8192x4096"), True) == 2 * 8192 * 4096 * 2 + 4096 * 2
    assert bench.algorithmic_bytes(spec("fwd_bf16_8192x4096"), True) == 134_225_920
    assert bench.algorithmic_bytes(spec("fwd_f32_64x512"), True) == 264_192
    assert bench.algorithmic_bytes(spec("fwd_bf16_32768x2048"), True) == 268_439_552
    assert bench.algorithmic_bytes(spec("fwd_bf16_32768x2048"), False) == 268_435_456
    # x, r read; y, residual_out written
    assert bench.algorithmic_bytes(spec("fwd_residual_bf16_16384x8192"), True) == 1_073_758_208
    # x, dy read; dx written; rrms read; w read; dw written
    assert bench.algorithmic_bytes(spec("bwd_bf16_8192x6144"), True) == 302_059_520
    assert bench.algorithmic_bytes(spec("bwd_residual_bf16_16384x8192"), True) == \
        4 * 16384 * 8192 * 2 + 16384 * 4 + 8192 * 2 + 8192 * 4
    # per-batch AdaLN reads 2 conditioning rows of scale and of shift
    assert bench.algorithmic_bytes(spec("adaln_bf16_2x4096x2048_batchcond"), True) == \
        2 * 8192 * 2048 * 2 + 2048 * 2 + 2 * 2 * 2048 * 2
    # RoPE: x and out, plus half of each float32 table row
    assert bench.algorithmic_bytes(spec("rope_bf16_2x8064x32x64"), True) == \
        2 * 2 * 8064 * 32 * 64 * 2 + 2 * 8064 * 32 * 4
    # residual + LayerNorm: x, r read, y and residual_out written, w and b once
    assert bench.algorithmic_bytes(spec("ln_residual_f32_16384x1024"), True) == 4 * 16384 * 1024 * 4 + 2 * 1024 * 4
    # a leading sample scales the row-proportional part only
    s = spec("fwd_bf16_8192x4096")
    assert bench.algorithmic_bytes(s, True, rows=1024) == 2 * 1024 * 4096 * 2 + 4096 * 2


def test_every_bench_workload_names_a_kernel_and_sources():
    for w, (name, _) in bench.WORKLOADS.items():
        kind = bench.kernel_kind(synthetic.WORKLOADS[name])
        assert kind in bench.KERNEL_KEY and kind in bench.KERNEL_SOURCES, w
        assert len(bench.kernel_source_digest(kind)) == 16


def test_ragged_forward_runs_the_off_grid_kernels():
    # rows of 8194 bytes leave the 16-byte grid; rows of 8192 bytes do not
    assert bench.kernel_kind(spec("fwd_bf16_8192x4097")) == "fwd_offgrid"
    assert bench.KERNEL_KEY["fwd_offgrid"] == "rmsnorm_fwd_kernel"
    assert bench.kernel_kind(spec("fwd_bf16_8192x4096")) == "fwd"
    assert bench.kernel_kind(spec("fwd_f32_64x512")) == "fwd"
    assert bench.algorithmic_bytes(spec("fwd_bf16_8192x4097"), True) == 2 * 8192 * 4097 * 2 + 4097 * 2
    # and so does the backward on them
    assert bench.kernel_kind(spec("bwd_bf16_8192x4097")) == "bwd_offgrid"
    assert bench.KERNEL_KEY["bwd_offgrid"] == "rmsnorm_bwd_kernel"
    assert bench.kernel_kind(spec("bwd_bf16_8192x6144")) == "bwd"


@pytest.mark.parametrize("argv,needle", [(["--gpus", "2"], "one GPU"), (["--graph", "--steps", "150"], "multiple")])
def test_guards_exit_before_touching_a_device(argv, needle):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=120)
    assert p.returncode == 2 and needle in p.stderr


def _counter_csv(path, counter, kernel, kernel_value, copy_value, copy_grid=4096):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size"])
        wr.writeheader()
        for _ in range(3):
            wr.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": kernel_value,
                         "Grid_Size": 1})
        wr.writerow({"Kernel_Name": "copyBuffer", "Counter_Name": counter, "Counter_Value": copy_value,
                     "Grid_Size": copy_grid})
        wr.writerow({"Kernel_Name": "copyBuffer", "Counter_Name": counter, "Counter_Value": 1.0, "Grid_Size": 8})


def test_traffic_summary_scales_by_the_copy_reference(tmp_path):
    w = "fwd_bf16_8192x4096"
    known_kib = 8192 * 4096 * 2 / 1024.0
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the fetch counter reads half of the copied bytes, the write counter all
    _counter_csv(fetch, "FETCH_SIZE", "rmsnorm_fwd_kernel<...>", known_kib / 2, known_kib / 2)
    _counter_csv(write, "WRITE_SIZE", "rmsnorm_fwd_kernel<...>", known_kib, known_kib)
    text = bench.summarize_pmc(str(fetch), str(write), w)
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line and not line.startswith("#"))
    assert float(fields["fetch_scale"]) == pytest.approx(2.0)
    assert float(fields["write_scale"]) == pytest.approx(1.0)
    assert float(fields["hbm_bytes_per_launch"]) == pytest.approx(2 * known_kib * 1024, rel=1e-9)
    assert int(fields["algorithmic_bytes_per_launch"]) == 134_225_920
    assert fields["kernel_source_digest"].strip() == bench.kernel_source_digest("fwd")
