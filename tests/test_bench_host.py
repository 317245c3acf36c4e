"""Host-side checks of bench.py (no GPU): the one-GPU contract, the algorithmic
bytes that the roofline line divides by the measured time, and the guard that
reports counter-derived traffic only for the kernel sources it was taken on."""
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench
from block_scaled_fp4_gemv_amd import synth as sy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# bytes per weight element of the codes and of the block scales, and the
# tensor scales per expert (NVFP4 only), from the format definitions
CODE_B = {1: 0.5, 2: 0.5, 3: 1.0}
SCALE_B = {1: 1 / 16, 2: 1 / 32, 3: 4 / 128}
TAU_B = {1: 12, 2: 0, 3: 0}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name", ["decode35b", "decode753b"])
@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_algorithmic_bytes_follow_the_formats(name, fmt):
    wl = sy.WORKLOADS[name]
    H, E, F, k = wl.H, wl.E, wl.F, wl.k
    expert = 3 * F * H * (CODE_B[fmt] + SCALE_B[fmt]) + TAU_B[fmt]
    nb = bench.algorithmic_bytes(wl, fmt)
    assert nb["expert"] == k * expert
    assert nb["router"] == E * H * 4
    # activations: x read by the router and by gate/up, h written and read, out
    # written, the routing (index + weight per pair) written and read
    act = 3 * H * 2 + 2 * k * F * 2 + 2 * k * 8
    assert nb["layer_total"] == k * expert + E * H * 4 + act


def test_decode35b_nvfp4_layer_bytes():
    # the figure the headline roofline divides by: 8 experts of three 512 x 2048
    # NVFP4 matrices (4 bits + one E4M3 byte per 16 weights, three fp32 tensor
    # scales), the 256 x 2048 fp32 router, and the activations
    assert bench.algorithmic_bytes(sy.WORKLOADS["decode35b"], 1)["layer_total"] == 16281824


def test_measured_traffic_only_for_the_recorded_sources(tmp_path, monkeypatch):
    # the committed record matches the committed kernel sources
    got = bench.measured_traffic(40, 40)
    rec = json.load(open(os.path.join(ROOT, "profiles", "decode35b_traffic.json")))
    assert got == int(rec["decode_layer_read_bytes"] + rec["decode_layer_write_bytes"])
    assert got > 16281824  # at least the algorithmic bytes
    # a run over fewer layers than the default is not the measured configuration
    assert bench.measured_traffic(8, 40) is None
    # a changed source (one byte appended to a kernel file) voids the record
    shutil.copytree(os.path.join(ROOT, "profiles"), tmp_path / "profiles")
    src = os.path.join(ROOT, "block_scaled_fp4_gemv_amd", "csrc")
    dst = tmp_path / "block_scaled_fp4_gemv_amd" / "csrc"
    shutil.copytree(src, dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(40, 40) == got
    with open(dst / "combine.hip", "a") as f:
        f.write("\n")
    assert bench.measured_traffic(40, 40) is None
