"""Host check of the grouped-GEMM schedule (csrc/schedule.h, used by the plan
kernel): compiled with the system C++ compiler and run over seeded expert size
patterns (uniform, Zipf-like, one hot expert, mostly empty, just over a
multiple of the M-tile), M-tiles of 256 / 128 / 64 rows, 1-120 N-tiles, 8-256
workgroups and K-split caps of 1-8. Every tile must be scheduled exactly once
(or each K-range of a split last-round tile once), each XCD's entries must
fill a prefix of its slots, the split round must take at most one short entry
per workgroup, and the K-ranges must partition K."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_schedule_covers_every_tile_once(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "check_schedule"
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "mixture_experts_ffn_top_amd", "csrc"),
                    os.path.join(ROOT, "tests", "schedule", "check_schedule.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300).stdout.strip()
    assert out.startswith("ok "), out
    assert int(out.split()[1]) > 300 and int(out.split()[2]) >= 50 and int(out.split()[3]) >= 50, out
