"""The workgroup orders of the kernels (csrc/grid_order.h), checked on the
host: tests/native/grid_order_check.cpp includes the same header the kernels
include and checks that grouped_order is a bijection onto the token-tile x
vocabulary-group grid for every window size the planner picks, and that
xcd_remap permutes the workgroup ids."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_cross_entropy_fp32_amd", "csrc")


def test_grid_orders_are_bijections(tmp_path):
    exe = tmp_path / "grid_order_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC,
                    os.path.join(ROOT, "tests", "native", "grid_order_check.cpp"), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok "), out.stdout
