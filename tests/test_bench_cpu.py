"""CPU tests of bench.py's command line: the multi-GPU request is refused with a
message, and the kernel-trace summary groups dispatches by kernel and grid."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, BENCH, "--gpus", str(n)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_trace_summary_groups_by_kernel_and_grid(tmp_path):
    rows = [
        ("attnblk::(anonymous namespace)::flash_fwd_f16_d128(attnblk::FlashArgs)", 524288, 512, 0, 1_000_000),
        ("attnblk::(anonymous namespace)::flash_fwd_f16_d128(attnblk::FlashArgs)", 524288, 512, 0, 3_000_000),
        ("attnblk::(anonymous namespace)::flash_fwd_f16_d128(attnblk::FlashArgs)", 262144, 512, 0, 500_000),
        ("attnblk::(anonymous namespace)::gemm_f16_nt(attnblk::GemmArgs)", 786432, 512, 10, 810),
    ]
    csv = tmp_path / "trace.csv"
    with open(csv, "w") as f:
        f.write("Kernel_Name,Grid_Size_X,Grid_Size_Y,Grid_Size_Z,Workgroup_Size_X,Start_Timestamp,End_Timestamp\n")
        for name, g, w, t0, t1 in rows:
            f.write(f"\"{name}\",{g},1,1,{w},{t0},{t1}\n")
    r = subprocess.run([sys.executable, BENCH, "--trace-summary", str(csv)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    assert lines[0].startswith("| kernel | grid threads")
    body = {tuple(c.strip() for c in ln.strip("|").split("|")[:4]): ln for ln in lines[2:]}
    # two dispatches of 1 ms and 3 ms: mean 2 ms, min 1, max 3
    big = body[("flash_fwd_f16_d128", "524288", "512", "2")]
    assert "| 2.0000 | 1.0000 | 3.0000 |" in big
    assert ("flash_fwd_f16_d128", "262144", "512", "1") in body
    assert ("gemm_f16_nt", "786432", "512", "1") in body
    # sorted by total time, largest first
    assert lines[2].startswith("| flash_fwd_f16_d128 | 524288")
