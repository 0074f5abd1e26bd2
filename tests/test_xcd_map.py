"""Workgroup-id maps of the attention kernels, checked on the host (no GPU).

tests/xcd_map_check.cpp includes the library's internal header and runs both maps
(xcd_remap: one contiguous range of query blocks per XCD; xcd_head_remap: every XCD
on the same head at a time, each on its own slice) over a grid of head counts and
query-block counts, including the video shapes (12 x 256, 40 x 591, 24 x 929),
grids smaller than the eight XCDs and counts that leave remainders. Each map must be
a bijection with the same number of ids per XCD, and the head-major one must walk
the heads in order on every XCD, each head's slice ascending and contiguous.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path_factory.mktemp("xcdmap") / "xcd_map_check"
    subprocess.run([hipcc, "-O1", "-std=c++17", "-Wno-unused-command-line-argument",
                    "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "block_sparse_attention_ibcs_amd", "csrc"),
                    os.path.join(HERE, "xcd_map_check.cpp"), "-o", str(exe)], check=True, capture_output=True)
    return str(exe)


def test_maps_are_balanced_bijections(checker):
    grids = [(nbh, nqb) for nbh in (1, 2, 3, 5, 7, 8, 9, 12, 13, 24, 40, 64)
             for nqb in list(range(1, 41)) + [63, 64, 65, 255, 256, 257, 591, 929]]
    res = subprocess.run([checker], input="".join(f"{a} {b}\n" for a, b in grids), capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip() == f"ok {len(grids)} grids"


def test_checker_catches_a_broken_map(checker, tmp_path):
    """The checker itself fails on a map that is not a bijection: the same program
    built against a header whose head-major map sends every id of XCD 1 to XCD 0's."""
    src = open(os.path.join(ROOT, "block_sparse_attention_ibcs_amd", "csrc", "ab_internal.h")).read()
    planted = src.replace("const int x = pid % kXcds, j = pid / kXcds;  // XCD and position in its sequence",
                          "const int x = (pid % kXcds) == 1 ? 0 : pid % kXcds, j = pid / kXcds;")
    assert planted != src
    (tmp_path / "ab_internal.h").write_text(planted)
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = tmp_path / "broken"
    subprocess.run([hipcc, "-O1", "-std=c++17", "-Wno-unused-command-line-argument", "-I" + str(tmp_path),
                    "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "block_sparse_attention_ibcs_amd", "csrc"),
                    os.path.join(HERE, "xcd_map_check.cpp"), "-o", str(exe)], check=True, capture_output=True)
    res = subprocess.run([str(exe)], input="12 256\n", capture_output=True, text=True)
    assert res.returncode != 0 and "not a bijection" in res.stdout
