"""The kernels' per-wave FULL block ranges agree with the block classifier block by block.

Host build of csrc/block_class.h (the same header every kernel includes) with g++; the check
program walks every block of many square and rectangular problems.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "online_softmax_fwd_flash_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_full_block_ranges_match_block_class(tmp_path):
    exe = str(tmp_path / "check_full_ranges")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC,
                    os.path.join(HERE, "native", "check_full_ranges.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout
