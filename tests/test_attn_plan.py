"""The balanced split plan of zha_attn at sizes where 32-bit sums would wrap (no GPU).

The plan functions (``csrc/zha_plan.hpp``, used by the attention kernel and its
merge) are compiled host-only with hipcc and checked on the CPU by
``tests/native/attn_plan_check.cpp``: at 2048 heads attending up to 2^31 - 3
tokens each (about 2^42 positions in one call) every position lies in exactly
one range, a head's segments cover its list in order, and partial slots are
unique and inside the scratch buffer.  A second build runs the same check
with the host's AddressSanitizer and UndefinedBehaviorSanitizer (signed
overflow, shifts, out-of-bounds indexing abort the check).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                    reason="hipcc not available")
def test_balanced_plan_at_overflow_sizes(tmp_path):
    exe = str(tmp_path / "attn_plan_check")
    cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "hierarchical_tree_indexed_04_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "attn_plan_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout[-4000:]
    assert ">= 2^31" in r.stdout


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                    reason="hipcc not available")
def test_balanced_plan_under_host_sanitizers(tmp_path):
    exe = str(tmp_path / "attn_plan_check_san")
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"):
        san += ["-Xarch_host", f]
    cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", *san,
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "hierarchical_tree_indexed_04_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "attn_plan_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), (r.stdout + r.stderr)[-4000:]
