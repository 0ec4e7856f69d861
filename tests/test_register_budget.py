"""The walk kernels keep the register budget that lets eight waves reside on
each SIMD (compiled here for gfx950; no GPU needed).

A kernel's scalar register count is its highest scalar register used, and on
MI355X it limits resident waves below what the compiler's occupancy estimate
reports: measured with per-wave timestamps, the walk held 8 waves per SIMD at
70 scalar registers, 7 at 90 and 6 at 96, and ran 7% faster at 68 than at 90.
The walk's assembly loop uses fixed scalar registers (s16..s49); a change that
moved them up, or that grew the compiler's own use, would cost resident waves
without changing any result, so the budget is checked here."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "barnes_hut_tree_amd", "csrc", "traverse.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

MAX_SGPR = 76    # next free scalar register, at most (8 waves measured at 70)
MAX_VGPR = 64    # 512 vector registers per SIMD lane / 8 waves


@pytest.fixture(scope="module")
def walk_kernels(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "traverse.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", SRC, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    text = open(out).read()
    kernels = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
        body = m.group(2)
        sgpr = int(re.search(r"\.amdhsa_next_free_sgpr (\d+)", body).group(1))
        vgpr = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", body).group(1))
        kernels[m.group(1)] = (sgpr, vgpr)
    # the walk itself (k_walk<...>), not its record-copy kernel k_walk_nodes
    return {k: v for k, v in kernels.items() if "k_walkI" in k}


def test_every_walk_kernel_fits_eight_waves(walk_kernels):
    # 2 (soft) x 2 (self) x 2 (count) x 2 (vote) x 2 (unsorted) instantiations
    assert len(walk_kernels) == 32, sorted(walk_kernels)
    over = {k: v for k, v in walk_kernels.items() if v[0] > MAX_SGPR or v[1] > MAX_VGPR}
    assert not over, over
