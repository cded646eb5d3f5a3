"""Host build and run of tile_map_check.cpp: the grouped GEMMs' workgroup ->
(m-tile, n-tile) map, compiled for the CPU from the library's own header, must
cover every tile exactly once, keep each XCD's valid positions a prefix, give
no XCD more than ceil(total/8) m-tiles, keep large m-tiles contiguous per XCD
and put the reserved smallest tiles last; the compact tiles' row split between
the two wave rows must cover every row within the stage and the accumulators.
No GPU needed."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("tile_map") / "tile_map_check")
    cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O2",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "combine_top_route_expert_amd", "csrc"),
           os.path.join(HERE, "tile_map_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.mark.parametrize("seed", [2024, 7])
def test_tile_map_properties(checker, seed):
    r = subprocess.run([checker, str(seed), "2000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert "0 failures" in r.stdout
