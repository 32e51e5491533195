"""The kernels' copy offsets evaluated on the host (no GPU): full coverage of every tile
copy, fine-stage reads confined to the selected cube or, for a plan entry outside [0, C),
past the end of the head's region, where the buffer range check returns zeros, the
one-call path's K and V copies from the token grid reading exactly what the cube-ordered copy
reads (padded V slots reading zeros), and its LDS transpose reads handing every P V MFMA lane
the V^T elements it needs, on 64 distinct banks per half wavefront."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_copy_offsets_on_the_host(tmp_path):
    exe = tmp_path / "tile_bounds"
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "video_diffusion_dit_amd", "csrc"),
           os.path.join(ROOT, "tests", "c", "tile_bounds.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
