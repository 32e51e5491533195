"""The boundary is a C ABI: a C99 program built with gcc against include/wf_attn.h links to
libwfattn.so and gets the size queries, status strings and argument checks right (no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "video_diffusion_dit_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_and_library_from_c(tmp_path):
    assert os.path.exists(os.path.join(LIBDIR, "libwfattn.so")), "build the library first"
    exe = tmp_path / "abi_from_c"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", LIBDIR, "-lwfattn",
           f"-Wl,-rpath,{LIBDIR}", "-lm", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
