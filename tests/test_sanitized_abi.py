"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Builds the library once more with the host half of every source instrumented
(each -fsanitize= applies to the host compilation only; device code is built as
usual), then runs against it the C99 program that exercises the header's size
queries, status strings and argument checks, and the Python ABI tests
(test_abi.py) with the sanitizer runtime preloaded.  Any sanitizer report fails
the run.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_diffusion_dit_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm compilers not available")


def _asan_runtime() -> str:
    return subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True).stdout.strip()


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    out = tmp_path_factory.mktemp("asan")
    sys.path.insert(0, os.path.join(ROOT, "video_diffusion_dit_amd"))
    import build  # the package's own source list and flags
    sys.path.pop(0)

    def one(src):
        obj = str(out / (os.path.splitext(src)[0] + ".o"))
        cmd = [HIPCC, *[f for f in build.FLAGS if f != "-O3"], "-O1", "-g", *SAN, "-c", os.path.join(CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        return obj
    with ThreadPoolExecutor(len(build.SOURCES)) as ex:
        objs = list(ex.map(one, build.SOURCES))
    lib = str(out / "libwfattn.so")
    r = subprocess.run([HIPCC, "--offload-arch=" + build.ARCH, "-shared", "-fPIC", "-shared-libsan", *SAN, *objs,
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return lib


def _env(lib):
    env = dict(os.environ)
    env.update(ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98", WF_LIB_PATH=lib)
    return env


def test_c_program_under_sanitizers(sanitized_lib, tmp_path):
    rt_dir = os.path.dirname(_asan_runtime())
    exe = str(tmp_path / "abi_from_c")
    lib_dir = os.path.dirname(sanitized_lib)
    r = subprocess.run([CLANG, "-std=c99", "-Wall", "-Wextra", "-Werror", "-g", "-fsanitize=address,undefined",
                        "-shared-libsan", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", lib_dir, "-lwfattn",
                        f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{rt_dir}", "-lm", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=_env(sanitized_lib))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr


def test_python_abi_tests_under_sanitizers(sanitized_lib):
    env = _env(sanitized_lib)
    env["ASAN_OPTIONS"] = "detect_leaks=0:exitcode=99"   # the interpreter keeps its allocations to the end
    env["LD_PRELOAD"] = _asan_runtime()
    probe = subprocess.run([sys.executable, "-c", "import video_diffusion_dit_amd as w; print(w.LIB_PATH)"],
                           capture_output=True, text=True, env=env, cwd=ROOT, timeout=120)
    assert probe.returncode == 0 and probe.stdout.strip() == sanitized_lib, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
