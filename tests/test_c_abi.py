"""The boundary from plain C: tests/c_abi/check_abi.c includes include/fbd.h
as ISO C99 (compiled with -pedantic -Werror), links against the built
libfbd.so and checks workspace sizes, status messages and the host-side
argument checks (every call it makes is rejected before anything is
enqueued, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "fwd_bwd_double_amd")
SRC = os.path.join(ROOT, "tests", "c_abi", "check_abi.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_and_library_from_c(tmp_path):
    assert os.path.exists(os.path.join(LIBDIR, "libfbd.so")), "build the library first"
    exe = tmp_path / "check_abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), SRC, "-L", LIBDIR, "-lfbd",
                    f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "check_abi: ok" in r.stdout
