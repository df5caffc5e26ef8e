"""The C ABI from a plain C11 caller (no GPU needed): tests/abi_consumer.c is compiled by gcc
against include/psffn.h alone (a C translation unit, so the header must be valid C), linked
against the in-tree libpsffn.so, and run.  It checks sizes, status strings and host-side argument
rejection; every call that takes device pointers is invalid, so nothing is enqueued."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "activation_sparse_ffn_psffn_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_caller_uses_the_abi(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "libpsffn.so")):
        pytest.skip("libpsffn.so not built")
    exe = str(tmp_path / "abi_consumer")
    subprocess.check_call([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
                           os.path.join(ROOT, "tests", "abi_consumer.c"), "-o", exe,
                           "-L", LIBDIR, "-lpsffn", "-Wl,-rpath," + LIBDIR, "-lm"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed" in r.stdout
