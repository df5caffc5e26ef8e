"""The layer end to end from a plain C11 caller on the GPU, with no Python or torch on the path:
tests/layer_consumer.c allocates with hipMalloc, calls psffn_workspace_init and psffn_layer at
batch 1 and 4, and checks logits, the active set and y against the C oracle compiled into the
same program.  The program is a few hundred lines of C: gcc builds it on the host in well under a
second, right before it runs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "activation_sparse_ffn_psffn_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.gpu
def test_c_caller_runs_the_layer(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = os.path.join(LIBDIR, "libpsffn.so")
    if not os.path.exists(lib):
        raise RuntimeError("libpsffn.so is not built: run __graft_entry__.build() first")
    exe = str(tmp_path / "layer_consumer")
    subprocess.check_call([gcc, "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
                           os.path.join(ROOT, "tests", "layer_consumer.c"), os.path.join(ROOT, "oracle", "psffn_oracle.c"),
                           "-o", exe, "-L", LIBDIR, "-lpsffn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                           "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"])
    print("running the C caller", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=90)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed" in r.stdout
