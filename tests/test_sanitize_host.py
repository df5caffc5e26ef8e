"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU):
  * the C oracle, built with gcc -fsanitize=address,undefined, runs its pin tests
    (tests/test_oracle_core.py);
  * the library's host side (argument validation and workspace arithmetic in api.hip), built with
    the sanitizers on the host pass only, runs the C-ABI rejection tests (tests/test_abi_host.py)
    and the binding's checks (tests/test_binding_host.py).
Each runs in a child process with the sanitizer runtime preloaded; any report aborts it."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:allocator_may_return_null=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def run_child(args, env_extra, tmp):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    env["PYTHONPATH"] = ROOT
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + args,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = str(tmp_path / "oracle_san.so")
    subprocess.check_call([gcc, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                           "-o", lib, os.path.join(ROOT, "oracle", "psffn_oracle.c"), "-lm"])
    asan = subprocess.check_output([gcc, "-print-file-name=libasan.so"], text=True).strip()
    ubsan = subprocess.check_output([gcc, "-print-file-name=libubsan.so"], text=True).strip()
    out = run_child(["tests/test_oracle_core.py"], {"PSFFN_ORACLE_LIB": lib, "LD_PRELOAD": asan + ":" + ubsan},
                    tmp_path)
    assert " passed" in out


def hipcc():
    c = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return c if os.path.exists(c) else shutil.which("hipcc")


def test_library_host_side_under_asan_ubsan(tmp_path):
    cc = hipcc()
    objs = sorted(glob.glob(os.path.join(ROOT, "activation_sparse_ffn_psffn_amd", "_build", "*.o")))
    objs = [o for o in objs if os.path.basename(o) != "api.o"]
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if cc is None or not objs or not rt:
        pytest.skip("hipcc, the library's object files (build() first) or clang's ASan runtime are missing")
    api = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libpsffn_san.so")
    inc = os.path.join(ROOT, "include")
    # the sanitizers on the host pass only (the device code of api.hip is the fill kernel's launch)
    subprocess.check_call([cc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                           "-Xclang", "-packed-fp32-ops", "-I", inc, "-Xarch_host", "-fsanitize=address",
                           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                           "-c", os.path.join(ROOT, "activation_sparse_ffn_psffn_amd", "csrc", "api.hip"), "-o", api],
                          stderr=subprocess.DEVNULL)
    subprocess.check_call([cc, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                           "-Xarch_host", "-fsanitize=undefined", "-o", lib, api] + objs, stderr=subprocess.DEVNULL)
    out = run_child(["tests/test_abi_host.py", "tests/test_binding_host.py"],
                    {"PSFFN_LIB": lib, "LD_PRELOAD": rt[0]}, tmp_path)
    assert " passed" in out
