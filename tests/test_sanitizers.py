"""CPU sanitizer pass over the host code (AddressSanitizer and
UndefinedBehaviorSanitizer, every report fatal):

  * the oracle, built with g++ -fsanitize=address,undefined, runs its pins;
  * the HIP library, built with the sanitizers on its host pass only
    (argument validation, workspace and plan layout, launch set-up; the
    gfx950 device code is not instrumented), runs the C-ABI host tests,
    which reach every validation path without touching a GPU.

Each runs in a child interpreter with the matching sanitizer runtime preloaded
(the interpreter itself is not instrumented), with leak reports off (they
would be the interpreter's own).  Skipped when the toolchain or a runtime is
missing."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_OPTIONS = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
UBSAN_OPTIONS = "halt_on_error=1:print_stacktrace=1"


def _run(code, env_extra, timeout):
    env = dict(os.environ, ASAN_OPTIONS=ASAN_OPTIONS, UBSAN_OPTIONS=UBSAN_OPTIONS, **env_extra)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=timeout, env=env,
                       cwd=ROOT)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def _pytest_child(patch, test_files):
    return ("import sys; sys.path.insert(0, %r)\n%s\nimport pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu'] + %r))\n"
            % (ROOT, patch, [os.path.join(ROOT, "tests", f) for f in test_files]))


def test_oracle_pins_under_asan_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    runtime = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("libasan not found")
    lib = str(tmp_path / "libmoe_oracle_asan.so")
    srcs = [os.path.join(ROOT, "oracle", f) for f in ("moe_oracle.cpp", "attn_oracle.cpp")]
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", lib, *srcs], check=True)
    patch = "import oracle.build as ob; ob.LIB = %r" % lib
    out = _run(_pytest_child(patch, ["test_oracle_pins.py", "test_attn_oracle_pins.py", "test_golden_shapes.py"]),
               {"LD_PRELOAD": runtime}, timeout=900)
    assert " passed" in out, out[-2000:]


def test_abi_host_validation_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc")
    runtimes = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if hipcc is None or not runtimes:
        pytest.skip("hipcc or the clang ASan runtime not found")
    sys.path.insert(0, ROOT)
    from mixture_experts_moe_amd import build as hip_build
    lib = str(tmp_path / "libmoe_asan.so")
    host_only = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-g"):
        host_only += ["-Xarch_host", f]
    hip_build.build(extra_flags=host_only, out=lib)
    patch = "from mixture_experts_moe_amd import moe; moe.LIB_PATH = %r" % lib
    out = _run(_pytest_child(patch, ["test_abi_host.py"]), {"LD_PRELOAD": runtimes[-1]}, timeout=600)
    assert " passed" in out, out[-2000:]
