"""The C-ABI validation layer under AddressSanitizer and UndefinedBehavior-
Sanitizer (host code only, no GPU).

tests/sanitize/abi_errors.cpp calls every entry point of include/rq.h with
the error cases of test_abi.py and with the extremes of every integer
argument; it is linked against csrc/rq_api.hip and csrc/noalloc.hip, built
with the sanitizers on their host side, and against launch stand-ins
(tests/sanitize/launch_stubs.cpp) that record any launch.  A signed overflow,
an out-of-bounds access or a launch that validation should have stopped fails
the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CXX = "/opt/rocm/bin/amdclang++"
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"]
# sanitizers on the host side of HIP sources only
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def run(cmd, cwd):
    p = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p


@pytest.mark.skipif(not os.path.exists(CXX), reason="amdclang++ not installed")
def test_c_abi_validation_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include")]
    csrc = os.path.join(ROOT, "rotation_w4a4_quantization_amd", "csrc")
    san = os.path.join(ROOT, "tests", "sanitize")
    objs = []
    # the C-ABI layer and the launch stand-ins: host code only
    for src in (os.path.join(csrc, "rq_api.hip"), os.path.join(san, "launch_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        run([CXX, "-x", "hip", "--offload-host-only", *FLAGS, *HOST_SAN, *inc, "-c", src,
             "-o", obj], tmp_path)
        objs.append(obj)
    # noalloc.hip holds a device array: built for gfx950, sanitizers on the host side
    obj = str(tmp_path / "noalloc.hip.o")
    run([CXX, "-x", "hip", "--offload-arch=gfx950", *FLAGS, *HOST_SAN, *inc, "-c",
         os.path.join(csrc, "noalloc.hip"), "-o", obj], tmp_path)
    objs.append(obj)
    obj = str(tmp_path / "abi_errors.o")
    run([CXX, *FLAGS, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *inc, "-c",
         os.path.join(san, "abi_errors.cpp"), "-o", obj], tmp_path)
    objs.append(obj)
    exe = str(tmp_path / "abi_sanitized")
    run([CXX, "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib", "-o", exe], tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], cwd=tmp_path, capture_output=True, text=True, timeout=120, env=env)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.startswith("ok:"), p.stdout + p.stderr
    assert "runtime error" not in p.stderr, p.stderr
    shutil.rmtree(tmp_path, ignore_errors=True)
