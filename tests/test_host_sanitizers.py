"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer run of the C ABI.

The entry-point sources of the library are rebuilt with the sanitizers on their host code only (device
code is built as usual), and the plain-C consumer in tests/c_abi_check.c drives every argument check
that returns before a HIP call.
CPU only: nothing here touches a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "all_gather_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not present")
def test_c_abi_under_asan_and_ubsan(tmp_path):
    from all_gather_amd import _build

    # The sources whose host code the C consumer reaches (argument checks, workspace and plan caches,
    # the engine and device-array entry points) are rebuilt with the sanitizers; debug info on the host
    # side only.  The kernel files' objects come from the library's own build when it is current (their
    # host code only launches kernels, which this CPU-only check never does), else are compiled here.
    sanitized = ("api", "noalloc", "sdma")
    base = ["--offload-arch=gfx950", "-O1", "-Xarch_host", "-g", "-std=c++17", "-fPIC",
            "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    names = [os.path.splitext(src)[0] for src in _build.SOURCES]
    procs, objs = [], []
    for name in names:
        src = os.path.join(CSRC, name + ".hip")
        built = os.path.join(_build.OBJ, name + ".o")
        if name not in sanitized and os.path.exists(built) and os.path.getmtime(built) >= max(
                os.path.getmtime(src), os.path.getmtime(os.path.join(CSRC, "mr_internal.h"))):
            objs.append(built)
            continue
        obj = str(tmp_path / (name + ".o"))
        flags = base + (HOST_SAN.split() if name in sanitized else [])
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", src, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.PIPE))
        objs.append(obj)
    for p in procs:
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, err.decode()[-2000:]
    lib = tmp_path / "libmr.so"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN.split(), *objs,
                        "-lhsa-runtime64", "-o", str(lib)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = tmp_path / "check"
    r = subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", str(tmp_path), "-lmr",
                        f"-Wl,-rpath,{tmp_path}", "-o", str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "c abi ok" in r.stdout, (r.stdout + r.stderr)[-3000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
