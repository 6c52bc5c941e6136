"""The host-side ABI code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tq_abi.cpp (argument checks, plans, the no-allocation entry point's set-up),
tq_codebook.cpp (Lloyd-Max tables) and tq_rotation.cpp (the seeded rotation draws) are
compiled with host-only sanitizers (every -fsanitize flag behind -Xarch_host: the device
code is built as usual) and linked with the in-tree build's other objects into a separate
library.  The ABI and rotation tests then run against it in a child Python process with
the sanitizer runtime preloaded; any report fails the test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "compressed_attention_rotate_amd")
CSRC = os.path.join(PKG, "csrc")
HOST_SRCS = ["tq_abi.cpp", "tq_codebook.cpp", "tq_rotation.cpp"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_tests_are_clean_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rt = _runtime()
    if not os.path.exists(hipcc) or rt is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from compressed_attention_rotate_amd import build as B
    hip_objs = [os.path.join(B.BUILD, os.path.basename(s) + ".o")
                for s in sorted(glob.glob(os.path.join(CSRC, "*.hip")))]
    if not all(os.path.exists(o) for o in hip_objs):
        B.build()
    objs = list(hip_objs)
    for src in HOST_SRCS:
        obj = str(tmp_path / (src + ".o"))
        cmd = [hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "-x", "hip", *B.DEVICE, *SAN,
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        objs.append(obj)
    lib = str(tmp_path / "libtq_asan.so")
    res = subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *SAN, *objs, "-o", lib],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    # the host code really is instrumented: the library calls into both runtimes
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env.update({"TQ_LIB_PATH": lib, "LD_PRELOAD": rt,
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py"),
                          os.path.join(ROOT, "tests", "test_rotation.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    # and the child loaded that library
    probe = subprocess.run([sys.executable, "-c", "import compressed_attention_rotate_amd as tq; "
                            "tq.load(); print(tq.LIB_PATH)"], cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip() == lib, probe.stdout + probe.stderr
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in run.stdout
