"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

kvq_abi.hip (every argument check and the host arithmetic: workspace sizes,
cache bytes, the Lloyd-Max levels) is rebuilt with both sanitizers on its host
code only (its device part is compiled as usual), linked with the other
objects of the regular build into a library of its own, and the argument-error
tests of test_abi_cpu.py run against that library in a child process with the
sanitizer runtime preloaded and halting on the first report.  Nothing here
touches a GPU: every call those tests make fails validation or is host-only.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "compressed_attention_fwht_amd")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"

# sanitizers on the host pass only (each flag behind -Xarch_host)
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined"]
LINK_SANITIZE = ["-fsanitize=address,undefined", "-shared-libsan"]


def _runtime():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return rt[-1] if rt else None


def test_validation_paths_under_asan_and_ubsan(tmp_path):
    others = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
              for s in __import__("compressed_attention_fwht_amd.build", fromlist=["SOURCES"]).SOURCES
              if s != "kvq_abi.hip"]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("the regular build's objects are missing (run the build first)")
    rt = _runtime()
    if rt is None or not os.path.exists(CLANGXX):
        pytest.skip("no sanitizer runtime in this toolchain")
    obj = str(tmp_path / "kvq_abi_san.o")
    lib = str(tmp_path / "libkvq_san.so")
    cc = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
          "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", *HOST_SANITIZE,
          "-c", os.path.join(PKG, "csrc", "kvq_abi.hip"), "-o", obj]
    r = subprocess.run(cc, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    ld = [CLANGXX, "-shared", *LINK_SANITIZE, obj, *others, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    r = subprocess.run(ld, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    child = ("import sys, pytest\n"
             "import compressed_attention_fwht_amd as kvq\n"
             f"kvq.LIB_PATH = {lib!r}\n"
             "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', "
             f"{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))\n")
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True,
                       timeout=600, cwd=ROOT, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "Sanitizer" not in out, out[-6000:]
    assert " passed" in r.stdout
