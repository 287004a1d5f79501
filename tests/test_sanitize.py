"""CPU sanitizer runs (AddressSanitizer + UndefinedBehaviorSanitizer, any report fatal):

* the oracle (oracle/lca_oracle.c) built with gcc -fsanitize=address,undefined, under the oracle's pin
  tests (tests/test_oracle_formats.py, tests/test_oracle_layer.py) in a child process that preloads the
  ASan runtime;
* the host side of the C ABI (long_context_attention_18_amd/csrc/capi.hip), its host pass built with the
  sanitizers (the device pass unchanged), linked with host stand-ins for the kernel launches and the HIP
  runtime (tests/sanitize/) and driven through every entry point by tests/sanitize/abi_driver.cpp.

No GPU is used: the stand-ins record the launches and check their arguments.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
FLAGS = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer"]
CLANG_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
# host pass only: each sanitizer flag behind -Xarch_host
HIPCC_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def _clean(out):
    return "AddressSanitizer" not in out and "runtime error:" not in out and "LeakSanitizer" not in out


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liblca_oracle_san.so")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "lca_oracle.c"), "-o", lib, "-lm"])
    assert rc == 0, out
    rc, asan = _run(["gcc", "-print-file-name=libasan.so"])
    assert rc == 0 and os.path.exists(asan.strip()), asan
    env = dict(os.environ, LD_PRELOAD=asan.strip(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    code = ("import sys, oracle._build as b\n"
            f"b.LIB = {lib!r}\n"
            "import oracle\n"
            "import pytest\n"
            "rc = pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider', "
            "'tests/test_oracle_formats.py', 'tests/test_oracle_layer.py'])\n"
            "assert oracle.lib()._name == b.LIB\n"
            "sys.exit(rc)\n")
    rc, out = _run([sys.executable, "-c", code], cwd=ROOT, env=env, timeout=900)
    assert rc == 0 and _clean(out), out[-4000:]
    assert " passed" in out


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    t = str(tmp_path)
    objs = []
    for src, name in ((os.path.join(ROOT, "long_context_attention_18_amd", "csrc", "capi.hip"), "capi.o"),
                      (os.path.join(SAN, "launch_stubs.hip"), "launch_stubs.o")):
        obj = os.path.join(t, name)
        rc, out = _run(["hipcc", "--offload-arch=gfx950"] + FLAGS + HIPCC_SAN + ["-c", src, "-o", obj])
        assert rc == 0, out
        objs.append(obj)
    for src in ("hip_stubs.cpp", "abi_driver.cpp"):
        obj = os.path.join(t, src + ".o")
        rc, out = _run([CLANG] + FLAGS + CLANG_SAN + ["-c", os.path.join(SAN, src), "-o", obj])
        assert rc == 0, out
        objs.append(obj)
    exe = os.path.join(t, "abi_driver")
    rc, out = _run([CLANG] + CLANG_SAN + ["-o", exe] + objs)
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and _clean(out), out[-4000:]
    assert "all checks passed" in out
