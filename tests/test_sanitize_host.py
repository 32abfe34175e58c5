"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the C ABI's host path (abk_api.cpp and the page allocator pool.cpp, built
by g++ with the kernel launchers replaced by ones that launch nothing) and the
oracle's C part (abk_oracle.c). The host-only pool tests (every call against
the independent page model, pages running out at each budget level, protocol
errors that must change nothing), the oracle's pins and the generator tests run
in a child process on these builds; any sanitizer report fails the run."""
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-O1", "-g"]
CSRC = os.path.join(ROOT, "long_reasoning_kv_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

# run in the child: the suites, then proof that the sanitized builds were the
# ones loaded
CHILD = r"""
import sys, pytest
rc = pytest.main(["-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + sys.argv[1:])
maps = open("/proc/self/maps").read()
import os
for var in ("ABK_LIB", "ABK_ORACLE_LIB"):
    if os.environ[var] not in maps:
        print("not loaded:", os.environ[var])
        rc = rc or 3
sys.exit(int(rc))
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not available")
    return path


def test_host_code_under_address_and_undefined_sanitizers(tmp_path):
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not available")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    abk_lib = str(tmp_path / "libabk_san.so")
    orc_lib = str(tmp_path / "liborc_san.so")
    subprocess.run(["g++", "-std=c++17", "-shared", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROCM}/include", "-o", abk_lib, os.path.join(CSRC, "abk_api.cpp"),
                    os.path.join(CSRC, "pool.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_only_launchers.cpp"),
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"], check=True)
    subprocess.run(["gcc", "-shared", "-fPIC", "-fopenmp", *SAN, "-o", orc_lib,
                    os.path.join(ROOT, "oracle", "abk_oracle.c"), "-lm"], check=True)
    env = dict(os.environ)
    env["ABK_LIB"] = abk_lib
    env["ABK_ORACLE_LIB"] = orc_lib
    # the sanitizer runtimes first, then whatever is preloaded already
    env["LD_PRELOAD"] = " ".join(x for x in (asan, ubsan, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    suites = [os.path.join(ROOT, "tests", f) for f in
              ("test_abi_host.py", "test_oracle_pins.py", "test_synth_and_pagemodel.py")]
    r = subprocess.run([sys.executable, "-c", CHILD, *suites], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    print(tail)
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
