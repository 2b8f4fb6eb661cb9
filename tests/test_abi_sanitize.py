"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): every source is compiled with the sanitizers on its host side,
linked with tests/sanitize/abi_sanitize.cpp, and run; the driver calls every
entry point with arguments that fail validation or only size a workspace,
so no HIP call is made and no GPU is needed."""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_lifted_gemv_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_sanitize.cpp")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# sanitizers on the host side only (device code is never instrumented)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-g"]
BASE = ["--offload-arch=gfx950", "-O1", "-std=c++20",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with tempfile.TemporaryDirectory() as tmp:
        def comp(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            r = subprocess.run([HIPCC, *BASE, *SAN, "-c", src, "-o", obj],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            return obj
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            objs = list(ex.map(comp, srcs + [DRIVER]))
        exe = os.path.join(tmp, "abi_sanitize")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address,undefined", *objs,
                            "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        assert "all checks passed" in r.stdout
