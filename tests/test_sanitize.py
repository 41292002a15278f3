"""Host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The library's sources are compiled with the sanitizers on the host side only
(each -fsanitize= behind -Xarch_host: the gfx950 device code is built as
usual and never runs here) and linked with tests/abi_driver.cpp, which drives
every entry point's argument validation and the host helpers, from two
threads at once, without a GPU.  Any sanitizer report, or a status or error
text other than the expected one, fails the test.
"""

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from paged_kv_mla_req_amd import build as B

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _flags():
    return [f for f in B.COMMON_FLAGS if f not in ("-O3", "-fPIC")] + ["-O1", "-g"]


def test_abi_host_code_under_asan_and_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        def compile_one(path):
            obj = os.path.join(d, os.path.basename(path) + ".o")
            cmd = [HIPCC, *_flags(), *B.SOURCE_FLAGS.get(os.path.basename(path), []), *SAN,
                   "-c", path, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj

        sources = [os.path.join(B.CSRC, s) for s in B.SOURCES]
        sources.append(os.path.join(os.path.dirname(__file__), "abi_driver.cpp"))
        with ThreadPoolExecutor(max_workers=8) as ex:
            objs = list(ex.map(compile_one, sources))
        exe = os.path.join(d, "abi_driver")
        r = subprocess.run([HIPCC, f"--offload-arch={B.ARCH}", *SAN, *objs, "-o", exe],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
                   HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out[-4000:]
        assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
        assert " 0 failures" in r.stdout, r.stdout[-2000:]
