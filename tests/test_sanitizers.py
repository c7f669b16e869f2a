"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer:

* the oracle (plain C) with a driver that calls every entry point on tiny
  valid and invalid inputs (tests/sanitize/oracle_driver.c);
* the C ABI's host side (argument validation, launch planning, workspace
  layout) with its kernel launchers replaced by stubs, driven through every
  entry point with bad, extreme and valid arguments
  (tests/sanitize/api_driver.cpp); no GPU is touched.
The sanitizers abort on any invalid memory access or undefined behaviour; the
drivers check the returned status codes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, (cmd, r.stdout[-2000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-fopenmp", "-std=c11", os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "sia_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_api_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "indexer_top_sparse_02_amd", "csrc")]
    base = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *SAN_HOST, *inc]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "drv.o", "api_driver"))
    _run([*base, "-c", os.path.join(ROOT, "indexer_top_sparse_02_amd", "csrc", "sia_api.hip"), "-o", api_o])
    _run([*base, "-x", "hip", "-c", os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"), "-o", drv_o])
    _run([HIPCC, "--offload-arch=gfx950", *SAN_HOST, api_o, drv_o, "-o", exe])
    # (the HIP runtime's own allocations are not ours: leak checking off)
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert "all checks passed" in r.stdout
