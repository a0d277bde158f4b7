"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/attn_oracle.c) is compiled with gcc and the
  sanitizers together with tests/sanitize/oracle_driver.c, which runs every
  public function on small inputs of every layout, mask and grouping, with
  NaN/Inf/subnormal values and argument errors.
* The HIP library's host side (argument checks, split plans, status strings
  of bf16_forward_attention_amd/csrc/attn_fwd.hip) is compiled with the
  sanitizers on its host pass only, with tests/sanitize/host_driver.cpp; the
  GPU code is built as usual and never launched (there is no GPU here, and
  the calls stop at their argument or device checks).

Either program aborts on a sanitizer finding and exits non-zero on a failed
check.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(exe):
    res = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, timeout=300)
    assert res.returncode == 0, f"{exe} failed ({res.returncode}):\n{res.stdout}\n{res.stderr[-4000:]}"
    assert "all checks passed" in res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-pthread",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "attn_oracle.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    _run(exe)


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from bf16_forward_attention_amd import build

    exe = str(tmp_path / "host_driver")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-O3", "-fPIC", "-shared")]
    # each sanitizer flag on the host pass only (-Xarch_host): the GPU code is built without it
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [build.hipcc(), *flags, "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"), build.SRC,
           os.path.join(HERE, "host_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    _run(exe)
