"""Host-code sanitizer runs (CPU only): the fp64 oracle and the C-ABI host
layer built with AddressSanitizer and UndefinedBehaviorSanitizer.

* tests/sanitize/oracle_driver.c calls every oracle entry point on small
  random inputs and edge cases (built with gcc, -fsanitize=address,undefined).
* tests/sanitize/abi_driver.cpp calls the C ABI's validation paths and the
  split-KV workspace sizing; the kernel launchers are replaced by host-only
  stand-ins (tests/sanitize/abi_stubs.cpp) that write every workspace
  region the kernels use, so that a workspace of exactly the queried size
  overflows under the sanitizer if the query and the layout ever disagree.
  Built host-only with hipcc, the sanitizer flags applied to the host pass.
Any sanitizer report aborts the driver, failing the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
           OMP_NUM_THREADS="4")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fopenmp", "-o", exe,
                    os.path.join(SAN, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "orthros_oracle.c"), "-lm"])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=300)
    assert rc == 0 and "ok" in out and "Sanitizer" not in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_c_abi_host_layer_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "long_context_prefill_swa_amd", "csrc")
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1",
           "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(csrc, "orthros_api.cpp"),
           os.path.join(csrc, "splitkv_plan.cpp"),
           os.path.join(SAN, "abi_stubs.cpp"),
           os.path.join(SAN, "abi_driver.cpp"), "-o", exe]
    rc, out = _run(cmd, timeout=600)
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=300)
    assert rc == 0 and "ok" in out and "Sanitizer" not in out, out
