"""AddressSanitizer and UndefinedBehaviorSanitizer over the host code: the
CPU oracle (oracle/bao_ref.c) driven through every entry point, and the
C-ABI validation layer (bit_qk_attention_amd/csrc/api.hip, host code only)
driven through every entry point with accepted and rejected arguments and
launcher stubs in place of the GPU kernels (tests/sanitize/). Any report
aborts the driver."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
# host-only sanitizer flags for hipcc: each one on the host side
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wno-unknown-pragmas", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "bao_ref.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failure(s)" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_abi_validation_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "bit_qk_attention_amd", "csrc")]
    objs = []
    for src in (os.path.join(ROOT, "bit_qk_attention_amd", "csrc", "api.hip"), os.path.join(SAN, "api_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-host-only", "-c", "-O1", "-g", "-std=c++17", *HOST_SAN, "-fno-omit-frame-pointer",
              *inc, src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "api_driver.o")
    _run([CLANG, "-c", "-O1", "-g", "-std=c11", "-Wall", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          *inc, os.path.join(SAN, "api_driver.c"), "-o", drv])
    exe = str(tmp_path / "api_driver")
    _run([CLANG + "++", "-fsanitize=address,undefined", *objs, drv, "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "0 failure(s)" in r.stdout
