"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/abi_sanitize.cpp calls every entry point with arguments that must fail
validation (so no device is touched) and checks the status codes. It is
linked against the library's own ABI, forward and decode sources, with both
sanitizers on their host code and the sanitizer reports made fatal."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_12_amd", "csrc")
# built whole for gfx950 with the sanitizers on their host code; the backward
# launchers are stubs in the driver (validation never reaches them)
SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_decode.hip"]

pytestmark = pytest.mark.slow


def test_abi_validation_under_asan_and_ubsan():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("no ROCm toolchain")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    # device code with the library's own device flags (build.DEVICE_FLAGS)
    from exact_attention_12_amd import build
    common = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, *build.DEVICE_FLAGS]
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        procs = []
        for src in SOURCES + ["abi_sanitize.cpp"]:
            path = os.path.join(CSRC if src != "abi_sanitize.cpp" else os.path.dirname(__file__), src)
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            procs.append(subprocess.Popen([hipcc, *common, *san, "-c", path, "-o", obj],
                                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        for p in procs:
            out = p.communicate()[0]
            assert p.returncode == 0, out.decode()[-2000:]
        exe = os.path.join(tmp, "abi_sanitize")
        link = subprocess.run([hipcc, "--offload-arch=gfx950", *san, *objs, "-o", exe],
                              capture_output=True, text=True)
        assert link.returncode == 0, link.stdout + link.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "passed: 0 failure(s)" in run.stdout
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report
