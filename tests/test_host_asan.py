"""Host-side argument fuzzing of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (host pass only; the device code is built as
usual and never launched).  tests/host/abi_fuzz.cpp drives every entry point
with edge-value shapes and pointers; each call is a pure host query or is
rejected by the host checks, so no GPU is needed.  The program exits 0 only
if every size, path and status it checks held and neither sanitizer fired
(undefined behaviour aborts)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_amd", "csrc")


@pytest.fixture(scope="module")
def fuzz_exe(tmp_path_factory):
    from mixture_experts_layer_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("asan") / "abi_fuzz")
    # each sanitizer flag applies to the host pass only
    sanitize = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = ([hipcc, "-O1", "-g", "-std=c++17", f"--offload-arch={B.ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + sanitize +
           ["-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(ROOT, "tests", "host", "abi_fuzz.cpp")] +
           [os.path.join(CSRC, s) for s in B.SOURCES] + ["-o", exe])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_abi_fuzz_under_sanitizers(fuzz_exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_exe, "40000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.startswith("ok 40000 cases")
