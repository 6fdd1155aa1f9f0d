"""CPU checks of the kernels' integer arithmetic shortcuts (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_int8_quantiser_shortcut_is_exact_for_every_float32(tmp_path):
    """trunc(clamp(v) + copysign(0.5 - 2^-25, v)) == sat127(RHAZ(v)) for all 2^32 patterns."""
    exe = tmp_path / "check_q8"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "native", "check_q8.c"), "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 mismatches" in r.stdout


def test_rounding_shift_arithmetic_form():
    """(v + 64 + (v >> 31)) >> 7 (arithmetic shifts) equals sign(v)*((|v| + 64) >> 7)
    for every product Q(Decay) * state the StatePassing update can form."""
    import numpy as np
    v = np.arange(-128 * 127, 128 * 127 + 1, dtype=np.int64)
    ref = np.sign(v) * ((np.abs(v) + 64) >> 7)
    fast = (v + 64 + (v >> 63)) >> 7
    assert np.array_equal(fast, ref)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    """ssd_api.cpp (validation, size arithmetic, workspace carving) built for
    the host with AddressSanitizer and UBSan, every error fatal, linked to
    counting stand-ins of the kernel launchers, and driven through every entry
    point's branches on fake device addresses."""
    repo = os.path.dirname(HERE)
    csrc = os.path.join(repo, "mamba_ssd_chunked_amd", "csrc")
    exe = tmp_path / "abi_san"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(repo, 'include')}", f"-I{csrc}", os.path.join(csrc, "ssd_api.cpp"),
           os.path.join(HERE, "native", "abi_stubs.cpp"), os.path.join(HERE, "native", "abi_sanitize.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " 0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
