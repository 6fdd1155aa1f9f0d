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
