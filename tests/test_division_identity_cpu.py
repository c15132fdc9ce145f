"""The encode and fit kernels normalize a weight w by its fp16 row scale s with
a per-row reciprocal and one correction step instead of a division:
y = RN(1/s), q0 = RN(w y), rem = fma(-q0, s, w), q = RN(rem y + q0). This
checks on the host, in IEEE fp32, that q is RN(w / s) (the oracle's division)
for every pair of significands, and at the edges of the range |w| in
[2^-100, 2^100] the kernels use it in (outside it they divide)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("divchk") / "recip_division_check")
    src = os.path.join(HERE, "recip_division_check.c")
    base = [gcc, "-O2", "-ffp-contract=off", src, "-o", exe, "-lm"]
    # fmaf must be the fused operation: hardware FMA where the host has it, else libm's
    with open("/proc/cpuinfo") as f:
        fma = "fma" in f.read().split()
    for extra in ((["-mfma"] if fma else []) + ["-fopenmp"], ["-fopenmp"], []):
        if subprocess.run(base[:2] + extra + base[2:], capture_output=True).returncode == 0:
            return exe
    pytest.skip("could not build the checker")


@pytest.mark.parametrize("mode", [0, 1])
def test_reciprocal_division_identity(checker, mode):
    r = subprocess.run([checker, str(mode)], capture_output=True, text=True, timeout=600)
    out = r.stdout.strip().splitlines()[-1]
    n, m = int(out.split()[1]), int(out.split()[3])
    assert m == 0 and r.returncode == 0, r.stdout
    assert n == (1 << 33) if mode == 0 else n > 10**6
