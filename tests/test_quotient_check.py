"""The quantizer computes x / scale from a per-row reciprocal and one FMA
correction instead of a division per element. tests/native/quotient_check.c
replays that exact binary32 sequence on the CPU for every (bf16 row maximum,
bf16 element of either sign) pair and checks the E4M3 codes equal those of
the correctly rounded quotient."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reciprocal_fma_quotient_gives_ieee_codes(tmp_path):
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "native", "quotient_check.c"), "-lm"],
                   check=True)
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(16, os.cpu_count() or 1)))
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env,
                         timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    assert "code_diffs=0" in res.stdout
    assert "pairs=1065402238" in res.stdout
