"""The oracle against what the pages and the mathematics fix (CPU only)."""
import os

import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_bf16_rounding_exhaustive(tmp_path):
    """Every fp32 pattern through the oracle's bf16 rounding against a
    definitional rounder (tests/exhaustive_bf16.c), 2^32 cases."""
    import subprocess
    here = os.path.dirname(os.path.abspath(__file__))
    odir = os.path.dirname(oracle.__file__)
    exe = tmp_path / "exhaustive_bf16"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(here, "exhaustive_bf16.c"), "-L", odir, "-loracle",
                    f"-Wl,-rpath,{odir}", "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
