"""Host check of the arithmetic the bulk append kernel uses in place of IEEE
division (Markstein-corrected quotients from one correctly rounded reciprocal,
codes packed through a rounding constant): tests/host/division_identity.c,
built with gcc, compares it with IEEE fp32 division + rint + clamp over
complete binades of a / 7 and over random draws of x / s, including a few
ulps around every half-integer quotient and bf16 inputs; the same for the
2- and 3-bit quantiser's divisors a / 1 and a / 3."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "division_identity.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path_factory.mktemp("divid") / "division_identity")
    subprocess.run([gcc, "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
                    SRC, "-o", exe, "-lm"], check=True)
    return exe


def test_div7_complete_binades(checker):
    r = subprocess.run([checker, "exhaustive"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 differ" in r.stdout


def test_quotients_and_code_words_random(checker):
    r = subprocess.run([checker, "random", "4000000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 quotients differ" in r.stdout and "0 words differ" in r.stdout


def test_bits_quotients_and_codes_random(checker):
    """The 2- and 3-bit bulk append's quotients (s = a / 1 and a / 3) and
    codes equal those of IEEE division."""
    r = subprocess.run([checker, "bits", "2000000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 quotients differ" in r.stdout and "0 codes differ" in r.stdout
