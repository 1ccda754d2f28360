"""The code quotient of the fused per-token quantization (qgemm_w8a8_fp8_dynamic
and _int8_dynamic) rounds to the same code as the IEEE quotient a / s for every
bf16 pair the quantizer can meet, whenever the row scale is at least 2^-100 --
checked exhaustively by a small C program (tests/native/dyn_quotient_check.c,
about 5 * 10^8 pairs per format).  Rows with smaller scales divide."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "tests", "native", "dyn_quotient_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("dynq") / "dyn_quotient_check")
    subprocess.run([cc, "-O2", "-std=c11", "-ffp-contract=off", "-o", exe, SRC, "-lm"], check=True)
    return exe


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_code_quotient_matches_division(checker, fmt):
    out = subprocess.run([checker, "f" if fmt == "fp8" else "i"], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert " 0 differing codes" in out.stdout, out.stdout
    assert int(out.stdout.split(":")[1].split()[0]) > 5 * 10**8      # every pair enumerated
