"""Planted mistakes in a scratch copy of the oracle must fail the pins.

Each case copies oracle/ to a temporary directory, applies one textual
mutation to the C source (a swapped prior, an off-by-one in the window or in
M, a dropped scale, a wrong sign, V read from K ...), and runs
tests/test_oracle_pins.py against the copy in a subprocess.  The pins pass on
the real oracle (test_oracle_pins.py itself) and must fail on every mutant.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "prior_swapped": ("? prior_local : prior_skip", "? prior_skip : prior_local"),
    "M_off_by_one": ("dist / pi <= M;", "dist / pi < M;"),
    "scale_dropped": ("sc[a] = scale * dot;", "sc[a] = dot;"),
    "prior_always": ("        if (has_skip)\n            sc[a] +=", "        if (1)\n            sc[a] +="),
    "window_off_by_one": ("return abs(i - j) <= k;", "return abs(i - j) < k;"),
    "softplus_sign": ("return -log1p(exp(-x));", "return -log1p(exp(x));"),
    "v_read_from_k": ("out[c] += w * load_elem(vv, vb + c, dt);",
                      "out[c] += w * load_elem(kk, vb + c, dt);"),
    # the backward
    "bwd_dk_scale_dropped": ("dk[ko + c] += scale * ds *", "dk[ko + c] += ds *"),
    "bwd_skip_gate_sign": ("? (1.0 - alpha) : -alpha)", "? (1.0 - alpha) : alpha)"),
    "bwd_dv_uses_dlogit": ("dv[ko + c] += sc[a] *", "dv[ko + c] += ds *"),
    "bwd_D_dropped": ("double ds = sc[a] * (dp[a] - D);", "double ds = sc[a] * dp[a];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(tmp_path, name):
    old, new = MUTATIONS[name]
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp*"))
    src = tmp_path / "oracle" / "piattn_oracle.c"
    text = src.read_text()
    assert text.count(old) == 1, "mutation anchor not found"
    src.write_text(text.replace(old, new))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    shutil.copy(os.path.join(ROOT, "tests", "test_oracle_pins.py"), tmp_path / "tests")
    (tmp_path / "tests" / "conftest.py").write_text(
        "import os, sys\nsys.path.insert(0, os.path.dirname(os.path.dirname(__file__)))\n"
        "import pytest\n@pytest.fixture(scope='session')\ndef oracle_lib():\n"
        "    import oracle\n    oracle.build()\n    return oracle\n")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 1, res.stdout[-2000:] + res.stderr[-2000:]
    assert "failed" in res.stdout
