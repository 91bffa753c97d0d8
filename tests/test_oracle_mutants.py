"""The oracle's pins have teeth: plant plausible mistakes in a copy of the oracle
(CPU only) and check that the pin suite fails on every one of them."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# (description, literal text in oracle/attention.py, replacement)
MUTANTS = [
    ("dropped scale", "s = (q[b, h, blk] @ k[b, h].T) * sc", "s = (q[b, h, blk] @ k[b, h].T)"),
    ("keys in reverse order", "s = (q[b, h, blk] @ k[b, h].T) * sc", "s = (q[b, h, blk] @ k[b, h, ::-1].T) * sc"),
    ("transposed value product", "out[b, h, pos:pos + r] = p[:, :n_valid] @ v[b, h, :n_valid]",
     "out[b, h, pos:pos + r] = (v[b, h, :n_valid].T @ p[:, :n_valid].T).T[:, ::-1]"),
    ("no mask applied", "s[~ok] = -np.inf", "pass"),
    ("sign flip in exponent", "e[live] = np.exp(s[live] - m[live, None])", "e[live] = np.exp(m[live, None] - s[live])"),
    ("strict causal", "ok &= j[None, :] <= i[:, None]", "ok &= j[None, :] < i[:, None]"),
    ("off-by-one key length", "ok = (j[None, :] < kv) & (i[:, None] >= qs)", "ok = (j[None, :] <= kv) & (i[:, None] >= qs)"),
    ("q_start ignored", "ok = (j[None, :] < kv) & (i[:, None] >= qs)", "ok = (j[None, :] < kv) & (i[:, None] >= 0)"),
    ("log2 in LSE", "m[live] + np.log(l[live])", "m[live] + np.log2(l[live])"),
    ("max not added back to LSE", "m[live] + np.log(l[live])", "np.log(l[live])"),
    ("unnormalised P", "p[live] = e[live] / l[live, None]", "p[live] = e[live]"),
    ("P times K instead of V", "out[b, h, pos:pos + r] = p[:, :n_valid] @ v[b, h, :n_valid]",
     "out[b, h, pos:pos + r] = p[:, :n_valid] @ k[b, h, :n_valid]"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, desc, old, new):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    src = (tmp_path / "oracle" / "attention.py").read_text(encoding="utf-8")
    assert old in src, f"mutation site for '{desc}' not found"
    (tmp_path / "oracle" / "attention.py").write_text(src.replace(old, new, 1), encoding="utf-8")
    (tmp_path / "tests").mkdir()
    shutil.copy(os.path.join(HERE, "test_oracle.py"), tmp_path / "tests")
    shutil.copytree(os.path.join(HERE, "golden"), tmp_path / "tests" / "golden")
    (tmp_path / "tests" / "conftest.py").write_text(
        "import os, sys\nsys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))\n")
    # only the pins of the two-pass definition; the online recurrence is a separate function
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_oracle.py", "-k", "not online"],
                         cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"no pin caught the planted mistake '{desc}'"
