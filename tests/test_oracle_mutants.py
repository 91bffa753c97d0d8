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
    ("bottom-right offset reversed", "return n_k - n_q if int(causal) == 2 else 0",
     "return n_q - n_k if int(causal) == 2 else 0"),
    ("bottom-right treated as top-left", "return n_k - n_q if int(causal) == 2 else 0", "return 0"),
    ("dense mask ignored", "                    ok = ok & dm", "                    pass"),
    ("dense mask inverted", "                    ok = ok & dm", "                    ok = ok & ~dm"),
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
    shutil.copy(os.path.join(ROOT, "workloads.py"), tmp_path)
    (tmp_path / "tests" / "conftest.py").write_text(
        "import os, sys\nsys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))\n")
    # only the pins of the two-pass definition; the online recurrence is a separate function
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_oracle.py", "-k", "not online"],
                         cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"no pin caught the planted mistake '{desc}'"


# (description, literal text in oracle/backward.py, replacement)
BWD_MUTANTS = [
    ("softmax correction dropped", "ds = pb * (dp - (pb * dp).sum(axis=1, keepdims=True))", "ds = pb * dp"),
    ("softmax correction sign", "ds = pb * (dp - (pb * dp).sum(axis=1, keepdims=True))",
     "ds = pb * (dp + (pb * dp).sum(axis=1, keepdims=True))"),
    ("correction summed over rows", "(pb * dp).sum(axis=1, keepdims=True)", "(pb * dp).sum(axis=0, keepdims=True)"),
    ("dK without scale", "dk[b, h] = sc * (ds.T @ q[b, h])", "dk[b, h] = ds.T @ q[b, h]"),
    ("dQ from V", "dq[b, h] = sc * (ds @ k[b, h])", "dq[b, h] = sc * (ds @ v[b, h])"),
    ("dP from K", "dp = g[b, h] @ v[b, h].T", "dp = g[b, h] @ k[b, h].T"),
    ("dV keys reversed", "dv[b, h] = pb.T @ g[b, h]", "dv[b, h] = pb.T[::-1] @ g[b, h]"),
    ("dK from untransposed dS", "dk[b, h] = sc * (ds.T @ q[b, h])", "dk[b, h] = sc * (ds[:, ::-1].T @ q[b, h])"),
]


@pytest.mark.parametrize("desc,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_backward_pins_catch_planted_mistake(tmp_path, desc, old, new):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    src = (tmp_path / "oracle" / "backward.py").read_text(encoding="utf-8")
    assert old in src, f"mutation site for '{desc}' not found"
    (tmp_path / "oracle" / "backward.py").write_text(src.replace(old, new, 1), encoding="utf-8")
    (tmp_path / "tests").mkdir()
    shutil.copy(os.path.join(HERE, "test_oracle_bwd.py"), tmp_path / "tests")
    (tmp_path / "tests" / "conftest.py").write_text(
        "import os, sys\nsys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))\n")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_oracle_bwd.py", "-k", "not checker"],
                         cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"no pin caught the planted mistake '{desc}'"


# (description, literal text in oracle/fp8.py, replacement)
FP8_MUTANTS = [
    ("exponent bias 8", "np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(1.0 + m / 8.0, e - 8)"),
    ("no implicit leading one", "np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(m / 8.0, e - 7)"),
    ("subnormal scale of a normal", "np.ldexp(m / 8.0, -6)", "np.ldexp(m / 8.0, -7)"),
    ("sign ignored", "out = np.where(s == 1, -mag, mag)", "out = mag"),
    ("S.1111.xxx all NaN", "(e == 15) & (m == 7)", "(e == 15)"),
    ("V not transposed", "v = np.swapaxes(e4m3_decode(vt8), -1, -2) * np.float64(v_descale)",
     "v = e4m3_decode(vt8).reshape(vt8.shape[:2] + (vt8.shape[3], vt8.shape[2])) * np.float64(v_descale)"),
    ("v_descale dropped", "v = np.swapaxes(e4m3_decode(vt8), -1, -2) * np.float64(v_descale)",
     "v = np.swapaxes(e4m3_decode(vt8), -1, -2)"),
    ("k_descale as q_descale", "k = e4m3_decode(k8) * np.float64(k_descale)",
     "k = e4m3_decode(k8) * np.float64(q_descale)"),
]


@pytest.mark.parametrize("desc,old,new", FP8_MUTANTS, ids=[m[0] for m in FP8_MUTANTS])
def test_fp8_pins_catch_planted_mistake(tmp_path, desc, old, new):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    shutil.copy(os.path.join(ROOT, "workloads.py"), tmp_path)
    src = (tmp_path / "oracle" / "fp8.py").read_text(encoding="utf-8")
    assert old in src, f"mutation site for '{desc}' not found"
    (tmp_path / "oracle" / "fp8.py").write_text(src.replace(old, new, 1), encoding="utf-8")
    (tmp_path / "tests").mkdir()
    shutil.copy(os.path.join(HERE, "test_oracle_fp8.py"), tmp_path / "tests")
    (tmp_path / "tests" / "conftest.py").write_text(
        "import os, sys\nsys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))\n")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_oracle_fp8.py", "-k", "not torch and not generator"],
                         cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"no pin caught the planted mistake '{desc}'"


@pytest.mark.parametrize("module,test_file,select", [("attention.py", "test_oracle.py", "not online"),
                                                      ("backward.py", "test_oracle_bwd.py", "not checker"),
                                                      ("fp8.py", "test_oracle_fp8.py", "not torch and not generator")])
def test_unmutated_copy_passes(tmp_path, module, test_file, select):
    """Control for the two tests above: the same harness passes the oracle as it is."""
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    (tmp_path / "tests").mkdir()
    shutil.copy(os.path.join(HERE, test_file), tmp_path / "tests")
    shutil.copytree(os.path.join(HERE, "golden"), tmp_path / "tests" / "golden")
    shutil.copy(os.path.join(ROOT, "workloads.py"), tmp_path)
    (tmp_path / "tests" / "conftest.py").write_text(
        "import os, sys\nsys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))\n")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          f"tests/{test_file}", "-k", select], cwd=tmp_path, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stdout[-2000:]
