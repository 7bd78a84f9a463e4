"""Seeded inputs are reproducible, and the oracle and the HIP path share no code."""
import ast
import os

import numpy as np

from synth import WORKLOADS, InputStream, LayerShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_same_seed_same_bytes():
    s = LayerShape("gdn", 3, 2, 8, 8, 2, 4)
    a, b = InputStream(s, 7), InputStream(s, 7)
    for _ in range(3):
        ra, rb = a.record(), b.record()
        for n in ra:
            assert ra[n].dtype == np.float32 and ra[n].flags.c_contiguous
            np.testing.assert_array_equal(ra[n], rb[n])
    np.testing.assert_allclose(np.linalg.norm(ra["k"], axis=-1), 1.0, rtol=1e-6)
    assert np.all((ra["alpha"] > 0) & (ra["alpha"] < 1) & (ra["beta"] > 0) & (ra["beta"] < 1))


def test_mamba2_params_and_shapes():
    s = WORKLOADS["mamba2_b2_h4_p16_n16_l4"]
    ins = InputStream(s, 0)
    assert np.all(ins.params["A"] <= -1.0) and np.all(ins.params["A"] >= -16.0)
    r = ins.record()
    assert r["x"].shape == (2, 4, 16) and r["B"].shape == (2, 1, 16) and r["dt"].shape == (2, 4)
    d = ins.drafts(3)
    assert d["x"].shape == (2, 3, 4, 16)
    assert np.all(r["dt"] > 0)


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def _py_files(d):
    for dirpath, _, files in os.walk(os.path.join(ROOT, d)):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(dirpath, f)


def test_oracle_imports_nothing_from_the_hip_path():
    for f in _py_files("oracle"):
        assert "hybrid_model_ssm_replay_amd" not in _imports(f), f
        assert "torch" not in _imports(f), f


def test_hip_path_never_imports_the_oracle():
    for f in _py_files("hybrid_model_ssm_replay_amd"):
        assert "oracle" not in _imports(f), f
    for dirpath, _, files in os.walk(os.path.join(ROOT, "hybrid_model_ssm_replay_amd", "csrc")):
        for f in files:
            txt = open(os.path.join(dirpath, f), errors="ignore").read()
            assert "oracle" not in txt.lower(), f


def test_synth_holds_no_decode_arithmetic():
    for f in _py_files("synth"):
        assert not ({"oracle", "hybrid_model_ssm_replay_amd"} & _imports(f))
