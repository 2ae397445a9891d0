"""The oracle and the HIP path share no code: neither imports the other, the
oracle touches no torch/ctypes/HIP, and the product never reaches the oracle."""
import ast
import os

from conftest import ROOT

PKG = "zero_sharded_mixed_bucketed_amd"


def _imports(path):
    tree = ast.parse(open(path).read(), path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name.split(".")[0]
        elif isinstance(node, ast.ImportFrom):
            if node.level == 0 and node.module:
                yield node.module.split(".")[0]


def _py_files(d):
    for base, _, files in os.walk(os.path.join(ROOT, d)):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(base, f)


def test_oracle_imports_only_numpy_and_stdlib():
    for f in _py_files("oracle"):
        bad = {m for m in _imports(f)} & {PKG, "torch", "ctypes", "synth", "bench"}
        assert not bad, (f, bad)


def test_product_never_imports_oracle():
    for f in _py_files(PKG):
        assert "oracle" not in set(_imports(f)), f
        assert "synth" not in set(_imports(f)), f


def test_product_sources_do_not_name_the_oracle():
    csrc = os.path.join(ROOT, PKG, "csrc")
    for base, _, files in os.walk(csrc):
        for f in files:
            text = open(os.path.join(base, f), errors="ignore").read()
            assert "oracle" not in text.lower(), f


def test_synth_holds_no_method_arithmetic():
    # the shared generator module must not import either side
    for f in _py_files("synth"):
        bad = set(_imports(f)) & {PKG, "oracle"}
        assert not bad, (f, bad)
