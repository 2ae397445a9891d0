"""The product path has no fallback: without the built HIP library, importing
the package fails and says how to build it (CPU test, no device)."""
import os
import shutil
import subprocess
import sys

from conftest import ROOT


def test_import_fails_loudly_without_the_library(tmp_path):
    pkg = "zero_sharded_mixed_bucketed_amd"
    dst = tmp_path / pkg
    shutil.copytree(os.path.join(ROOT, pkg), dst,
                    ignore=shutil.ignore_patterns("*.so", "*.so.*", "__pycache__"))
    assert not any(p.name.endswith(".so") for p in dst.iterdir())
    code = f"import sys; sys.path.insert(0, {str(tmp_path)!r}); import {pkg}"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=str(tmp_path))
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libzero.so is missing" in r.stderr
    assert "_build" in r.stderr
