"""Host: the product path has no fallback and no route to the oracle.

* Without its HIP library the package refuses to import (a loud ImportError),
  so no call can silently run elsewhere.
* No module of the package, and none of the seeded input generators that both
  sides share, imports the oracle (it is test infrastructure only)."""
import ast
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "decode_attention_paged_fp8kv_amd"


def test_import_without_the_library_fails_loudly(tmp_path):
    dst = tmp_path / PKG
    dst.mkdir()
    for f in os.listdir(os.path.join(ROOT, PKG)):
        if f.endswith(".py"):
            shutil.copy(os.path.join(ROOT, PKG, f), dst / f)
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    r = subprocess.run([sys.executable, "-c", f"import {PKG}"], capture_output=True, text=True,
                       timeout=120, cwd=str(tmp_path), env=env)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "no non-HIP fallback" in r.stderr


def _imports(path):
    tree = ast.parse(open(path).read(), path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            yield from (a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_product_and_generators_never_import_the_oracle():
    files = []
    for d in (PKG, "workloads"):
        files += [os.path.join(ROOT, d, f) for f in os.listdir(os.path.join(ROOT, d))
                  if f.endswith(".py")]
    assert len(files) >= 5
    for f in files:
        bad = [m for m in _imports(f) if m == "oracle" or m.startswith("oracle.")]
        assert not bad, (f, bad)
