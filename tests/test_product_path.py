"""Host-side rules of the product path (CPU only):
  * the binding refuses to run without the HIP library (no CPU fallback);
  * the package never imports the oracle, and bench.py touches it only inside
    its CPU-baseline leg;
  * bench.py measures one GPU and says so when asked for more.
"""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_raises(monkeypatch):
    from eagle_feature_space_amd import binding as E
    monkeypatch.setattr(E, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libeagle.so"))
    monkeypatch.setattr(E, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        E.lib()


def _imports(tree):
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield node, a.name
        elif isinstance(node, ast.ImportFrom):
            yield node, node.module or ""


def test_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "eagle_feature_space_amd")
    for fn in sorted(os.listdir(pkg)):
        if not fn.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(pkg, fn)).read())
        for _, mod in _imports(tree):
            assert not mod.split(".")[0] == "oracle", f"{fn} imports {mod}"
            assert not mod.startswith("tests"), f"{fn} imports {mod}"


def test_bench_uses_the_oracle_only_in_the_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    owner = {}
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                owner.setdefault(id(node), fn.name)
    for node, mod in _imports(tree):
        if mod.split(".")[0] == "oracle":
            assert owner.get(id(node)) == "cpu_baseline", f"oracle imported outside cpu_baseline: {mod}"


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
