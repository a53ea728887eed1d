"""The product path and the oracle stay apart, and the binding has no fallback.

Checked statically (AST over the sources) and with a subprocess, so these run
on the CPU:
  * nothing in the package (``grouped_gemm_moe_amd``) or in ``workloads``
    imports the oracle, and the oracle imports neither of them;
  * ``bench.py`` imports the oracle only inside its CPU-baseline function;
  * loading the binding without the HIP library raises instead of falling
    back to anything.
"""
from __future__ import annotations

import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _py_files(rel):
    top = os.path.join(ROOT, rel)
    for dirpath, _, files in os.walk(top):
        if "__pycache__" in dirpath:
            continue
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(dirpath, f)


def _imported_modules(tree):
    """(top-level module name, enclosing function name or None) per import."""
    out = []

    def visit(node, func):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else func
            if isinstance(child, ast.Import):
                out.extend((a.name.split(".")[0], func) for a in child.names)
            elif isinstance(child, ast.ImportFrom) and child.module and child.level == 0:
                out.append((child.module.split(".")[0], func))
            visit(child, f)

    visit(tree, None)
    return out


def _imports_of(path):
    with open(path, encoding="utf-8") as fh:
        return _imported_modules(ast.parse(fh.read(), filename=path))


def test_product_and_workloads_never_import_the_oracle():
    files = list(_py_files("grouped_gemm_moe_amd")) + list(_py_files("workloads"))
    assert files
    for path in files:
        mods = {m for m, _ in _imports_of(path)}
        assert "oracle" not in mods, f"{os.path.relpath(path, ROOT)} imports the oracle"


def test_oracle_imports_neither_the_package_nor_torch():
    files = list(_py_files("oracle"))
    assert files
    for path in files:
        mods = {m for m, _ in _imports_of(path)}
        assert "grouped_gemm_moe_amd" not in mods, f"{os.path.relpath(path, ROOT)} imports the HIP path"
        assert "torch" not in mods, f"{os.path.relpath(path, ROOT)} imports torch"


def test_bench_uses_the_oracle_only_for_the_cpu_baseline():
    uses = [(m, f) for m, f in _imports_of(os.path.join(ROOT, "bench.py")) if m == "oracle"]
    assert uses, "bench.py is expected to time the oracle in its CPU baseline"
    assert all(f == "cpu_baseline" for _, f in uses), uses


def test_binding_raises_without_the_library(tmp_path):
    missing = str(tmp_path / "no_such_libmoegmm.so")
    code = ("import grouped_gemm_moe_amd as g\n"
            "try:\n"
            "    g.library()\n"
            "except ImportError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    raise SystemExit('loaded without a library')\n")
    env = dict(os.environ, MOEGMM_LIB=missing, PYTHONPATH=ROOT)
    p = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "raised:" in p.stdout and "no fallback" in p.stdout
