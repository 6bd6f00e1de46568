"""The product path stands on the HIP library alone: the package refuses to
import without libaxr.so (no CPU fallback), and nothing outside the test
suite, the smoke check and the benchmark's CPU-baseline leg reaches the
oracle."""

import ast
import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "lut_attention_scoring_amd")


def test_import_fails_loudly_without_the_library(tmp_path):
    # a copy of the package's Python files with no libaxr.so beside them
    dst = tmp_path / "lut_attention_scoring_amd"
    dst.mkdir()
    for fn in os.listdir(PKG):
        if fn.endswith(".py"):
            shutil.copy(os.path.join(PKG, fn), dst / fn)
    assert not (dst / "libaxr.so").exists()
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    proc = subprocess.run([sys.executable, "-c", "import lut_attention_scoring_amd"],
                          cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=300)
    assert proc.returncode != 0
    assert "ImportError" in proc.stderr and "libaxr.so is missing" in proc.stderr


def _imports_oracle(tree):
    """Nodes of a module that import the oracle package."""
    hits = []
    for node in ast.walk(tree):
        if isinstance(node, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in node.names):
            hits.append(node)
        elif isinstance(node, ast.ImportFrom) and (node.module or "").split(".")[0] == "oracle":
            hits.append(node)
    return hits


def test_product_sources_never_reach_the_oracle():
    for top in ("lut_attention_scoring_amd", "workloads", "include"):
        for dirpath, _, files in os.walk(os.path.join(ROOT, top)):
            for fn in files:
                path = os.path.join(dirpath, fn)
                if fn.endswith(".py"):
                    with open(path) as f:
                        tree = ast.parse(f.read(), path)
                    assert not _imports_oracle(tree), path
                elif fn.endswith((".hip", ".cpp", ".h", ".c")):
                    with open(path) as f:
                        text = f.read()
                    assert not re.search(r'#\s*include\s*["<][^">]*oracle', text), path


def _functions_importing_oracle(path):
    with open(path) as f:
        tree = ast.parse(f.read(), path)
    owners = set()
    for fn in ast.walk(tree):
        if isinstance(fn, (ast.FunctionDef, ast.AsyncFunctionDef)):
            if any(_imports_oracle(stmt) for stmt in fn.body):
                owners.add(fn.name)
    # an import at module level would make every path depend on the oracle
    top_level = [n for n in tree.body
                 if not isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef))
                 and _imports_oracle(n)]
    return owners, top_level


def test_bench_uses_the_oracle_only_for_the_cpu_baseline():
    owners, top = _functions_importing_oracle(os.path.join(ROOT, "bench.py"))
    assert not top
    assert owners == {"cpu_baseline"}


def test_graft_entry_uses_the_oracle_only_in_smoke():
    owners, top = _functions_importing_oracle(os.path.join(ROOT, "__graft_entry__.py"))
    assert not top
    assert owners == {"smoke"}
