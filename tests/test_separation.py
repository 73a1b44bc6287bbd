"""The oracle and the HIP path share no code: neither imports the other, the
seeded input module imports neither, and no product source (the package, its
HIP sources, the header, the benchmark's GPU legs) reaches into the oracle
except the benchmark's CPU-baseline leg."""
import ast
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(path):
    tree = ast.parse(open(path).read(), path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def _py_files(d):
    for base, _, files in os.walk(os.path.join(ROOT, d)):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(base, f)


@pytest.mark.parametrize("pkg,forbidden", [("self_speculative_lm_amd", "oracle"),
                                           ("oracle", "self_speculative_lm_amd"),
                                           ("seeded", "oracle"), ("seeded", "self_speculative_lm_amd")])
def test_no_imports_across(pkg, forbidden):
    for f in _py_files(pkg):
        assert forbidden not in _imports(f), f


def test_native_sources_do_not_reference_the_oracle():
    for d in ("self_speculative_lm_amd/csrc", "include"):
        for base, _, files in os.walk(os.path.join(ROOT, d)):
            for f in files:
                text = open(os.path.join(base, f), errors="replace").read()
                assert "oracle" not in text.lower(), f


def test_bench_uses_the_oracle_only_in_its_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    users = set()
    for fn in [n for n in ast.walk(tree) if isinstance(n, ast.FunctionDef)]:
        for node in ast.walk(fn):
            if isinstance(node, ast.ImportFrom) and node.module and node.module.split(".")[0] == "oracle":
                users.add(fn.name)
            if isinstance(node, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in node.names):
                users.add(fn.name)
    assert users <= {"cpu_baseline"}, users
