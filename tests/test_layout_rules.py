"""Structural rules checked on the CPU: the product never reaches the oracle
or the input generators, the oracle never reaches the product, and the
benchmark refuses more than one GPU before touching any."""

import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def _py_files(pkg):
    for dirpath, _, files in os.walk(os.path.join(ROOT, pkg)):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(dirpath, f)


def test_product_does_not_import_oracle_or_generators():
    for path in _py_files("tenant_linear_layers_amd"):
        bad = _imports(path) & {"oracle", "synthetic"}
        assert not bad, f"{path} imports {bad}"


def test_oracle_does_not_import_product():
    for path in _py_files("oracle"):
        bad = _imports(path) & {"tenant_linear_layers_amd", "synthetic", "torch"}
        assert not bad, f"{path} imports {bad}"


def test_hip_sources_do_not_include_oracle_code():
    csrc = os.path.join(ROOT, "tenant_linear_layers_amd", "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f)).read()
        assert "oracle" not in text.lower(), f


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
