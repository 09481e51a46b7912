"""The product path and the oracle stay apart, and bench.py refuses more than one GPU."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "segmented_gather_matmul_amd")


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_package_never_imports_the_oracle():
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            assert "oracle" not in _imports(os.path.join(PKG, f)), f


def test_oracle_does_not_import_the_hip_path():
    for f in ("__init__.py",):
        names = _imports(os.path.join(ROOT, "oracle", f))
        assert "segmented_gather_matmul_amd" not in names
    src = open(os.path.join(ROOT, "oracle", "lora_oracle.c")).read()
    includes = [l.split()[1] for l in src.splitlines() if l.strip().startswith("#include")]
    assert all(i.startswith("<") for i in includes), includes
    assert not any("hip" in i for i in includes), includes


def test_workload_generator_holds_no_method_arithmetic():
    path = os.path.join(PKG, "workloads.py")
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        assert not (isinstance(node, ast.BinOp) and isinstance(node.op, ast.MatMult))
        if isinstance(node, ast.Attribute):
            assert node.attr not in ("matmul", "einsum", "dot", "tensordot", "bmm", "mm"), node.attr
    assert _imports(path) <= {"__future__", "math", "dataclasses", "numpy"}


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
