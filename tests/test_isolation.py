"""The oracle and the product path share no code: nothing under the package imports the
oracle, the oracle imports nothing of the package or its HIP sources, and bench.py reaches
the oracle only inside its cpu_baseline legs."""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_attention_11_amd")


def _imports(path):
    tree = ast.parse(open(path).read())
    out = []
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            out += [(a.name, node) for a in node.names]
        elif isinstance(node, ast.ImportFrom) and node.module:
            out.append((node.module, node))
    return out


def test_package_does_not_import_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            p = os.path.join(dirpath, f)
            if f.endswith(".py"):
                assert not any(m.split(".")[0] == "oracle" for m, _ in _imports(p)), p
            elif f.endswith((".hip", ".h", ".cpp")):
                assert not re.search(r'#include\s+"[^"]*oracle', open(p).read()), p


def test_oracle_does_not_import_the_package():
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            mods = [m.split(".")[0] for m, _ in _imports(os.path.join(ROOT, "oracle", f))]
            assert "long_context_attention_11_amd" not in mods and "synth" not in mods, f


def test_bench_uses_the_oracle_only_for_the_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    for fn in ast.walk(tree):
        if not isinstance(fn, ast.FunctionDef):
            continue
        for node in ast.walk(fn):
            if isinstance(node, (ast.Import, ast.ImportFrom)):
                names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                if any(n.split(".")[0] == "oracle" for n in names):
                    assert fn.name.startswith("cpu_baseline"), fn.name
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    for node in top:
        names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
        assert not any(n.split(".")[0] == "oracle" for n in names)
