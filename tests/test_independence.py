"""The oracle and the HIP path share no code: no module of either imports the other, and the seeded
input generators that both use import neither (static check of every module's imports)."""

import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _modules(pkg):
    for dirpath, _, files in os.walk(os.path.join(ROOT, pkg)):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(dirpath, f)


def _imports(path):
    tree = ast.parse(open(path, encoding="utf-8").read(), filename=path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def test_oracle_imports_nothing_of_the_hip_path():
    for path in _modules("oracle"):
        assert "long_context_online_amd" not in _imports(path), path
        text = open(path, encoding="utf-8").read()
        assert "csrc" not in text and "libblasst" not in text, path


def test_hip_path_never_imports_the_oracle():
    for path in _modules("long_context_online_amd"):
        assert "oracle" not in _imports(path), path
    for dirpath, _, files in os.walk(os.path.join(ROOT, "long_context_online_amd", "csrc")):
        for f in files:
            if f.endswith((".hip", ".hpp", ".cpp", ".h")):
                assert "oracle" not in open(os.path.join(dirpath, f), encoding="utf-8").read().lower(), f
    for f in os.listdir(os.path.join(ROOT, "include")):
        assert "oracle" not in open(os.path.join(ROOT, "include", f), encoding="utf-8").read().lower(), f


def test_input_generators_import_neither_side():
    for path in _modules("synth"):
        imported = _imports(path)
        assert "oracle" not in imported and "long_context_online_amd" not in imported, path
