"""The GPU path and the fp64 oracle share no code, and the product has no fallback.

Static checks over the sources (imports and includes), plus the loader's behaviour
when the library has not been built.  CPU only.
"""
import ast
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "oasis_score_summaries_amd")


def _py_imports(path):
    """(module, enclosing function or None) for every import statement of a file."""
    tree = ast.parse(open(path).read(), path)
    out = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            name = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(child, ast.Import):
                out.extend((a.name, fn) for a in child.names)
            elif isinstance(child, ast.ImportFrom):
                out.append(("." * child.level + (child.module or ""), fn))
            visit(child, name)

    visit(tree, None)
    return out


def _files(top, exts):
    for dirpath, _, names in os.walk(top):
        if "__pycache__" in dirpath:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(dirpath, n)


def test_package_never_imports_the_oracle():
    for path in _files(PKG, (".py",)):
        for mod, _ in _py_imports(path):
            assert not mod.split(".")[0] == "oracle", f"{path} imports {mod}"
    for path in _files(PKG, (".cpp", ".hip", ".h")):
        for inc in re.findall(r'#include\s+[<"]([^>"]+)[>"]', open(path).read()):
            assert "oracle" not in inc, f"{path} includes {inc}"
    for path in _files(os.path.join(ROOT, "include"), (".h",)):
        assert "oracle" not in "".join(re.findall(r"#include.*", open(path).read())), path


def test_oracle_never_imports_the_package():
    for path in _files(os.path.join(ROOT, "oracle"), (".py",)):
        for mod, _ in _py_imports(path):
            top = mod.lstrip(".").split(".")[0]
            assert top not in ("oasis_score_summaries_amd", "bench", "synth"), f"{path} imports {mod}"


def test_input_generator_depends_on_neither_side():
    for path in _files(os.path.join(ROOT, "synth"), (".py",)):
        for mod, _ in _py_imports(path):
            top = mod.lstrip(".").split(".")[0]
            assert top not in ("oracle", "oasis_score_summaries_amd"), f"{path} imports {mod}"


def test_bench_uses_the_oracle_only_for_the_cpu_baseline():
    users = {fn for mod, fn in _py_imports(os.path.join(ROOT, "bench.py")) if mod.split(".")[0] == "oracle"}
    assert users == {"cpu_baseline"}, users


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from oasis_score_summaries_amd import _lib

    monkeypatch.setattr(_lib, "_lib", None)   # as in a process that has loaded nothing yet
    with pytest.raises(ImportError, match="missing"):
        _lib.load(str(tmp_path / "liboasis.so"))
