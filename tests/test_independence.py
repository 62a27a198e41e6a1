"""The oracle and the HIP path share no code, and the oracle serves only as
test infrastructure. This is checked statically over the sources' imports
and includes:

* the package (Python binding, metadata, HIP sources) never imports or
  includes anything from ``oracle/``;
* the oracle never imports the package or the input generators;
* the input generators (``workloads/``) import neither side;
* ``bench.py`` imports the oracle only inside its CPU-baseline functions
  (``cpu_*``), and ``__graft_entry__.py`` only inside ``smoke()``.
"""

import ast
import pathlib
import re

ROOT = pathlib.Path(__file__).resolve().parents[1]
PKG = "paged_kv_cache_slot_amd"


def _top_imports(tree):
    """(top-level module name, innermost enclosing function or None) for
    every absolute import in the tree."""
    found = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            name = fn
            if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)):
                name = child.name
            if isinstance(child, ast.Import):
                found.extend((a.name.split(".")[0], fn) for a in child.names)
            elif isinstance(child, ast.ImportFrom) and child.level == 0:
                found.append((child.module.split(".")[0], fn))
            visit(child, name)

    visit(tree, None)
    return found


def _py_files(sub):
    files = sorted((ROOT / sub).rglob("*.py"))
    assert files, sub
    return files


def _imports_of(path):
    return _top_imports(ast.parse(path.read_text(), filename=str(path)))


def test_package_never_uses_the_oracle():
    for p in _py_files(PKG):
        mods = {m for m, _ in _imports_of(p)}
        assert "oracle" not in mods, p
    sources = [p for p in (ROOT / PKG / "csrc").iterdir()
               if p.suffix in (".hip", ".cpp", ".h")]
    assert sources
    for p in sources:
        for inc in re.findall(r'#include\s*[<"]([^>"]+)[>"]', p.read_text()):
            assert "oracle" not in inc, (p, inc)


def test_oracle_never_uses_the_package_or_the_generators():
    for p in _py_files("oracle"):
        mods = {m for m, _ in _imports_of(p)}
        assert not mods & {PKG, "workloads", "torch"}, (p, mods)


def test_generators_import_neither_side():
    for p in _py_files("workloads"):
        mods = {m for m, _ in _imports_of(p)}
        assert not mods & {PKG, "oracle"}, (p, mods)


def test_bench_and_entry_use_the_oracle_only_where_allowed():
    bench = [(m, fn) for m, fn in _imports_of(ROOT / "bench.py")
             if m == "oracle"]
    assert bench, "bench.py's CPU baseline times the oracle"
    for _, fn in bench:
        assert fn is not None and fn.startswith("cpu_"), fn
    entry = [(m, fn) for m, fn in _imports_of(ROOT / "__graft_entry__.py")
             if m == "oracle"]
    for _, fn in entry:
        assert fn == "smoke", fn
