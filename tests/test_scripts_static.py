"""Static name check of the top-level scripts that only run in full on a machine
with a GPU (bench.py, __graft_entry__.py): every function they call by plain name must be
defined, imported or bound somewhere in scope, so that a helper removed by
mistake fails here instead of midway through a GPU run."""
import ast
import builtins
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bound_names(node):
    """Names bound anywhere inside `node` (parameters, assignments, imports,
    loop and comprehension targets, with-as, except-as, nested defs)."""
    names = set()
    for n in ast.walk(node):
        if isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            names.add(n.name)
        if isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.Lambda)):
            a = n.args
            for arg in a.posonlyargs + a.args + a.kwonlyargs:
                names.add(arg.arg)
            if a.vararg:
                names.add(a.vararg.arg)
            if a.kwarg:
                names.add(a.kwarg.arg)
        elif isinstance(n, ast.Name) and isinstance(n.ctx, ast.Store):
            names.add(n.id)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            for al in n.names:
                names.add((al.asname or al.name).split(".")[0])
        elif isinstance(n, ast.ExceptHandler) and n.name:
            names.add(n.name)
    return names


@pytest.mark.parametrize("script", ["bench.py", "__graft_entry__.py"])
def test_called_names_resolve(script):
    tree = ast.parse(open(os.path.join(ROOT, script)).read())
    module_names = set()
    for n in tree.body:
        module_names |= _bound_names(n) if not isinstance(
            n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)) else {n.name}
    missing = []
    for fn in [n for n in ast.walk(tree) if isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef))]:
        local = _bound_names(fn)
        for call in [c for c in ast.walk(fn) if isinstance(c, ast.Call)]:
            if isinstance(call.func, ast.Name):
                name = call.func.id
                if name not in local and name not in module_names and not hasattr(builtins, name):
                    missing.append(f"{fn.name}: {name}")
    assert not missing, missing


def test_kernel_hash_ignores_comments_and_layout_only():
    import sys
    sys.path.insert(0, ROOT)
    import bench
    src = 'int a = 1; // note\n/* block\n comment */\nasm("s_nop 0\\n\\tx // kept");  char c = \'"\';\n'
    assert bench.strip_comments(src) == 'int a = 1; asm("s_nop 0\\n\\tx // kept"); char c = \'"\';'
    assert bench.strip_comments(src) == bench.strip_comments(src.replace("note", "other note"))
    assert bench.strip_comments(src) != bench.strip_comments(src.replace("a = 1", "a = 2"))


def _imports(path):
    """(module names, enclosing top-level function or None) of every import in a file."""
    import ast
    tree = ast.parse(open(path).read())
    out = []
    for top in tree.body:
        owner = top.name if isinstance(top, (ast.FunctionDef, ast.AsyncFunctionDef)) else None
        for node in ast.walk(top):
            if isinstance(node, ast.Import):
                out += [(a.name, owner) for a in node.names]
            elif isinstance(node, ast.ImportFrom) and node.module:
                out.append((node.module, owner))
    return out


def test_oracle_and_hip_path_stay_apart():
    """The product package never imports the oracle, the oracle never imports
    the product (or the HIP library), and bench.py uses the oracle only in its
    CPU-baseline functions."""
    import glob
    pkg = glob.glob(os.path.join(ROOT, "async_stage_tile_amd", "**", "*.py"), recursive=True)
    assert pkg
    for f in pkg:
        assert not [m for m, _ in _imports(f) if m.split(".")[0] == "oracle"], f
    for f in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        bad = [m for m, _ in _imports(f) if m.split(".")[0] in ("async_stage_tile_amd", "torch")]
        assert not bad, (f, bad)
        assert "libpipetile" not in open(f).read(), f
    owners = {o for m, o in _imports(os.path.join(ROOT, "bench.py")) if m.split(".")[0] == "oracle"}
    assert owners <= {"cpu_baseline", "cpu_oracle_extras"}, owners
