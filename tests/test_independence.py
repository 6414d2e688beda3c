"""The oracle and the HIP path share no code: no module of the package
imports the oracle (nor the test helpers that wrap it), the oracle imports
nothing of the package, and the only module both sides use is the seeded
input generator, which holds none of the method's arithmetic."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "hierarchical_sparse_attention_block_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            if node.level:   # relative: a module of the same package
                continue
            base = node.module or ""
            names.add(base)
            names.update(f"{base}.{a.name}" if base else a.name for a in node.names)
    return names


def _py_files(d):
    for dirpath, _, files in os.walk(d):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(dirpath, f)


def test_package_never_imports_the_oracle():
    for path in _py_files(PKG):
        bad = {n for n in _imports(path) if n.split(".")[0] in ("oracle", "tests", "hsab_testlib")}
        assert not bad, f"{os.path.relpath(path, ROOT)} imports {sorted(bad)}"


def test_oracle_imports_nothing_of_the_package():
    for path in _py_files(ORACLE):
        bad = {n for n in _imports(path) if "hierarchical_sparse_attention_block_amd" in n or n.startswith("hsab")}
        assert not bad, f"{os.path.relpath(path, ROOT)} imports {sorted(bad)}"


def test_native_sources_do_not_reach_the_oracle():
    csrc = os.path.join(PKG, "csrc")
    for f in os.listdir(csrc):
        if f.endswith((".hip", ".h", ".cpp", ".c")):
            text = open(os.path.join(csrc, f)).read()
            assert "oracle" not in text.lower(), f"csrc/{f} mentions the oracle"


def test_input_generator_holds_no_method_arithmetic():
    """workloads.py draws inputs only: it imports neither side and defines
    none of the operator's steps (bounds, top-k, softmax, attention)."""
    path = os.path.join(PKG, "workloads.py")
    names = _imports(path)
    assert not {n for n in names if n.split(".")[0] in ("oracle", "torch")}, names
    tree = ast.parse(open(path).read())
    defs = {n.name for n in ast.walk(tree) if isinstance(n, ast.FunctionDef)}
    for banned in ("softmax", "topk", "top_k", "attend", "block_bound", "upper_bound", "select_blocks",
                   "select_tokens", "decode_step"):
        assert not any(banned in d for d in defs), (banned, sorted(defs))
