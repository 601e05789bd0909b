"""The product path and the oracle stay apart (no device needed).

- Nothing in the package (Python binding, HIP sources, headers) imports,
  includes or loads anything from oracle/.
- In bench.py and __graft_entry__.py the oracle is imported only inside the
  functions allowed to use it: the CPU-baseline leg, build() (which compiles
  it) and smoke() (which checks against it).
- Without the built HIP library the binding raises instead of computing
  anything another way."""
import ast
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_delta_rule_86_amd")


def _package_sources():
    for d, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                yield os.path.join(d, f)


def _oracle_imports(tree):
    """(enclosing function name or None, line) of every import of oracle."""
    found = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            name = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(child, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in child.names):
                found.append((fn, child.lineno))
            elif isinstance(child, ast.ImportFrom) and (child.module or "").split(".")[0] == "oracle":
                found.append((fn, child.lineno))
            visit(child, name)

    visit(tree, None)
    return found


def test_package_never_touches_the_oracle():
    sources = list(_package_sources())
    assert any(p.endswith("gdr2.py") for p in sources) and any(p.endswith(".hip") for p in sources)
    for path in sources:
        text = open(path).read()
        if path.endswith(".py"):
            assert not _oracle_imports(ast.parse(text)), path
            assert "libgdr2_oracle" not in text and "gdr2_oracle" not in text, path
        else:
            assert not re.search(r'#\s*include\s*[<"][^>"]*oracle', text), path


@pytest.mark.parametrize("script,allowed", [
    ("bench.py", {"cpu_baseline"}),
    ("__graft_entry__.py", {"build", "smoke"}),
])
def test_oracle_imported_only_where_allowed(script, allowed):
    found = _oracle_imports(ast.parse(open(os.path.join(ROOT, script)).read()))
    assert found, f"{script} no longer uses the oracle: update this test"
    bad = [(fn, line) for fn, line in found if fn not in allowed]
    assert not bad, f"{script}: oracle imported outside {sorted(allowed)}: {bad}"


def test_missing_library_fails_loudly(tmp_path):
    missing = str(tmp_path / "libgdr2.so")
    code = ("from gated_delta_rule_86_amd import gdr2\n"
            f"gdr2.load_library({missing!r})\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "RuntimeError" in r.stderr and "is not built" in r.stderr
