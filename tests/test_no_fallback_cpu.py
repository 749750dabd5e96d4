"""The product path has no fallback (CPU).

Without the built library the binding refuses to import, and no module of
the package or of the product's launch path (the binding, the build script,
the benchmark's GPU legs) imports the float64 oracle, which is test
infrastructure only.
"""
import ast
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_attention_rnn_amd")


def test_binding_without_library_raises(tmp_path):
    pkg = tmp_path / "linear_attention_rnn_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(PKG, "__init__.py"), pkg / "__init__.py")
    shutil.copy(os.path.join(PKG, "wkv7.py"), pkg / "wkv7.py")
    code = ("import sys\n"
            "try:\n"
            "    from linear_attention_rnn_amd import wkv7\n"
            "except ImportError as e:\n"
            "    print('refused:', e)\n"
            "    sys.exit(0)\n"
            "sys.exit(3)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode == 0, (r.stdout, r.stderr)
    assert "no fallback" in r.stdout


def _imports(path):
    with open(path) as f:
        tree = ast.parse(f.read(), path)
    out = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            out |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom) and node.module:
            out.add(node.module.split(".")[0])
    return out


def test_package_does_not_import_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for name in files:
            if name.endswith(".py"):
                p = os.path.join(dirpath, name)
                assert "oracle" not in _imports(p), p


def test_package_sources_do_not_name_the_oracle_library():
    """The native sources link nothing of the oracle's C code."""
    for dirpath, _, files in os.walk(os.path.join(PKG, "csrc")):
        for name in files:
            with open(os.path.join(dirpath, name), errors="replace") as f:
                text = f.read()
            assert "wkv7ref" not in text and "oracle/" not in text, name


def test_benchmark_imports_the_oracle_only_in_its_cpu_baseline():
    """bench.py may time the oracle (its cpu_baseline leg) and nothing
    else: every import of the oracle sits in a function whose name says
    so."""
    with open(os.path.join(ROOT, "bench.py")) as f:
        tree = ast.parse(f.read())
    assert "oracle" not in {a.name.split(".")[0] for n in tree.body
                            if isinstance(n, ast.Import) for a in n.names}
    assert not any(isinstance(n, ast.ImportFrom) and n.module and
                   n.module.split(".")[0] == "oracle" for n in tree.body)
    for fn in ast.walk(tree):
        if not isinstance(fn, ast.FunctionDef):
            continue
        for node in ast.walk(fn):
            if isinstance(node, ast.ImportFrom) and node.module and \
                    node.module.split(".")[0] == "oracle":
                assert "cpu" in fn.name or "oracle" in fn.name, fn.name
