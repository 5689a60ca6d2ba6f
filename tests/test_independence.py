"""The library and the oracle are independent, and the library has no
fallback: nothing in the product package imports the oracle (or the tests),
nothing in the oracle imports the product package or the native sources,
and the binding refuses to run when libpa.so is missing instead of computing
anything another way."""
import ast
import os
import subprocess
import sys

from tests.conftest import ROOT

PKG = os.path.join(ROOT, "paged_kv_cache_355_amd")
ORACLE = os.path.join(ROOT, "oracle")


def imported_modules(path):
    tree = ast.parse(open(path, encoding="utf-8").read(), filename=path)
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.level == 0 and node.module:
            mods.add(node.module.split(".")[0])
    return mods


def python_files(top):
    for dirpath, _, files in os.walk(top):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(dirpath, f)


def test_product_package_never_imports_the_oracle_or_tests():
    for path in python_files(PKG):
        bad = imported_modules(path) & {"oracle", "tests"}
        assert not bad, (path, bad)


def test_native_sources_do_not_mention_the_oracle():
    csrc = os.path.join(PKG, "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f), encoding="utf-8").read()
        assert "oracle" not in text.lower(), f


def test_oracle_never_imports_the_product_package():
    for path in python_files(ORACLE):
        bad = imported_modules(path) & {"paged_kv_cache_355_amd", "tests", "bench"}
        assert not bad, (path, bad)


def test_binding_refuses_to_run_without_the_library():
    code = (
        "import paged_kv_cache_355_amd._lib as L\n"
        "L.LIB_PATH = '/nonexistent/libpa.so'\n"
        "L._lib = None\n"
        "try:\n"
        "    L.lib()\n"
        "except RuntimeError as e:\n"
        "    print('refused:', e)\n"
        "else:\n"
        "    raise SystemExit('loaded without a library')\n"
    )
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert proc.returncode == 0, proc.stderr
    assert "refused:" in proc.stdout and "is not built" in proc.stdout
