"""The product path has no CPU fallback: without the HIP library every call
raises, and nothing in the package imports the oracle."""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_sequence_causal_cp_amd")


def test_missing_library_raises():
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import long_sequence_causal_cp_amd.binding as b\n"
        "b._lib = None\n"
        "b.load_library.__defaults__ = ('/nonexistent/libcp_attn.so',)\n"
        "try:\n"
        "    b.cp_zigzag_chunks(8, 0, 2048, 0)\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(3)\n" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "not built" in r.stdout


def _imports(path):
    tree = ast.parse(open(path).read(), path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(PKG) if f.endswith(".py")))
def test_package_does_not_import_oracle(name):
    mods = list(_imports(os.path.join(PKG, name)))
    assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)
