"""The oracle and the product path share no code: the package (Python binding and HIP
sources) never imports or names the oracle module, the oracle never imports the package,
and the binding fails loudly instead of falling back when the library is missing."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "selective_state_space_mamba2_amd")


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            p = os.path.join(dirpath, f)
            if f.endswith(".py"):
                assert "oracle" not in _imports(p), p
            elif f.endswith((".hip", ".cpp", ".h")):
                assert "oracle" not in open(p).read().lower(), p


def test_oracle_never_imports_the_package():
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            names = _imports(os.path.join(ROOT, "oracle", f))
            assert "selective_state_space_mamba2_amd" not in names, f


def test_binding_refuses_to_run_without_the_library(tmp_path):
    """With the library path pointing at a missing file the first call raises; there is no
    fallback path."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from selective_state_space_mamba2_amd import _abi\n"
        "_abi.LIB_PATH = %r\n"
        "try:\n"
        "    _abi.lib()\n"
        "except Exception as e:\n"
        "    print('raised', type(e).__name__)\n"
        "else:\n"
        "    print('loaded')\n" % (ROOT, str(tmp_path / "missing.so")))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert "raised" in out.stdout, out.stdout + out.stderr
