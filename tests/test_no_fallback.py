"""The product path has no CPU fallback: without the HIP library it fails
loudly, and nothing in the package imports the oracle."""
import ast
import os

import pytest

from online_softmax_tiled_amd import fa

PKG = os.path.dirname(os.path.abspath(fa.__file__))


def test_missing_library_raises(monkeypatch):
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "_LIB_NAME", "libfa_mi355x_missing.so")
    with pytest.raises(FileNotFoundError, match="is not built"):
        fa.load_library()


def test_package_never_imports_the_oracle():
    for name in sorted(os.listdir(PKG)):
        if not name.endswith(".py"):
            continue
        with open(os.path.join(PKG, name)) as f:
            tree = ast.parse(f.read(), name)
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            else:
                continue
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), f"{name} imports {mods}"
