"""The product path has one implementation, the HIP library: without it
every entry point raises, and no module of the package reaches the oracle
(which is test infrastructure only)."""
import ast
import os

import pytest

from mixed_precision_sharded_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixed_precision_sharded_amd")


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libmps_adamw.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


def package_sources():
    for d, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                yield os.path.join(d, f)


def test_package_never_imports_the_oracle():
    seen = 0
    for path in package_sources():
        text = open(path, encoding="utf-8").read()
        seen += 1
        if path.endswith(".py"):
            for node in ast.walk(ast.parse(text)):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                assert not any(n.split(".")[0] == "oracle" for n in names), path
        else:
            for line in text.splitlines():
                if line.lstrip().startswith("#include"):
                    assert "oracle" not in line, (path, line)
    assert seen > 5


def test_oracle_shares_no_code_with_the_library():
    """The oracle reaches neither the package nor its kernel headers."""
    odir = os.path.join(ROOT, "oracle")
    for f in os.listdir(odir):
        path = os.path.join(odir, f)
        if f.endswith(".py"):
            for node in ast.walk(ast.parse(open(path, encoding="utf-8").read())):
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                else:
                    continue
                assert not any(n.startswith("mixed_precision_sharded_amd") for n in names), path
        elif f.endswith((".c", ".h")):
            for line in open(path, encoding="utf-8"):
                if line.lstrip().startswith("#include"):
                    assert "csrc" not in line and "mps_" not in line, (path, line)
