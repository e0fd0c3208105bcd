"""The oracle and the HIP path stay apart (static checks, no GPU):

* nothing in the product package imports, includes or loads anything under oracle/, so no
  product call can route through the CPU oracle;
* the oracle includes and imports nothing from the product package (it takes the seeded
  inputs as arrays);
* bench.py touches the oracle only in its CPU leg, the functions cpu_baseline (the
  headline's sample and parity spot check) and cpu_baselines (a sample of every workload);
* the binding has no fallback: with the library missing, every call raises.
"""
import ast
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dense_gemm_operand_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _sources(top, exts):
    for d, dirs, files in os.walk(top):
        dirs[:] = [x for x in dirs if not x.startswith(("_build", "__pycache__"))]
        for f in files:
            if f.endswith(exts):
                yield os.path.join(d, f)


def _imported_modules(path):
    tree = ast.parse(open(path, encoding="utf-8").read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name.split(".")[0], node
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            yield node.module.split(".")[0], node


def test_product_package_never_reaches_the_oracle():
    for path in _sources(PKG, (".py",)):
        mods = {m for m, _ in _imported_modules(path)}
        assert "oracle" not in mods, path
        assert "liboracle" not in open(path, encoding="utf-8").read(), path
    for path in _sources(PKG, (".hip", ".hpp", ".cpp", ".h")):
        text = open(path, encoding="utf-8").read()
        for inc in re.findall(r'#include\s+"([^"]+)"', text):
            assert "oracle" not in inc, (path, inc)
        assert "liboracle" not in text, path


def test_oracle_takes_nothing_from_the_product_package():
    for path in _sources(ORACLE, (".py",)):
        mods = {m for m, _ in _imported_modules(path)}
        assert "dense_gemm_operand_amd" not in mods, path
        assert "libdgemm" not in open(path, encoding="utf-8").read(), path
    for path in _sources(ORACLE, (".c", ".h")):
        text = open(path, encoding="utf-8").read()
        for inc in re.findall(r'#include\s+["<]([^">]+)[">]', text):
            assert "dense_gemm" not in inc and "csrc" not in inc and "dgemm" not in inc, (path, inc)


def test_bench_uses_the_oracle_only_in_its_cpu_leg():
    path = os.path.join(ROOT, "bench.py")
    tree = ast.parse(open(path, encoding="utf-8").read())
    funcs = {n.name: n for n in tree.body if isinstance(n, ast.FunctionDef)}
    assert "cpu_baseline" in funcs and "cpu_baselines" in funcs
    leg = set(map(id, ast.walk(funcs["cpu_baseline"]))) | set(map(id, ast.walk(funcs["cpu_baselines"])))
    for node in ast.walk(tree):
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
            if any(n.split(".")[0] == "oracle" for n in names):
                assert id(node) in leg, f"bench.py imports the oracle outside cpu_baseline (line {node.lineno})"


def test_binding_has_no_fallback_without_the_library(tmp_path):
    import dense_gemm_operand_amd as dg
    saved_path, saved_lib = dg.LIB_PATH, dg._lib
    dg.LIB_PATH, dg._lib = str(tmp_path / "missing.so"), None
    try:
        with pytest.raises(RuntimeError, match="no fallback"):
            dg.gemm_plan(64, 64, 64, "row", "col", "f16", "f16", "f16", 1)
        with pytest.raises(RuntimeError, match="no fallback"):
            dg.attn_fwd(0x10000, 0x20000, 0x30000, 0x40000, 1, 64, 64, 128, "f16", 0.125, stream=0)
    finally:
        dg.LIB_PATH, dg._lib = saved_path, saved_lib
