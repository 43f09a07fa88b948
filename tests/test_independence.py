"""The HIP path and the CPU oracle share no code, and nothing that runs reads
the pages' copy: static checks over the committed sources (CPU)."""

import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _files(top, exts):
    for d, _, names in os.walk(os.path.join(ROOT, top)):
        if "__pycache__" in d:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    out = []
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            out += [(a.name.split(".")[0], node) for a in node.names]
        elif isinstance(node, ast.ImportFrom) and node.module:
            out.append((node.module.split(".")[0], node))
    return out


def test_product_never_touches_the_oracle():
    for f in _files("mxfp8_decode_gemm_amd", (".py",)):
        assert "oracle" not in [m for m, _ in _imports(f)], f
    for f in _files("mxfp8_decode_gemm_amd", (".hip", ".h", ".cpp")):
        text = open(f).read()
        assert not re.search(r'#include\s+"[^"]*oracle', text), f
    for f in _files("include", (".h",)):
        assert "oracle" not in open(f).read(), f


def test_oracle_and_generators_never_touch_the_product():
    for top in ("oracle", "workloads"):
        for f in _files(top, (".py",)):
            mods = [m for m, _ in _imports(f)]
            assert "mxfp8_decode_gemm_amd" not in mods, f
            if top == "workloads":
                assert "oracle" not in mods, f  # inputs hold none of the method's arithmetic
    for f in _files("oracle", (".py",)):
        text = open(f).read()
        assert "csrc" not in text and "libmxgemm" not in text, f


def test_bench_imports_the_oracle_only_inside_functions():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    for node in tree.body:  # module level only
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            names = [a.name for a in node.names] + [getattr(node, "module", "") or ""]
            assert not any(n.split(".")[0] == "oracle" for n in names)


def test_nothing_that_runs_reads_the_page_copy():
    runs = list(_files("mxfp8_decode_gemm_amd", (".py", ".hip", ".h"))) + list(
        _files("tests", (".py",))) + list(_files("workloads", (".py",))) + list(
        _files("oracle", (".py",)))
    runs += [os.path.join(ROOT, f) for f in ("bench.py", "__graft_entry__.py")]
    for f in runs:
        if os.path.abspath(f) == os.path.abspath(__file__):
            continue
        assert "/root/reference" not in open(f).read(), f
