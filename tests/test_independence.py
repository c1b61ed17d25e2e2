"""The HIP path and the oracle share no code: the package never imports or
links the oracle, and the oracle never includes the package's kernels or
headers.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
reach the oracle."""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "qat_nvfp4_quantize_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _files(top, exts):
    for d, _, fs in os.walk(top):
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(d, f)


def test_package_never_reaches_the_oracle():
    for path in _files(PKG, (".py", ".hip", ".h", ".cpp")):
        text = open(path, encoding="utf-8").read()
        if path.endswith(".py"):
            for node in ast.walk(ast.parse(text)):
                if isinstance(node, ast.Import):
                    assert not any(a.name.split(".")[0] == "oracle" for a in node.names), path
                if isinstance(node, ast.ImportFrom):
                    assert (node.module or "").split(".")[0] != "oracle", path
        assert "nvfp4_oracle" not in text and "liboracle" not in text, path


def test_oracle_includes_nothing_from_the_package():
    for path in _files(ORACLE, (".cpp", ".c", ".h", ".py")):
        text = open(path, encoding="utf-8").read()
        for inc in re.findall(r'#include\s*[<"]([^>"]+)[>"]', text):
            assert not inc.startswith("nvq") and "csrc" not in inc, (path, inc)
        assert "qat_nvfp4_quantize_amd.nvq" not in text and "libnvq" not in text, path


def test_bench_calls_the_oracle_only_in_its_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read())
    owners = []
    for fn in ast.walk(tree):
        if isinstance(fn, (ast.FunctionDef, ast.AsyncFunctionDef)):
            for node in ast.walk(fn):
                if isinstance(node, ast.Import) and any(a.name == "oracle" for a in node.names):
                    owners.append(fn.name)
    top_level = [n for n in tree.body if isinstance(n, ast.Import)
                 and any(a.name == "oracle" for a in n.names)]
    assert not top_level
    assert owners and set(owners) == {"cpu_baseline"}, owners
