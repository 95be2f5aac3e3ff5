"""The product path has no CPU fallback: without the built HIP library every entry point raises, the
package never imports the oracle (test infrastructure), and tensors off the GPU are refused."""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "taylor_feature_map_amd")


def test_missing_library_raises():
    code = ("import taylor_feature_map_amd._lib as L\n"
            "L.LIB_PATH = '/nonexistent/libbased.so'\n"
            "L._lib = None\n"
            "from taylor_feature_map_amd import plan\n"
            "plan(1, 64, 1, 16, 64)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "is missing" in r.stderr


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, f)).read())
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                assert not any(n == "oracle" or n.startswith("oracle.") for n in names), f


def test_cpu_tensors_refused():
    torch = pytest.importorskip("torch")
    from taylor_feature_map_amd import based_forward
    q = torch.zeros((1, 4, 1, 16), dtype=torch.bfloat16)
    v = torch.zeros((1, 4, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        based_forward(q, q, v)
