"""The product path has no fallback: without the HIP library every call
raises, and no module of the package imports the oracle or computes the
method with torch.  Host-only checks (no GPU)."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "autoregressive_video_diffusion_ring_amd")


def test_missing_library_raises_on_first_use():
    code = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from autoregressive_video_diffusion_ring_amd import _lib\n"
        "_lib.LIB_PATH = '/nonexistent/librc.so'\n"
        "import autoregressive_video_diffusion_ring_amd as rc\n"
        "for call in (lambda: rc.rc_qkv_workspace_bytes(757, 5120), lambda: rc.rc_ring_v_ld(5788)):\n"
        "    try:\n"
        "        call()\n"
        "    except ImportError as e:\n"
        "        assert 'librc.so is missing' in str(e), e\n"
        "    else:\n"
        "        raise SystemExit('a call succeeded without the library')\n"
        "print('raised')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "raised"


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_package_never_imports_the_oracle():
    for name in os.listdir(PKG):
        if name.endswith(".py"):
            imported = _imports(os.path.join(PKG, name))
            assert "oracle" not in imported, name
            assert "synthetic_inputs" not in imported, name


def test_package_python_does_no_method_arithmetic():
    """The binding marshals arguments only: no torch math on the method's
    tensors (softmax, matmul, exponentials, trigonometry, reductions)."""
    banned = {"softmax", "matmul", "bmm", "einsum", "exp", "exp2", "sin", "cos", "logsumexp", "baddbmm",
              "amax", "cumsum", "topk", "sort", "polar", "view_as_complex"}
    for name in ("__init__.py", "_lib.py"):
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        used = {n.attr for n in ast.walk(tree) if isinstance(n, ast.Attribute)}
        assert not (used & banned), (name, used & banned)
