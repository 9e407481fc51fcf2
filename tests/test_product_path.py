"""The product path stands alone: it never reaches the oracle (or the input
generator), and without its HIP library it fails at once instead of falling
back to anything on the CPU."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "llama_transformer_decode_amd")


def test_package_imports_neither_oracle_nor_generator():
    for name in os.listdir(PKG):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        for node in ast.walk(tree):
            mods = []
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            for m in mods:
                assert m.split(".")[0] not in ("oracle", "synth"), f"{name} imports {m}"


def test_hip_sources_share_nothing_with_the_oracle():
    csrc = os.path.join(PKG, "csrc")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name)).read()
        assert "oracle" not in text.lower(), name
    for name in os.listdir(os.path.join(ROOT, "include")):
        assert "oracle" not in open(os.path.join(ROOT, "include", name)).read().lower(), name


def test_missing_library_fails_loudly():
    code = (
        "import llama_transformer_decode_amd.ld as ld\n"
        "ld._SO = '/nonexistent/libld.so'\n"
        "try:\n"
        "    ld.library()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('loaded')\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "no CPU fallback" in r.stdout
