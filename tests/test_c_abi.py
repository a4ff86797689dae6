"""The C ABI from C: tests/c_abi_check.c includes include/attn.h as C99,
links libattn.so with gcc and checks argument rejection and status strings
(no call reaches HIP, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "causal_gqa_attention_fa2_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_compiles_as_c_and_links(tmp_path):
    exe = tmp_path / "c_abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "c_abi_check.c"),
           f"-L{PKG}", "-lattn", f"-Wl,-rpath,{PKG}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("\n") == 8
