"""The header is plain C: a C99 program compiled with gcc against it links
to the library and gets every validation answer before any device work
(no GPU needed)."""
import os
import shutil
import subprocess

import pytest

from vision_transformer_attention_psa_amd.build import LIB_PATH, PKG_DIR, ROOT


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c99_consumer(tmp_path):
    if not os.path.exists(LIB_PATH):
        pytest.fail(f"{LIB_PATH} not built; run __graft_entry__.build() first")
    exe = tmp_path / "abi_check"
    src = os.path.join(ROOT, "tests", "c", "abi_check.c")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}",
           src, "-o", str(exe), f"-L{PKG_DIR}", "-lpsa_attn", f"-Wl,-rpath,{PKG_DIR}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    assert "abi_check ok" in run.stdout
