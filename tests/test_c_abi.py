"""The boundary from plain C: tests/c/abi_check.c is compiled with the system C compiler
against include/medusa.h and linked to libmedusa.so, then run (host-only calls)."""
import os
import shutil
import subprocess

import pytest

from speculative_decoding_amd import LIB_PATH

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_c_client(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_check"
    lib_dir = os.path.dirname(LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        os.path.join(HERE, "c", "abi_check.c"), "-o", str(exe), "-L", lib_dir,
                        "-lmedusa", f"-Wl,-rpath,{lib_dir}", "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
