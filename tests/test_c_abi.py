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


def _clang_asan_runtime():
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return os.path.dirname(hits[-1]) if hits else None


def test_c_client_under_address_and_ub_sanitizers(tmp_path):
    """The library's host code (argument checks, plans, status strings, the profiler) built
    with AddressSanitizer and UndefinedBehaviorSanitizer on the host side only, linked with
    the ordinary kernel objects, and driven by the C client with leak detection on."""
    from speculative_decoding_amd import build as b
    clang = "/opt/rocm/llvm/bin/clang"
    rt = _clang_asan_runtime()
    kernels = [os.path.join(b.BUILD, os.path.basename(s) + ".o") for s in b.sources()
               if s.endswith(".hip")]
    if not os.path.exists(clang) or rt is None or not all(os.path.exists(k) for k in kernels):
        pytest.skip("ROCm clang, its sanitizer runtime or the built kernel objects are missing")
    # host-side instrumentation only: each flag goes to the host pass (-Xarch_host)
    san = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
    san += ["-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in b.sources():
        if not src.endswith(".cpp"):
            continue
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([b.hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={b.ARCH}",
                            *san, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        objs.append(obj)
    lib = str(tmp_path / "libmedusa.so")
    r = subprocess.run([b.hipcc(), "-shared", "-fPIC", f"--offload-arch={b.ARCH}", *san,
                        "-shared-libasan", *objs, *kernels, "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "abi_check")
    r = subprocess.run([clang, "-std=c99", "-g", "-fsanitize=address,undefined", "-shared-libasan",
                        "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c", "abi_check.c"),
                        "-o", exe, "-L", str(tmp_path), "-lmedusa", f"-Wl,-rpath,{tmp_path}",
                        f"-Wl,-rpath,{rt}", "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:protect_shadow_gap=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "0 failures" in r.stdout
