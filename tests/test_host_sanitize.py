"""The C ABI's host code (plan.cpp, abi.cpp and the host parts of the kernel sources) built with
the address and undefined-behaviour sanitizers (host code only; device code is unchanged) and
driven by ``host_sanitize/abi_driver.cpp``: key ranges and scan order over 1380 shapes against the
frame rules, argument validation, status strings and the allocation-free forward's host checks.
No GPU is used; the sanitizers abort the driver on any report."""

import glob
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _clang_rt(name):
    hits = sorted(glob.glob(f"/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.{name}-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") or _clang_rt("asan") is None,
                    reason="needs hipcc and the clang sanitizer runtime")
def test_abi_host_code_under_sanitizers(tmp_path):
    from linear_video_attention_amd import build as b
    lib = str(tmp_path / "libvdn_asan.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    b.build(lib_path=lib, extra_flags=san)
    exe = str(tmp_path / "abi_driver")
    clang = shutil.which("clang++", path="/opt/rocm/llvm/bin") or "/opt/rocm/llvm/bin/clang++"
    cmd = [clang, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(HERE, "host_sanitize", "abi_driver.cpp"), lib, f"-Wl,-rpath,{tmp_path}",
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout, res.stderr[-3000:])
    assert res.returncode == 0, res.stderr[-3000:]
    assert "all checks passed" in res.stdout
