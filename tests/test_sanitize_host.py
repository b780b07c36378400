"""The host code of libdmel (argument validation, workspace sizes, host
tables) under AddressSanitizer and UndefinedBehaviorSanitizer: the library is
rebuilt with the sanitizers on its host side only (device code unchanged,
-Xarch_host before each sanitizer flag) and driven by
tests/sanitize/validate_main.cpp, which needs no GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "encoder_free_audio_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _hipcc():
    cand = os.path.join(ROCM, "bin", "hipcc")
    return cand if os.path.exists(cand) else shutil.which("hipcc")


@pytest.mark.timeout(900)
def test_host_code_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None or not os.path.exists(CLANG):
        pytest.skip("hipcc / clang++ not available")
    from encoder_free_audio_amd import build as b
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    objs = []
    for src in b.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [hipcc, f"--offload-arch={b.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
               "-c", os.path.join(CSRC, src), "-o", obj] + host_san
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
            cmd += b.DEVICE_FLAGS
        else:
            cmd += ["-D__HIP_PLATFORM_AMD__"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    lib = str(tmp_path / "libdmel_san.so")
    r = subprocess.run([hipcc, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", lib] + objs + host_san,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the host code really is instrumented
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms
    exe = str(tmp_path / "validate")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", CSRC,
                        "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "sanitize", "validate_main.cpp"),
                        "-o", exe, lib, f"-Wl,-rpath,{tmp_path}", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                        f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"] + SAN, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
