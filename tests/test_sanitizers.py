"""CPU sanitizer runs of the C and C++ code that runs on the host.

* The oracle's loops (oracle/svoracle.c) built with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer (every report fatal); the oracle pins rerun in a
  child process against that build.
* The library's host side -- descriptor validation, workspace sizing, the
  argument checks of every entry point -- built by hipcc for the host only with
  the same sanitizers (clang's runtimes); the C-ABI tests rerun against it.

Neither build runs GPU code: the ABI tests launch nothing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_child(tests, extra_env):
    env = dict(os.environ, **SAN_ENV, **extra_env)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-std=gnu11", "-shared", "-fPIC",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(lib),
                    os.path.join(ROOT, "oracle", "svoracle.c"), "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(asan), "gcc has no AddressSanitizer runtime"
    out = _run_child(["tests/test_oracle_pins.py", "tests/test_golden.py", "tests/test_oracle_composition.py"],
                     {"LD_PRELOAD": asan, "SVO_ORACLE_LIB": str(lib)})
    assert " passed" in out


def _clang_asan_runtime():
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_side_argument_checks_under_asan_and_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime next to hipcc")
    from concurrent.futures import ThreadPoolExecutor
    csrc = os.path.join(ROOT, "mtp_draft_verification_amd", "csrc")

    def compile_one(src):
        # device code as in the product build; the sanitizers apply to the host code only
        obj = tmp_path / (src + ".o")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-g", "-std=c++17", "-fPIC",
                            "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                            "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                            "-c", os.path.join(csrc, src), "-o", str(obj)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return str(obj)
    srcs = ("api.hip", "attn.hip", "lmhead.hip", "accept.hip", "stack.hip")
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = tmp_path / "libspecverify_san.so"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", str(lib), *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = _run_child(["tests/test_abi.py"], {"LD_PRELOAD": rt, "SV_LIBRARY": str(lib)})
    assert " passed" in out
