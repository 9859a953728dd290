"""CPU sanitizer runs of the host code (address + undefined-behaviour).

Two builds of the same sources, each exercised by the existing CPU tests in
a child process with the matching sanitizer runtime preloaded:
  - the CPU oracle, built with g++ -fsanitize=address,undefined, running the
    layer and Philox pin tests (small shapes, every oracle entry point);
  - the host side of the C-ABI library (argument validation, workspace
    planning, tap tables), built by hipcc with the sanitizers on the host
    compilation only, running the host ABI tests (no GPU calls).
A sanitizer report or a failing test fails this test.  The device code is
not sanitized (no GPU sanitizer here)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "deep_cnn_image_amd", "csrc")
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")

pytestmark = pytest.mark.slow


def _child(env_extra, tests, tmp):
    logdir = os.path.join(str(tmp), "sanitizer_logs")
    os.makedirs(logdir, exist_ok=True)
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={logdir}/asan"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:halt_on_error=1:log_path={logdir}/ubsan"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    logs = sorted(glob.glob(os.path.join(logdir, "*")))
    report = "".join(open(f, errors="replace").read() for f in logs)
    assert not logs, report[-4000:]
    for rep in REPORTS:
        assert rep not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    libasan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("g++ has no AddressSanitizer runtime")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["g++", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fopenmp",
                    "-fPIC", "-shared", "-std=c++17", "-fno-fast-math", "-ffp-contract=off",
                    os.path.join(ROOT, "oracle", "alexnet_oracle.cpp"), "-o", lib], check=True)
    out = _child({"ORACLE_LIB": lib, "LD_PRELOAD": libasan},
                 ["tests/test_oracle_layers.py", "tests/test_oracle_philox.py"], tmp_path)
    print(out.strip().splitlines()[-1])


def test_host_abi_under_asan_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    hipcc = "/opt/rocm/bin/hipcc"
    if not rt or not os.path.exists(hipcc):
        pytest.skip("no clang AddressSanitizer runtime or hipcc")
    objs = []
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    base = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared-libsan",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    for src in ("kernels.hip", "plan.cpp", "alexnet.cpp"):
        obj = str(tmp_path / (src.split(".")[0] + ".o"))
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        subprocess.run([hipcc, *base, *san, *lang, "-c", os.path.join(CSRC, src), "-o", obj], check=True,
                       capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "libalexnet_san.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *san, *objs, "-o", lib],
                   check=True, capture_output=True)
    out = _child({"ALEXNET_LIB": lib, "LD_PRELOAD": rt[-1]}, ["tests/test_abi_host.py"], tmp_path)
    print(out.strip().splitlines()[-1])
