"""Memory and undefined-behaviour checks of the host code, on the CPU.

* The float64 oracle (oracle/kda_oracle.c) built with gcc's AddressSanitizer
  and UndefinedBehaviorSanitizer runs its pins.
* The library's argument validation (kda_api.hip, host code only: the
  sanitizers instrument the host pass, the GPU code is untouched) runs every
  case of tests/test_abi.py.  No call there reaches a kernel launch.

Each run happens in a child process with the sanitizer runtime preloaded;
any report makes that process fail.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=97",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=98"}


def _child(env_extra, *pytest_args):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *pytest_args]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc has no AddressSanitizer runtime")
    lib = str(tmp_path / "libkda_oracle_san.so")
    san = "-fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer".split()
    subprocess.run([gcc, "-O1", "-g", "-fopenmp", "-shared", "-fPIC", "-std=c11", *san, "-o", lib,
                    os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm"], check=True)
    r = _child({"LD_PRELOAD": asan, "KDA_ORACLE_LIBRARY": lib},
               "tests/test_oracle_pins.py", "tests/test_gate_pins.py", "tests/test_sanitizer_probe.py")
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]


def test_host_validation_under_asan_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    rts = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(hipcc) or not rts:
        pytest.skip("hipcc or its AddressSanitizer runtime not found")
    sys.path.insert(0, ROOT)
    from gated_delta_rule_101_amd import build_lib
    objs = [o for o in glob.glob(os.path.join(build_lib.BUILD, "*.o")) if not o.endswith("kda_api.hip.o")]
    if len(objs) < 2:
        build_lib.build_library()
        objs = [o for o in glob.glob(os.path.join(build_lib.BUILD, "*.o")) if not o.endswith("kda_api.hip.o")]
    # host pass only: every sanitizer flag goes to the host compiler
    san = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
           "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
    obj = str(tmp_path / "kda_api_san.o")
    lib = str(tmp_path / "libkda_san.so")
    flags = [f for f in build_lib.HIPCC_FLAGS if not f.startswith("-O")]
    subprocess.run([hipcc, *flags, "-O1", "-g", *san, "-c", os.path.join(build_lib.CSRC, "kda_api.hip"),
                    "-o", obj], check=True, capture_output=True)
    subprocess.run([hipcc, f"--offload-arch={build_lib.ARCH}", "-shared", "-fPIC", *san[:4], "-shared-libsan",
                    "-o", lib, obj, *objs], check=True, capture_output=True)
    r = _child({"LD_PRELOAD": rts[0], "KDA_LIBRARY": lib}, "tests/test_abi.py", "tests/test_sanitizer_probe.py")
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
