"""The CPU code under the address and undefined-behaviour sanitizers.

Builds the oracle (oracle.c), the input generator (synth.c) and the
host-only validation library (validate.cpp) with -fsanitize=address,undefined
into a scratch directory, then runs the CPU test files that exercise them in
a child process with the sanitizer runtime preloaded and every library
loaded from that directory.  Any sanitizer report fails the run."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _host_builder():
    spec = importlib.util.spec_from_file_location(
        "_moe_build", os.path.join(ROOT, "w4a16_routed_expert_sigmoid_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_cpu_code_clean_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("no libasan runtime")
    d = str(tmp_path)
    subprocess.check_call(["gcc", "-std=c11", "-D_DEFAULT_SOURCE", "-shared", "-fPIC", "-pthread", *SAN,
                           "-o", os.path.join(d, "liboracle.so"), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    subprocess.check_call(["gcc", "-fopenmp", "-shared", "-fPIC", *SAN, "-o", os.path.join(d, "libsynth.so"),
                           os.path.join(ROOT, "synth", "synth.c"), "-lm"])
    _host_builder().build_host(out=os.path.join(d, "libmoe_host.so"), extra_flags=SAN)
    env = dict(os.environ, MOE_HOST_LIB_DIR=d, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=0:exitcode=97",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=98")
    files = ["tests/test_oracle_pins.py", "tests/test_oracle_attn.py", "tests/test_synth.py", "tests/test_compare_helper.py",
             "tests/test_abi.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "-k", "not hip and not exports", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout
