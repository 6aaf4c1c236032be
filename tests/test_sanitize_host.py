"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host translation units (argument validation, bank addressing,
workspace sizing, the page manager, the span-slot helper) are built with g++
and -fsanitize=address,undefined against stand-ins for the HIP runtime and
the launchers (tests/sanitize/host_stubs.cpp: no device, every launch
fails), and the oracle's C source with gcc and the same sanitizers. The CPU
tests of both (oracle pins and invariants, page manager parity, C-ABI
validation) then run against those builds with the sanitizer runtimes
preloaded; any report fails the test. No GPU code is built or run here."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_kvcache_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def runtime(name: str) -> str:
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build_oracle(src: str, out: str) -> str:
    subprocess.run(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "oracle"), src, "-o", out, "-lm"], check=True)
    return out


def sanitizer_env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join([runtime("libasan.so"), runtime("libubsan.so")])
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.setdefault("OMP_NUM_THREADS", "4")
    return env


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitize")
    lib = str(d / "libpagedkv_host_san.so")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-fPIC", "-shared",
                    os.path.join(CSRC, "pagedkv.cpp"), os.path.join(CSRC, "page_mgr.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"), "-o", lib],
                   check=True)
    orc = build_oracle(os.path.join(ROOT, "oracle", "oracle.c"), str(d / "liborc_san.so"))
    return lib, orc


def test_host_code_under_sanitizers(builds):
    lib, orc = builds
    env = sanitizer_env()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize",
                                                     "run_host_tests.py"), lib, orc],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out


PLANTED = """
import ctypes, sys
import numpy as np
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
from paged_kv_attention_kvcache_amd import synth
from cases import oracle_decode_case
oracle._lib = oracle._bind(ctypes.CDLL({lib!r}))
case = synth.make_decode_case(0, "f32", 2, (17, 40), 2, 1, 64, num_pages=8)
oracle_decode_case(case)
print("no report")
"""


def test_sanitizers_report_a_planted_overflow(tmp_path):
    # the same build and preload catch a mistake planted in a copy of the
    # oracle: the per-query accumulator cleared one element past its end
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    good = "for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;"
    assert src.count(good) == 1
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(good, "for (int32_t d = 0; d <= D; ++d) acc[d] = 0.0;"))
    lib = build_oracle(str(mutant), str(tmp_path / "liborc_mutant.so"))
    code = PLANTED.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       env=sanitizer_env(), cwd=ROOT, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode != 0 and "heap-buffer-overflow" in out, out[-3000:]
