"""Runs the CPU tests of the host code against sanitizer builds of the
library's host code and of the oracle (paths given as arguments), in a
process that has the sanitizer runtimes preloaded. Test infrastructure only;
started by tests/test_sanitize_host.py."""
from __future__ import annotations

import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
ROOT = os.path.dirname(TESTS)
sys.path[:0] = [ROOT, TESTS]

import paged_kv_attention_kvcache_amd as pkv  # noqa: E402
import oracle  # noqa: E402

# the sanitizer runtime must be loaded, or nothing below is checked
assert hasattr(ctypes.CDLL(None), "__asan_init"), "AddressSanitizer runtime not preloaded"
pkv_lib, orc_lib = sys.argv[1], sys.argv[2]
pkv.LIB_PATH = pkv_lib
pkv.lib()
oracle._lib = oracle._bind(ctypes.CDLL(orc_lib))

import pytest  # noqa: E402

files = ["test_oracle_pins.py", "test_oracle_invariants.py", "test_oracle_latest.py",
         "test_oracle_lotus.py", "test_page_mgr.py", "test_abi_host.py"]
args = [os.path.join(TESTS, f) for f in files] + [
    "-q", "-m", "not gpu", "-p", "no:cacheprovider",
    # these two read the real library's binary (exports, code-object targets)
    "--deselect", "tests/test_abi_host.py::test_library_is_gfx950_only",
    "--deselect", "tests/test_abi_host.py::test_exports_every_declared_symbol",
]
sys.exit(pytest.main(args + sys.argv[3:]))
