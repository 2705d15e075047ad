"""Run CPU test files with the library and the oracle replaced by builds whose
host code carries AddressSanitizer and UndefinedBehaviorSanitizer checks.

Started by test_sanitizers.py in a process of its own, with the sanitizer
runtime preloaded. Usage: sanitize_run.py LIBSSD ORACLE_LIB TEST_FILE...
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
from mamba_ssd_sequence_fwd_amd import _lib  # noqa: E402

lib_path, oracle_path, files = sys.argv[1], sys.argv[2], sys.argv[3:]
_lib._lib = None
_lib.load(lib_path)                   # cached: every later load() returns it
oracle._lib = oracle._load(oracle_path)

import pytest  # noqa: E402

sys.exit(pytest.main(["-q", "-m", "not gpu", "-p", "no:cacheprovider", *files]))
