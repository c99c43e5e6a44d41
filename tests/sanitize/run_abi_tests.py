"""Runs tests/test_abi_cpu.py against a sanitizer build of the C ABI's host
code (argv[1]: the shared library built from api.cpp, shapes.cpp and the
stub launchers), by pointing the binding's library handle at it.  Started as
a subprocess with the AddressSanitizer runtime preloaded; test
infrastructure only."""

import ctypes
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import bitlinear_rmsnorm_absmax_amd as bl  # noqa: E402
from bitlinear_rmsnorm_absmax_amd import _lib  # noqa: E402

san = ctypes.CDLL(sys.argv[1])
for name, args in _lib._SIGNATURES.items():
    fn = getattr(san, name)
    fn.argtypes = args
    fn.restype = ctypes.c_int
san.bitlinear_last_error.restype = ctypes.c_char_p
_lib.lib = san
bl.lib = san
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider",
                      os.path.join(ROOT, "tests", "test_abi_cpu.py")]))
