"""Pytest plugin of test_host_sanitized.py: binds the package's library
handle to the sanitized host-only build named by BCG_SANITIZED_HOST_LIB, so
the ``host`` cases of test_host_lib.py call instrumented code.  Loaded with
``-p sanitized_host`` in a child process whose environment preloads the
AddressSanitizer runtime."""
import ctypes
import os

from bucketed_classifier_free_amd import _lib as L


def pytest_configure(config):
    L._lib = L.configure(ctypes.CDLL(os.environ["BCG_SANITIZED_HOST_LIB"]), L.HOST_EXPORTS)
