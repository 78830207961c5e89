"""GPU check of the plain-read ceiling helper (libkvattn_probe.so) that the
benchmark uses for context: a small read runs and reports finite positive
times for every policy and grid size."""
import ctypes
import math

import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def test_probe_read_ceiling_small():
    from long_context_attention_amd import build as hipbuild
    P = ctypes.CDLL(hipbuild.PROBE_LIB)
    fn = P.kvattn_probe_read_ceiling
    fn.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_double),
                   ctypes.POINTER(ctypes.c_double)]
    fn.restype = ctypes.c_int
    us = (ctypes.c_double * 8)()
    best = ctypes.c_double()
    nbytes = 4 * 1024 * 1024 + 48  # a ragged tail of three 16-byte words
    assert fn(nbytes, 2, 2, us, ctypes.byref(best)) == 0
    assert all(math.isfinite(u) and u > 0 for u in us)
    assert math.isfinite(best.value) and best.value > 0
    assert abs(best.value - max(nbytes / u / 1e3 for u in us)) <= 1e-6 * best.value
