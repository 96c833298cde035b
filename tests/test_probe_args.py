"""The measurement probes' argument checks (libkascade_probe.so, used by
bench.py --probe). No GPU is needed: every call here is rejected by host code
before anything is launched, and no pointer passed here is dereferenced.
"""
import ctypes
import os

import pytest

from long_context_amd import build as B

FAKE = 0x10000  # never dereferenced by the checks exercised here


@pytest.fixture(scope="module")
def P():
    if not os.path.exists(B.PROBE_LIBRARY):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(B.PROBE_LIBRARY)
    lib.kascade_probe_mix.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 2
    lib.kascade_probe_mix.restype = ctypes.c_int
    lib.kascade_probe_gather.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 6 + [ctypes.c_void_p] * 2
    lib.kascade_probe_gather.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("kind, mode, d, wps, iters, out", [
    (0, 0, 96, 4, 16, FAKE),     # d other than 64 or 128
    (0, 0, 128, 0, 16, FAKE),    # no wavefronts
    (0, 0, 128, 7, 16, FAKE),    # more than six wavefronts per SIMD
    (0, 0, 128, 4, 0, FAKE),     # no iterations
    (0, 0, 128, 4, 16, None),    # no output
    (2, 0, 128, 2, 16, FAKE),    # unknown kind
    (1, 5, 128, 2, 16, FAKE),    # unknown attention mode
    (1, -1, 64, 2, 16, FAKE),
    (1, 2, 128, 4, 16, FAKE),    # attention above three wavefronts per SIMD
    (1, 0, 128, 3, 16, FAKE),    # a step ahead at d = 128 needs the two-wavefront budget
    (1, 3, 128, 3, 16, FAKE),
    (1, 4, 128, 3, 16, FAKE),
])
def test_mix_rejects(P, kind, mode, d, wps, iters, out):
    assert P.kascade_probe_mix(kind, mode, d, wps, iters, out, None) == 1


@pytest.mark.parametrize("k, v, idx, units, n, length, splits, inflight, contiguous, sink", [
    (FAKE, FAKE, FAKE, 0, 1024, 64, 4, 2, 0, FAKE),      # no units
    (FAKE, FAKE, FAKE, 4, 0, 64, 4, 2, 0, FAKE),         # no keys
    (FAKE, FAKE, FAKE, 4, 1024, 2048, 4, 2, 0, FAKE),    # list longer than the keys
    (FAKE, FAKE, FAKE, 4, 1024, 64, 0, 2, 0, FAKE),      # no splits
    (None, FAKE, FAKE, 4, 1024, 64, 4, 2, 0, FAKE),      # no K
    (FAKE, FAKE, None, 4, 1024, 64, 4, 2, 0, FAKE),      # gathered without a list
    (FAKE, FAKE, FAKE, 4, 1024, 64, 4, 2, 0, None),      # no sink
    (FAKE, FAKE, FAKE, 4, 1024, 64, 4, 3, 0, FAKE),      # rows in flight other than 1, 2, 4, 8
    (FAKE, FAKE, None, 4, 1024, 64, 4, 16, 1, FAKE),
])
def test_gather_rejects(P, k, v, idx, units, n, length, splits, inflight, contiguous, sink):
    assert P.kascade_probe_gather(k, v, idx, units, n, length, splits, inflight, contiguous, sink, None) == 1
