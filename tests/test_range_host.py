"""Host checks of the prefill's buffer ranges (no GPU).

The prefill addresses its inputs and outputs through raw buffer descriptors
with a 32-bit byte range; accesses beyond the range read 0 or are dropped.
The range of a chunk's descriptor is its own window of tokens, computed by
``gdn2::window_bytes`` (``csrc/gdn2_range.hpp``, the same function the kernels
call). These tests compile that header on the host with g++ and check the
range at sequence spans where a 32-bit product of (tokens left) x (token
stride) wraps: exactly 2^32 bytes, 2^32 plus one token, and 2^33.
"""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_83_amd", "csrc")

_SRC = r"""
#include "gdn2_range.hpp"
extern "C" unsigned window_bytes_c(long long t0, long long len, long long window, unsigned stride) {
  return gdn2::window_bytes(t0, len, window, stride);
}
extern "C" int window_fits_c(long long hqk, long long hv, long long dk, long long dv) {
  return gdn2::window_fits(hqk, hv, dk, dv) ? 1 : 0;
}
"""


@pytest.fixture(scope="module")
def rng_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("range")
    src, lib = d / "range.cpp", d / "librange.so"
    src.write_text(_SRC)
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-I", CSRC, str(src), "-o", str(lib)])
    L = ctypes.CDLL(str(lib))
    L.window_bytes_c.restype = ctypes.c_uint32
    L.window_bytes_c.argtypes = [ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_uint32]
    L.window_fits_c.restype = ctypes.c_int
    L.window_fits_c.argtypes = [ctypes.c_longlong] * 4
    return L


def expected(t0, n, window, stride):
    return max(0, min(n - t0, window)) * stride


def wrapped_rest_of_sequence(t0, n, stride):
    """The range a 32-bit product of (tokens left) x stride would give."""
    return ((n - t0) * stride) & 0xFFFFFFFF if t0 < n else 0


# token strides of the wide rows: bf16 values at 32 value heads (8 KiB), bf16
# gate pre-activations at 64 value heads (16 KiB), fp32 gates at 32 (16 KiB)
STRIDES = [32 * 128 * 2, 64 * 128 * 2, 32 * 128 * 4]


@pytest.mark.parametrize("stride", STRIDES)
@pytest.mark.parametrize("extra_tokens", [0, 1, None])  # span 2^32, 2^32 + one token, 2^33
def test_window_at_wrapping_spans(rng_lib, stride, extra_tokens):
    n = (1 << 32) // stride + (extra_tokens if extra_tokens is not None else (1 << 32) // stride)
    window = 32
    starts = list(range(0, 4 * window, window)) + [n - 5, n - window, n - 1, n, n + 7]
    starts += list(range(0, n, max(window, (n // 997) // window * window)))
    wrapped_somewhere = False
    for t0 in starts:
        got = rng_lib.window_bytes_c(t0, n, window, stride)
        assert got == expected(t0, n, window, stride), (t0, n, stride, got)
        # where the old whole-rest-of-sequence range wrapped below the window,
        # the chunk's requests past it would have read zeros
        if t0 < n and wrapped_rest_of_sequence(t0, n, stride) < expected(t0, n, window, stride):
            wrapped_somewhere = True
    assert wrapped_somewhere, "the chosen spans must exercise the 32-bit wrap"


def test_window_edges(rng_lib):
    assert rng_lib.window_bytes_c(0, 0, 32, 512) == 0
    assert rng_lib.window_bytes_c(10, 10, 32, 512) == 0
    assert rng_lib.window_bytes_c(9, 10, 32, 512) == 512
    assert rng_lib.window_bytes_c(0, 10, 0, 512) == 0
    assert rng_lib.window_bytes_c(0, 1 << 40, 64, 32 * 1024) == 64 * 32 * 1024
    # beyond the descriptor's range the value saturates (the interface
    # rejects such problems before any launch)
    assert rng_lib.window_bytes_c(0, 1 << 40, 64, 1 << 26) == 0x7FFFFFFF


def test_window_fits_bound(rng_lib):
    assert rng_lib.window_fits_c(16, 32, 128, 128) == 1
    assert rng_lib.window_fits_c(65535, 65535, 128, 128) == 1
    assert rng_lib.window_fits_c(1, 65536, 128, 128) == 0
    assert rng_lib.window_fits_c(65536, 65536, 16, 16) == 1


def test_interface_rejects_too_wide_rows():
    """gdn2_chunk_forward_plan (host only) refuses rows whose chunk window
    exceeds a descriptor's range, and accepts the widest that fits."""
    import gated_delta_rule_83_amd as g
    st, _, _ = g.gdn2_chunk_forward_plan(g.make_desc(1, 1024, 1, 65536, 128, 128, 64, g.GDN2_BF16))
    assert st == g.GDN2_ERR_UNSUPPORTED
    st, c, n = g.gdn2_chunk_forward_plan(g.make_desc(1, 1024, 1, 65535, 128, 128, 64, g.GDN2_BF16))
    assert st == g.GDN2_OK and c in (16, 32, 64) and n >= 1
