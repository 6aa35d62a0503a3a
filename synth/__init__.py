"""Seeded synthetic inputs shared by the oracle's tests, the GPU tests and the benchmark.

The generator (``gen.c``) draws counter-based normals (SplitMix64 + Box-Muller) addressed by
(sequence, head, position, element), so any slice of a cache regenerates bit-identically.
This package holds no attention arithmetic: it only makes the Q, K, V buffers, and the
workload descriptions in :mod:`synth.workloads`.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

F32 = 0
BF16 = 1


def build(force=False):
    """Compile gen.c into libsynth.so with gcc (OpenMP, no fast-math)."""
    if os.path.exists(_LIB_PATH) and not force:
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                           os.path.join(_HERE, "gen.c"), "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_double]
        lib.synth_fill.restype = None
        lib.synth_lengths.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int64]
        lib.synth_lengths.restype = None
        lib.synth_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
        lib.synth_uniform.restype = ctypes.c_double
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
        lib.synth_normal.restype = ctypes.c_double
        _lib = lib
    return _lib


def fill(dtype, seed, stream, seq, head0, nheads, pos0, npos, d, layout, span_size=1, offset_norm=0.0, out=None):
    """Normals for heads [head0, head0+nheads) x positions [pos0, pos0+npos) x d elements.

    dtype: ``F32`` (float32 array) or ``BF16`` (uint16 bit patterns).
    layout 0 -> shape [nheads][npos][d] (cache slab); layout 1 -> [npos][nheads][d] (query rows).
    offset_norm > 0 adds the per-(head, span) direction of that norm (span = pos // span_size).
    """
    shape = (nheads, npos, d) if layout == 0 else (npos, nheads, d)
    np_dtype = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty(shape, dtype=np_dtype)
    assert out.dtype == np_dtype and out.flags.c_contiguous and out.size == nheads * npos * d
    assert 0 <= seq < 4096 and 0 <= head0 and head0 + nheads <= 256 and d <= 256
    assert 0 <= pos0 and pos0 + npos < (1 << 36)
    if npos > 0 and nheads > 0:
        _load().synth_fill(out.ctypes.data, dtype, seed, stream, seq, head0, nheads, pos0, npos, d, layout,
                           max(1, int(span_size)), float(offset_norm))
    return out


def lengths(seed, n, lo, hi):
    """n integer lengths drawn uniformly from [lo, hi] (inclusive) from stream 5."""
    out = np.empty(n, dtype=np.int64)
    _load().synth_lengths(out.ctypes.data, seed, n, lo, hi)
    return out


def uniform(seed, stream, idx):
    return _load().synth_uniform(seed, stream, idx)


def normal(seed, stream, idx):
    return _load().synth_normal(seed, stream, idx)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
