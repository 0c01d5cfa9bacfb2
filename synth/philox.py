"""Philox-4x32-10 counter-based generator and a Box-Muller normal stream.

Philox-4x32-10 follows its published definition (Salmon, Moraes, Dror, Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11, section 3.2): ten rounds
of a multiply-high/low bijection on four 32-bit words, with the two-word key
bumped by the Weyl constants between rounds.

Stream layout used by every tensor of a workload:
  key     = (seed, tensor_id)
  counter = (i mod 2**32, i div 2**32, 0, 0) for block i = 0, 1, 2, ...
  block i yields two 64-bit words r0 = x0 | x1 << 32 and r1 = x2 | x3 << 32,
  each mapped to a uniform u = ((r >> 11) + 1/2) * 2**-53 in (0, 1),
  and the Box-Muller pair
      z0 = sqrt(-2 ln u0) cos(2 pi u1),  z1 = sqrt(-2 ln u0) sin(2 pi u1)
  supplies elements 2i and 2i + 1 of the tensor (row-major order).

The bulk generator is C (synth/philox_words.c, OpenMP); the numpy functions
here are its slow twin, used to check it.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Apply Philox-4x32-10 to arrays of counters (uint64 arrays holding 32-bit
    values) under the key (k0, k1).  Returns the four output words as uint64
    arrays holding 32-bit values."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
        p0 = c0 * PHILOX_M0          # exact: 32 x 32 -> 64 bits
        p1 = c2 * PHILOX_M1
        hi0, lo0 = p0 >> _S32, p0 & _MASK32
        hi1, lo1 = p1 >> _S32, p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
    return c0, c1, c2, c3


def _words_numpy(seed: int, tensor_id: int, first_pair: int, n_pairs: int):
    i = np.arange(first_pair, first_pair + n_pairs, dtype=np.uint64)
    zero = np.zeros_like(i)
    x0, x1, x2, x3 = philox4x32_10(i & _MASK32, i >> _S32, zero, zero, seed, tensor_id)
    return x0 | (x1 << _S32), x2 | (x3 << _S32)


_CLIB = None
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_philox_words.so")


def _clib():
    global _CLIB
    if _CLIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_philox_words.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32,
                                           ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_philox_words.restype = None
        lib.synth_normals_f32.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p]
        lib.synth_normals_f32.restype = None
        _CLIB = lib
    return _CLIB


def philox_words(seed: int, tensor_id: int, first_pair: int, n_pairs: int, use_c: bool = True):
    """The two 64-bit words (r0, r1) of blocks first_pair .. first_pair + n_pairs - 1."""
    if not use_c:
        return _words_numpy(seed, tensor_id, first_pair, n_pairs)
    r0 = np.empty(n_pairs, dtype=np.uint64)
    r1 = np.empty(n_pairs, dtype=np.uint64)
    _clib().synth_philox_words(first_pair, n_pairs, int(seed) & 0xFFFFFFFF,
                               int(tensor_id) & 0xFFFFFFFF, r0.ctypes.data, r1.ctypes.data)
    return r0, r1


def normals_f32(seed: int, tensor_id: int, n: int, std: float = 1.0) -> np.ndarray:
    """First ``n`` values of the stream as float32: each Box-Muller value is
    computed in double, multiplied by ``std`` in double and rounded once to
    float32."""
    n = int(n)
    if n < 0:
        raise ValueError("n must be non-negative")
    out = np.empty(n, dtype=np.float32)
    _clib().synth_normals_f32(0, n, int(seed) & 0xFFFFFFFF, int(tensor_id) & 0xFFFFFFFF,
                              float(std), out.ctypes.data)
    return out


def normals_reference(seed: int, tensor_id: int, n: int, std: float = 1.0) -> np.ndarray:
    """Pure-numpy evaluation of the same definition (slow; checks the C build).
    Its transcendentals come from numpy rather than libm, so a value may differ
    from ``normals_f32`` by one float32 ulp in rare cases."""
    n_pairs = (int(n) + 1) // 2
    r0, r1 = _words_numpy(seed, tensor_id, 0, n_pairs)
    scale = 2.0 ** -53
    u0 = ((r0 >> np.uint64(11)).astype(np.float64) + 0.5) * scale
    u1 = ((r1 >> np.uint64(11)).astype(np.float64) + 0.5) * scale
    rad = np.sqrt(-2.0 * np.log(u0))
    ang = 2.0 * np.pi * u1
    z = np.empty(2 * n_pairs, dtype=np.float64)
    z[0::2] = rad * np.cos(ang)
    z[1::2] = rad * np.sin(ang)
    return (std * z[:int(n)]).astype(np.float32)
