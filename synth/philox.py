"""Counter-based random numbers for the synthetic workloads (host side, numpy).

Two published generators are implemented from their definitions:

* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; the 64-bit finaliser popularised by Vigna):
  add the golden-ratio increment, then two xor-shift-multiply rounds and a
  final xor-shift.  Used only to derive one Philox key per (seq, layer, head).
* Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
  easy as 1, 2, 3", SC 2011): ten rounds of two 32x32->64 multiplies whose
  halves are xored with the other counter words and the round key, with a
  Weyl key schedule.

Element recipe (identical on the device, ``synth/csrc/synth_gen.hip``):
counter = (row low 32 bits, row high 32 bits, column, stream), key = unit key.
The four 32-bit outputs are split into eight 16-bit halves; their sum minus
its mean (8 * 32767.5 = 262140) is an exact integer x with variance close to
8 * 65536^2 / 12 (Irwin-Hall of order 8).  A value with standard deviation
sigma is float32(x) * float32(sigma * sqrt(1.5) / 65536), one fp32 product
rounded to nearest even, so the host and the device agree bit for bit.
"""
from __future__ import annotations

import math

import numpy as np

STREAM_K = 0
STREAM_V = 1
STREAM_Q = 2
STREAM_SIGMA = 3
STREAM_ROT = 4

_M64 = (1 << 64) - 1
_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = 0x9E3779B9
_PHILOX_W1 = 0xBB67AE85
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

#: fp32 multiplier that turns the Irwin-Hall integer into a unit-variance value.
NORMAL_MULT = np.float32(math.sqrt(1.5) / 65536.0)


def splitmix64(x: int) -> int:
    """One splitmix64 output for state ``x`` (python int, 64-bit wrap)."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def unit_key(seed: int, seq: int, layer: int, head: int) -> tuple[int, int]:
    """Philox key (k0, k1) of one (sequence, layer, KV head) unit."""
    z = splitmix64((seed ^ (seq << 40) ^ (layer << 20) ^ head) & _M64)
    return z & 0xFFFFFFFF, z >> 32


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on arrays of 32-bit counter words.

    Returns four uint32 arrays.  ``c*`` may be numpy arrays or ints; they are
    broadcast against each other.
    """
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & _LO32 for c in (c0, c1, c2, c3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    ka, kb = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for r in range(10):
        if r:
            ka = (ka + _PHILOX_W0) & 0xFFFFFFFF
            kb = (kb + _PHILOX_W1) & 0xFFFFFFFF
        p0 = x0 * _PHILOX_M0
        p1 = x2 * _PHILOX_M1
        hi0, lo0 = p0 >> _S32, p0 & _LO32
        hi1, lo1 = p1 >> _S32, p1 & _LO32
        x0 = hi1 ^ x1 ^ np.uint64(ka)
        x1 = lo1
        x2 = hi0 ^ x3 ^ np.uint64(kb)
        x3 = lo0
    return tuple(v.astype(np.uint32) for v in (x0, x1, x2, x3))


def irwin_hall8_int(key: tuple[int, int], rows, cols, stream: int) -> np.ndarray:
    """Centred sum of eight 16-bit uniforms for every (row, col) pair.

    ``rows`` and ``cols`` are 1-D integer arrays; the result has shape
    (len(rows), len(cols)) and dtype int32.
    """
    r = np.asarray(rows, dtype=np.uint64)[:, None]
    c = np.asarray(cols, dtype=np.uint64)[None, :]
    words = philox4x32_10(r & _LO32, r >> _S32, c, stream, key[0], key[1])
    total = np.zeros(np.broadcast(r, c).shape, dtype=np.int64)
    for w in words:
        w = w.astype(np.int64)
        total += (w & 0xFFFF) + (w >> 16)
    return (total - 262140).astype(np.int32)


def normal_values(key, rows, cols, stream: int, mult) -> np.ndarray:
    """fp32 values float32(x) * mult[col] (mult broadcast over columns)."""
    x = irwin_hall8_int(key, rows, cols, stream).astype(np.float32)
    return x * np.asarray(mult, dtype=np.float32)


def uniform01(key, rows, cols, stream: int) -> np.ndarray:
    """fp64 uniforms in (0, 1) from the first Philox word: (u + 0.5) / 2^32."""
    r = np.asarray(rows, dtype=np.uint64)[:, None]
    c = np.asarray(cols, dtype=np.uint64)[None, :]
    w = philox4x32_10(r & _LO32, r >> _S32, c, stream, key[0], key[1])[0]
    return (w.astype(np.float64) + 0.5) / 4294967296.0
