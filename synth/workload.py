"""Host-side regeneration of any part of a synthetic workload.

Layout only: rows of a unit are drawn with ``synth.philox`` and stored the way
the cache stores them (fp32 or bfloat16 key rows, bfloat16 value rows,
bfloat16 queries).  The device generator in ``synth/csrc/synth_gen.hip``
produces the same bits for every element.
"""
from __future__ import annotations

import numpy as np

from .configs import Config
from .philox import NORMAL_MULT, STREAM_K, STREAM_Q, STREAM_V, normal_values


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rotate_rows(rot: np.ndarray, z: np.ndarray) -> np.ndarray:
    """k = R z per row: fp64 running sum over j in ascending order, then fp32."""
    r = np.asarray(rot, dtype=np.float64)
    zz = np.asarray(z, dtype=np.float64)
    acc = np.zeros((zz.shape[0], r.shape[0]), dtype=np.float64)
    for j in range(r.shape[1]):
        acc = acc + zz[:, j:j + 1] * r[None, :, j]
    return acc.astype(np.float32)


def key_values(cfg: Config, seq: int, layer: int, head: int, rows) -> np.ndarray:
    """fp32 key values before storage rounding, (len(rows), D)."""
    rows = np.asarray(rows, dtype=np.int64)
    key = cfg.key(seq, layer, head)
    x = normal_values(key, rows, np.arange(cfg.dim), STREAM_K, cfg.k_mult(seq, layer, head))
    if cfg.rotated:
        x = rotate_rows(cfg.rotation(layer, head), x)
    return x


def key_rows(cfg: Config, seq: int, layer: int, head: int, rows):
    """Stored key rows: (bits, values).  bits is float32 or uint16 (bf16)."""
    x = key_values(cfg, seq, layer, head, rows)
    if cfg.k_dtype == "f32":
        return x, x
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)


def value_rows(cfg: Config, seq: int, layer: int, head: int, rows):
    """Stored value rows (bf16): (bits, values)."""
    rows = np.asarray(rows, dtype=np.int64)
    x = normal_values(cfg.key(seq, layer, head), rows, np.arange(cfg.dim), STREAM_V,
                      NORMAL_MULT)
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)


def query(cfg: Config, seq: int, layer: int, head: int, step: int = 0):
    """Queries of the unit's G heads at decode step ``step``: (bits, values)."""
    rows = np.arange(cfg.group, dtype=np.int64) + step * cfg.group
    x = normal_values(cfg.key(seq, layer, head), rows, np.arange(cfg.dim), STREAM_Q,
                      NORMAL_MULT)
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)
