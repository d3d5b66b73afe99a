"""The five synthetic workloads and their seeded per-unit parameters.

A *unit* is one (sequence, layer, KV head).  Keys of a unit are drawn per
channel j with standard deviation sigma_j; V and q are unit-variance.  The
workloads stand in for the key caches of Qwen3-8B-shaped (36 layers, 8 KV
heads of 128 channels, 4 query heads per KV head) and Llama-3.1-8B-shaped
(32 layers) models described on the Fathom page (§1 and §2); no model weights
or datasets are used.

sigma_j recipes:
* log-uniform on [0.1, 4]: sigma = exp(ln 0.1 + U ln 40);
* heavy-tailed (Pareto, alpha = 1.5): sigma = 0.1 * U^(-1/1.5), capped at 1000.
U comes from the unit's Philox stream ``STREAM_SIGMA`` (row 0, column j).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .philox import (NORMAL_MULT, STREAM_ROT, STREAM_SIGMA, normal_values,
                     uniform01, unit_key)

BLOCK = 64
ROT_SEQ = 0xFFFFF  # sequence slot of the per-(layer, head) rotation keys


@dataclass(frozen=True)
class Config:
    name: str
    seqs: int
    layers: int
    heads: int
    n: int                     # tokens per sequence when the step starts
    k: int                     # top-k per query head
    budgets: tuple             # plane budgets P
    seed: int
    group: int = 4
    dim: int = 128
    k_dtype: str = "bf16"      # dtype of the stored key rows ("f32" or "bf16")
    pareto_from_head: int = -1  # KV heads >= this use Pareto sigmas (-1: none)
    rotated: bool = False      # keys pre-rotated by a per-(layer, head) orthogonal R
    append_steps: int = 0      # decode steps that each append one token per sequence
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def units(self) -> int:
        return self.seqs * self.layers * self.heads

    @property
    def capacity(self) -> int:
        total = self.n + self.append_steps
        return (total + BLOCK - 1) // BLOCK * BLOCK

    def unit_index(self, seq: int, layer: int, head: int) -> int:
        return (seq * self.layers + layer) * self.heads + head

    def unit_coords(self, u: int) -> tuple[int, int, int]:
        head = u % self.heads
        layer = (u // self.heads) % self.layers
        seq = u // (self.heads * self.layers)
        return seq, layer, head

    def key(self, seq: int, layer: int, head: int):
        return unit_key(self.seed, seq, layer, head)

    def sigma(self, seq: int, layer: int, head: int) -> np.ndarray:
        """fp64 per-channel standard deviations of the unit's keys."""
        u = uniform01(self.key(seq, layer, head), [0], np.arange(self.dim), STREAM_SIGMA)[0]
        if 0 <= self.pareto_from_head <= head:
            return np.minimum(0.1 * u ** (-1.0 / 1.5), 1000.0)
        return np.exp(math.log(0.1) + u * math.log(40.0))

    def chan_var(self, seq: int, layer: int, head: int) -> np.ndarray:
        """sigma_j^2 in fp32: the channel variance handed to the depth rule."""
        return (self.sigma(seq, layer, head) ** 2).astype(np.float32)

    def k_mult(self, seq: int, layer: int, head: int) -> np.ndarray:
        """fp32 per-channel multipliers of the key generator."""
        return (self.sigma(seq, layer, head) * (math.sqrt(1.5) / 65536.0)).astype(np.float32)

    def rotation(self, layer: int, head: int) -> np.ndarray:
        """Seeded Haar-orthogonal D x D matrix (fp32) of one (layer, head).

        QR of a seeded Gaussian matrix, columns sign-fixed so that the
        triangular factor has a positive diagonal.
        """
        key = unit_key(self.seed, ROT_SEQ, layer, head)
        g = normal_values(key, np.arange(self.dim), np.arange(self.dim), STREAM_ROT,
                          NORMAL_MULT).astype(np.float64)
        qm, rm = np.linalg.qr(g)
        qm = qm * np.sign(np.diag(rm))[None, :]
        return qm.astype(np.float32)


CONFIGS = [
    Config("c1", seqs=1, layers=1, heads=1, n=4096, k=64, budgets=(64,), seed=1000,
           k_dtype="f32",
           description="single layer, 1 KV head, n=4096, fp32 keys, P=64, k=64"),
    Config("c2", seqs=1, layers=1, heads=8, n=32768, k=512, budgets=(64, 88, 128), seed=1001,
           description="Qwen3-8B-shaped single layer, 8 KV heads, n=32768"),
    Config("c3", seqs=4, layers=36, heads=8, n=131072, k=512, budgets=(88,), seed=1002,
           description="full decode step, 36 layers x 8 KV heads x 4 sequences, n=131072"),
    Config("c4", seqs=1, layers=36, heads=8, n=1048576, k=512, budgets=(64, 88, 128), seed=1003,
           pareto_from_head=4,
           description="long context, 36 layers x 8 KV heads, n=1048576, heads 4-7 Pareto"),
    Config("c5", seqs=8, layers=32, heads=8, n=131072, k=512, budgets=(88,), seed=1004,
           rotated=True, append_steps=64,
           description="Llama-3.1-8B-shaped, 32 layers x 8 KV heads x 8 sequences, "
                       "rotated keys, one appended token per step"),
]


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
