"""Build a resident synthetic workload on the GPU through the library.

Rows are drawn on the device by ``synth.device`` (the same bits as the host
generator), the per-unit channel variances, rotations and queries come from
``synth``, and the bit planes are written by the library's own
``encode_append``.  Used by the benchmark, the smoke check and the GPU tests.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from synth import Config
from synth import device as synth_device
from synth import workload as synth_workload

from ._lib import Cache, encode_append


def build_cache(cfg: Config, n: int | None = None, device: str = "cuda",
                host_resident: bool = False, values: bool = False) -> Cache:
    """Allocate the cache of ``cfg``, fill n tokens of rows and encode them.
    With host_resident the rows, planes and scales end in pinned host memory
    (built on the GPU, then copied); with values the cache also holds value
    planes."""
    n = cfg.n if n is None else n
    if host_resident:
        dev = build_cache(cfg, n, device, values=values)
        cache = Cache(cfg.seqs, cfg.layers, cfg.heads, cfg.capacity, group=cfg.group,
                      k_dtype=cfg.k_dtype, rotated=cfg.rotated, device=device,
                      host_resident=True, values=values)
        names = ["k_rows", "v_rows", "planes", "scales", "chan_var"]
        names += ["v_planes", "v_scales"] if values else []
        for name in names:
            getattr(cache, name).copy_(getattr(dev, name))
        if cfg.rotated:
            cache.rot.copy_(dev.rot)
        cache.n_tokens[:] = dev.n_tokens
        del dev
        torch.cuda.synchronize()
        return cache
    cache = Cache(cfg.seqs, cfg.layers, cfg.heads, cfg.capacity, group=cfg.group,
                  k_dtype=cfg.k_dtype, rotated=cfg.rotated, device=device, values=values)
    var = np.zeros((cfg.seqs, cfg.layers, cfg.heads, cfg.dim), dtype=np.float32)
    for s in range(cfg.seqs):
        for l in range(cfg.layers):
            for h in range(cfg.heads):
                var[s, l, h] = cfg.chan_var(s, l, h)
    cache.chan_var.copy_(torch.from_numpy(var))
    if cfg.rotated:
        rot = np.stack([np.stack([cfg.rotation(l, h) for h in range(cfg.heads)])
                        for l in range(cfg.layers)])
        cache.rot.copy_(torch.from_numpy(rot))
    fill_tokens(cfg, cache, 0, n)
    for s in range(cfg.seqs):
        encode_append(cache, s, None, None, n)
    torch.cuda.synchronize()
    return cache


def fill_tokens(cfg: Config, cache: Cache, row0: int, rows: int) -> None:
    """Write rows [row0, row0 + rows) of K and V of every unit in place."""
    chunk = 1 << 16
    ktab = synth_device.unit_tables(cfg, "k")
    vtab = synth_device.unit_tables(cfg, "v")
    for r in range(row0, row0 + rows, chunk):
        m = min(chunk, row0 + rows - r)
        synth_device.fill_rows(cfg, cache.k_rows, "k", r, m, rot=cache.rot, tables=ktab)
        synth_device.fill_rows(cfg, cache.v_rows, "v", r, m, tables=vtab)


def queries(cfg: Config, l0: int = 0, l1: int | None = None, step: int = 0,
            device: str = "cuda") -> torch.Tensor:
    """bf16 queries [S][l1-l0][H][G][D] of decode step ``step``."""
    l1 = cfg.layers if l1 is None else l1
    q = np.zeros((cfg.seqs, l1 - l0, cfg.heads, cfg.group, cfg.dim), dtype=np.uint16)
    for s in range(cfg.seqs):
        for l in range(l0, l1):
            for h in range(cfg.heads):
                q[s, l - l0, h] = synth_workload.query(cfg, s, l, h, step)[0]
    return torch.from_numpy(q.view(np.int16)).to(device).view(torch.bfloat16)


def softmax_scale(cfg: Config) -> float:
    return 1.0 / math.sqrt(cfg.dim)
