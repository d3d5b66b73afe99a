"""Device-side fill of a workload's key and value rows (binding of libbpk_synth.so).

Produces, directly in GPU memory, the same bits as ``synth.workload`` does on
the host.  Used by the tests and the benchmark to build large caches without
host round trips.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from .configs import Config
from .philox import NORMAL_MULT, STREAM_K, STREAM_V

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbpk_synth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built (python bit_plane_key_amd/build.py)")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
        lib.synth_fill_rows.restype = ctypes.c_int
        lib.synth_fill_rows.argtypes = [P, P, P, I, I, LL, LL, LL, I, I, P, P]
        lib.synth_stream_read.restype = ctypes.c_int
        lib.synth_stream_read.argtypes = [P, LL, I, P, P]
        _lib = lib
    return _lib


def unit_tables(cfg: Config, which: str):
    """Per-unit Philox keys [units][2] (uint32) and multipliers [units][D] (fp32)."""
    keys = np.zeros((cfg.units, 2), dtype=np.uint32)
    mult = np.zeros((cfg.units, cfg.dim), dtype=np.float32)
    for u in range(cfg.units):
        s, l, h = cfg.unit_coords(u)
        keys[u] = cfg.key(s, l, h)
        mult[u] = cfg.k_mult(s, l, h) if which == "k" else NORMAL_MULT
    return keys, mult


def fill_rows(cfg: Config, out: torch.Tensor, which: str, row0: int, rows: int,
              rot: torch.Tensor | None = None, tables=None) -> None:
    """Fill rows [row0, row0 + rows) of every unit of ``out`` ([S][L][H][cap][D])."""
    lib = _load()
    keys, mult = tables if tables is not None else unit_tables(cfg, which)
    dev = out.device
    keys_d = torch.from_numpy(keys.view(np.int32).copy()).to(dev)
    mult_d = torch.from_numpy(mult).to(dev)
    cap = out.shape[-2]
    bf16 = out.dtype == torch.bfloat16
    rc = lib.synth_fill_rows(keys_d.data_ptr(), mult_d.data_ptr(),
                             None if rot is None else rot.data_ptr(),
                             cfg.layers * cfg.heads, cfg.units, row0, rows, cap,
                             STREAM_K if which == "k" else STREAM_V, int(bf16),
                             out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_rows failed ({rc})")
    torch.cuda.current_stream().synchronize()


def stream_read(buf: torch.Tensor, out: torch.Tensor, ptr: int | None = None) -> None:
    """Read every byte of ``buf`` (a benchmark probe of the read bandwidth);
    ``out`` is an int32 tensor of one word per workgroup; ``ptr`` is the
    address the GPU reads buf at (default buf.data_ptr())."""
    lib = _load()
    rc = lib.synth_stream_read(buf.data_ptr() if ptr is None else ptr,
                               buf.numel() * buf.element_size() // 16,
                               out.numel(), out.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_stream_read failed ({rc})")
