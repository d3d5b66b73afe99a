"""ctypes binding of libbpk.so: argument marshalling only.

Every entry point of ``include/bpk.h`` has a function of the same name here
(without the ``bpk_`` prefix).  Tensors are torch tensors on the GPU; the
functions check dtypes, shapes and devices, pass raw pointers and the current
torch stream, and raise ``BpkError`` on a nonzero return.  No step of the
computation runs in Python, and there is no fallback: importing this module
without the built library raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbpk.so")

BPK_OK, BPK_EINVAL, BPK_EUNSUPPORTED, BPK_EWORKSPACE, BPK_ECAPACITY, BPK_EHIP = 0, -1, -2, -3, -4, -5
BPK_F32, BPK_BF16 = 0, 1
BPK_OP_SELECT, BPK_OP_ATTEND, BPK_OP_DECODE, BPK_OP_POOLED = 3, 4, 5, 6
BPK_OP_ATTEND_V, BPK_OP_DECODE_V = 7, 8
BPK_DEPTH_WATERFILL, BPK_DEPTH_SPARQ, BPK_DEPTH_CHANNELS, BPK_DEPTH_UNIFORM = 0, 1, 2, 3
HEAD_DIM, BLOCK, PLANES = 128, 64, 4

EXPORTS = ("bpk_encode_append", "bpk_alloc_depth", "bpk_fixed_depth", "bpk_pooled_planes",
           "bpk_layer_budgets", "bpk_alloc_depth_layers", "bpk_scan_scores", "bpk_select_topk",
           "bpk_sparse_attend", "bpk_decode_step", "bpk_decode_step_depth",
           "bpk_decode_step_noalloc", "bpk_decode_fallback_units", "bpk_value_depth",
           "bpk_sparse_attend_v", "bpk_decode_step_v", "bpk_workspace_bytes", "bpk_last_error",
           "bpk_trace_enable", "bpk_trace_read")
STAGES = ("alloc", "sample", "threshold", "scan", "select", "fallback", "attend")


def block_stride(capacity: int) -> int:
    """Words per plane row (and scales per scale row): BPK_BLOCK_STRIDE."""
    return (capacity // BLOCK + 7) // 8 * 8


class BpkError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"bpk error {code}: {message}")
        self.code = code


class BpkCacheStruct(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("k_dtype", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("n_tokens", ctypes.POINTER(ctypes.c_int64)),
        ("k_rows", ctypes.c_void_p),
        ("v_rows", ctypes.c_void_p),
        ("planes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("chan_var", ctypes.c_void_p),
        ("rot", ctypes.c_void_p),
        ("v_planes", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python bit_plane_key_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    C = ctypes.POINTER(BpkCacheStruct)
    sig = {
        "bpk_encode_append": (ctypes.c_int, [C, I32, P, P, I64, P]),
        "bpk_alloc_depth": (ctypes.c_int, [C, P, I32, I32, I32, P, P, P]),
        "bpk_fixed_depth": (ctypes.c_int, [C, P, I32, I32, I32, I32, P, P, P, P]),
        "bpk_pooled_planes": (ctypes.c_int, [C, P, I32, I32, I32, P, P, SZ, P]),
        "bpk_layer_budgets": (ctypes.c_int, [C, P, I32, I32, I32, I32, P, P]),
        "bpk_alloc_depth_layers": (ctypes.c_int, [C, P, I32, I32, P, P, P, P]),
        "bpk_scan_scores": (ctypes.c_int, [C, P, P, I32, I32, P, P]),
        "bpk_select_topk": (ctypes.c_int, [C, P, I32, I32, I32, P, P, SZ, P]),
        "bpk_sparse_attend": (ctypes.c_int, [C, P, P, I32, I32, I32, F, P, P, SZ, P]),
        "bpk_decode_step": (ctypes.c_int, [C, P, I32, I32, I32, I32, F, P, P, P, P, SZ, P]),
        "bpk_decode_step_depth": (ctypes.c_int, [C, P, P, P, I32, I32, I32, I32, F, P, P, P, SZ, P]),
        "bpk_decode_step_noalloc": (ctypes.c_int, [C, P, I32, I32, I32, I32, F, P, P, P, P]),
        "bpk_decode_fallback_units": (ctypes.c_int, [C, I32, I32, I32, P, SZ, P, P]),
        "bpk_value_depth": (ctypes.c_int, [C, I32, I32, P, P, I32, P, I32, P, P]),
        "bpk_sparse_attend_v": (ctypes.c_int, [C, P, P, I32, I32, I32, F, I32, P, P, P, P, SZ, P]),
        "bpk_decode_step_v": (ctypes.c_int, [C, P, I32, I32, I32, I32, F, I32, P, P, P, P, P, P,
                                             SZ, P]),
        "bpk_workspace_bytes": (ctypes.c_size_t, [C, I32, I32, I32, I32]),
        "bpk_last_error": (ctypes.c_char_p, []),
        "bpk_trace_enable": (ctypes.c_int, [I32]),
        "bpk_trace_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64), I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


LIB = _load()


def last_error() -> str:
    return LIB.bpk_last_error().decode()


def _check(rc: int) -> None:
    if rc != BPK_OK:
        raise BpkError(rc, last_error())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")


_HIP = None


def _device_pointer(t: torch.Tensor) -> int:
    """The device address of a tensor: its data pointer on the GPU, or for a
    pinned host tensor (hipHostMalloc memory) the address under which the
    GPU reads it over the host link."""
    global _HIP
    if t.device.type == "cuda":
        return t.data_ptr()
    if not t.is_pinned():
        raise ValueError("host arrays of a cache must be pinned (pin_memory=True)")
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipHostGetDevicePointer.restype = ctypes.c_int
        _HIP.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                 ctypes.c_uint]
    dptr = ctypes.c_void_p()
    rc = _HIP.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
    if rc != 0:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({rc})")
    return dptr.value


class Cache:
    """Caller-owned storage of a bit-plane key cache (see include/bpk.h).

    Arrays are torch tensors on the GPU; with ``host_resident`` the key and
    value rows, the planes and the scales are pinned host memory instead,
    which the GPU reads over the host link (the regime of the Fathom page's
    measurements, §1 and §3.1).  With ``values`` the cache also holds value
    planes and per-token value scales (ReadKV §5.3), coded on append.
    ``n_tokens`` is a host int64 array the caller advances after appends.
    """

    def __init__(self, num_seqs: int, num_layers: int, num_kv_heads: int, capacity: int,
                 group: int = 4, k_dtype: str = "bf16", rotated: bool = False,
                 device: str = "cuda", host_resident: bool = False, values: bool = False):
        if capacity % BLOCK:
            raise ValueError("capacity must be a multiple of 64")
        S, L, H, D = num_seqs, num_layers, num_kv_heads, HEAD_DIM
        self.S, self.L, self.H, self.G, self.capacity = S, L, H, group, capacity
        self.k_dtype = k_dtype
        self.host_resident = host_resident
        kt = torch.float32 if k_dtype == "f32" else torch.bfloat16
        big = dict(device="cpu", pin_memory=True) if host_resident else dict(device=device)
        self.k_rows = torch.empty((S, L, H, capacity, D), dtype=kt, **big)
        self.v_rows = torch.empty((S, L, H, capacity, D), dtype=torch.bfloat16, **big)
        nb = block_stride(capacity)
        self.planes = torch.zeros((S, L, H, D, PLANES, nb), dtype=torch.int64, **big)
        self.scales = torch.zeros((S, L, H, D, nb), dtype=torch.float16, **big)
        self.v_planes = self.v_scales = None
        names = ["k_rows", "v_rows", "planes", "scales"]
        if values:
            self.v_planes = torch.zeros((S, L, H, capacity, PLANES, D // 8), dtype=torch.uint8,
                                        **big)
            self.v_scales = torch.zeros((S, L, H, capacity), dtype=torch.float16, **big)
            names += ["v_planes", "v_scales"]
        self._ptrs = {name: _device_pointer(getattr(self, name)) for name in names}
        self.chan_var = torch.ones((S, L, H, D), dtype=torch.float32, device=device)
        self.rot = (torch.empty((L, H, D, D), dtype=torch.float32, device=device)
                    if rotated else None)
        self.n_tokens = np.zeros(S, dtype=np.int64)
        self._struct = BpkCacheStruct()

    def struct(self) -> ctypes.POINTER(BpkCacheStruct):
        s = self._struct
        s.num_seqs, s.num_layers, s.num_kv_heads = self.S, self.L, self.H
        s.head_dim, s.group = HEAD_DIM, self.G
        s.k_dtype = BPK_F32 if self.k_dtype == "f32" else BPK_BF16
        s.capacity = self.capacity
        s.n_tokens = self.n_tokens.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        s.k_rows, s.v_rows = self._ptrs["k_rows"], self._ptrs["v_rows"]
        s.planes, s.scales = self._ptrs["planes"], self._ptrs["scales"]
        s.chan_var = self.chan_var.data_ptr()
        s.rot = None if self.rot is None else self.rot.data_ptr()
        s.v_planes = self._ptrs.get("v_planes")
        s.v_scales = self._ptrs.get("v_scales")
        return ctypes.pointer(s)

    def units(self, l0: int, l1: int) -> int:
        return self.S * (l1 - l0) * self.H


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def workspace_bytes(cache: Cache, op: int, l0: int, l1: int, k: int) -> int:
    return int(LIB.bpk_workspace_bytes(cache.struct(), op, l0, l1, k))


def encode_append(cache: Cache, seq: int, k_new=None, v_new=None, n_new: int | None = None,
                  stream=None) -> None:
    """Append tokens to sequence ``seq`` and encode the blocks they complete.

    With ``k_new``/``v_new`` None the rows are already in place and ``n_new``
    must be given.  Advances ``cache.n_tokens[seq]``.
    """
    if k_new is not None:
        n_new = k_new.shape[2]
        kt = torch.float32 if cache.k_dtype == "f32" else torch.bfloat16
        _need(k_new, "k_new", kt, (cache.L, cache.H, n_new, HEAD_DIM))
        _need(v_new, "v_new", torch.bfloat16, (cache.L, cache.H, n_new, HEAD_DIM))
    _check(LIB.bpk_encode_append(cache.struct(), seq, _ptr(k_new), _ptr(v_new), int(n_new),
                                 _stream(stream)))
    cache.n_tokens[seq] += int(n_new)


def alloc_depth(cache: Cache, q: torch.Tensor, l0: int, l1: int, budget: int, depth=None,
                q_basis=None, stream=None):
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    if depth is None:
        depth = torch.empty((*u, HEAD_DIM), dtype=torch.uint8, device=q.device)
    if q_basis is None:
        q_basis = torch.empty((*u, cache.G, HEAD_DIM), dtype=torch.float32, device=q.device)
    _need(depth, "depth", torch.uint8, (*u, HEAD_DIM))
    _need(q_basis, "q_basis", torch.float32, (*u, cache.G, HEAD_DIM))
    _check(LIB.bpk_alloc_depth(cache.struct(), q.data_ptr(), l0, l1, int(budget),
                               depth.data_ptr(), q_basis.data_ptr(), _stream(stream)))
    return depth, q_basis


def fixed_depth(cache: Cache, q: torch.Tensor, l0: int, l1: int, rule: int, param: int,
                channels=None, depth=None, q_basis=None, stream=None):
    """A baseline depth rule (BPK_DEPTH_SPARQ / _CHANNELS / _UNIFORM, see bpk.h);
    channels: uint8 [L][H][param] on the GPU for BPK_DEPTH_CHANNELS."""
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    if depth is None:
        depth = torch.empty((*u, HEAD_DIM), dtype=torch.uint8, device=q.device)
    if q_basis is None:
        q_basis = torch.empty((*u, cache.G, HEAD_DIM), dtype=torch.float32, device=q.device)
    _need(depth, "depth", torch.uint8, (*u, HEAD_DIM))
    _need(q_basis, "q_basis", torch.float32, (*u, cache.G, HEAD_DIM))
    if channels is not None:
        _need(channels, "channels", torch.uint8, (cache.L, cache.H, param))
    _check(LIB.bpk_fixed_depth(cache.struct(), q.data_ptr(), l0, l1, int(rule), int(param),
                               _ptr(channels), depth.data_ptr(), q_basis.data_ptr(),
                               _stream(stream)))
    return depth, q_basis


def pooled_planes(cache: Cache, q: torch.Tensor, l0: int, l1: int, budget: int, counts=None,
                  ws=None, stream=None):
    """Planes each unit of layers [l0, l1) gets when the call's whole budget
    is water-filled over all its units (int32 [S][nl][H])."""
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    if counts is None:
        counts = torch.empty(u, dtype=torch.int32, device=q.device)
    _need(counts, "counts", torch.int32, u)
    if ws is None:
        ws = torch.empty(workspace_bytes(cache, BPK_OP_POOLED, l0, l1, 1), dtype=torch.uint8,
                         device=q.device)
    _check(LIB.bpk_pooled_planes(cache.struct(), q.data_ptr(), l0, l1, int(budget),
                                 counts.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))
    return counts


def layer_budgets(cache: Cache, counts: torch.Tensor, l0: int, l1: int, budget: int, out=None,
                  stream=None):
    """Per-layer budgets [nl] from pooled counts [queries][S][nl][H]."""
    nq = counts.shape[0]
    _need(counts, "counts", torch.int32, (nq, cache.S, l1 - l0, cache.H))
    if out is None:
        out = torch.empty(l1 - l0, dtype=torch.int32, device=counts.device)
    _need(out, "out", torch.int32, (l1 - l0,))
    _check(LIB.bpk_layer_budgets(cache.struct(), counts.data_ptr(), nq, l0, l1, int(budget),
                                 out.data_ptr(), _stream(stream)))
    return out


def alloc_depth_layers(cache: Cache, q: torch.Tensor, l0: int, l1: int, budgets: torch.Tensor,
                       depth=None, q_basis=None, stream=None):
    """alloc_depth with a budget per layer (int32 [l1 - l0] on the GPU)."""
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    _need(budgets, "budgets", torch.int32, (l1 - l0,))
    if depth is None:
        depth = torch.empty((*u, HEAD_DIM), dtype=torch.uint8, device=q.device)
    if q_basis is None:
        q_basis = torch.empty((*u, cache.G, HEAD_DIM), dtype=torch.float32, device=q.device)
    _need(depth, "depth", torch.uint8, (*u, HEAD_DIM))
    _need(q_basis, "q_basis", torch.float32, (*u, cache.G, HEAD_DIM))
    _check(LIB.bpk_alloc_depth_layers(cache.struct(), q.data_ptr(), l0, l1, budgets.data_ptr(),
                                      depth.data_ptr(), q_basis.data_ptr(), _stream(stream)))
    return depth, q_basis


def scan_scores(cache: Cache, q_basis: torch.Tensor, depth: torch.Tensor, l0: int, l1: int,
                scores=None, stream=None):
    u = (cache.S, l1 - l0, cache.H)
    _need(q_basis, "q_basis", torch.float32, (*u, cache.G, HEAD_DIM))
    _need(depth, "depth", torch.uint8, (*u, HEAD_DIM))
    if scores is None:
        scores = torch.zeros((*u, cache.G, cache.capacity), dtype=torch.float32,
                             device=q_basis.device)
    _need(scores, "scores", torch.float32, (*u, cache.G, cache.capacity))
    _check(LIB.bpk_scan_scores(cache.struct(), q_basis.data_ptr(), depth.data_ptr(), l0, l1,
                               scores.data_ptr(), _stream(stream)))
    return scores


def select_topk(cache: Cache, scores: torch.Tensor, l0: int, l1: int, k: int, idx=None,
                stream=None):
    u = (cache.S, l1 - l0, cache.H)
    _need(scores, "scores", torch.float32, (*u, cache.G, cache.capacity))
    if idx is None:
        idx = torch.empty((*u, cache.G, k), dtype=torch.int32, device=scores.device)
    _need(idx, "idx", torch.int32, (*u, cache.G, k))
    _check(LIB.bpk_select_topk(cache.struct(), scores.data_ptr(), l0, l1, int(k),
                               idx.data_ptr(), None, 0, _stream(stream)))
    return idx


def sparse_attend(cache: Cache, q: torch.Tensor, idx: torch.Tensor, l0: int, l1: int, k: int,
                  softmax_scale: float, out=None, ws=None, stream=None):
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    _need(idx, "idx", torch.int32, (*u, cache.G, k))
    if out is None:
        out = torch.empty((*u, cache.G, HEAD_DIM), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (*u, cache.G, HEAD_DIM))
    need = workspace_bytes(cache, BPK_OP_ATTEND, l0, l1, k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(LIB.bpk_sparse_attend(cache.struct(), q.data_ptr(), idx.data_ptr(), l0, l1, int(k),
                                 float(softmax_scale), out.data_ptr(), ws.data_ptr(),
                                 ws.numel(), _stream(stream)))
    return out


def decode_step(cache: Cache, q: torch.Tensor, l0: int, l1: int, budget: int, k: int,
                softmax_scale: float, out=None, depth_out=None, idx_out=None, ws=None,
                stream=None):
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    if out is None:
        out = torch.empty((*u, cache.G, HEAD_DIM), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (*u, cache.G, HEAD_DIM))
    if depth_out is not None:
        _need(depth_out, "depth_out", torch.uint8, (*u, HEAD_DIM))
    if idx_out is not None:
        _need(idx_out, "idx_out", torch.int32, (*u, cache.G, k))
    need = workspace_bytes(cache, BPK_OP_DECODE, l0, l1, k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(LIB.bpk_decode_step(cache.struct(), q.data_ptr(), l0, l1, int(budget), int(k),
                               float(softmax_scale), out.data_ptr(), _ptr(depth_out),
                               _ptr(idx_out), ws.data_ptr(), ws.numel(), _stream(stream)))
    return out


def decode_step_depth(cache: Cache, q: torch.Tensor, q_basis: torch.Tensor, depth: torch.Tensor,
                      l0: int, l1: int, k: int, softmax_scale: float, out=None, idx_out=None,
                      ws=None, stream=None, max_rows: int = 0):
    """decode_step on given depths (from alloc_depth or fixed_depth); max_rows:
    a bound on the plane rows (sum of depths) of every unit, 0 if not known."""
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    _need(q_basis, "q_basis", torch.float32, (*u, cache.G, HEAD_DIM))
    _need(depth, "depth", torch.uint8, (*u, HEAD_DIM))
    if out is None:
        out = torch.empty((*u, cache.G, HEAD_DIM), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (*u, cache.G, HEAD_DIM))
    if idx_out is not None:
        _need(idx_out, "idx_out", torch.int32, (*u, cache.G, k))
    need = workspace_bytes(cache, BPK_OP_DECODE, l0, l1, k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(LIB.bpk_decode_step_depth(cache.struct(), q.data_ptr(), q_basis.data_ptr(),
                                     depth.data_ptr(), int(max_rows), l0, l1, int(k),
                                     float(softmax_scale),
                                     out.data_ptr(), _ptr(idx_out), ws.data_ptr(), ws.numel(),
                                     _stream(stream)))
    return out


def decode_fallback_units(cache: Cache, l0: int, l1: int, k: int, ws: torch.Tensor,
                          stream=None) -> int:
    """Units that the last decode_step on ``ws`` redid unfused (see bpk.h);
    waits for the stream."""
    out = torch.zeros(1, dtype=torch.int32, device=ws.device)
    _check(LIB.bpk_decode_fallback_units(cache.struct(), l0, l1, int(k), ws.data_ptr(),
                                         ws.numel(), out.data_ptr(), _stream(stream)))
    return int(out.item())


NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_step_noalloc(cache: Cache, q: torch.Tensor, l0: int, l1: int, budget: int, k: int,
                        softmax_scale: float, out: torch.Tensor, depth_out=None, idx_out=None,
                        stream=None):
    """decode_step on the library's own scratch array: nothing is allocated,
    so ``out`` (and the optional outputs) must be given."""
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    _need(out, "out", torch.float32, (*u, cache.G, HEAD_DIM))
    if depth_out is not None:
        _need(depth_out, "depth_out", torch.uint8, (*u, HEAD_DIM))
    if idx_out is not None:
        _need(idx_out, "idx_out", torch.int32, (*u, cache.G, k))
    _check(LIB.bpk_decode_step_noalloc(cache.struct(), q.data_ptr(), l0, l1, int(budget), int(k),
                                       float(softmax_scale), out.data_ptr(), _ptr(depth_out),
                                       _ptr(idx_out), _stream(stream)))
    return out


def value_depth(cache: Cache, l0: int, l1: int, rows: torch.Tensor, n_rows: torch.Tensor,
                weights: torch.Tensor, v_budget: int, depth=None, stream=None):
    """Per-row value depths from given importances (see bpk.h)."""
    u = (cache.S, l1 - l0, cache.H)
    ld = rows.shape[-1]
    _need(rows, "rows", torch.int32, (*u, ld))
    _need(n_rows, "n_rows", torch.int32, u)
    _need(weights, "weights", torch.float32, (*u, ld))
    if depth is None:
        depth = torch.empty((*u, ld), dtype=torch.uint8, device=rows.device)
    _need(depth, "depth", torch.uint8, (*u, ld))
    _check(LIB.bpk_value_depth(cache.struct(), l0, l1, rows.data_ptr(), n_rows.data_ptr(), int(ld),
                               weights.data_ptr(), int(v_budget), depth.data_ptr(),
                               _stream(stream)))
    return depth


def _value_outputs(cache, u, k, union_out, v_depth_out):
    if union_out is not None:
        _need(union_out, "union_out", torch.int32, (*u, cache.G * k))
    if v_depth_out is not None:
        _need(v_depth_out, "v_depth_out", torch.uint8, (*u, cache.G * k))


def sparse_attend_v(cache: Cache, q: torch.Tensor, idx: torch.Tensor, l0: int, l1: int, k: int,
                    softmax_scale: float, v_budget: int, out=None, union_out=None,
                    v_depth_out=None, ws=None, stream=None):
    """Sparse attention with value rows read at per-token depths."""
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    _need(idx, "idx", torch.int32, (*u, cache.G, k))
    if out is None:
        out = torch.empty((*u, cache.G, HEAD_DIM), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (*u, cache.G, HEAD_DIM))
    _value_outputs(cache, u, k, union_out, v_depth_out)
    need = workspace_bytes(cache, BPK_OP_ATTEND_V, l0, l1, k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(LIB.bpk_sparse_attend_v(cache.struct(), q.data_ptr(), idx.data_ptr(), l0, l1, int(k),
                                   float(softmax_scale), int(v_budget), out.data_ptr(),
                                   _ptr(union_out), _ptr(v_depth_out), ws.data_ptr(), ws.numel(),
                                   _stream(stream)))
    return out


def decode_step_v(cache: Cache, q: torch.Tensor, l0: int, l1: int, budget: int, k: int,
                  softmax_scale: float, v_budget: int, out=None, depth_out=None, idx_out=None,
                  union_out=None, v_depth_out=None, ws=None, stream=None):
    """decode_step whose attention reads the value rows at per-token depths."""
    u = (cache.S, l1 - l0, cache.H)
    _need(q, "q", torch.bfloat16, (*u, cache.G, HEAD_DIM))
    if out is None:
        out = torch.empty((*u, cache.G, HEAD_DIM), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (*u, cache.G, HEAD_DIM))
    if depth_out is not None:
        _need(depth_out, "depth_out", torch.uint8, (*u, HEAD_DIM))
    if idx_out is not None:
        _need(idx_out, "idx_out", torch.int32, (*u, cache.G, k))
    _value_outputs(cache, u, k, union_out, v_depth_out)
    need = workspace_bytes(cache, BPK_OP_DECODE_V, l0, l1, k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(LIB.bpk_decode_step_v(cache.struct(), q.data_ptr(), l0, l1, int(budget), int(k),
                                 float(softmax_scale), int(v_budget), out.data_ptr(),
                                 _ptr(depth_out), _ptr(idx_out), _ptr(union_out),
                                 _ptr(v_depth_out), ws.data_ptr(), ws.numel(), _stream(stream)))
    return out


def trace_enable(on: bool = True) -> None:
    """Turn stage tracing of decode_step on or off for the calling thread."""
    _check(LIB.bpk_trace_enable(1 if on else 0))


def trace_read(reset: bool = True) -> tuple[dict, int]:
    """Summed milliseconds per decode_step stage over the traced calls, and
    the number of calls (waits for the recorded events)."""
    ms = (ctypes.c_double * len(STAGES))()
    calls = ctypes.c_int64(0)
    _check(LIB.bpk_trace_read(ms, ctypes.byref(calls), 1 if reset else 0))
    return {name: ms[i] for i, name in enumerate(STAGES)}, int(calls.value)
