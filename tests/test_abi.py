"""The C ABI library: it loads, exports every declared symbol, and rejects bad
arguments from the host before anything is enqueued (no GPU needed: every
call here fails validation, so no HIP call is reached)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bpk.h")


@pytest.fixture(scope="module")
def lib():
    from bit_plane_key_amd import _lib
    return _lib


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bpk_[a-z_]+)\s*\(", text)))


def test_header_declares_the_six_calls():
    names = declared_symbols()
    for call in ("encode_append", "alloc_depth", "scan_scores", "select_topk",
                 "sparse_attend", "decode_step"):
        assert f"bpk_{call}" in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib.LIB, name), name
    assert set(lib.EXPORTS) == set(declared_symbols())


def _cache(lib, **over):
    n = np.array([over.pop("n", 4096)], dtype=np.int64)
    s = lib.BpkCacheStruct()
    s.num_seqs, s.num_layers, s.num_kv_heads = 1, 2, 8
    s.head_dim, s.group, s.k_dtype = 128, 4, lib.BPK_BF16
    s.capacity = 8192
    fake = 0x10000  # never dereferenced: every call below fails validation
    s.k_rows = s.v_rows = s.planes = s.scales = s.chan_var = fake
    s.rot = None
    for k, v in over.items():
        setattr(s, k, v)
    s.n_tokens = n.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    return s, n


FAKE = 0x20000


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, -2),
    ("group", 3, -2),
    ("num_seqs", 0, -2),
    ("num_seqs", 65, -2),
    ("capacity", 100, -2),
    ("k_dtype", 7, -1),
    ("planes", None, -1),
])
def test_bad_cache_rejected(lib, field, value, code):
    s, n = _cache(lib, **{field: value})
    rc = lib.LIB.bpk_alloc_depth(ctypes.pointer(s), FAKE, 0, 1, 88, FAKE, FAKE, None)
    assert rc == code
    assert lib.last_error()


def test_null_cache_and_outputs(lib):
    assert lib.LIB.bpk_scan_scores(None, FAKE, FAKE, 0, 1, FAKE, None) == -1
    s, n = _cache(lib)
    assert lib.LIB.bpk_scan_scores(ctypes.pointer(s), None, FAKE, 0, 1, FAKE, None) == -1
    assert lib.LIB.bpk_alloc_depth(ctypes.pointer(s), FAKE, 0, 1, -1, FAKE, FAKE, None) == -1


def test_bad_layer_range(lib):
    s, n = _cache(lib)
    for l0, l1 in ((1, 1), (-1, 1), (0, 3), (2, 1)):
        assert lib.LIB.bpk_scan_scores(ctypes.pointer(s), FAKE, FAKE, l0, l1, FAKE, None) == -1


def test_n_tokens_beyond_capacity(lib):
    s, n = _cache(lib, n=8193)
    assert lib.LIB.bpk_scan_scores(ctypes.pointer(s), FAKE, FAKE, 0, 1, FAKE, None) == -1


def test_append_past_capacity(lib):
    s, n = _cache(lib, n=8000)
    assert lib.LIB.bpk_encode_append(ctypes.pointer(s), 0, None, None, 193, None) == -4
    assert lib.LIB.bpk_encode_append(ctypes.pointer(s), 1, None, None, 1, None) == -1
    assert lib.LIB.bpk_encode_append(ctypes.pointer(s), 0, FAKE, None, 1, None) == -1
    assert lib.LIB.bpk_encode_append(ctypes.pointer(s), 0, None, None, -1, None) == -1


def test_k_must_cover_kept_tokens(lib):
    s, n = _cache(lib, n=4096)
    assert lib.LIB.bpk_select_topk(ctypes.pointer(s), FAKE, 0, 1, 35, FAKE, None, 0, None) == -1
    s, n = _cache(lib, n=4096 + 50)   # open block of 50 tokens is kept whole
    assert lib.LIB.bpk_select_topk(ctypes.pointer(s), FAKE, 0, 1, 53, FAKE, None, 0, None) == -1
    assert lib.LIB.bpk_select_topk(ctypes.pointer(s), FAKE, 0, 1, 0, FAKE, None, 0, None) == -1
    assert lib.LIB.bpk_select_topk(ctypes.pointer(s), FAKE, 0, 1, 4097, FAKE, None, 0, None) == -1


def test_workspace_checked(lib):
    s, n = _cache(lib)
    need = lib.LIB.bpk_workspace_bytes(ctypes.pointer(s), lib.BPK_OP_DECODE, 0, 1, 512)
    assert need > 8 * 4 * 8192 * 4           # holds the scores of the call's units
    rc = lib.LIB.bpk_decode_step(ctypes.pointer(s), FAKE, 0, 1, 88, 512, 0.088, FAKE, None, None,
                                 FAKE, need - 1, None)
    assert rc == -3
    need_att = lib.LIB.bpk_workspace_bytes(ctypes.pointer(s), lib.BPK_OP_ATTEND, 0, 1, 512)
    rc = lib.LIB.bpk_sparse_attend(ctypes.pointer(s), FAKE, FAKE, 0, 1, 512, 0.088, FAKE, None,
                                   need_att, None)
    assert rc == -3
    assert lib.LIB.bpk_workspace_bytes(ctypes.pointer(s), 99, 0, 1, 512) == 0
    assert lib.LIB.bpk_workspace_bytes(None, lib.BPK_OP_DECODE, 0, 1, 512) == 0
    assert lib.LIB.bpk_workspace_bytes(ctypes.pointer(s), lib.BPK_OP_SELECT, 0, 1, 512) == 0


def test_noalloc_refuses_more_than_its_scratch(lib):
    """The allocation-free decode step rejects, before any launch, a call whose
    workspace would not fit its scratch array; a small call passes the size
    check (here it then fails on the null q, still before any launch)."""
    s, n = _cache(lib, n=1 << 20, capacity=1 << 20)
    need = lib.LIB.bpk_workspace_bytes(ctypes.pointer(s), lib.BPK_OP_DECODE, 0, 2, 512)
    assert need > lib.NOALLOC_SCRATCH_BYTES
    rc = lib.LIB.bpk_decode_step_noalloc(ctypes.pointer(s), FAKE, 0, 2, 88, 512, 0.088, FAKE,
                                         None, None, None)
    assert rc == -3 and "scratch" in lib.last_error()
    rc = lib.LIB.bpk_decode_step_noalloc(ctypes.pointer(s), None, 0, 1, 88, 512, 0.088, FAKE,
                                         None, None, None)
    assert rc == -1


def test_fixed_depth_validates(lib):
    s, n = _cache(lib)
    c = ctypes.pointer(s)
    assert lib.LIB.bpk_fixed_depth(c, FAKE, 0, 1, 0, 88, None, FAKE, FAKE, None) == -1   # waterfill
    assert lib.LIB.bpk_fixed_depth(c, FAKE, 0, 1, 9, 1, None, FAKE, FAKE, None) == -1
    assert lib.LIB.bpk_fixed_depth(c, FAKE, 0, 1, lib.BPK_DEPTH_SPARQ, 129, None, FAKE, FAKE,
                                   None) == -1
    assert lib.LIB.bpk_fixed_depth(c, FAKE, 0, 1, lib.BPK_DEPTH_UNIFORM, 5, None, FAKE, FAKE,
                                   None) == -1
    assert lib.LIB.bpk_fixed_depth(c, FAKE, 0, 1, lib.BPK_DEPTH_CHANNELS, 32, None, FAKE, FAKE,
                                   None) == -1
    assert lib.LIB.bpk_fixed_depth(c, None, 0, 1, lib.BPK_DEPTH_UNIFORM, 2, None, FAKE, FAKE,
                                   None) == -1
    rc = lib.LIB.bpk_decode_step_depth(c, FAKE, None, FAKE, 0, 0, 1, 512, 0.088, FAKE, None, FAKE,
                                       1 << 30, None)
    assert rc == -1
    rc = lib.LIB.bpk_decode_step_depth(c, FAKE, FAKE, FAKE, -1, 0, 1, 512, 0.088, FAKE, None,
                                       FAKE, 1 << 30, None)
    assert rc == -1 and "max_rows" in lib.last_error()


def test_product_has_no_cpu_path():
    """The package never imports the oracle or any CPU implementation."""
    pkg = os.path.join(ROOT, "bit_plane_key_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            src = open(os.path.join(pkg, f)).read()
            assert "oracle" not in src.replace("no CPU", ""), f


def test_trace_calls_validate_and_start_empty(lib):
    """Stage tracing: NULL outputs are rejected, and with nothing recorded a
    read returns zeros without touching the GPU."""
    assert lib.LIB.bpk_trace_read(None, None, 0) == -1
    assert lib.LIB.bpk_trace_enable(1) == 0
    ms, calls = lib.trace_read()
    assert calls == 0 and set(ms) == set(lib.STAGES) and all(v == 0.0 for v in ms.values())
    assert lib.LIB.bpk_trace_enable(0) == 0


def test_value_entry_points_validate(lib):
    """Value-depth calls need value planes, a non-negative budget and a row
    stride within [1, BPK_MAX_SELECTED]; v_planes and v_scales go together."""
    s, n = _cache(lib)
    c = ctypes.pointer(s)
    # no value planes in the cache
    assert lib.LIB.bpk_value_depth(c, 0, 1, FAKE, FAKE, 64, FAKE, 10, FAKE, None) == -1
    assert "value planes" in lib.last_error()
    assert lib.LIB.bpk_sparse_attend_v(c, FAKE, FAKE, 0, 1, 512, 0.088, 10, FAKE, None, None,
                                       FAKE, 1 << 30, None) == -1
    assert lib.LIB.bpk_decode_step_v(c, FAKE, 0, 1, 88, 512, 0.088, 10, FAKE, None, None, None,
                                     None, FAKE, 1 << 30, None) == -1
    s, n = _cache(lib, v_planes=FAKE)            # scales missing
    assert lib.LIB.bpk_alloc_depth(ctypes.pointer(s), FAKE, 0, 1, 88, FAKE, FAKE, None) == -1
    s, n = _cache(lib, v_planes=FAKE, v_scales=FAKE)
    c = ctypes.pointer(s)
    assert lib.LIB.bpk_value_depth(c, 0, 1, FAKE, FAKE, 0, FAKE, 10, FAKE, None) == -1
    assert lib.LIB.bpk_value_depth(c, 0, 1, FAKE, FAKE, 8193, FAKE, 10, FAKE, None) == -1
    assert lib.LIB.bpk_value_depth(c, 0, 1, FAKE, FAKE, 64, FAKE, -1, FAKE, None) == -1
    assert lib.LIB.bpk_value_depth(c, 0, 1, FAKE, None, 64, FAKE, 1, FAKE, None) == -1
    assert lib.LIB.bpk_sparse_attend_v(c, FAKE, FAKE, 0, 1, 512, 0.088, -1, FAKE, None, None,
                                       FAKE, 1 << 30, None) == -1
    need = lib.LIB.bpk_workspace_bytes(c, lib.BPK_OP_ATTEND_V, 0, 1, 512)
    assert need > lib.LIB.bpk_workspace_bytes(c, lib.BPK_OP_ATTEND, 0, 1, 512)
    assert lib.LIB.bpk_sparse_attend_v(c, FAKE, FAKE, 0, 1, 512, 0.088, 10, FAKE, None, None,
                                       FAKE, need - 1, None) == -3
    need_d = lib.LIB.bpk_workspace_bytes(c, lib.BPK_OP_DECODE_V, 0, 1, 512)
    assert need_d >= lib.LIB.bpk_workspace_bytes(c, lib.BPK_OP_DECODE, 0, 1, 512)
    assert lib.LIB.bpk_decode_step_v(c, FAKE, 0, 1, 88, 512, 0.088, 10, FAKE, None, None, None,
                                     None, FAKE, need_d - 1, None) == -3
    assert lib.LIB.bpk_decode_step_v(c, FAKE, 0, 1, 88, 512, 0.088, -2, FAKE, None, None, None,
                                     None, FAKE, need_d, None) == -1


def test_bench_sample_plan_matches_the_library():
    """bench.py counts the sampled scan's bytes with the library's sample plan
    (the first SAMPLE_GROUP blocks of every SAMPLE_STRIDE)."""
    import bench
    src = open(os.path.join(ROOT, "bit_plane_key_amd", "csrc", "bpk_internal.h")).read()
    stride = int(re.search(r"SAMPLE_STRIDE\s*=\s*(\d+)", src).group(1))
    group = int(re.search(r"SAMPLE_GROUP\s*=\s*(\d+)", src).group(1))
    assert (bench.SAMPLE_STRIDE, bench.SAMPLE_GROUP) == (stride, group)
    assert bench.sampled_blocks(64 * (2 * stride + 10)) == 2 * group + 10
    assert bench.sampled_blocks(64 * 20) == 20
