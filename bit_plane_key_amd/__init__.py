"""MI355X (gfx950) top-k sparse decode attention over a bit-plane 4-bit key cache.

The computation lives in ``libbpk.so`` (hand-written HIP, C ABI declared in
``include/bpk.h``); this package is its Python binding.  Importing it without
the built library raises ImportError: there is no fallback path.
"""
from ._lib import (  # noqa: F401
    BLOCK,
    BPK_OP_ATTEND,
    BPK_OP_DECODE,
    BPK_OP_POOLED,
    BPK_OP_SELECT,
    BPK_DEPTH_CHANNELS,
    BPK_DEPTH_SPARQ,
    BPK_DEPTH_UNIFORM,
    BPK_DEPTH_WATERFILL,
    EXPORTS,
    HEAD_DIM,
    LIB_PATH,
    PLANES,
    STAGES,
    BpkError,
    Cache,
    alloc_depth,
    alloc_depth_layers,
    decode_step,
    decode_step_depth,
    fixed_depth,
    layer_budgets,
    pooled_planes,
    decode_fallback_units,
    decode_step_noalloc,
    NOALLOC_SCRATCH_BYTES,
    encode_append,
    last_error,
    scan_scores,
    select_topk,
    sparse_attend,
    trace_enable,
    trace_read,
    workspace_bytes,
)
