"""The allocation-free decode step (bpk_decode_step_noalloc) against
bpk_decode_step with a caller workspace: the same kernels, so every output
must be identical.  Calls in a row, the second on a smaller input (the
library's scratch array keeps the earlier call's contents).  The refusal of a
call larger than the scratch array is checked on the CPU (tests/test_abi.py)."""
import numpy as np
import pytest
import torch

from synth import config_by_name

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _both(bpk, cfg, cache, q, l0, l1, budget, k):
    scale = bpk.workloads.softmax_scale(cfg)
    u = (cfg.seqs, l1 - l0, cfg.heads)
    res = []
    for noalloc in (False, True):
        out = torch.full((*u, cfg.group, 128), float("nan"), dtype=torch.float32, device="cuda")
        depth = torch.full((*u, 128), 255, dtype=torch.uint8, device="cuda")
        idx = torch.full((*u, cfg.group, k), -7, dtype=torch.int32, device="cuda")
        if noalloc:
            bpk.decode_step_noalloc(cache, q, l0, l1, budget, k, scale, out, depth_out=depth,
                                    idx_out=idx)
        else:
            bpk.decode_step(cache, q, l0, l1, budget, k, scale, out=out, depth_out=depth,
                            idx_out=idx)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), depth.cpu().numpy(), idx.cpu().numpy()))
    (o0, d0, i0), (o1, d1, i1) = res
    assert np.array_equal(d0, d1), "depths differ"
    assert np.array_equal(i0, i1), "selected indices differ"
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), "outputs differ"
    assert np.isfinite(o1).all()


def test_noalloc_matches_workspace_step_twice():
    import bit_plane_key_amd as bpk
    from bit_plane_key_amd import workloads
    bpk.workloads = workloads
    big = config_by_name("c2")        # 8 units x 32768 tokens
    small = config_by_name("c1")      # 1 unit x 4096 tokens
    _say("noalloc: building c2 and c1 caches")
    cache_b = workloads.build_cache(big)
    cache_s = workloads.build_cache(small)
    need_b = bpk.workspace_bytes(cache_b, bpk.BPK_OP_DECODE, 0, big.layers, big.k)
    need_s = bpk.workspace_bytes(cache_s, bpk.BPK_OP_DECODE, 0, small.layers, small.k)
    assert need_s < need_b <= bpk.NOALLOC_SCRATCH_BYTES
    _say("noalloc: c2, P=88, k=512")
    _both(bpk, big, cache_b, workloads.queries(big), 0, big.layers, 88, big.k)
    _say("noalloc: c1, P=64, k=64 (smaller, after the larger call)")
    _both(bpk, small, cache_s, workloads.queries(small), 0, small.layers, 64, small.k)
    _say("noalloc: c2 again at P=128")
    _both(bpk, big, cache_b, workloads.queries(big, step=1), 0, big.layers, 128, big.k)
