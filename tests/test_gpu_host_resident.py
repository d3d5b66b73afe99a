"""Host-resident caches: rows, planes and scales in pinned host memory that
the kernels read over the host link (the regime the Fathom page measures,
§1 and §3.1).  Same kernels, so every result must be bit-identical to the
device-resident cache's."""
import numpy as np
import pytest
import torch

from synth import config_by_name

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_host_resident_matches_device():
    import bit_plane_key_amd as b
    from bit_plane_key_amd import workloads as wl
    cfg = config_by_name("c2")
    _say("host-resident: building c2 on the device and in pinned host memory")
    dev = wl.build_cache(cfg)
    host = wl.build_cache(cfg, host_resident=True)
    assert host.planes.device.type == "cpu" and host.planes.is_pinned()
    q = wl.queries(cfg)
    scale = wl.softmax_scale(cfg)
    res = []
    for cache in (dev, host):
        idx = torch.empty((1, 1, cfg.heads, cfg.group, cfg.k), dtype=torch.int32, device="cuda")
        out = b.decode_step(cache, q, 0, 1, 88, cfg.k, scale, idx_out=idx)
        depth, qb = b.alloc_depth(cache, q, 0, 1, 88)
        sc = b.scan_scores(cache, qb, depth, 0, 1)
        torch.cuda.synchronize()
        res.append((idx.cpu(), out.cpu(), sc.cpu()))
    assert torch.equal(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1])
    assert torch.equal(res[0][2], res[1][2])


def test_host_resident_append_encodes_over_the_link():
    """encode_append writes planes and scales into pinned host memory."""
    import bit_plane_key_amd as b
    from bit_plane_key_amd._lib import Cache
    rng = np.random.default_rng(4)
    n = 64 * 37 + 5
    kb = (rng.standard_normal((1, 2, n, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    k_dev = torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16)
    caches = [Cache(1, 1, 2, 64 * 40), Cache(1, 1, 2, 64 * 40, host_resident=True)]
    for c in caches:
        b.encode_append(c, 0, k_dev, k_dev, n)
    torch.cuda.synchronize()
    assert torch.equal(caches[0].planes.cpu(), caches[1].planes)
    assert torch.equal(caches[0].scales.cpu(), caches[1].scales)
    assert torch.equal(caches[0].k_rows[..., :n, :].cpu(), caches[1].k_rows[..., :n, :])
