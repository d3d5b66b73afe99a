"""GPU parity of the per-layer budget calibration (a reading of Fathom §3's
optional calibration): pooled plane counts of every unit bit-exact against
the oracle's pooled water-filling, per-layer budgets equal to the oracle's,
and a decode step run per layer at those budgets reading exactly them."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import config_by_name
from synth import workload as W

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def c4small():
    """The long-context workload's 36 layers x 8 KV heads (channel variances
    of both kinds and the queries), over a cache of 2048 tokens."""
    import bit_plane_key_amd as b
    from bit_plane_key_amd import workloads as wl
    cfg = config_by_name("c4")
    _say("calibration: building the 288 units' variances and queries")
    cache = b.Cache(1, cfg.layers, cfg.heads, 2048, group=cfg.group)
    var = np.stack([np.stack([cfg.chan_var(0, l, h) for h in range(cfg.heads)])
                    for l in range(cfg.layers)])[None]
    cache.chan_var.copy_(torch.from_numpy(var))
    qs = [wl.queries(cfg, step=s) for s in range(3)]
    gains = []
    for s in range(3):
        g = np.zeros((cfg.layers, cfg.heads, 128), dtype=np.float32)
        for l in range(cfg.layers):
            for h in range(cfg.heads):
                g[l, h] = O.channel_gains(W.query(cfg, 0, l, h, s)[1], cfg.chan_var(0, l, h))
        gains.append(g.reshape(-1, 128))
    return b, wl, cfg, cache, qs, gains


@pytest.mark.parametrize("budget", [0, 1, 64, 88, 128, 511, 600])
def test_pooled_counts_bit_exact(c4small, budget):
    b, wl, cfg, cache, qs, gains = c4small
    counts = b.pooled_planes(cache, qs[0], 0, cfg.layers, budget)
    torch.cuda.synchronize()
    ref = O.pooled_plane_counts(gains[0], budget)
    got = counts.cpu().numpy().reshape(-1)
    assert np.array_equal(got, ref), (budget, np.abs(got - ref).max())


def test_layer_budgets_and_per_layer_decode(c4small):
    b, wl, cfg, cache, qs, gains = c4small
    P = 88
    counts = torch.stack([b.pooled_planes(cache, q, 0, cfg.layers, P) for q in qs])
    budgets = b.layer_budgets(cache, counts, 0, cfg.layers, P)
    torch.cuda.synchronize()
    ref_counts = np.stack([O.pooled_plane_counts(g, P) for g in gains])
    assert np.array_equal(counts.cpu().numpy().reshape(3, -1), ref_counts)
    ref = O.calibrate_layer_budgets(ref_counts.reshape(3, cfg.layers, cfg.heads), P)
    got = budgets.cpu().numpy()
    assert np.array_equal(got, ref) and got.sum() == cfg.layers * P
    # the layer sub-range [4, 9) on its own
    sub = b.layer_budgets(cache, counts[:, :, 4:9].contiguous(), 4, 9, P)
    torch.cuda.synchronize()
    assert np.array_equal(sub.cpu().numpy(),
                          O.calibrate_layer_budgets(ref_counts.reshape(3, cfg.layers, cfg.heads)[:, 4:9], P))
    # each layer's allocation at its budget reads exactly that many planes per unit
    for l in (0, 17, 35):
        depth, _ = b.alloc_depth(cache, qs[0][:, l:l + 1].contiguous(), l, l + 1, int(got[l]))
        torch.cuda.synchronize()
        assert (depth.cpu().numpy().reshape(-1, 128).sum(axis=1) == min(int(got[l]), 512)).all()


def test_alloc_depth_layers_matches_per_layer_calls(c4small):
    """One call with a budget per layer equals one alloc_depth call per layer."""
    b, wl, cfg, cache, qs, gains = c4small
    budgets = torch.tensor([(17 * l) % 130 for l in range(cfg.layers)], dtype=torch.int32,
                           device="cuda")
    depth, qb = b.alloc_depth_layers(cache, qs[1], 0, cfg.layers, budgets)
    torch.cuda.synchronize()
    for l in range(cfg.layers):
        d1, _ = b.alloc_depth(cache, qs[1][:, l:l + 1].contiguous(), l, l + 1, int(budgets[l]))
        torch.cuda.synchronize()
        assert torch.equal(depth[:, l:l + 1], d1), l
