"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (decode_step over every layer of the cache at once).

The oracle cannot take a whole step, so it checks sampled units: their key
and value rows are read back from the rows the device generator drew (a few
of them re-derived on the host, which pins them to the host generator), and
the oracle encodes, allocates, scans, selects and attends on them.  Over all
units, decode_step's indices equal select_topk(scan_scores(...)).

Bars: planes, scales and depths bit-exact; scores within 1e-4 of their L1
scale; top-k sets equal up to near-tie swaps; attention within 2e-3.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import config_by_name
from synth import device as synth_device
from synth import workload as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def bpk():
    import bit_plane_key_amd as b
    from bit_plane_key_amd import workloads
    return b, workloads


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rows_f32(t):
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return W.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))


def _check_unit(cfg, cache, s, l, h, n, budget, k, scale, step, depth, idx, out, scores=None):
    where = f"{cfg.name} unit ({s},{l},{h}) n={n} P={budget}"
    _say("oracle on", where)
    kv = _rows_f32(cache.k_rows[s, l, h, :n])
    vv = _rows_f32(cache.v_rows[s, l, h, :n])
    # pin the read-back rows to the host generator on a few rows
    rows = np.array([0, 1, n // 2, n - 1])
    hk = W.key_rows(cfg, s, l, h, rows)[1]
    hv = W.value_rows(cfg, s, l, h, rows)[1]
    assert np.array_equal(kv[rows], hk) and np.array_equal(vv[rows], hv), where
    q = W.query(cfg, s, l, h, step)[1]
    rot = cfg.rotation(l, h) if cfg.rotated else None
    ref = O.decode_unit(q, cfg.chan_var(s, l, h), kv, vv, n, budget, k, scale, rot=rot)
    nb = n // 64
    planes = cache.planes[s, l, h, :, :, :nb].cpu().numpy().view(np.uint64)
    assert np.array_equal(planes, ref["planes"]), where
    gs = cache.scales[s, l, h, :, :nb].cpu().numpy().view(np.uint16)
    assert np.array_equal(gs, np.asarray(ref["scales"]).view(np.uint16)), where
    assert np.array_equal(depth[s, l, h].cpu().numpy(), ref["depth"]), where
    if scores is not None:
        P.check_scores(scores[s, l, h, :, : nb * 64].cpu().numpy(), ref["scores"], ref["l1"], where)
    ix = idx[s, l, h].cpu().numpy()
    P.check_selection(ix, ref["idx"], ref["scores"], ref["l1"], n, k, where)
    P.check_attention(out[s, l, h].cpu().numpy(), O.attend(q, kv, vv, ix, scale), where)


def _step_all(b, cfg, cache, q, budget, scale):
    S, L, H, G, k = cfg.seqs, cfg.layers, cfg.heads, cfg.group, cfg.k
    depth = torch.empty((S, L, H, 128), dtype=torch.uint8, device="cuda")
    idx = torch.empty((S, L, H, G, k), dtype=torch.int32, device="cuda")
    out = b.decode_step(cache, q, 0, L, budget, k, scale, depth_out=depth, idx_out=idx)
    return depth, idx, out


@pytest.mark.parametrize("name,budget", [("c3", 88), ("c4", 64), ("c4", 88), ("c4", 128)])
def test_fullsize_decode_step(bpk, name, budget):
    b, wl = bpk
    cfg = config_by_name(name)
    _say(f"building {name}")
    cache = wl.build_cache(cfg)
    q = wl.queries(cfg)
    scale = wl.softmax_scale(cfg)
    depth, idx, out = _step_all(b, cfg, cache, q, budget, scale)
    d2, qb = b.alloc_depth(cache, q, 0, cfg.layers, budget)
    scores = b.scan_scores(cache, qb, d2, 0, cfg.layers)
    idx2 = b.select_topk(cache, scores, 0, cfg.layers, cfg.k)
    torch.cuda.synchronize()
    _say(f"{name} P={budget}: fused == unfused over {cfg.units} units")
    assert torch.equal(depth, d2)
    assert torch.equal(idx, idx2)
    units = [(0, 0, 0), (cfg.seqs - 1, cfg.layers - 1, cfg.heads - 1)]
    if name == "c4":
        units.append((0, 17, 5))  # a heavy-tailed head
    for (s, l, h) in units:
        _check_unit(cfg, cache, s, l, h, cfg.n, budget, cfg.k, scale, 0, depth, idx, out, scores)


def test_fullsize_c5_append_loop(bpk):
    """Rotated keys; each of 64 decode steps appends one token per sequence,
    so the open tail block grows from 1 to 63 tokens and then completes."""
    b, wl = bpk
    cfg = config_by_name("c5")
    _say("building c5")
    cache = wl.build_cache(cfg)
    scale = wl.softmax_scale(cfg)
    budget = cfg.budgets[0]
    ktab = synth_device.unit_tables(cfg, "k")
    vtab = synth_device.unit_tables(cfg, "v")
    q = None
    checks = {0: [(0, 0, 0)], 40: [(3, 11, 2)], 63: [(7, 31, 7), (5, 20, 6)]}
    for t in range(cfg.append_steps):
        row = cfg.n + t
        synth_device.fill_rows(cfg, cache.k_rows, "k", row, 1, rot=cache.rot, tables=ktab)
        synth_device.fill_rows(cfg, cache.v_rows, "v", row, 1, tables=vtab)
        for s in range(cfg.seqs):
            b.encode_append(cache, s, None, None, 1)
        if q is None or t in checks:
            q = wl.queries(cfg, step=t)
        depth, idx, out = _step_all(b, cfg, cache, q, budget, scale)
        if t in checks:
            torch.cuda.synchronize()
            n = row + 1
            _say(f"c5 step {t}: n = {n}")
            for (s, l, h) in checks[t]:
                _check_unit(cfg, cache, s, l, h, n, budget, cfg.k, scale, t, depth, idx, out)
