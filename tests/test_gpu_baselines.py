"""GPU parity of the fixed-depth baselines (Fathom §2: SparQ r = 16 / 32,
Double Sparsity c = 32, the 2-bit thumbnail) run on the same planes:
depth vectors bit-exact against the oracle's rules, scores within 1e-4 of
their L1 mass, and the decode step on those depths equal to the unfused
scan + select and, up to near-ties, to the oracle's selection."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import config_by_name
from tests import parity as P

pytestmark = pytest.mark.gpu

ABS_MEAN = math.sqrt(2.0 / math.pi)   # E|x| of a standard normal


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def c2():
    import bit_plane_key_amd as b
    from bit_plane_key_amd import workloads as wl
    cfg = config_by_name("c2")
    _say("baselines: building c2")
    cache = wl.build_cache(cfg)
    q = wl.queries(cfg)
    inps = [P.unit_inputs(cfg, 0, 0, h, cfg.n) for h in range(cfg.heads)]
    return b, wl, cfg, cache, q, inps


def ds_channels(cfg, c):
    """Double Sparsity's offline channel sets [L][H][c]: the calibration
    statistics of the synthetic workload are its generator's, mean|q_j| =
    E|N(0,1)| for every channel and mean|k_j| = sigma_j E|N(0,1)|."""
    out = np.zeros((cfg.layers, cfg.heads, c), dtype=np.uint8)
    for l in range(cfg.layers):
        for h in range(cfg.heads):
            sig = np.sqrt(cfg.chan_var(0, l, h).astype(np.float64))
            out[l, h] = O.double_sparsity_channels(np.full(128, ABS_MEAN), sig * ABS_MEAN, c)
    return out


RULES = [("sparq", 16), ("sparq", 32), ("ds", 32), ("uniform", 2), ("uniform", 4)]


def _depths(b, cfg, cache, q, rule, param):
    if rule == "sparq":
        return b.fixed_depth(cache, q, 0, 1, b.BPK_DEPTH_SPARQ, param)
    if rule == "ds":
        ch = torch.from_numpy(ds_channels(cfg, param)).cuda()
        return b.fixed_depth(cache, q, 0, 1, b.BPK_DEPTH_CHANNELS, param, channels=ch)
    return b.fixed_depth(cache, q, 0, 1, b.BPK_DEPTH_UNIFORM, param)


def _oracle_depth(cfg, inp, h, rule, param):
    if rule == "sparq":
        return O.sparq_depth(inp["q"], param)
    if rule == "ds":
        return O.channel_set_depth(ds_channels(cfg, param)[0, h])
    return O.uniform_depth(param)


@pytest.mark.parametrize("rule,param", RULES)
def test_baseline_depths_and_scores(c2, rule, param):
    b, wl, cfg, cache, q, inps = c2
    depth, qb = _depths(b, cfg, cache, q, rule, param)
    scores = b.scan_scores(cache, qb, depth, 0, 1)
    torch.cuda.synchronize()
    d = depth.cpu().numpy()
    sc = scores.cpu().numpy()
    for h in range(cfg.heads):
        ref_d = _oracle_depth(cfg, inps[h], h, rule, param)
        assert np.array_equal(d[0, 0, h], ref_d), (rule, param, h)
        if h in (0, 5):
            planes, scales = P.oracle_encode(inps[h], cfg.n)
            ref, l1 = O.scan_scores(inps[h]["q"], ref_d, planes, scales, cfg.n)
            P.check_scores(sc[0, 0, h, :, :cfg.n], ref, l1, f"{rule} {param} head {h}")


@pytest.mark.parametrize("rule,param", [("sparq", 16), ("ds", 32), ("uniform", 2)])
def test_baseline_decode_step(c2, rule, param):
    b, wl, cfg, cache, q, inps = c2
    n, k = cfg.n, cfg.k
    scale = wl.softmax_scale(cfg)
    depth, qb = _depths(b, cfg, cache, q, rule, param)
    idx = torch.empty((1, 1, cfg.heads, cfg.group, k), dtype=torch.int32, device="cuda")
    out = b.decode_step_depth(cache, q, qb, depth, 0, 1, k, scale, idx_out=idx)
    # the rule's bound on the rows a unit reads (4 r, 4 c, 128 t) gives the
    # same result with only the scan variants that hold that many rows
    bound = {"sparq": 4 * param, "ds": 4 * param, "uniform": 128 * param}[rule]
    idx_b = torch.empty_like(idx)
    out_b = b.decode_step_depth(cache, q, qb, depth, 0, 1, k, scale, idx_out=idx_b, max_rows=bound)
    scores = b.scan_scores(cache, qb, depth, 0, 1)
    idx2 = b.select_topk(cache, scores, 0, 1, k)
    out2 = b.sparse_attend(cache, q, idx2, 0, 1, k, scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)
    assert torch.equal(idx_b, idx) and torch.equal(out_b, out)
    ix = idx.cpu().numpy()
    ot = out.cpu().numpy()
    for h in (1, 6):
        inp = inps[h]
        planes, scales = P.oracle_encode(inp, n)
        ref, l1 = O.scan_scores(inp["q"], _oracle_depth(cfg, inp, h, rule, param), planes, scales, n)
        full = np.zeros((cfg.group, n))
        full[:, : ref.shape[1]] = ref
        P.check_selection(ix[0, 0, h], O.select_topk(full, n, k), full, l1, n, k, f"{rule} head {h}")
        P.check_attention(ot[0, 0, h], O.attend(inp["q"], inp["k"], inp["v"], ix[0, 0, h], scale),
                          f"{rule} head {h}")


def test_decode_step_depth_bound_below_the_rows_read(c2):
    """A bound below the rows the units read (SparQ r = 32: 128 rows, bound
    64) leaves every unit unscanned: the call still completes, and every
    selected index is a token of the unit (the result itself is undefined)."""
    b, wl, cfg, cache, q, inps = c2
    n, k = cfg.n, cfg.k
    scale = wl.softmax_scale(cfg)
    depth, qb = _depths(b, cfg, cache, q, "sparq", 32)
    idx = torch.empty((1, 1, cfg.heads, cfg.group, k), dtype=torch.int32, device="cuda")
    ws = torch.zeros(b.workspace_bytes(cache, b.BPK_OP_DECODE, 0, 1, k), dtype=torch.uint8,
                     device="cuda")
    out = b.decode_step_depth(cache, q, qb, depth, 0, 1, k, scale, idx_out=idx, ws=ws, max_rows=64)
    torch.cuda.synchronize()
    ix = idx.cpu().numpy()
    assert ((ix >= 0) & (ix < n)).all()
    assert torch.isfinite(out).all()
