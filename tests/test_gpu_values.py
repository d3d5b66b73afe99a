"""GPU parity of the value-side depths (ReadKV §5.3, §5.4) against the oracle.

Bars: value planes and scales bit-exact; depths from given importances
bit-exact; in the attention with value depths, the union exact, the depths
equal to the oracle's except for plane values within 1e-4 (relative) of the
cut (the GPU's probabilities are fp32), the number of planes granted exact,
and outputs within 2e-3 of the oracle's per head plus what the near-cut
depths may move.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import config_by_name
from tests import parity as P

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128.0)
CUT_RTOL = 1e-4


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def lib():
    import bit_plane_key_amd as b
    from bit_plane_key_amd import workloads as wl
    return b, wl


def _bf16(x: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16)


def _custom_cache(b, rng, seqs, n_list, group, cap, row_scale=True):
    """A one-layer, one-head cache of seeded bf16 rows: keys N(0, 1), values
    N(0, 1) times a per-token factor exp(U(-2, 2)).  Returns the cache and the
    host float32 values of every sequence's rows."""
    cache = b.Cache(seqs, 1, 1, cap, group=group, k_dtype="bf16", values=True)
    cache.chan_var.fill_(1.0)
    host = []
    for s, n in enumerate(n_list):
        k = _bf16(rng.standard_normal((1, 1, n, 128)))
        f = np.exp(rng.uniform(-2, 2, n))[:, None] if row_scale else 1.0
        v = _bf16(rng.standard_normal((1, 1, n, 128)) * f)
        if n:
            b.encode_append(cache, s, k.cuda(), v.cuda())
        host.append((k.float().numpy()[0, 0], v.float().numpy()[0, 0]))
    torch.cuda.synchronize()
    return cache, host


def _idx_lists(rng, n, g, k, shared=0.6):
    """Per head: the first 4 and last 32 tokens, then a share of the rest from
    a pool common to the group and the remainder drawn per head (strictly
    ascending, -1 padding when n < k)."""
    out = np.full((g, k), -1, dtype=np.int32)
    if n <= k:
        out[:, :n] = np.arange(n)
        return out
    fixed = np.concatenate([np.arange(4), np.arange(n - 32, n)])
    middle = np.arange(4, n - 32)
    rest = k - len(fixed)
    pool = rng.choice(middle, size=min(len(middle), rest), replace=False)
    for h in range(g):
        m = int(shared * rest)
        a = rng.choice(pool, size=m, replace=False)
        others = np.setdiff1d(middle, a)
        c = rng.choice(others, size=rest - m, replace=False)
        out[h] = np.sort(np.concatenate([fixed, a, c]))
    return out


def _check_depths(gpu_depth, ref, vscales, budget, where):
    """Depths equal to the oracle's except candidates within CUT_RTOL of the
    cut value; the number of planes granted equal.  Returns the rows whose
    depth may differ."""
    s = vscales[ref["union"]].astype(np.float64)
    vals = (ref["a"] * s * s)[:, None] * 0.25 ** np.arange(4)[None, :]
    pos = np.sort(vals[vals > 0])[::-1]
    amb = np.zeros_like(vals, dtype=bool)
    if 0 < budget < len(pos):
        cut = pos[budget - 1]
        amb = np.abs(vals - cut) <= CUT_RTOL * cut
    t = np.arange(4)[None, :]
    tr = t < ref["depth"][:, None]
    tg = t < gpu_depth[:, None]
    assert int(tg.sum()) == int(tr.sum()) == min(budget, len(pos)), where
    bad = (tr != tg) & ~amb
    assert not bad.any(), f"{where}: {int(bad.sum())} plane grants differ away from the cut"
    return np.nonzero((tr != tg).any(axis=1))[0]


def _check_out(gpu_out, ref, gpu_depth, moved, vscales, where):
    """|gpu - oracle| <= 2e-3 max|oracle| per head, plus, for each row whose
    depth moved by a near-cut plane, p_hr * 4 s_r 2^-t (a quarter of the
    coarser cell: the most one plane moves a rebuilt value)."""
    extra = np.zeros(ref["out"].shape[0])
    for r in moved:
        t = min(int(gpu_depth[r]), int(ref["depth"][r]))
        extra += ref["p"][:, r] * 4.0 * float(vscales[ref["union"][r]]) * 2.0 ** -t
    for h in range(ref["out"].shape[0]):
        err = np.max(np.abs(gpu_out[h].astype(np.float64) - ref["out"][h]))
        tol = P.ATT_RTOL * max(np.max(np.abs(ref["out"][h])), 1e-30) + extra[h] * (1 + 1e-6)
        assert err <= tol, f"{where}: head {h} off by {err:.3g} > {tol:.3g}"


# ---------------------------------------------------------------------------
# encoding
# ---------------------------------------------------------------------------

def test_value_encode_bit_exact_c1(lib):
    b, wl = lib
    cfg = config_by_name("c1")
    _say("values: building c1 with value planes")
    cache = wl.build_cache(cfg, values=True)
    inp = P.unit_inputs(cfg, 0, 0, 0, cfg.n)
    planes, scales = O.encode_values(inp["v"])
    gp = cache.v_planes[0, 0, 0, : cfg.n].cpu().numpy()
    gs = cache.v_scales[0, 0, 0, : cfg.n].cpu().numpy()
    assert np.array_equal(gs.view(np.uint16), scales.view(np.uint16))
    assert np.array_equal(gp, planes)


def test_value_encode_appends_and_edge_rows(lib):
    """Appends of 1, 63, 64, 100 and 7 tokens code each token at once; edge
    rows: all zero, -0, a row at exact code boundaries, a row whose maximum
    saturates the fp16 scale, a row of tiny values."""
    b, wl = lib
    rng = np.random.default_rng(11)
    sizes = [1, 63, 64, 100, 7]
    n = sum(sizes)
    v = rng.standard_normal((n, 128)).astype(np.float32)
    v[0] = 0.0
    v[1] = -0.0
    v[2] = (np.arange(128) % 16 - 8).astype(np.float32) * 0.5    # codes on the grid, s = 0.5
    v[2, 0] = 4.0
    v[3] = rng.standard_normal(128) * 1e30
    v[4] = rng.standard_normal(128) * 1e-30
    vt = _bf16(v)
    kt = _bf16(rng.standard_normal((n, 128)))
    cache = b.Cache(1, 1, 1, 512, group=4, k_dtype="bf16", values=True)
    r0 = 0
    for m in sizes:
        b.encode_append(cache, 0, kt[r0:r0 + m][None, None].contiguous().cuda(),
                        vt[r0:r0 + m][None, None].contiguous().cuda())
        r0 += m
    torch.cuda.synchronize()
    planes, scales = O.encode_values(vt.float().numpy())
    assert np.array_equal(cache.v_scales[0, 0, 0, :n].cpu().numpy().view(np.uint16),
                          scales.view(np.uint16))
    assert np.array_equal(cache.v_planes[0, 0, 0, :n].cpu().numpy(), planes)
    assert float(scales[3]) == 65504.0 and float(scales[0]) == 0.0


# ---------------------------------------------------------------------------
# depths from given importances (bit-exact)
# ---------------------------------------------------------------------------

def test_value_depth_bit_exact(lib):
    b, wl = lib
    rng = np.random.default_rng(12)
    n_list = [9000, 3000, 50, 0, 8192]
    cache, host = _custom_cache(b, rng, len(n_list), n_list, 4, 9024)
    ld = 8192
    rows = np.zeros((len(n_list), 1, 1, ld), dtype=np.int32)
    nrows = np.zeros((len(n_list), 1, 1), dtype=np.int32)
    wts = np.zeros((len(n_list), 1, 1, ld), dtype=np.float32)
    counts = [5000, 1, 37, 0, 8192]
    for s, (n, c) in enumerate(zip(n_list, counts)):
        if n == 0 or c == 0:
            continue
        r = np.sort(rng.choice(n, size=c, replace=False)).astype(np.int32)
        w = (rng.uniform(0, 1, c) ** 3).astype(np.float32)
        w[rng.uniform(size=c) < 0.1] = 0.0
        rows[s, 0, 0, :c] = r
        nrows[s, 0, 0] = c
        wts[s, 0, 0, :c] = w
    # equal weights on two tokens of equal scale: plant a copy of a row
    tie_a, tie_b = int(rows[0, 0, 0, 10]), int(rows[0, 0, 0, 11])
    cache.v_rows[0, 0, 0, tie_b] = cache.v_rows[0, 0, 0, tie_a]
    cache.n_tokens[0] = tie_b
    b.encode_append(cache, 0, None, None, 1)          # re-code token tie_b in place
    cache.n_tokens[0] = n_list[0]
    wts[0, 0, 0, 11] = wts[0, 0, 0, 10] = 0.25
    vrows = host[0][1].copy()
    vrows[tie_b] = vrows[tie_a]
    host[0] = (host[0][0], vrows)
    # padding past n_rows is never read: fill it with junk
    for s, c in enumerate(counts):
        wts[s, 0, 0, c:] = np.nan
        rows[s, 0, 0, c:] = -7
    dev = lambda x: torch.from_numpy(x).cuda()
    for budget in (0, 1, 777, 4 * 5000, 4 * 8192 + 5):
        d = b.value_depth(cache, 0, 1, dev(rows), dev(nrows), dev(wts), budget)
        torch.cuda.synchronize()
        d = d.cpu().numpy()
        for s, c in enumerate(counts):
            if c == 0:
                assert not d[s, 0, 0].any()
                continue
            _, vscales = O.encode_values(host[s][1][: n_list[s]])
            r = rows[s, 0, 0, :c]
            ref = O.alloc_value_depth(wts[s, 0, 0, :c], vscales[r], budget)
            assert np.array_equal(d[s, 0, 0, :c], ref), (budget, s)
            assert not d[s, 0, 0, c:].any()
        if budget == 1:
            assert d[0, 0, 0].sum() == 1


def test_value_depth_exact_ties_bit_exact(lib):
    """Every value row the same (equal scales) and weights from {1/4, 1/2, 1}:
    plane values tie within a plane and across planes (1/4 at plane 0 equals
    1 at plane 1), so most budgets cut through a run of equal values, which
    are handed out in (row, plane) order."""
    b, wl = lib
    rng = np.random.default_rng(31)
    n, ld = 6000, 8192
    cache = b.Cache(2, 1, 1, 6016, group=4, k_dtype="bf16", values=True)
    cache.chan_var.fill_(1.0)
    row = rng.standard_normal(128)
    for s, m in enumerate((n, 300)):
        k = _bf16(rng.standard_normal((1, 1, m, 128)))
        v = _bf16(np.broadcast_to(row, (1, 1, m, 128)))
        b.encode_append(cache, s, k.cuda(), v.cuda())
    torch.cuda.synchronize()
    _, vscales = O.encode_values(_bf16(row[None, :]).float().numpy())
    counts = [5000, 300]
    rows = np.full((2, 1, 1, ld), -7, dtype=np.int32)
    nrows = np.array(counts, dtype=np.int32).reshape(2, 1, 1)
    wts = np.full((2, 1, 1, ld), np.nan, dtype=np.float32)
    for s, c in enumerate(counts):
        rows[s, 0, 0, :c] = np.sort(rng.choice(n if s == 0 else 300, size=c, replace=False))
        wts[s, 0, 0, :c] = rng.choice(np.array([0.25, 0.5, 1.0], dtype=np.float32), size=c)
    dev = lambda x: torch.from_numpy(x).cuda()
    for budget in (1, 2, 777, 1500, 4999, 5001, 9000, 4 * 5000 - 3):
        d = b.value_depth(cache, 0, 1, dev(rows), dev(nrows), dev(wts), budget)
        torch.cuda.synchronize()
        d = d.cpu().numpy()
        for s, c in enumerate(counts):
            ref = O.alloc_value_depth(wts[s, 0, 0, :c], np.full(c, vscales[0]), budget)
            assert np.array_equal(d[s, 0, 0, :c], ref), (budget, s)
            assert int(d[s, 0, 0, :c].sum()) == min(budget, 4 * c), (budget, s)


# ---------------------------------------------------------------------------
# attention with value depths
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def c2v(lib):
    b, wl = lib
    cfg = config_by_name("c2")
    _say("values: building c2 with value planes")
    cache = wl.build_cache(cfg, values=True)
    q = wl.queries(cfg)
    inps = [P.unit_inputs(cfg, 0, 0, h, cfg.n) for h in range(cfg.heads)]
    enc = [O.encode_values(inp["v"]) for inp in inps]
    return cfg, cache, q, inps, enc


@pytest.mark.parametrize("budget", [0, 1, 300, 1024, 2048, 10 ** 6])
def test_sparse_attend_v_c2(lib, c2v, budget):
    b, wl = lib
    cfg, cache, q, inps, enc = c2v
    rng = np.random.default_rng(100 + budget % 97)
    idx = np.stack([_idx_lists(rng, cfg.n, cfg.group, cfg.k) for _ in range(cfg.heads)])
    idx_t = torch.from_numpy(idx[None, None]).cuda()
    sel = cfg.group * cfg.k
    uo = torch.empty((1, 1, cfg.heads, sel), dtype=torch.int32, device="cuda")
    vd = torch.empty((1, 1, cfg.heads, sel), dtype=torch.uint8, device="cuda")
    out = b.sparse_attend_v(cache, q, idx_t, 0, 1, cfg.k, SCALE, budget, union_out=uo,
                            v_depth_out=vd)
    torch.cuda.synchronize()
    out, uo, vd = out.cpu().numpy(), uo.cpu().numpy(), vd.cpu().numpy()
    for h in range(cfg.heads):
        planes, scales = enc[h]
        ref = O.attend_values(inps[h]["q"], inps[h]["k"], planes, scales, idx[h], SCALE, budget)
        nu = len(ref["union"])
        where = f"budget {budget} head {h}"
        assert np.array_equal(uo[0, 0, h, :nu], ref["union"]), where
        assert np.all(uo[0, 0, h, nu:] == -1) and not vd[0, 0, h, nu:].any(), where
        moved = _check_depths(vd[0, 0, h, :nu], ref, scales, budget, where)
        _check_out(out[0, 0, h], ref, vd[0, 0, h, :nu], moved, scales, where)
        if budget >= 4 * nu:
            assert np.all(vd[0, 0, h, :nu] == 4)


def test_decode_step_v_matches_its_stages(lib, c2v):
    """decode_step_v selects as decode_step does and then equals
    sparse_attend_v on its own selection, bit for bit."""
    b, wl = lib
    cfg, cache, q, inps, enc = c2v
    u = (1, 1, cfg.heads)
    idx_v = torch.empty((*u, cfg.group, cfg.k), dtype=torch.int32, device="cuda")
    idx_e = torch.empty_like(idx_v)
    sel = cfg.group * cfg.k
    uo = torch.empty((*u, sel), dtype=torch.int32, device="cuda")
    vd = torch.empty((*u, sel), dtype=torch.uint8, device="cuda")
    out_v = b.decode_step_v(cache, q, 0, 1, 88, cfg.k, SCALE, 1024, idx_out=idx_v, union_out=uo,
                            v_depth_out=vd)
    b.decode_step(cache, q, 0, 1, 88, cfg.k, SCALE, idx_out=idx_e)
    uo2 = torch.empty_like(uo)
    vd2 = torch.empty_like(vd)
    out_s = b.sparse_attend_v(cache, q, idx_v, 0, 1, cfg.k, SCALE, 1024, union_out=uo2,
                              v_depth_out=vd2)
    torch.cuda.synchronize()
    assert torch.equal(idx_v, idx_e)
    assert torch.equal(uo, uo2) and torch.equal(vd, vd2)
    assert torch.equal(out_v, out_s)


@pytest.mark.parametrize("group,k,n", [(8, 1024, 20000), (1, 64, 300), (2, 200, 5000)])
def test_sparse_attend_v_shapes(lib, group, k, n):
    """Largest union (G k = 8192 rows), a single head, and a pair; a second
    sequence holds fewer tokens than k (every token kept, -1 padding) and a
    third none at all."""
    b, wl = lib
    rng = np.random.default_rng(group * 1000 + k)
    n_list = [n, min(50, k - 1), 0]
    cache, host = _custom_cache(b, rng, 3, n_list, group, (n + 63) // 64 * 64)
    q = rng.standard_normal((3, 1, 1, group, 128))
    qt = _bf16(q).cuda()
    qv = _bf16(q).float().numpy()
    idx = np.stack([_idx_lists(rng, m, group, k, shared=0.3) if m else
                    np.full((group, k), -1, dtype=np.int32) for m in n_list])[:, None, None]
    sel = group * k
    uo = torch.empty((3, 1, 1, sel), dtype=torch.int32, device="cuda")
    vd = torch.empty((3, 1, 1, sel), dtype=torch.uint8, device="cuda")
    for budget in (0, 3000, 4 * sel):
        out = b.sparse_attend_v(cache, qt, torch.from_numpy(np.ascontiguousarray(idx)).cuda(), 0, 1,
                                k, SCALE, budget, union_out=uo, v_depth_out=vd)
        torch.cuda.synchronize()
        o, u_, d_ = out.cpu().numpy(), uo.cpu().numpy(), vd.cpu().numpy()
        for s, m in enumerate(n_list):
            where = f"G={group} k={k} seq {s} budget {budget}"
            if m == 0:
                assert np.all(u_[s, 0, 0] == -1) and not d_[s, 0, 0].any(), where
                assert not o[s, 0, 0].any(), where
                continue
            keys, vals = host[s]
            planes, scales = O.encode_values(vals)
            ref = O.attend_values(qv[s, 0, 0], keys, planes, scales, idx[s, 0, 0], SCALE, budget)
            nu = len(ref["union"])
            assert np.array_equal(u_[s, 0, 0, :nu], ref["union"]), where
            moved = _check_depths(d_[s, 0, 0, :nu], ref, scales, budget, where)
            _check_out(o[s, 0, 0], ref, d_[s, 0, 0, :nu], moved, scales, where)
