"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Bars: codes, planes, scales and depths bit-exact; scores within 1e-4 of their
L1 scale; top-k sets equal up to near-tie swaps (and always a valid top-k of
the GPU's own scores); attention within 2e-3 relative per head.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import config_by_name, Config
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def bpk():
    import bit_plane_key_amd as b
    from bit_plane_key_amd import workloads
    return b, workloads


def _planes_np(cache, s, l, h, nb):
    p = cache.planes[s, l, h, :, :, :nb].cpu().numpy().view(np.uint64)
    sc = cache.scales[s, l, h, :, :nb].cpu().numpy()
    return p, sc


@pytest.fixture(scope="module")
def c1(bpk):
    b, wl = bpk
    cfg = config_by_name("c1")
    _say("building c1 cache")
    cache = wl.build_cache(cfg)
    q = wl.queries(cfg)
    inp = P.unit_inputs(cfg, 0, 0, 0, cfg.n)
    return cfg, cache, q, inp


@pytest.fixture(scope="module")
def c2(bpk):
    b, wl = bpk
    cfg = config_by_name("c2")
    _say("building c2 cache")
    cache = wl.build_cache(cfg)
    q = wl.queries(cfg)
    inps = [P.unit_inputs(cfg, 0, 0, h, cfg.n) for h in range(cfg.heads)]
    return cfg, cache, q, inps


# ---------------------------------------------------------------------------
# inputs and encode
# ---------------------------------------------------------------------------

def test_device_generator_matches_host(c1, c2):
    cfg, cache, q, inp = c1
    k = cache.k_rows[0, 0, 0, : cfg.n].cpu().numpy()
    assert np.array_equal(k.view(np.uint32), inp["k"].view(np.uint32))
    v = cache.v_rows[0, 0, 0, : cfg.n].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(v, inp["v_bits"])
    assert np.array_equal(q[0, 0, 0].cpu().view(torch.int16).numpy().view(np.uint16), inp["q_bits"])
    cfg2, cache2, q2, inps2 = c2
    for h in (0, 5):
        kb = cache2.k_rows[0, 0, h, : cfg2.n].cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(kb, inps2[h]["k_bits"])


def test_encode_bit_exact_c1(c1):
    cfg, cache, q, inp = c1
    planes, scales = P.oracle_encode(inp, cfg.n)
    gp, gs = _planes_np(cache, 0, 0, 0, cfg.n // 64)
    assert np.array_equal(gs.view(np.uint16), scales.view(np.uint16))
    assert np.array_equal(gp, planes)


def test_encode_bit_exact_c2(c2):
    cfg, cache, q, inps = c2
    for h in range(cfg.heads):
        planes, scales = P.oracle_encode(inps[h], cfg.n)
        gp, gs = _planes_np(cache, 0, 0, h, cfg.n // 64)
        assert np.array_equal(gs.view(np.uint16), scales.view(np.uint16)), h
        assert np.array_equal(gp, planes), h


def test_encode_append_in_pieces_matches_bulk(bpk, c2):
    """Appends that cross block boundaries produce the planes of a bulk encode."""
    b, wl = bpk
    cfg, cache, q, inps = c2
    n = 64 * 5 + 17
    small = b.Cache(1, 1, 8, 1024, group=4)
    small.chan_var.copy_(cache.chan_var)
    k_all = cache.k_rows[0, :, :, :n].contiguous()
    v_all = cache.v_rows[0, :, :, :n].contiguous()
    for a, z in ((0, 50), (50, 150), (150, 150), (150, 200), (200, n)):
        b.encode_append(small, 0, k_all[:, :, a:z].contiguous(), v_all[:, :, a:z].contiguous())
    torch.cuda.synchronize()
    assert small.n_tokens[0] == n
    nb = n // 64
    assert torch.equal(small.planes[0, :, :, :, :, :nb], cache.planes[0, :, :, :, :, :nb])
    assert torch.equal(small.scales[0, :, :, :, :nb].view(torch.int16),
                       cache.scales[0, :, :, :, :nb].view(torch.int16))
    assert torch.equal(small.k_rows[0, :, :, :n], cache.k_rows[0, :, :, :n])
    assert int(small.planes[0, :, :, :, :, nb:].abs().sum()) == 0   # open block not encoded


def test_encode_edge_values(bpk):
    """Zero blocks, scale saturation, exact multiples of the scale (fp32 keys)."""
    b, wl = bpk
    cache = b.Cache(1, 1, 1, 256, group=4, k_dtype="f32")
    rng = np.random.default_rng(7)
    k = (rng.standard_normal((256, 128)) * np.exp(rng.uniform(-8, 8, 128))).astype(np.float32)
    k[:64, 0] = 0.0                              # zero block -> scale 0, codes 8
    k[64:128, 1] = 1e9 * np.sign(k[64:128, 1])   # fp16 overflow -> 65504
    s = O.block_scales(k[128:192])
    for j in range(2, 20):                       # exact multiples m * s
        k[128:144, j] = (np.arange(-8, 8) * np.float64(s[j])).astype(np.float32)
        k[144:160, j] = np.nextafter(k[128:144, j], np.float32(-np.inf))
    v = np.zeros((256, 128), dtype=np.uint16)
    b.encode_append(cache, 0, torch.from_numpy(k).cuda()[None, None],
                    torch.from_numpy(v.view(np.int16)).cuda().view(torch.bfloat16)[None, None])
    torch.cuda.synchronize()
    planes, scales = O.encode_unit(k)
    gp, gs = _planes_np(cache, 0, 0, 0, 4)
    assert np.array_equal(gs.view(np.uint16), scales.view(np.uint16))
    assert np.array_equal(gp, planes)


# ---------------------------------------------------------------------------
# depth allocation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("budget", [0, 1, 17, 64, 88, 128, 300, 511, 512, 600])
def test_alloc_depth_bit_exact(bpk, c2, budget):
    b, wl = bpk
    cfg, cache, q, inps = c2
    depth, qb = b.alloc_depth(cache, q, 0, 1, budget)
    torch.cuda.synchronize()
    for h in range(cfg.heads):
        ref = O.alloc_depth(inps[h]["q"], inps[h]["var"], budget)
        assert np.array_equal(depth[0, 0, h].cpu().numpy(), ref), (budget, h)
        assert np.array_equal(qb[0, 0, h].cpu().numpy(), inps[h]["q"])


def test_alloc_depth_ties(bpk):
    """Equal gains (zero and repeated queries) fill low channels first."""
    b, wl = bpk
    cache = b.Cache(1, 1, 2, 64, group=4)
    q = torch.zeros((1, 1, 2, 4, 128), dtype=torch.bfloat16, device="cuda")
    q[0, 0, 1] = 1.0
    for budget in (1, 5, 9, 100, 255):
        depth, _ = b.alloc_depth(cache, q, 0, 1, budget)
        ones = np.ones(128, dtype=np.float32)
        for h, qq in ((0, np.zeros((4, 128), np.float32)), (1, np.ones((4, 128), np.float32))):
            assert np.array_equal(depth[0, 0, h].cpu().numpy(), O.alloc_depth(qq, ones, budget))


# ---------------------------------------------------------------------------
# scan, select, attend (single calls)
# ---------------------------------------------------------------------------

def _oracle_unit(inp, n, budget, k, scale):
    return O.decode_unit(inp["q"], inp["var"], inp["k"], inp["v"], n, budget, k, scale,
                         rot=inp["rot"])


@pytest.mark.parametrize("budget", [64, 88, 128, 200, 512])
def test_calls_c2(bpk, c2, budget):
    b, wl = bpk
    cfg, cache, q, inps = c2
    n, k = cfg.n, cfg.k
    scale = wl.softmax_scale(cfg)
    depth, qb = b.alloc_depth(cache, q, 0, 1, budget)
    scores = b.scan_scores(cache, qb, depth, 0, 1)
    idx = b.select_topk(cache, scores, 0, 1, k)
    out = b.sparse_attend(cache, q, idx, 0, 1, k, scale)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    ix = idx.cpu().numpy()
    ot = out.cpu().numpy()
    for h in range(cfg.heads):
        ref = _oracle_unit(inps[h], n, budget, k, scale)
        where = f"c2 P={budget} head {h}"
        P.check_scores(sc[0, 0, h, :, :n], ref["scores"], ref["l1"], where)
        P.check_topk_valid(sc[0, 0, h, :, :n], ix[0, 0, h], n, k, where)
        P.check_selection(ix[0, 0, h], ref["idx"], ref["scores"], ref["l1"], n, k, where)
        att = O.attend(inps[h]["q"], inps[h]["k"], inps[h]["v"], ix[0, 0, h], scale)
        P.check_attention(ot[0, 0, h], att, where)


def test_sparse_attend_list_forms(bpk, c2):
    """The union stage merges ascending lists of different lengths (-1 padding
    at the end) by rank and sorts unordered lists (padding anywhere) whole:
    attention matches the oracle over each head's own set, a head with no row
    outputs zeros, and an unordered copy of the lists gives the same result
    bit for bit."""
    b, wl = bpk
    cfg, cache, q, inps = c2
    scale = wl.softmax_scale(cfg)
    n, k = cfg.n, cfg.k
    rng = np.random.default_rng(11)
    G = q.shape[3]
    lens = [k, k // 3, 1, 0, k - 1, 37, k, 2]
    idx = np.full((1, 1, cfg.heads, G, k), -1, dtype=np.int32)
    for h in range(cfg.heads):
        for g in range(G):
            m = lens[(h + g) % len(lens)]
            idx[0, 0, h, g, :m] = np.sort(rng.choice(n, size=m, replace=False))
    shuffled = idx.copy()
    for h in range(cfg.heads):
        for g in range(G):
            shuffled[0, 0, h, g] = rng.permutation(shuffled[0, 0, h, g])
    out = b.sparse_attend(cache, q, torch.from_numpy(idx).cuda(), 0, 1, k, scale)
    out2 = b.sparse_attend(cache, q, torch.from_numpy(shuffled).cuda(), 0, 1, k, scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    ot = out.cpu().numpy()
    for h in range(cfg.heads):
        att = O.attend(inps[h]["q"], inps[h]["k"], inps[h]["v"], idx[0, 0, h], scale)
        P.check_attention(ot[0, 0, h], att, f"list forms head {h}")
        for g in range(G):
            if lens[(h + g) % len(lens)] == 0:
                assert not ot[0, 0, h, g].any()


def test_decode_step_c1(bpk, c1):
    b, wl = bpk
    cfg, cache, q, inp = c1
    scale = wl.softmax_scale(cfg)
    budget = cfg.budgets[0]
    depth = torch.empty((1, 1, 1, 128), dtype=torch.uint8, device="cuda")
    idx = torch.empty((1, 1, 1, 4, cfg.k), dtype=torch.int32, device="cuda")
    out = b.decode_step(cache, q, 0, 1, budget, cfg.k, scale, depth_out=depth, idx_out=idx)
    torch.cuda.synchronize()
    ref = _oracle_unit(inp, cfg.n, budget, cfg.k, scale)
    assert np.array_equal(depth[0, 0, 0].cpu().numpy(), ref["depth"])
    ix = idx[0, 0, 0].cpu().numpy()
    P.check_selection(ix, ref["idx"], ref["scores"], ref["l1"], cfg.n, cfg.k, "c1")
    att = O.attend(inp["q"], inp["k"], inp["v"], ix, scale)
    P.check_attention(out[0, 0, 0].cpu().numpy(), att, "c1")
    if np.array_equal(ix, ref["idx"]):
        P.check_attention(out[0, 0, 0].cpu().numpy(), ref["out"], "c1 end-to-end")


def test_decode_step_matches_single_calls(bpk, c2):
    b, wl = bpk
    cfg, cache, q, inps = c2
    scale = wl.softmax_scale(cfg)
    idx = torch.empty((1, 1, 8, 4, cfg.k), dtype=torch.int32, device="cuda")
    out = b.decode_step(cache, q, 0, 1, 88, cfg.k, scale, idx_out=idx)
    depth, qb = b.alloc_depth(cache, q, 0, 1, 88)
    idx2 = b.select_topk(cache, b.scan_scores(cache, qb, depth, 0, 1), 0, 1, cfg.k)
    out2 = b.sparse_attend(cache, q, idx2, 0, 1, cfg.k, scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)


def test_stage_trace_times_decode_step(bpk, c2):
    """Stage tracing records every stage a fused decode step runs and leaves
    its results unchanged."""
    b, wl = bpk
    cfg, cache, q, inps = c2
    scale = wl.softmax_scale(cfg)
    idx = torch.empty((1, 1, 8, 4, cfg.k), dtype=torch.int32, device="cuda")
    out = b.decode_step(cache, q, 0, 1, 88, cfg.k, scale, idx_out=idx)
    b.trace_enable(True)
    try:
        idx2 = torch.empty_like(idx)
        out2 = b.decode_step(cache, q, 0, 1, 88, cfg.k, scale, idx_out=idx2)
        out3 = b.decode_step(cache, q, 0, 1, 88, cfg.k, scale)
        ms, calls = b.trace_read()
    finally:
        b.trace_enable(False)
    torch.cuda.synchronize()
    assert calls == 2
    for stage in b.STAGES:
        assert ms[stage] > 0.0, stage
    assert torch.equal(idx, idx2) and torch.equal(out, out2) and torch.equal(out, out3)
    assert b.trace_read() == ({s: 0.0 for s in b.STAGES}, 0)


def test_scan_mixed_row_counts(bpk, c2):
    """One scan over units that read up to 128 plane rows and units that read
    more: each unit's scores equal those of a call over that unit's budget."""
    b, wl = bpk
    cfg, cache, q, inps = c2
    n = cfg.n
    d_small, qb = b.alloc_depth(cache, q, 0, 1, 88)
    d_big, _ = b.alloc_depth(cache, q, 0, 1, 200)
    depth = d_small.clone()
    depth[0, 0, 1::2] = d_big[0, 0, 1::2]  # odd KV heads read 200 rows
    scores = b.scan_scores(cache, qb, depth, 0, 1)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    for h in range(cfg.heads):
        budget = 200 if h % 2 else 88
        ref = _oracle_unit(inps[h], n, budget, cfg.k, wl.softmax_scale(cfg))
        P.check_scores(sc[0, 0, h, :, :n], ref["scores"], ref["l1"], f"mixed head {h} P={budget}")


@pytest.mark.parametrize("budget", [88, 200])
def test_decode_step_matches_single_calls_budgets(bpk, c2, budget):
    b, wl = bpk
    cfg, cache, q, inps = c2
    scale = wl.softmax_scale(cfg)
    idx = torch.empty((1, 1, 8, 4, cfg.k), dtype=torch.int32, device="cuda")
    out = b.decode_step(cache, q, 0, 1, budget, cfg.k, scale, idx_out=idx)
    depth, qb = b.alloc_depth(cache, q, 0, 1, budget)
    idx2 = b.select_topk(cache, b.scan_scores(cache, qb, depth, 0, 1), 0, 1, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _small_cache(b, cfg_like: Config, n, group=4, cap=None, heads=1):
    cap = cap or max(64, (n + 63) // 64 * 64)
    cache = b.Cache(1, 1, heads, cap, group=group)
    return cache


@pytest.mark.parametrize("n", [0, 1, 37, 64, 100, 64 * 9 + 40, 64 * 20, 64 * 20 + 7])
@pytest.mark.parametrize("group", [1, 4, 8])
def test_small_and_ragged(bpk, n, group):
    """Empty, shorter-than-k, open trailing blocks, and every supported group."""
    b, wl = bpk
    rng = np.random.default_rng(n * 31 + group)
    cap = max(64, (n + 63) // 64 * 64)
    cache = b.Cache(1, 1, 1, cap, group=group)
    k_rows = (rng.standard_normal((max(n, 1), 128)) * np.exp(rng.uniform(-2, 1.4, 128))).astype(np.float32)
    from synth.workload import f32_to_bf16_bits, bf16_bits_to_f32
    kb = f32_to_bf16_bits(k_rows)[:n]
    vb = f32_to_bf16_bits(rng.standard_normal((max(n, 1), 128)).astype(np.float32))[:n]
    qb = f32_to_bf16_bits(rng.standard_normal((group, 128)).astype(np.float32))
    var = np.exp(rng.uniform(-4.6, 2.8, 128)).astype(np.float32)
    cache.chan_var.copy_(torch.from_numpy(var)[None, None, None])
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    if n:
        b.encode_append(cache, 0, to_dev(kb)[None, None], to_dev(vb)[None, None])
    q = to_dev(qb)[None, None, None]
    k = 64 if group < 8 else 40
    if n > k and k < 4 + O.kept_tail(n):
        k = 4 + O.kept_tail(n) + 8
    scale = 1 / math.sqrt(128)
    depth = torch.empty((1, 1, 1, 128), dtype=torch.uint8, device="cuda")
    idx = torch.empty((1, 1, 1, group, k), dtype=torch.int32, device="cuda")
    out = b.decode_step(cache, q, 0, 1, 88, k, scale, depth_out=depth, idx_out=idx)
    depth2, qbasis = b.alloc_depth(cache, q, 0, 1, 88)
    scores = b.scan_scores(cache, qbasis, depth2, 0, 1)
    torch.cuda.synchronize()
    kv, vv, qv = bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), bf16_bits_to_f32(qb)
    ref = O.decode_unit(qv, var, kv, vv, n, 88, k, scale)
    assert np.array_equal(depth[0, 0, 0].cpu().numpy(), ref["depth"])
    ix = idx[0, 0, 0].cpu().numpy()
    nb = n // 64
    P.check_scores(scores[0, 0, 0, :, : nb * 64].cpu().numpy(), ref["scores"], ref["l1"], f"n={n}")
    full = np.zeros((group, n))
    full[:, : nb * 64] = scores[0, 0, 0, :, : nb * 64].cpu().numpy()
    P.check_topk_valid(full, ix, n, k, f"n={n}")
    P.check_selection(ix, ref["idx"], ref["scores"], ref["l1"], n, k, f"n={n}")
    assert (ix[:, min(n, k):] == -1).all()
    o = out[0, 0, 0].cpu().numpy()
    if n == 0:
        assert (o == 0).all()
    else:
        P.check_attention(o, O.attend(qv, kv, vv, ix, scale), f"n={n}")


def test_all_ties_pick_lowest_indices(bpk):
    """Budget 0: every score is 0, so the winners are the lowest candidate indices."""
    b, wl = bpk
    n, k = 64 * 30, 100
    cache = b.Cache(1, 1, 1, n, group=4)
    rng = np.random.default_rng(3)
    from synth.workload import f32_to_bf16_bits
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    kb = f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    b.encode_append(cache, 0, to_dev(kb)[None, None], to_dev(kb)[None, None])
    q = to_dev(f32_to_bf16_bits(rng.standard_normal((4, 128)).astype(np.float32)))[None, None, None]
    depth, qb = b.alloc_depth(cache, q, 0, 1, 0)
    scores = b.scan_scores(cache, qb, depth, 0, 1)
    idx = b.select_topk(cache, scores, 0, 1, k)
    torch.cuda.synchronize()
    assert float(scores[..., :n].abs().max()) == 0.0
    want = np.concatenate([np.arange(4), np.arange(4, 4 + k - 36), np.arange(n - 32, n)])
    for h in range(4):
        assert np.array_equal(idx[0, 0, 0, h].cpu().numpy(), want)


def test_multi_layer_multi_seq_call(bpk):
    """Per-call arrays cover [S][l1-l0][H]: a layer-range call equals per-layer calls."""
    b, wl = bpk
    cfg = Config("tiny", seqs=2, layers=3, heads=2, n=64 * 40 + 5, k=96, budgets=(88,),
                 seed=77)
    cache = wl.build_cache(cfg)
    q_all = wl.queries(cfg)
    scale = wl.softmax_scale(cfg)
    out_all = b.decode_step(cache, q_all[:, 1:3].contiguous(), 1, 3, 88, cfg.k, scale)
    for l in (1, 2):
        out_l = b.decode_step(cache, q_all[:, l:l + 1].contiguous(), l, l + 1, 88, cfg.k, scale)
        torch.cuda.synchronize()
        assert torch.equal(out_all[:, l - 1], out_l[:, 0])
    # and one unit of it against the oracle
    inp = P.unit_inputs(cfg, 1, 2, 1, cfg.n)
    ref = _oracle_unit(inp, cfg.n, 88, cfg.k, scale)
    idx = torch.empty((2, 1, 2, 4, cfg.k), dtype=torch.int32, device="cuda")
    out = b.decode_step(cache, q_all[:, 2:3].contiguous(), 2, 3, 88, cfg.k, scale, idx_out=idx)
    torch.cuda.synchronize()
    ix = idx[1, 0, 1].cpu().numpy()
    P.check_selection(ix, ref["idx"], ref["scores"], ref["l1"], cfg.n, cfg.k, "tiny")
    P.check_attention(out[1, 0, 1].cpu().numpy(), O.attend(inp["q"], inp["k"], inp["v"], ix, scale),
                      "tiny")
