"""GPU: decode_step's fused selection (sampled threshold -> candidate scan ->
exact top-k among the candidates, with a full scan + radix select for the
units it cannot settle) selects exactly what select_topk(scan_scores(...))
selects, and matches the oracle.

Bars as in test_gpu_parity: top-k sets equal to the oracle's up to near-tie
swaps; fused and unfused index arrays identical; attention within 2e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import config_by_name
from synth.workload import bf16_bits_to_f32, f32_to_bf16_bits
from tests import parity as P

pytestmark = pytest.mark.gpu

# the plan of the fused path: the first 64 blocks of every 4096 are sampled;
# a scan workgroup of wb blocks keeps its candidates per head in four parts
# (one per wavefront: wavefront w scores blocks 4w .. 4w+3 of every 16), each
# of 2 wb slots; more than 4096 candidates per head are not taken
SAMPLE_STRIDE, SAMPLE_GROUP, CAND_CAP = 4096, 64, 4096


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def bpk():
    import bit_plane_key_amd as b
    from bit_plane_key_amd import workloads
    return b, workloads


def _to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _unit_cache(b, kb, vb, var, group):
    n = kb.shape[0]
    cache = b.Cache(1, 1, 1, max(64, (n + 63) // 64 * 64), group=group)
    cache.chan_var.copy_(torch.from_numpy(var)[None, None, None])
    b.encode_append(cache, 0, _to_dev(kb)[None, None], _to_dev(vb)[None, None])
    return cache


def _unfused(b, cache, q, budget, k, scale):
    depth, qb = b.alloc_depth(cache, q, 0, 1, budget)
    scores = b.scan_scores(cache, qb, depth, 0, 1)
    idx = b.select_topk(cache, scores, 0, 1, k)
    return scores, idx


def _fused(b, cache, q, budget, k, scale, group):
    """decode_step on a workspace of its own; also returns how many units it
    redid unfused."""
    idx = torch.empty((1, 1, 1, group, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(b.workspace_bytes(cache, b.BPK_OP_DECODE, 0, 1, k), dtype=torch.uint8,
                     device="cuda")
    out = b.decode_step(cache, q, 0, 1, budget, k, scale, idx_out=idx, ws=ws)
    return idx, out, b.decode_fallback_units(cache, 0, 1, k, ws)


def _wg_blocks(nb, units=1):
    wb = 16
    while wb < 1024 and (nb * units // (2 * wb) >= 2048 or nb > 1024 * wb):
        wb *= 2
    return wb


def _key_floor(x):
    """The sampled threshold as the kernel keeps it: score x with the low 16
    bits of its order key cleared (the sample stores the upper halves)."""
    u = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
    if (u << 1) & 0xFFFFFFFF == 0:
        u = 0
    key = (~u & 0xFFFFFFFF) if u & 0x80000000 else (u | 0x80000000)
    key &= 0xFFFF0000
    bits = (key & 0x7FFFFFFF) if key & 0x80000000 else (~key & 0xFFFFFFFF)
    return float(np.array([bits], dtype=np.uint32).view(np.float32)[0])


def _fused_plan(scores_h, n, k, units=1):
    """The fused plan on one head's exact scores: (tokens at or above the
    sampled threshold, the largest count of them in one wavefront part, the
    part size).  The scan's own test may keep a few more just below it."""
    w = O.kept_tail(n)
    hi, want = n - w, k - 4 - w
    nb = n // 64
    toks = np.concatenate([np.arange(g * SAMPLE_STRIDE * 64,
                                     min(g * SAMPLE_STRIDE + SAMPLE_GROUP, nb) * 64)
                           for g in range((nb + SAMPLE_STRIDE - 1) // SAMPLE_STRIDE)])
    toks = toks[(toks >= 4) & (toks < hi)]
    m, nc = len(toks), hi - 4
    r = (2 * want * m + nc - 1) // nc + 8
    tau = -np.inf if r > m else _key_floor(np.sort(scores_h[toks])[::-1][r - 1])
    passed = np.zeros(nb * 64, dtype=bool)
    passed[4:hi] = scores_h[4:hi] >= tau
    wb = _wg_blocks(nb, units)
    blk = np.arange(nb * 64) // 64
    part = (blk // wb) * 4 + (blk % 16) // 4
    per_part = np.bincount(part[passed], minlength=part.max() + 1)
    return int(passed.sum()), int(per_part.max()), 2 * wb


@pytest.mark.parametrize("budget", [64, 88, 128])
def test_fused_equals_unfused_c2(bpk, budget):
    b, wl = bpk
    cfg = config_by_name("c2")
    cache = wl.build_cache(cfg)
    q = wl.queries(cfg)
    scale = wl.softmax_scale(cfg)
    idx = torch.empty((1, 1, 8, 4, cfg.k), dtype=torch.int32, device="cuda")
    out = b.decode_step(cache, q, 0, 1, budget, cfg.k, scale, idx_out=idx)
    depth, qb = b.alloc_depth(cache, q, 0, 1, budget)
    idx2 = b.select_topk(cache, b.scan_scores(cache, qb, depth, 0, 1), 0, 1, cfg.k)
    out2 = b.sparse_attend(cache, q, idx2, 0, 1, cfg.k, scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("n,group", [(4096 * 64 * 3 + 1000, 4), (4096 * 64 + 77, 1),
                                     (4096 * 64 * 2 + 64 * 7, 8)])
def test_fused_many_sample_groups_against_oracle(bpk, n, group):
    """Several sampled groups, a ragged tail, G = 1, 4, 8."""
    b, wl = bpk
    _say(f"fused n={n} G={group}")
    rng = np.random.default_rng(n + group)
    sig = np.exp(rng.uniform(math.log(0.1), math.log(4.0), 128))
    kb = f32_to_bf16_bits((rng.standard_normal((n, 128)) * sig).astype(np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    qb = f32_to_bf16_bits(rng.standard_normal((group, 128)).astype(np.float32))
    var = (sig ** 2).astype(np.float32)
    cache = _unit_cache(b, kb, vb, var, group)
    q = _to_dev(qb)[None, None, None]
    k, budget, scale = 512 if group < 8 else 256, 88, 1 / math.sqrt(128)
    idx, out, flagged = _fused(b, cache, q, budget, k, scale, group)
    scores, idx2 = _unfused(b, cache, q, budget, k, scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    kv, vv, qv = bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), bf16_bits_to_f32(qb)
    ref = O.decode_unit(qv, var, kv, vv, n, budget, k, scale)
    ix = idx[0, 0, 0].cpu().numpy()
    P.check_selection(ix, ref["idx"], ref["scores"], ref["l1"], n, k, f"n={n}")
    P.check_attention(out[0, 0, 0].cpu().numpy(), O.attend(qv, kv, vv, ix, scale), f"n={n}")
    sc = scores[0, 0, 0].cpu().numpy()
    for h in range(group):
        count, part_max, part_size = _fused_plan(sc[h], n, k)
        # comfortably inside the plan's limits: the fused path settles it
        assert k - 4 - O.kept_tail(n) <= count <= CAND_CAP // 2 and part_max <= part_size // 2
    assert flagged == 0


def test_fused_too_few_candidates_falls_back(bpk):
    """Keys of the sampled blocks score far above the rest, so the sampled
    threshold passes fewer than k - 4 - W tokens: the unit is redone by the
    full scan and radix select, and the result is still exact."""
    b, wl = bpk
    n, group, k, budget = 4096 * 64 * 2 + 64 * 100, 4, 512, 88
    rng = np.random.default_rng(11)
    k_f = rng.standard_normal((n, 128)).astype(np.float32) * 0.5
    for g in range(3):
        t0 = g * SAMPLE_STRIDE * 64
        k_f[t0:t0 + SAMPLE_GROUP * 64] = np.abs(k_f[t0:t0 + SAMPLE_GROUP * 64]) + 2.0
    kb = f32_to_bf16_bits(k_f)
    vb = f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    qb = f32_to_bf16_bits(np.ones((group, 128), dtype=np.float32))
    var = np.ones(128, dtype=np.float32)
    cache = _unit_cache(b, kb, vb, var, group)
    q = _to_dev(qb)[None, None, None]
    scale = 1 / math.sqrt(128)
    idx, out, flagged = _fused(b, cache, q, budget, k, scale, group)
    scores, idx2 = _unfused(b, cache, q, budget, k, scale)
    torch.cuda.synchronize()
    sc = scores[0, 0, 0].cpu().numpy()
    for h in range(group):
        count, _, _ = _fused_plan(sc[h], n, k)
        assert count < k - 4 - O.kept_tail(n)   # too few at or above the threshold
    assert flagged == 1
    assert torch.equal(idx, idx2)
    P.check_topk_valid(sc[:, :n].astype(np.float64), idx[0, 0, 0].cpu().numpy(), n, k, "few")


def test_fused_ties_at_threshold_take_lowest_indices(bpk):
    """Many candidates tie at the k-th score without overflowing: channel 0
    holds 7 on every 50th token and -8 elsewhere (every block scale 1), the
    query reads only channel 0 (one plane), so every such token scores the
    same top value.  The fused selection takes the lowest indices among the
    ties, as the unfused radix select does, without redoing the unit."""
    b, wl = bpk
    n, k, group = 64 * 600, 300, 4
    rng = np.random.default_rng(50)
    k32 = rng.uniform(-0.5, 0.5, (n, 128)).astype(np.float32)
    k32[:, 0] = -8.0
    top = np.arange(0, n, 50)
    k32[top, 0] = 7.0
    kb = f32_to_bf16_bits(k32)
    vb = f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    q32 = np.zeros((group, 128), dtype=np.float32)
    q32[:, 0] = 1.0 + 0.25 * np.arange(group)
    cache = _unit_cache(b, kb, vb, np.ones(128, dtype=np.float32), group)
    q = _to_dev(f32_to_bf16_bits(q32))[None, None, None]
    scale = 1 / math.sqrt(128)
    idx, out, flagged = _fused(b, cache, q, 1, k, scale, group)
    scores, idx2 = _unfused(b, cache, q, 1, k, scale)
    torch.cuda.synchronize()
    assert flagged == 0
    assert torch.equal(idx, idx2)
    w = O.kept_tail(n)
    want = k - 4 - w
    cand = top[(top >= 4) & (top < n - w)]
    assert len(cand) > want  # the k-th score is tied
    expect = np.concatenate([np.arange(4), cand[:want], np.arange(n - w, n)])
    for h in range(group):
        assert np.array_equal(idx[0, 0, 0, h].cpu().numpy(), expect)


def test_fused_overflow_falls_back(bpk):
    """Budget 0 makes every score 0: all candidates tie at the threshold and
    overflow the buffer; the fallback takes the lowest indices."""
    b, wl = bpk
    n, k = 64 * 100, 100
    rng = np.random.default_rng(5)
    kb = f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    cache = _unit_cache(b, kb, kb, np.ones(128, dtype=np.float32), 4)
    q = _to_dev(f32_to_bf16_bits(rng.standard_normal((4, 128)).astype(np.float32)))[None, None, None]
    idx, out, flagged = _fused(b, cache, q, 0, k, 1 / math.sqrt(128), 4)
    torch.cuda.synchronize()
    assert flagged == 1
    want = np.concatenate([np.arange(4), np.arange(4, 4 + k - 36), np.arange(n - 32, n)])
    for h in range(4):
        assert np.array_equal(idx[0, 0, 0, h].cpu().numpy(), want)


def test_large_k_takes_unfused_path(bpk):
    """k above the fused limit (1024) runs the unfused scan + radix select."""
    b, wl = bpk
    n, k = 64 * 600 + 9, 2000
    rng = np.random.default_rng(9)
    kb = f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    cache = _unit_cache(b, kb, vb, np.ones(128, dtype=np.float32), 2)
    q = _to_dev(f32_to_bf16_bits(rng.standard_normal((2, 128)).astype(np.float32)))[None, None, None]
    scale = 1 / math.sqrt(128)
    idx, out, flagged = _fused(b, cache, q, 88, k, scale, 2)
    scores, idx2 = _unfused(b, cache, q, 88, k, scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert flagged == 0


def test_fused_long_unit_radix_threshold(bpk):
    """One unit of 1,310,720 tokens: its sample (5 groups of 64 blocks, 20480
    scores per head) is too large for the register threshold kernels, so the
    radix threshold kernel sets the thresholds.  Fused = unfused, no unit
    redone, the selection a valid top-k of the scores, and the scores right
    on a seeded sample of tokens against the oracle."""
    b, wl = bpk
    n, group, k, budget = 1310720, 4, 512, 88
    _say(f"fused long unit n={n}")
    rng = np.random.default_rng(1310720)
    sig = np.exp(rng.uniform(math.log(0.1), math.log(4.0), 128))
    kb = f32_to_bf16_bits((rng.standard_normal((n, 128)) * sig).astype(np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    qb = f32_to_bf16_bits(rng.standard_normal((group, 128)).astype(np.float32))
    var = (sig ** 2).astype(np.float32)
    cache = _unit_cache(b, kb, vb, var, group)
    q = _to_dev(qb)[None, None, None]
    scale = 1 / math.sqrt(128)
    idx, out, flagged = _fused(b, cache, q, budget, k, scale, group)
    scores, idx2 = _unfused(b, cache, q, budget, k, scale)
    torch.cuda.synchronize()
    assert flagged == 0
    assert torch.equal(idx, idx2)
    sc = scores[0, 0, 0, :, :n].cpu().numpy()
    P.check_topk_valid(sc.astype(np.float64), idx[0, 0, 0].cpu().numpy(), n, k, "long unit")
    qv, kv = bf16_bits_to_f32(qb), bf16_bits_to_f32(kb)
    depth = O.alloc_depth(qv, var, budget)
    assert np.array_equal(b.alloc_depth(cache, q, 0, 1, budget)[0][0, 0, 0].cpu().numpy(), depth)
    blocks = np.sort(rng.choice(n // 64, 64, replace=False))
    toks = (blocks[:, None] * 64 + np.arange(64)[None, :]).ravel()
    planes, scales = O.encode_unit(kv[toks])      # the sampled blocks, re-encoded
    ref, l1 = O.scan_scores(qv, depth, planes, scales, len(toks))
    P.check_scores(sc[:, toks], ref, l1, "long unit sample")


def _random_cases(count=8, seed=2026):
    """Seeded random decode shapes: ragged n, every group size, k up to the
    fused limit, budgets from none to the wide kernel's row counts."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        group = int(rng.choice([1, 2, 4, 8]))
        n = int(rng.integers(1200, 40000))
        k = int(rng.integers(40, min(1024, n // 2)))
        budget = int(rng.choice([0, 1, 37, 88, 128, 200, 512]))
        cases.append((i, n, group, k, budget))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"n{c[1]}-G{c[2]}-k{c[3]}-P{c[4]}")
def test_fused_random_shapes_against_oracle(bpk, case):
    """Random shapes with heavy-tailed channel scales and one outlier
    channel: the fused step selects what the unfused path selects, its sets
    pass the oracle's top-k bar and its attention is within 2e-3."""
    b, wl = bpk
    i, n, group, k, budget = case
    _say(f"random case {i}: n={n} G={group} k={k} P={budget}")
    rng = np.random.default_rng(1000 + i)
    sig = np.exp(rng.uniform(math.log(0.05), math.log(3.0), 128))
    sig[int(rng.integers(128))] *= 12.0  # an outlier channel
    kb = f32_to_bf16_bits((rng.standard_t(4, (n, 128)) * sig).astype(np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    qb = f32_to_bf16_bits(rng.standard_normal((group, 128)).astype(np.float32))
    var = (sig ** 2).astype(np.float32)
    cache = _unit_cache(b, kb, vb, var, group)
    q = _to_dev(qb)[None, None, None]
    scale = 1 / math.sqrt(128)
    idx, out, flagged = _fused(b, cache, q, budget, k, scale, group)
    scores, idx2 = _unfused(b, cache, q, budget, k, scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    kv, vv, qv = bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), bf16_bits_to_f32(qb)
    ref = O.decode_unit(qv, var, kv, vv, n, budget, k, scale)
    ix = idx[0, 0, 0].cpu().numpy()
    where = f"case {i} n={n} G={group} k={k} P={budget}"
    P.check_selection(ix, ref["idx"], ref["scores"], ref["l1"], n, k, where)
    P.check_attention(out[0, 0, 0].cpu().numpy(), O.attend(qv, kv, vv, ix, scale), where)
