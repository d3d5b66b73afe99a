"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types an oracle formula: each checks the oracle against an
independent route (exact rationals, brute force, a library routine, a bound,
or a number the Fathom page prints).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _blocks(rng, nb, d, sigma=None):
    sigma = np.ones(d) if sigma is None else sigma
    return (rng.standard_normal((nb * 64, d)) * sigma).astype(np.float32)


# --------------------------------------------------------------------------
# quantizer and scales (Fathom §3.2)
# --------------------------------------------------------------------------

def test_scale_is_nearest_fp16_of_blockmax_over_8(rng):
    k = _blocks(rng, 4, 16, sigma=np.exp(rng.uniform(-6, 6, 16)))
    for b in range(4):
        blk = k[b * 64:(b + 1) * 64]
        s = O.block_scales(blk)
        for j in range(16):
            target = Fraction(float(np.max(np.abs(blk[:, j])))) / 8
            got = Fraction(float(s[j]))
            for nb_ in (np.nextafter(s[j], np.float16(np.inf)), np.nextafter(s[j], np.float16(0))):
                assert abs(got - target) <= abs(Fraction(float(nb_)) - target)


def test_scale_zero_block_and_saturation():
    blk = np.zeros((64, 3), dtype=np.float32)
    blk[5, 1] = 1e9           # beyond fp16 range after /8
    blk[7, 2] = -3.0
    s = O.block_scales(blk)
    assert s[0] == 0 and s[1] == np.float16(65504) and s[2] == np.float16(0.375)
    c = O.quantize_codes(blk, s)
    assert np.all(c[:, 0] == 8)          # zero scale -> code 8 (zero)
    assert c[5, 1] == 15                 # clipped at the top code
    assert c[7, 2] == 0                  # -3 / 0.375 = -8 exactly


def test_codes_match_exact_rational_floor(rng):
    k = _blocks(rng, 2, 8, sigma=np.exp(rng.uniform(-3, 3, 8)))
    # plant exact multiples of the scale and their neighbours
    s = O.block_scales(k[:64])
    for j in range(8):
        k[63, j] = np.float32(8 * float(s[j]))      # keeps the block scale at s
        for i, m in enumerate(range(-8, 8)):
            v = np.float32(m * float(s[j]))
            k[i, j] = v
            k[16 + i, j] = np.nextafter(v, np.float32(-np.inf))
    s2 = O.block_scales(k[:64])
    assert np.array_equal(s2, s)
    c = O.quantize_codes(k[:64], s)
    for i in range(64):
        for j in range(8):
            q = Fraction(float(k[i, j])) / Fraction(float(s[j]))
            m = math.floor(q)
            assert c[i, j] == min(max(m, -8), 7) + 8


def test_top_plane_is_sign_and_token_i_is_bit_i(rng):
    """Fathom §3.2: code 8 is zero and the most significant bit is the sign."""
    k = _blocks(rng, 3, 8)
    planes, scales = O.encode_unit(k)
    for b in range(3):
        for j in range(8):
            w = int(planes[j, 0, b])
            for i in range(64):
                assert ((w >> i) & 1) == int(k[64 * b + i, j] >= 0)


def test_open_block_has_no_planes(rng):
    k = _blocks(rng, 3, 4)[: 64 * 2 + 17]
    planes, scales = O.encode_unit(k)
    assert planes.shape == (4, 4, 2) and scales.shape == (4, 2)


# --------------------------------------------------------------------------
# prefix identity (Fathom §1 observation 2)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("t", [0, 1, 2, 3, 4])
def test_plane_prefix_is_the_t_bit_quantizer(rng, t):
    """Reading t planes equals quantizing k directly with t bits and cell s*2^(4-t)."""
    k = _blocks(rng, 4, 6, sigma=np.exp(rng.uniform(-2, 2, 6)))
    planes, scales = O.encode_unit(k)
    for j in range(6):
        pre = O.codes_from_planes(planes, t, j, np.arange(4))
        vals = O.prefix_values(pre, t)
        for i in range(0, 256, 3):
            s = Fraction(float(scales[j, i // 64]))
            if t == 0:
                expect = Fraction(0)
            else:
                w = s * 2 ** (4 - t)
                half = 2 ** (t - 1)
                cell = min(max(math.floor(Fraction(float(k[i, j])) / w), -half), half - 1)
                expect = (cell + Fraction(1, 2)) * w
            assert Fraction(vals[i]) * s == expect


def test_prefix_all_codes_all_depths():
    """Exhaustive over the 16 codes: a t-bit prefix reconstructs the midpoint of
    the 2^(4-t)-code cell that contains the code."""
    k = np.zeros((64, 1), dtype=np.float32)
    for i in range(64):
        k[i, 0] = (i % 16 - 8 + 0.25)          # code i % 16 under s = 1
    k[63, 0] = 7.25
    k[0, 0] = -8.0
    planes, scales = O.encode_unit(k * 1.0)
    assert float(scales[0, 0]) == 1.0
    for t in range(5):
        vals = O.prefix_values(O.codes_from_planes(planes, t, 0, np.arange(1)), t)
        for i in range(64):
            c = int(math.floor(k[i, 0])) + 8
            if t == 0:
                assert vals[i] == 0
                continue
            width = 2 ** (4 - t)
            lo = (c // width) * width - 8
            assert vals[i] == lo + width / 2


def test_error_quarters_per_bit(rng):
    """Fathom §1 observation 1: each further bit cuts the squared error ~4x."""
    k = _blocks(rng, 64, 32)
    planes, scales = O.encode_unit(k)
    mse = []
    for t in range(1, 5):
        err = 0.0
        for j in range(32):
            v = O.prefix_values(O.codes_from_planes(planes, t, j, np.arange(64)), t)
            v = v * np.repeat(scales[j].astype(np.float64), 64)
            err += np.mean((v - k[:, j]) ** 2)
        mse.append(err / 32)
    ratios = [mse[i] / mse[i + 1] for i in range(3)]
    assert all(3.3 < r < 4.8 for r in ratios), ratios


def test_reconstruction_error_bound(rng):
    """|k - k_hat| <= s * 2^(3-t) (+ fp16 rounding slack of the scale)."""
    k = _blocks(rng, 8, 16, sigma=np.exp(rng.uniform(-4, 4, 16)))
    planes, scales = O.encode_unit(k)
    for t in range(5):
        for j in range(16):
            v = O.prefix_values(O.codes_from_planes(planes, t, j, np.arange(8)), t)
            s = np.repeat(scales[j].astype(np.float64), 64)
            bound = s * 2.0 ** (3 - t) + s * 8 * 2.0 ** -10
            assert np.all(np.abs(v * s - k[:, j]) <= bound)


# --------------------------------------------------------------------------
# depth allocation (Fathom §1 observation 1, ReadKV §5.2 / §5.4)
# --------------------------------------------------------------------------

def _objective(g, t):
    return sum(Fraction(float(gj)) / 4 ** int(tj) for gj, tj in zip(g, t))


@pytest.mark.parametrize("d", [1, 2, 3, 5])
def test_alloc_brute_force_optimal(rng, d):
    for trial in range(12):
        q = rng.standard_normal((4, d)).astype(np.float32)
        var = np.exp(rng.uniform(-3, 3, d)).astype(np.float32)
        if trial == 0:
            var[:] = 1.0
            q[:] = 1.0        # all gains equal: ties everywhere
        g = O.channel_gains(q, var)
        import itertools
        allt = list(itertools.product(range(5), repeat=d))
        for p in range(0, 4 * d + 2):
            t = O.alloc_depth(q, var, p)
            assert int(t.sum()) == min(p, 4 * d)
            best = min(_objective(g, tt) for tt in allt if sum(tt) == min(p, 4 * d))
            assert _objective(g, t) == best


def test_alloc_gain_sums_group_heads():
    """ReadKV §5.2: channel importance sums the squared components of all heads."""
    var = np.ones(4, dtype=np.float32)
    q = np.zeros((4, 4), dtype=np.float32)
    q[0, 0] = 1.0           # channel 0: one head at 1
    q[:, 1] = 0.6           # channel 1: four heads at 0.6 -> 1.44 > 1
    t = O.alloc_depth(q, var, 1)
    assert list(t) == [0, 1, 0, 0]


def test_gain_is_channel_share_of_score_variance(rng):
    """Fathom §1 observation 1: g_j is channel j's contribution to the score
    variance, here summed over the heads that share the KV head [ReadKV §5.2].

    Monte Carlo with independent channels k_j ~ N(0, sigma_j^2), sigma_j far
    from 1: the empirical sum over heads of Var_i(q_hj k_ij) must match g_j,
    and the shares must add up to the summed variance of the real scores."""
    sigma = np.array([0.3, 0.55, 1.0, 1.7, 2.6, 4.0], dtype=np.float64)
    q = np.array([[0.9, -1.6, 0.2, 0.05, -0.7, 0.3],
                  [-0.4, 0.1, 1.3, -0.2, 0.0, -0.35],
                  [1.8, 0.6, -0.5, 0.9, 0.25, 0.1],
                  [0.0, -0.3, 0.8, 1.1, -0.15, 0.2]], dtype=np.float32)
    var = (sigma ** 2).astype(np.float32)
    g = O.channel_gains(q, var).astype(np.float64)
    n = 400_000
    k = rng.standard_normal((n, 6)) * sigma
    qd = q.astype(np.float64)
    share = np.array([sum(np.var(qd[h, j] * k[:, j]) for h in range(4)) for j in range(6)])
    np.testing.assert_allclose(g, share, rtol=0.02)
    total = sum(np.var(k @ qd[h]) for h in range(4))
    assert abs(g.sum() - total) <= 0.02 * total


def test_gain_predicts_next_plane_error_drop(rng):
    """Fathom §1 observation 1: one more plane of channel j cuts the summed
    squared score error by an amount proportional to g_j 4^-t_j.  Measured on
    the oracle's own encoder: at each depth the drop divided by g_j must be the
    same for every channel (the quantizer is scale-free), so a gain that weighs
    sigma instead of sigma^2, or |q| instead of q^2, fails."""
    sigma = np.array([0.25, 1.0, 3.0, 0.6], dtype=np.float64)
    q = np.array([[1.5, -0.2, 0.4, 0.0],
                  [0.3, 0.9, -0.1, 2.0],
                  [-0.6, 0.4, 0.05, 0.7],
                  [0.2, -1.2, 0.3, 0.1]], dtype=np.float32)
    g = O.channel_gains(q, (sigma ** 2).astype(np.float32)).astype(np.float64)
    n = 64 * 2048
    keys = (rng.standard_normal((n, 4)) * sigma).astype(np.float32)
    planes, scales = O.encode_unit(keys)
    blocks = np.arange(n // 64)
    qd = q.astype(np.float64)
    err = np.zeros((4, 5))
    for j in range(4):
        s = np.repeat(scales[j].astype(np.float64), 64)
        for t in range(5):
            rec = s * O.prefix_values(O.codes_from_planes(planes, t, j, blocks), t)
            e2 = np.mean((keys[:, j].astype(np.float64) - rec) ** 2)
            err[j, t] = e2 * float(np.sum(qd[:, j] ** 2))   # summed over heads
    for t in range(1, 4):
        ratio = (err[:, t] - err[:, t + 1]) / (g * 0.25 ** t)
        assert ratio.max() <= 1.03 * ratio.min(), (t, ratio)


def test_gain_two_channel_hand_worked():
    """Hand-worked: heads (3, 2) and (0, 2) on channels 0, 1 with variances 4
    and 1.  Gains: 4 (9 + 0) = 36 and 1 (4 + 4) = 8, so the planes are worth
    36, 9, 2.25, 0.5625 (channel 0) and 8, 2, 0.5, 0.125 (channel 1).  Taking
    them in value order gives the depths below.  (With sigma in place of
    sigma^2, sum |q| in place of sum q^2, or no variance at all, the second
    plane would go to channel 1.)"""
    q = np.array([[3.0, 2.0], [0.0, 2.0]], dtype=np.float32)
    var = np.array([4.0, 1.0], dtype=np.float32)
    assert list(O.channel_gains(q, var)) == [36.0, 8.0]
    expect = {0: [0, 0], 1: [1, 0], 2: [2, 0], 3: [2, 1], 4: [3, 1], 5: [3, 2],
              6: [4, 2], 7: [4, 3], 8: [4, 4], 9: [4, 4]}
    for p, t in expect.items():
        assert list(O.alloc_depth(q, var, p)) == t, p
        assert list(O.alloc_depth_greedy(q, var, p)) == t, p


def test_alloc_sort_form_equals_greedy_loop(rng):
    for trial in range(6):
        q = rng.standard_normal((4, 128)).astype(np.float32)
        var = np.exp(rng.uniform(-4.6, 2.8, 128)).astype(np.float32)
        for p in (0, 1, 64, 88, 128, 511, 512, 600):
            assert np.array_equal(O.alloc_depth(q, var, p), O.alloc_depth_greedy(q, var, p))


def test_alloc_water_filling_threshold(rng):
    """Closed form: some level lam splits planes worth more / less than lam."""
    q = rng.standard_normal((4, 128)).astype(np.float32)
    var = np.exp(rng.uniform(-4.6, 2.8, 128)).astype(np.float32)
    g = O.channel_gains(q, var).astype(np.float64)
    for p in (17, 64, 88, 128, 300):
        t = O.alloc_depth(q, var, p)
        vals = np.sort((g[:, None] * 0.25 ** np.arange(4)[None, :]).ravel())[::-1]
        lam = vals[p - 1]
        above = (g[:, None] * 0.25 ** np.arange(4)[None, :] > lam).sum(1)
        atleast = (g[:, None] * 0.25 ** np.arange(4)[None, :] >= lam).sum(1)
        assert np.all(t >= above) and np.all(t <= atleast)
        with np.errstate(divide="ignore"):
            closed = np.clip(np.floor(np.log(g / lam) / np.log(4.0)) + 1, 0, 4)
        clean = (above == atleast)
        assert np.array_equal(t[clean], closed[clean].astype(np.uint8))


def test_alloc_zero_gains_fill_low_channels_first():
    q = np.zeros((4, 8), dtype=np.float32)
    var = np.ones(8, dtype=np.float32)
    assert list(O.alloc_depth(q, var, 9)) == [4, 4, 1, 0, 0, 0, 0, 0]
    assert list(O.alloc_depth(q, var, 0)) == [0] * 8
    assert list(O.alloc_depth(q, var, 99)) == [4] * 8


# --------------------------------------------------------------------------
# scan (Fathom §1, §3.2)
# --------------------------------------------------------------------------

def test_scan_full_depth_equals_dequantized_codes(rng):
    k = _blocks(rng, 5, 128, sigma=np.exp(rng.uniform(-2.3, 1.4, 128)))
    q = rng.standard_normal((4, 128)).astype(np.float32)
    planes, scales = O.encode_unit(k)
    sc, _ = O.scan_scores(q, np.full(128, 4), planes, scales, k.shape[0])
    # independent route: codes straight from the quantizer, no planes
    ref = np.zeros_like(sc)
    for b in range(5):
        blk = k[b * 64:(b + 1) * 64]
        s = O.block_scales(blk).astype(np.float64)
        c = O.quantize_codes(blk, O.block_scales(blk)).astype(np.float64)
        khat = (c - 8 + 0.5) * s[None, :]
        ref[:, b * 64:(b + 1) * 64] = q.astype(np.float64) @ khat.T
    assert np.allclose(sc, ref, rtol=1e-12, atol=1e-12)


def test_scan_depth_zero_is_zero(rng):
    k = _blocks(rng, 2, 128)
    planes, scales = O.encode_unit(k)
    sc, l1 = O.scan_scores(rng.standard_normal((4, 128)), np.zeros(128), planes, scales, 128)
    assert np.all(sc == 0) and np.all(l1 == 0)


def test_scan_within_quantizer_bound_of_exact_dot(rng):
    sig = np.exp(rng.uniform(-2.3, 1.4, 128))
    k = _blocks(rng, 6, 128, sigma=sig)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    planes, scales = O.encode_unit(k)
    depth = O.alloc_depth(q, (sig ** 2).astype(np.float32), 88)
    sc, _ = O.scan_scores(q, depth, planes, scales, k.shape[0])
    exact = q.astype(np.float64) @ k.astype(np.float64).T
    s = np.repeat(scales.astype(np.float64), 64, axis=1)          # (D, n)
    half = s * (2.0 ** (3 - depth.astype(np.float64)))[:, None] + s * 8 * 2.0 ** -10
    bound = np.abs(q.astype(np.float64)) @ half
    assert np.all(np.abs(sc - exact) <= bound + 1e-9)


def test_more_planes_never_hurt_on_average(rng):
    sig = np.exp(rng.uniform(-2.3, 1.4, 128))
    k = _blocks(rng, 32, 128, sigma=sig)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    planes, scales = O.encode_unit(k)
    exact = q.astype(np.float64) @ k.astype(np.float64).T
    errs = []
    for p in (32, 64, 88, 128, 256, 512):
        depth = O.alloc_depth(q, (sig ** 2).astype(np.float32), p)
        sc, _ = O.scan_scores(q, depth, planes, scales, k.shape[0])
        errs.append(np.mean((sc - exact) ** 2))
    assert all(errs[i] > errs[i + 1] for i in range(len(errs) - 1)), errs


# --------------------------------------------------------------------------
# selection (Fathom §2 Top-k decoding)
# --------------------------------------------------------------------------

def _check_topk_property(scores, n, k, idx):
    w = O.kept_tail(n)
    fixed = set(range(4)) | set(range(n - w, n))
    for h in range(scores.shape[0]):
        sel = set(idx[h].tolist())
        assert len(sel) == k and fixed <= sel
        assert list(idx[h]) == sorted(idx[h])
        chosen = sel - fixed
        rest = set(range(4, n - w)) - chosen
        for a in chosen:
            for b in rest:
                assert scores[h, a] > scores[h, b] or (scores[h, a] == scores[h, b] and a < b)


@pytest.mark.parametrize("n", [100, 128, 150, 191])
def test_select_is_a_top_k(rng, n):
    scores = np.round(rng.standard_normal((4, n)) * 3) / 2     # many exact ties
    for k in (70, 80, n - 1):
        if k < 4 + O.kept_tail(n):
            continue
        idx = O.select_topk(scores, n, k)
        _check_topk_property(scores, n, k, idx)


def test_select_keeps_open_block():
    n = 64 * 3 + 40
    scores = np.zeros((1, n))
    idx = O.select_topk(scores, n, 60)
    assert set(range(n - 40, n)) <= set(idx[0].tolist())
    assert O.kept_tail(n) == 40 and O.kept_tail(64 * 3) == 32 and O.kept_tail(64 * 3 + 5) == 32


def test_select_all_when_k_covers_n():
    idx = O.select_topk(np.zeros((2, 50)), 50, 64)
    assert idx.shape == (2, 50) and np.array_equal(idx[1], np.arange(50))


# --------------------------------------------------------------------------
# attention (Fathom §2)
# --------------------------------------------------------------------------

def test_k_equals_n_is_dense_attention(rng):
    n = 300
    q = rng.standard_normal((4, 128)).astype(np.float32)
    kr = rng.standard_normal((n, 128)).astype(np.float32)
    vr = rng.standard_normal((n, 128)).astype(np.float32)
    sig = np.ones(128, dtype=np.float32)
    r = O.decode_unit(q, sig, kr, vr, n, 88, n, 1 / math.sqrt(128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[:, None, :],
        torch.from_numpy(kr.astype(np.float64))[None].expand(4, n, 128),
        torch.from_numpy(vr.astype(np.float64))[None].expand(4, n, 128),
        scale=1 / math.sqrt(128))[:, 0, :].numpy()
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_attention_two_keys_closed_form():
    q = np.zeros((1, 2))
    q[0, 0] = 1.0
    kr = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    vr = np.array([[1.0, 0.0], [0.0, 1.0]])
    out = O.attend(q, kr, vr, np.array([[0, 1]]), 1.0)
    assert np.allclose(out[0], [0.25, 0.75], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# rotated basis
# --------------------------------------------------------------------------

def test_rotation_matches_matmul_and_inverts(rng):
    a = rng.standard_normal((128, 128))
    r, _ = np.linalg.qr(a)
    r = r.astype(np.float32)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    z = O.rotate_basis(r, x)
    assert np.allclose(z, x.astype(np.float64) @ r.astype(np.float64), rtol=0, atol=1e-5)
    assert np.array_equal(O.rotate_basis(np.eye(128, dtype=np.float32), x), x)
    back = z.astype(np.float64) @ r.astype(np.float64).T
    assert np.allclose(back, x, atol=1e-4)


# --------------------------------------------------------------------------
# byte accounting (Fathom §1, §2; numbers the page prints)
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# per-layer budget calibration (Fathom §3; the rule is a reading)
# --------------------------------------------------------------------------

def test_pooled_allocation_of_one_unit_is_the_unit_rule(rng):
    q = rng.standard_normal((4, 128)).astype(np.float32)
    var = np.exp(rng.uniform(-4.6, 2.8, 128)).astype(np.float32)
    g = O.channel_gains(q, var)[None, :]
    for p in (0, 1, 64, 88, 512, 700):
        assert list(O.pooled_plane_counts(g, p)) == [int(O.alloc_depth(q, var, p).sum())]


def test_pooled_allocation_brute_force_optimal(rng):
    """Two units of two channels: with the pooled counts, the units' own
    depth rule reaches the best summed error sum_u sum_j g_uj 4^-t_uj over
    every split of the pooled budget (brute force over {0..4}^4)."""
    import itertools

    def err(g, t):
        return sum(Fraction(float(g[i // 2, i % 2])) / 4 ** t[i] for i in range(4))

    for trial in range(8):
        g = np.exp(rng.uniform(-3, 3, (2, 2))).astype(np.float32)
        if trial == 0:
            g[:] = 1.0          # ties everywhere
        allt = list(itertools.product(range(5), repeat=4))
        for p in range(0, 9):
            counts = O.pooled_plane_counts(g, p)
            total = min(2 * p, 16)
            assert counts.sum() == total
            best = min(err(g, t) for t in allt if sum(t) == total)
            with_counts = min(err(g, t) for t in allt
                              if t[0] + t[1] == counts[0] and t[2] + t[3] == counts[1])
            assert with_counts == best, (g, p, counts)


def test_layer_budgets_sum_and_follow_the_gains():
    """Largest-remainder rounding keeps the total L * P; a layer whose units
    take more planes in the pooled allocations gets the larger budget.
    Hand-worked: 3 layers x 2 units, P = 88, two queries whose pooled counts
    each sum to 528; per-layer means 97.5, 52.5, 114 -> floors 97, 52, 114
    (263), the one plane left goes to the larger remainder, the lower layer
    on the tie between layers 0 and 1."""
    counts = np.array([[[100, 90], [60, 50], [118, 110]],
                       [[110, 90], [50, 50], [108, 120]]])
    assert (counts.sum(axis=(1, 2)) == 528).all()
    assert list(O.calibrate_layer_budgets(counts, 88)) == [98, 52, 114]
    flat = np.full((1, 4, 8), 88)
    assert list(O.calibrate_layer_budgets(flat, 88)) == [88, 88, 88, 88]


# --------------------------------------------------------------------------
# fixed-depth baselines (Fathom §2: SparQ, Double Sparsity, thumbnail scan)
# --------------------------------------------------------------------------

def test_baseline_depths_cost_the_page_bits(rng):
    """The depth vectors of the baselines cost the bits the page prints:
    SparQ r = 16 / 32 at 4 bits 68 / 136, Double Sparsity c = 32 136 bits
    = 17 bytes, the thumbnail (all channels, two planes) 288."""
    g = json.load(open(os.path.join(GOLDEN, "fathom_bit_accounting.json")))
    q = rng.standard_normal((4, 128)).astype(np.float32)
    assert O.scan_bits_per_token(O.sparq_depth(q, g["sparq_68"]["channels"])) == \
        g["sparq_68"]["bits_per_token"]
    assert O.scan_bits_per_token(O.sparq_depth(q, g["scan_136"]["channels"])) == \
        g["scan_136"]["bits_per_token"]
    chans = O.double_sparsity_channels(rng.uniform(0.1, 1, 128), rng.uniform(0.1, 4, 128),
                                       g["label_cache_bytes_per_token"]["channels"])
    t = O.channel_set_depth(chans)
    assert O.scan_bits_per_token(t) == g["scan_136"]["bits_per_token"]
    assert O.scan_bits_per_token(t) / 8 == g["label_cache_bytes_per_token"]["bytes"]
    assert O.scan_bits_per_token(O.uniform_depth(g["thumbnail_288"]["depth"])) == \
        g["thumbnail_288"]["bits_per_token"]


def test_sparq_sums_abs_q_over_the_group():
    """Fathom §2 SparQ: |q| summed over the heads sharing the KV head, not
    q^2 and not per head.  Channel 0: one head at 3 (sum |q| 3, sum q^2 9);
    channel 1: four heads at 1 (sum |q| 4, sum q^2 4); channel 2: -2.5 on two
    heads (5, 12.5).  r = 1 takes channel 2, r = 2 adds channel 1 (a rule on
    q^2 would add channel 0)."""
    q = np.zeros((4, 6), dtype=np.float32)
    q[0, 0] = 3.0
    q[:, 1] = 1.0
    q[1:3, 2] = -2.5
    assert list(O.sparq_depth(q, 1)) == [0, 0, 4, 0, 0, 0]
    assert list(O.sparq_depth(q, 2)) == [0, 4, 4, 0, 0, 0]
    assert list(O.sparq_depth(q, 3)) == [4, 4, 4, 0, 0, 0]
    # equal sums: the lower channel first (channels 3..5 all zero)
    assert list(O.sparq_depth(q, 4)) == [4, 4, 4, 4, 0, 0]
    assert list(O.sparq_depth(q, 9)) == [4] * 6


def test_double_sparsity_ranks_the_product():
    """Fathom §2 Double Sparsity: channels ranked by mean|q| x mean|k|."""
    mq = np.array([1.0, 0.5, 2.0, 0.1, 1.0])
    mk = np.array([1.0, 3.0, 0.4, 9.0, 1.0])
    # products 1, 1.5, 0.8, 0.9, 1: the two largest are channels 1 and 0 (0 before 4)
    assert list(O.double_sparsity_channels(mq, mk, 2)) == [0, 1]
    assert list(O.double_sparsity_channels(mq, mk, 3)) == [0, 1, 4]
    assert list(O.channel_set_depth([0, 4], 5)) == [4, 0, 0, 0, 4]


def test_uniform_full_depth_scan_is_the_4bit_dot(rng):
    """At t = 4 on every channel the scan is the dot with the dequantized
    4-bit keys; at t = 2 each key is its 2-bit quantizer's cell midpoint."""
    k = _blocks(rng, 3, 128, sigma=np.exp(rng.uniform(-2, 1.4, 128)))
    q = rng.standard_normal((4, 128)).astype(np.float32)
    planes, scales = O.encode_unit(k)
    s4, _ = O.scan_scores(q, O.uniform_depth(4), planes, scales, k.shape[0])
    codes = np.stack([O.quantize_codes(k[b * 64:(b + 1) * 64], O.block_scales(k[b * 64:(b + 1) * 64]))
                      for b in range(3)]).reshape(-1, 128).astype(np.float64)
    deq = (codes - 8.0 + 0.5) * np.repeat(scales.T.astype(np.float64), 64, axis=0)
    np.testing.assert_allclose(s4, q.astype(np.float64) @ deq.T, rtol=1e-12, atol=1e-12)
    s2, _ = O.scan_scores(q, O.uniform_depth(2), planes, scales, k.shape[0])
    mid2 = (np.floor(codes / 4) * 4 + 2 - 8) * np.repeat(scales.T.astype(np.float64), 64, axis=0)
    np.testing.assert_allclose(s2, q.astype(np.float64) @ mid2.T, rtol=1e-12, atol=1e-12)


def test_bit_accounting_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "fathom_bit_accounting.json")))
    m = g["model"]
    t = np.zeros(128, dtype=np.int64)
    t[: g["scan_136"]["channels"]] = g["scan_136"]["depth"]
    assert O.scan_bits_per_token(t) == g["scan_136"]["bits_per_token"]
    t2 = np.full(128, g["thumbnail_288"]["depth"])
    assert O.scan_bits_per_token(t2) == g["thumbnail_288"]["bits_per_token"]
    assert O.scan_bits_per_token(t) / 8 == g["label_cache_bytes_per_token"]["bytes"]
    n32 = g["scan_bytes_per_pair_32k"]["tokens"]
    per_pair = O.scan_bytes_unit(t, n32)
    assert round(per_pair / 1000) == g["scan_bytes_per_pair_32k"]["kilobytes"]
    pairs = m["layers"] * m["kv_heads"]
    assert round(per_pair * pairs / 1e6) == g["scan_bytes_per_step_32k"]["megabytes"]
    n1m = g["scan_bytes_per_step_1m"]["tokens"]
    assert round(O.scan_bytes_unit(t, n1m) * pairs / 1e9, 1) == g["scan_bytes_per_step_1m"]["gigabytes"]
    dense = 2 * n32 * m["head_dim"] * 2 * pairs
    assert round(dense / 1e9, 1) == g["dense_kv_bytes_per_step_32k"]["gigabytes"]
    assert m["q_per_kv"] * g["union_rows_per_kv_head_max"]["k"] == g["union_rows_per_kv_head_max"]["rows"]


# --------------------------------------------------------------------------
# value-side depths (ReadKV §5.3, §5.4)
# --------------------------------------------------------------------------

def _value_rows(rng, n, row_scale=None):
    sc = np.ones(n) if row_scale is None else row_scale
    return (rng.standard_normal((n, 128)) * sc[:, None]).astype(np.float32)


def test_value_planes_hand_worked():
    """One row: channel 0 = 4, channel 9 = -4, the rest 0.  The row maximum 4
    gives s = 0.5; codes are floor(v / s) + 8 clipped: channel 0 -> 8 + 8 = 16
    -> 15 (0b1111), channel 9 -> -8 + 8 = 0 (0b0000), zeros -> 8 (0b1000).
    Plane 0 (the top bit) is 1 everywhere but channel 9 (byte 1, bit 1):
    bytes FF FD FF ...; planes 1-3 are 1 only on channel 0: byte 0 = 01."""
    v = np.zeros((1, 128), dtype=np.float32)
    v[0, 0], v[0, 9] = 4.0, -4.0
    planes, scales = O.encode_values(v)
    assert float(scales[0]) == 0.5
    assert list(planes[0, 0, :3]) == [0xFF, 0xFD, 0xFF] and np.all(planes[0, 0, 2:] == 0xFF)
    for p in (1, 2, 3):
        assert planes[0, p, 0] == 0x01 and np.all(planes[0, p, 1:] == 0)


def test_value_plane_bit_layout(rng):
    """Channel j of plane p is bit j % 8 of byte j // 8 and carries bit 3 - p
    of the code, read back here with explicit shifts (no bit packing)."""
    v = _value_rows(rng, 5, np.exp(rng.uniform(-3, 3, 5)))
    planes, scales = O.encode_values(v)
    for i in range(5):
        s = Fraction(float(scales[i]))
        assert s == Fraction(float(np.float16(np.max(np.abs(v[i])) / np.float32(8))))
        for j in range(128):
            code = min(max(math.floor(Fraction(float(v[i, j])) / s), -8), 7) + 8
            for p in range(4):
                bit = (int(planes[i, p, j // 8]) >> (j % 8)) & 1
                assert bit == (code >> (3 - p)) & 1


@pytest.mark.parametrize("t", [0, 1, 2, 3, 4])
def test_value_prefix_is_the_t_bit_quantizer(rng, t):
    """Rebuilding a token from t planes equals quantising its values directly
    with t bits and cell s_i 2^(4-t) (exact rationals)."""
    v = _value_rows(rng, 6, np.exp(rng.uniform(-2, 2, 6)))
    planes, scales = O.encode_values(v)
    rec = O.value_prefix_rows(planes, scales, np.arange(6), [t] * 6)
    for i in range(6):
        s = Fraction(float(scales[i]))
        for j in range(0, 128, 7):
            if t == 0:
                expect = Fraction(0)
            else:
                w = s * 2 ** (4 - t)
                half = 2 ** (t - 1)
                cell = min(max(math.floor(Fraction(float(v[i, j])) / w), -half), half - 1)
                expect = (cell + Fraction(1, 2)) * w
            assert Fraction(rec[i, j]) == expect


def _value_objective(w, t):
    return sum(Fraction(float(wi)) / 4 ** int(ti) for wi, ti in zip(w, t))


def test_value_alloc_brute_force_optimal(rng):
    """ReadKV §5.4: for non-negative diminishing gains the greedy grants are
    optimal for the proxy.  Every depth vector of up to four tokens is tried;
    the allocation must reach the least sum_i w_i 4^-t_i and spend
    min(budget, planes with a positive gain)."""
    import itertools
    for trial in range(40):
        n = int(rng.integers(1, 5))
        a = (rng.uniform(0, 1, n) ** 3).astype(np.float32)
        if trial % 4 == 0:
            a[rng.integers(0, n)] = 0.0
        s = np.float16(np.exp(rng.uniform(-3, 2, n)))
        w = O.value_gains(a, s)
        for budget in range(0, 4 * n + 2):
            t = O.alloc_value_depth(a, s, budget)
            useful = 4 * int(np.count_nonzero(w > 0))
            assert int(t.sum()) == min(budget, useful)
            best = min(_value_objective(w, c) for c in itertools.product(range(5), repeat=n)
                       if sum(c) <= budget)
            assert _value_objective(w, t) == best


def test_value_alloc_literal_greedy_loop(rng):
    """The sort form equals the literal loop: grant the next plane to the token
    whose next plane is worth the most (lower token on ties), stop when the
    budget is spent or nothing is worth more than zero."""
    for trial in range(6):
        n = 40
        a = (rng.uniform(0, 1, n) ** 4).astype(np.float32)
        a[::7] = 0.0
        a[3] = a[5]                         # an exact tie between two tokens
        s = np.float16(np.exp(rng.uniform(-2, 2, n)))
        s[5] = s[3]
        s[11] = 0
        w = O.value_gains(a, s)
        for budget in (0, 1, 17, 60, 200):
            depth = np.zeros(n, dtype=np.int64)
            for _ in range(budget):
                best, best_v = -1, 0.0
                for i in range(n):
                    if depth[i] < 4:
                        val = float(np.float32(w[i] * np.float32(0.25) ** np.float32(depth[i])))
                        if val > best_v:
                            best, best_v = i, val
                if best < 0:
                    break
                depth[best] += 1
            np.testing.assert_array_equal(O.alloc_value_depth(a, s, budget), depth)


def test_value_alloc_equal_gains_round_robin():
    """Equal gains: plane 0 of every token outranks every plane 1, so the
    budget goes round the tokens in order: t_i = B // n + (i < B % n)."""
    n = 7
    a = np.full(n, 0.125, dtype=np.float32)
    s = np.full(n, 2.0, dtype=np.float16)
    for budget in range(0, 4 * n + 3):
        b = min(budget, 4 * n)
        expect = [b // n + (i < b % n) for i in range(n)]
        assert list(O.alloc_value_depth(a, s, budget)) == expect


def test_value_gain_predicts_output_error(rng):
    """ReadKV §5.3/§5.4: with independent per-token rebuild errors, the summed
    squared output error over the heads is sum_i (sum_h p_hi^2) E|e_i|^2, and
    a uniform cell of width 16 s 2^-t gives E|e_i|^2 = D (64/3) s_i^2 4^-t.
    Measured with the encoder on value rows spread over their whole range,
    for scales and depths that differ per token: the ratio of the measured
    error to (64 D / 3) sum_i w_i 4^-t_i must be 1 (a gain that squares no
    probability, drops s^2 or halves per bit fails)."""
    g, n, trials = 4, 12, 300
    logits = rng.standard_normal((g, n)) * 1.5
    p = np.exp(logits) / np.exp(logits).sum(axis=1, keepdims=True)
    a = (p * p).sum(axis=0).astype(np.float32)
    row_scale = np.exp(rng.uniform(-2, 2, n))
    for depth in ([0] * n, [4] * n, list(rng.integers(0, 5, n))):
        err = 0.0
        pred = 0.0
        for _ in range(trials):
            v = (rng.uniform(-1, 1, (n, 128)) * row_scale[:, None]).astype(np.float32)
            planes, scales = O.encode_values(v)
            rec = O.value_prefix_rows(planes, scales, np.arange(n), depth)
            e = v.astype(np.float64) - rec
            err += float(np.sum((p @ e) ** 2))
            w = O.value_gains(a, scales).astype(np.float64)
            pred += 128 * 64 / 3 * float(np.sum(w * 0.25 ** np.asarray(depth, dtype=np.float64)))
        assert abs(err / pred - 1) < 0.06, (depth, err / pred)


def _attend_values_case(rng, g=4, n=300, k=40):
    q = rng.standard_normal((g, 128)).astype(np.float32)
    keys = rng.standard_normal((n, 128)).astype(np.float32)
    vals = _value_rows(rng, n, np.exp(rng.uniform(-1, 1, n)))
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(g)])
    return q, keys, vals, idx


def test_attend_values_full_budget_is_4bit_values(rng):
    """A budget that covers every plane rebuilds every union row at full
    depth, the 4-bit cell midpoints s_i (c - 7.5), so the output is plain
    attention over those rows (computed here by the dense routine)."""
    q, keys, vals, idx = _attend_values_case(rng)
    planes, scales = O.encode_values(vals)
    r = O.attend_values(q, keys, planes, scales, idx, 0.09, 10 ** 6)
    assert np.all(r["depth"] == 4)
    s = scales.astype(np.float64)[:, None]
    codes = np.clip(np.floor(vals.astype(np.float64) / s), -8, 7) + 8
    v4 = s * (codes - 7.5)
    for h in range(q.shape[0]):
        expect = O.attend(q[h:h + 1], keys, v4, idx[h:h + 1], 0.09)
        np.testing.assert_allclose(r["out"][h], expect[0], rtol=1e-12, atol=1e-12)
    assert list(r["union"]) == sorted(set(idx.ravel().tolist()))


def test_attend_values_zero_budget_is_zero(rng):
    q, keys, vals, idx = _attend_values_case(rng)
    planes, scales = O.encode_values(vals)
    r = O.attend_values(q, keys, planes, scales, idx, 0.09, 0)
    assert np.all(r["depth"] == 0) and np.all(r["out"] == 0)


def test_attend_values_error_within_cell_bound(rng):
    """|o_hd - o_exact_hd| <= sum_i p_hi s_i 2^(3 - t_i) (half a cell; the
    depth-0 rebuild errs by at most |v| <= 8 s), whatever the budget."""
    q, keys, vals, idx = _attend_values_case(rng)
    planes, scales = O.encode_values(vals)
    exact = O.attend(q, keys, vals, idx, 0.09)
    for budget in (0, 30, 100, 250, 400):
        r = O.attend_values(q, keys, planes, scales, idx, 0.09, budget)
        s = scales[r["union"]].astype(np.float64)
        bound = r["p"] @ (s * 2.0 ** (3 - r["depth"].astype(np.float64)))
        assert np.all(np.abs(r["out"] - exact) <= bound[:, None] * (1 + 1e-3) + 1e-12)


def test_attend_values_hand_worked_union_weights():
    """Two heads: head 0 selects tokens {0, 1}, head 1 selects {1, 2}, every
    logit equal, so each head puts 1/2 on each of its rows.  The union
    0, 1, 2 has a = (1/4, 1/2, 1/4); all scales are 1 (row maximum 8).
    Plane values: token 1: 1/2, 1/8, ...; tokens 0 and 2: 1/4, 1/16, ...
    Budget 2 -> (1, 1, 0) (the tie goes to the lower token); budget 3 ->
    (1, 1, 1); budget 4 -> (1, 2, 1); budget 5 -> (2, 2, 1)."""
    q = np.zeros((2, 128), dtype=np.float32)
    keys = np.ones((3, 128), dtype=np.float32)
    vals = np.zeros((3, 128), dtype=np.float32)
    vals[:, 0] = 8.0
    idx = np.array([[0, 1], [1, 2]])
    planes, scales = O.encode_values(vals)
    assert np.all(scales == 1.0)
    expect = {2: [1, 1, 0], 3: [1, 1, 1], 4: [1, 2, 1], 5: [2, 2, 1]}
    for budget, dep in expect.items():
        r = O.attend_values(q, keys, planes, scales, idx, 1.0, budget)
        np.testing.assert_allclose(r["a"], [0.25, 0.5, 0.25])
        assert list(r["depth"]) == dep, budget


def test_value_bytes_full_depth():
    """Four planes of 128 bits and a 2-byte scale: 66 bytes against the
    256 bytes of a bf16 row; depth 0 reads nothing."""
    assert O.value_bytes([4]) == 66.0 and O.value_bytes([0, 0]) == 0.0
    assert O.value_bytes([1, 2, 0]) == 16 * 3 + 2 * 2
