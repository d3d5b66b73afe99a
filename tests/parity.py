"""Helpers of the GPU parity tests: host regeneration of a unit's inputs, the
oracle on them, and the comparison rules (bars stated with each function)."""
from __future__ import annotations

import numpy as np

import oracle as O
from synth import Config
from synth import workload as W

SCORE_RTOL = 1e-4   # |gpu - oracle| <= 1e-4 * sum_j |q_hj s_bj m_ij|
ATT_RTOL = 2e-3     # ||gpu - oracle||_inf <= 2e-3 * ||oracle||_inf per head


def unit_inputs(cfg: Config, s: int, l: int, h: int, n: int, rows=None, step: int = 0):
    """Host copies (float32 values) of one unit: K rows, V rows, q, chan_var."""
    rows = np.arange(n) if rows is None else np.asarray(rows)
    k_bits, k = W.key_rows(cfg, s, l, h, rows)
    v_bits, v = W.value_rows(cfg, s, l, h, rows)
    q_bits, q = W.query(cfg, s, l, h, step)
    return dict(k=k, k_bits=k_bits, v=v, v_bits=v_bits, q=q, q_bits=q_bits,
                var=cfg.chan_var(s, l, h),
                rot=cfg.rotation(l, h) if cfg.rotated else None)


def oracle_encode(inp, n):
    keys = inp["k"][:n] if inp["rot"] is None else O.rotate_basis(inp["rot"], inp["k"][:n])
    return O.encode_unit(keys)


def check_scores(gpu, ref, l1, where=""):
    err = np.abs(gpu.astype(np.float64) - ref)
    bound = SCORE_RTOL * l1 + 1e-30
    bad = err > bound
    assert not bad.any(), (f"{where}: {bad.sum()} scores off; worst ratio "
                           f"{(err / bound).max():.3g}")


def check_selection(gpu_idx, ref_idx, ref_scores, ref_l1, n, k, where=""):
    """Sets equal, except swaps among keys whose oracle score lies within
    1e-4 (of the score's own L1 scale) of the threshold score."""
    for h in range(gpu_idx.shape[0]):
        g = set(int(i) for i in gpu_idx[h] if i >= 0)
        r = set(int(i) for i in ref_idx[h] if i >= 0)
        assert len(g) == len(r) == min(n, k), where
        diff = g ^ r
        if not diff:
            continue
        w = O.kept_tail(n)
        fixed = set(range(4)) | set(range(n - w, n))
        assert not (diff & fixed), f"{where}: always-kept token missing"
        chosen = sorted(r - fixed, key=lambda i: (-ref_scores[h, i], i))
        tau = ref_scores[h, chosen[-1]]
        for i in diff:
            tol = SCORE_RTOL * max(ref_l1[h, i], abs(tau)) + 1e-30
            assert abs(ref_scores[h, i] - tau) <= tol, (
                f"{where}: head {h} token {i} swapped but {ref_scores[h, i]} vs {tau}")


def check_topk_valid(scores, idx, n, k, where=""):
    """idx is a correct top-k of `scores` under the selection rule (exact)."""
    for h in range(idx.shape[0]):
        sel = idx[h][idx[h] >= 0]
        assert list(sel) == sorted(sel), where
        if n <= k:
            assert np.array_equal(sel, np.arange(n)), where
            continue
        w = O.kept_tail(n)
        assert len(sel) == k
        mask = np.zeros(n, dtype=bool)
        mask[sel] = True
        assert mask[:4].all() and mask[n - w:].all(), where
        cand = np.arange(4, n - w)
        ins, outs = cand[mask[cand]], cand[~mask[cand]]
        if len(ins) == 0 or len(outs) == 0:
            continue
        s = scores[h].astype(np.float64)
        worst_in = s[ins].min()
        best_out = s[outs].max()
        assert worst_in >= best_out, f"{where}: head {h} {worst_in} < {best_out}"
        if worst_in == best_out:
            tie_in = ins[s[ins] == worst_in]
            tie_out = outs[s[outs] == worst_in]
            assert tie_in.max() < tie_out.min(), f"{where}: tie not broken by index"


def check_attention(gpu, ref, where=""):
    for h in range(ref.shape[0]):
        scale = np.abs(ref[h]).max()
        err = np.abs(gpu[h].astype(np.float64) - ref[h]).max()
        assert err <= ATT_RTOL * scale + 1e-30, f"{where}: head {h} err {err} vs {scale}"
