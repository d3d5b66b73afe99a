"""Precision of the key scan where its fixed-point frame is weakest, against
the oracle (1e-4 of each score's L1 mass, element by element).

One unit of 2^18 tokens whose channel 0 dominates: every block has one token
at 8 s on channel 0 (which sets the block's scale s) and the others in
[-s, s), i.e. codes 7 and 8 (cell midpoints -1/2 and +1/2), so the score's
L1 mass is little more than |q_h0| s / 2 while every other read row weighs
about 2^-17 of channel 0's top row.  The rounding of those rows' fixed-point
weights is then the whole error budget (Fathom §3.2 prefix decode)."""
import numpy as np
import pytest
import torch

import oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu

N = 1 << 18


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def unit():
    import bit_plane_key_amd as b
    rng = np.random.default_rng(20261203)
    keys = (rng.standard_normal((N, 128)) * 3e-4).astype(np.float32)
    keys[:, 0] = rng.uniform(-16.0, 16.0, N).astype(np.float32)
    keys[5::64, 0] = 128.0                      # the block maximum: s = 16, code 15
    keys[rng.integers(0, N, 32), 0] = -16.0     # exact cell edges (code 7)
    var = np.full(128, 9e-8, dtype=np.float32)
    var[0] = 100.0
    q_bits = (rng.standard_normal((4, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q = O.bf16_bits_to_f32(q_bits)
    v_bits = (rng.standard_normal((N, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    cache = b.Cache(1, 1, 1, N, group=4, k_dtype="f32")
    cache.k_rows[0, 0, 0].copy_(torch.from_numpy(keys))
    cache.v_rows[0, 0, 0].copy_(torch.from_numpy(v_bits.view(np.int16)).view(torch.bfloat16))
    cache.chan_var[0, 0, 0].copy_(torch.from_numpy(var))
    b.encode_append(cache, 0, None, None, N)
    qt = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).reshape(1, 1, 1, 4, 128).cuda()
    torch.cuda.synchronize()
    _say("precision unit built; encoding the oracle's planes")
    planes, scales = O.encode_unit(keys)
    assert np.array_equal(cache.planes[0, 0, 0, :, :, :N // 64].cpu().numpy().view(np.uint64), planes)
    return b, cache, qt, q, var, keys, planes, scales, O.bf16_bits_to_f32(v_bits)


@pytest.mark.parametrize("budget", [88, 128, 300])
def test_dominant_channel_scores(unit, budget):
    b, cache, qt, q, var, keys, planes, scales, v = unit
    depth, qb = b.alloc_depth(cache, qt, 0, 1, budget)
    scores = b.scan_scores(cache, qb, depth, 0, 1)
    torch.cuda.synchronize()
    d = depth[0, 0, 0].cpu().numpy()
    ref_d = O.alloc_depth(q, var, budget)
    assert np.array_equal(d, ref_d) and d[0] == 4
    ref, l1 = O.scan_scores(q, ref_d, planes, scales, N)
    got = scores[0, 0, 0].cpu().numpy().astype(np.float64)
    ratio = np.abs(got - ref) / (P.SCORE_RTOL * l1)
    _say(f"P={budget}: rows {int(d.sum())}, worst error / (1e-4 L1) = {ratio.max():.3g}")
    P.check_scores(got, ref, l1, f"dominant channel, P={budget}")


def test_dominant_channel_decode_step(unit):
    """The fused selection on the same unit: equal to the unfused path, and a
    top-k of the oracle's scores up to near-ties."""
    b, cache, qt, q, var, keys, planes, scales, v = unit
    k = 512
    idx = torch.empty((1, 1, 1, 4, k), dtype=torch.int32, device="cuda")
    b.decode_step(cache, qt, 0, 1, 88, k, 0.088, idx_out=idx)
    depth, qb = b.alloc_depth(cache, qt, 0, 1, 88)
    idx2 = b.select_topk(cache, b.scan_scores(cache, qb, depth, 0, 1), 0, 1, k)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    ref, l1 = O.scan_scores(q, O.alloc_depth(q, var, 88), planes, scales, N)
    ref_idx = O.select_topk(ref, N, k)
    P.check_selection(idx[0, 0, 0].cpu().numpy(), ref_idx, ref, l1, N, k, "dominant channel step")
