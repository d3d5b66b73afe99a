"""CPU oracle: top-k sparse decode attention over a bit-plane 4-bit key cache.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the
HIP library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or run it; the product
path never does.  It shares no code, header, table or helper with the HIP
library and does not import it.

Sources (cited by section; no sentence of them is reproduced):

* [Fathom] the page "Fathom：针对卸载KV缓存的稀疏解码逐查询读取深度", a
  translation of arXiv 2609.17652 -- §1 (observations 1 and 2), §2 ("Top-k
  decoding", "SparQ"), §3.1 (cost model, Eq. 1), §3.2 (bit-plane K cache).
  The extraction stops inside §3.2, so the plane word layout and the
  prefix-decode formula take the plainest reading: plane p holds bit 3 - p
  of each offset code (the top bit first), and a t-bit prefix decodes to its
  cell midpoint (see ``prefix_values``).
* [ReadKV] the page "AI存储论文解读:ReadKV：KV 存得更细、每步少读..." --
  §5.2 (key-channel importance summed over the query heads that share a KV
  head), §5.3 (value depth per token from the heads' squared attention
  probabilities), §5.4 (greedy allocation by largest predicted error drop),
  §6.1 (append-only planes).

Every floating-point decision that produces an integer (a code, a depth) is
taken here in the precision the GPU takes it: codes from the exact real floor
of k / s with s the stored fp16 scale, depths from fp32 gains compared
exactly.  Everything else (scores, attention) is fp64.

Parity pins: every function below is pinned by a ``-m "not gpu"`` test
(tests/test_oracle_pins.py) against closed forms, brute force or a library
routine; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

D = 128          # channels per KV head (head dimension)
BLOCK = 64       # tokens per quantisation block [Fathom §3.2]
PLANES = 4       # bits per code [Fathom §3.2]
FIRST_KEPT = 4   # always-kept leading tokens [Fathom §2, Top-k decoding]
LAST_KEPT = 32   # always-kept trailing tokens [Fathom §2, Top-k decoding]
FP16_MAX = 65504.0

__all__ = [
    "D", "BLOCK", "PLANES", "FIRST_KEPT", "LAST_KEPT",
    "bf16_bits_to_f32", "block_scales", "quantize_codes", "encode_unit",
    "codes_from_planes", "prefix_values", "channel_gains", "alloc_depth",
    "alloc_depth_greedy", "pooled_plane_counts", "calibrate_layer_budgets", "sparq_depth", "double_sparsity_channels", "channel_set_depth",
    "uniform_depth", "scan_scores", "kept_tail", "select_topk",
    "attend", "dense_attention", "rotate_basis", "decode_unit",
    "scan_bits_per_token", "scan_bytes_unit", "encode_values", "value_prefix_rows",
    "value_gains", "alloc_value_depth", "attend_values", "value_bytes",
]


# ----------------------------------------------------------------------------
# storage format
# ----------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to the float32 values they denote."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def block_scales(k_block: np.ndarray) -> np.ndarray:
    """fp16 scale of each channel of one 64-token block.

    [Fathom §3.2] the block maximum a = max_i |k_ij| gives the cell width
    s = a / 8, stored as one fp16 number per (block, channel).  a / 8 is exact
    in fp32; the fp16 rounding is round-to-nearest-even and values beyond the
    fp16 range saturate to 65504 (reading: a saturating store).
    """
    amax = np.max(np.abs(k_block.astype(np.float32)), axis=0)
    with np.errstate(over="ignore"):
        s = (amax / np.float32(8.0)).astype(np.float16)
    s[np.isinf(s)] = np.float16(FP16_MAX)
    return s


def quantize_codes(k_block: np.ndarray, s: np.ndarray) -> np.ndarray:
    """4-bit codes c = clip(floor(k / s), -8, 7) + 8 of one block.

    [Fathom §3.2] symmetric uniform code, code 8 is zero and the top bit is
    the sign.  The floor is the exact real floor of k / s (s = the stored fp16
    scale): the fp64 quotient is corrected with the exact products m*s.  A
    zero scale gives code 8 for every token.
    """
    k = k_block.astype(np.float64)
    sc = s.astype(np.float64)[None, :]
    safe = np.where(sc == 0.0, 1.0, sc)
    m = np.floor(k / safe)
    m = m - (m * safe > k)
    m = m + ((m + 1.0) * safe <= k)
    c = np.clip(m, -8, 7) + 8
    c = np.where(sc == 0.0, 8, c)
    return c.astype(np.uint8)


def encode_unit(keys: np.ndarray):
    """Bit planes and scales of every complete 64-token block of one unit.

    ``keys`` is (n, D) float32 (values of the stored key rows, or of the
    rotated keys).  Returns ``planes`` uint64 [D][4][nb] and ``scales``
    float16 [D][nb] with nb = n // 64: the open trailing block has no planes
    yet (append-only planes, [ReadKV §6.1]).

    [Fathom §3.2] for block b, channel j and bit p (p = 0 the most
    significant bit), the 64 codes' bit p forms one 64-bit word; bit i of the
    word belongs to token 64 b + i.  Words are stored channel-major.
    """
    n = keys.shape[0]
    nb = n // BLOCK
    blocks = keys[: nb * BLOCK].reshape(nb, BLOCK, keys.shape[1])
    planes = np.zeros((keys.shape[1], PLANES, nb), dtype=np.uint64)
    scales = np.zeros((keys.shape[1], nb), dtype=np.float16)
    weights = np.uint64(1) << np.arange(BLOCK, dtype=np.uint64)
    for b in range(nb):
        s = block_scales(blocks[b])
        c = quantize_codes(blocks[b], s)                 # (64, D)
        scales[:, b] = s
        for p in range(PLANES):
            bit = ((c >> (PLANES - 1 - p)) & 1).astype(np.uint64)   # (64, D)
            planes[:, p, b] = (bit * weights[:, None]).sum(axis=0, dtype=np.uint64)
    return planes, scales


def codes_from_planes(planes: np.ndarray, t: int, j: int, blocks: np.ndarray) -> np.ndarray:
    """The t-bit prefix code of channel j for every token of ``blocks``.

    Reads only planes p < t of channel j.  Returns an int64 array of shape
    (len(blocks) * 64,) in token order.
    """
    out = np.zeros(len(blocks) * BLOCK, dtype=np.int64)
    shifts = np.arange(BLOCK, dtype=np.uint64)
    for p in range(t):
        words = planes[j, p, blocks]
        bits = ((words[:, None] >> shifts[None, :]) & np.uint64(1)).astype(np.int64)
        out = out * 2 + bits.reshape(-1)
    return out


def prefix_values(prefix: np.ndarray, t: int) -> np.ndarray:
    """Cell midpoint, in units of s, of a t-bit prefix code.

    [Fathom §1 observation 2] the first t planes are the channel's t-bit
    mid-rise quantizer with the same block scale: the prefix names a cell of
    2^(4-t) consecutive codes whose midpoint is
    (prefix + 1/2) * 2^(4-t) - 8.  Depth 0 reads nothing and reconstructs 0.
    """
    if t == 0:
        return np.zeros(prefix.shape, dtype=np.float64)
    return (prefix.astype(np.float64) + 0.5) * 2.0 ** (PLANES - t) - 8.0


# ----------------------------------------------------------------------------
# per-query depth allocation
# ----------------------------------------------------------------------------

def channel_gains(q_basis: np.ndarray, chan_var: np.ndarray) -> np.ndarray:
    """g_j = var_j * sum_h q_hj^2 in fp32, h ascending, one rounding per op.

    [Fathom §1 observation 1] g_j is channel j's share of this query's score
    variance; [ReadKV §5.2] the importance of a key channel sums the squared
    query components of every query head sharing the KV head.
    """
    q = np.asarray(q_basis, dtype=np.float32)
    acc = np.zeros(q.shape[1], dtype=np.float32)
    for h in range(q.shape[0]):
        acc = (acc + q[h] * q[h]).astype(np.float32)
    return (np.asarray(chan_var, dtype=np.float32) * acc).astype(np.float32)


def alloc_depth(q_basis: np.ndarray, chan_var: np.ndarray, budget: int) -> np.ndarray:
    """Depths t_j by reverse water-filling of ``budget`` planes (sort form).

    [Fathom §1 observation 1, §3] the t-th plane of channel j is worth
    g_j * 4^-t (each extra bit cuts the quantisation error by 4).  The budget
    goes to the min(budget, 4 D) most valuable (channel, plane) candidates;
    equal values go to the lower channel, then the lower plane.
    """
    g = channel_gains(q_basis, chan_var)
    nd = g.shape[0]
    take = min(max(int(budget), 0), PLANES * nd)
    j = np.repeat(np.arange(nd), PLANES)
    t = np.tile(np.arange(PLANES), nd)
    v = (g[j] * np.float32(0.25) ** t.astype(np.float32)).astype(np.float32)
    order = np.lexsort((t, j, -v.astype(np.float64)))
    depth = np.zeros(nd, dtype=np.int64)
    np.add.at(depth, j[order[:take]], 1)
    return depth.astype(np.uint8)


def alloc_depth_greedy(q_basis: np.ndarray, chan_var: np.ndarray, budget: int) -> np.ndarray:
    """The same depths as the literal greedy loop.

    [ReadKV §5.4] repeatedly give the next bit to the channel whose next
    plane is worth the most (g_j * 4^-t_j), lower channel on ties, until the
    budget is spent.
    """
    g = channel_gains(q_basis, chan_var)
    nd = g.shape[0]
    depth = np.zeros(nd, dtype=np.int64)
    for _ in range(min(max(int(budget), 0), PLANES * nd)):
        best, best_v = -1, -1.0
        for jj in range(nd):
            if depth[jj] < PLANES:
                val = float(np.float32(g[jj] * np.float32(0.25) ** np.float32(depth[jj])))
                if val > best_v:
                    best, best_v = jj, val
        depth[best] += 1
    return depth.astype(np.uint8)


# ----------------------------------------------------------------------------
# per-layer budget calibration
# ----------------------------------------------------------------------------

def pooled_plane_counts(gains: np.ndarray, budget: int) -> np.ndarray:
    """Planes each unit receives when the whole budget of units * budget
    planes is water-filled across units at once.

    [Fathom §3, per-layer budget calibration; the rule itself is not on the
    page] Reading: the value of a unit's t-th plane of channel j is
    g_uj * 4^-t as within one unit (Fathom §1 observation 1), and the pooled
    budget goes to the most valuable (unit, channel, plane) candidates, equal
    values to the lower unit, then channel, then plane.  ``gains`` is
    float32 [units][D]; returns int64 [units].
    """
    g = np.asarray(gains, dtype=np.float32)
    nu, nd = g.shape
    take = min(max(int(budget), 0) * nu, PLANES * nd * nu)
    u = np.repeat(np.arange(nu), nd * PLANES)
    j = np.tile(np.repeat(np.arange(nd), PLANES), nu)
    t = np.tile(np.arange(PLANES), nd * nu)
    v = (g[u, j] * np.float32(0.25) ** t.astype(np.float32)).astype(np.float32)
    order = np.lexsort((t, j, u, -v.astype(np.float64)))
    counts = np.zeros(nu, dtype=np.int64)
    np.add.at(counts, u[order[:take]], 1)
    return counts


def calibrate_layer_budgets(plane_counts: np.ndarray, budget: int) -> np.ndarray:
    """Per-layer plane budgets from pooled allocations of calibration queries.

    ``plane_counts`` is [queries][layers][units per layer] (the pooled
    allocation of each calibration query, pooled over every unit of every
    layer).  Reading: a layer's budget is the mean count of its units over
    the queries, rounded by largest remainder (ties to the lower layer) so
    that the budgets sum to layers * budget, the total a uniform budget
    spends.
    """
    c = np.asarray(plane_counts, dtype=np.int64)
    nl = c.shape[1]
    per = c.sum(axis=(0, 2))                       # planes of each layer, all queries
    denom = c.shape[0] * c.shape[2]
    base = per // denom
    rem = per - base * denom
    short = max(nl * int(budget) - int(base.sum()), 0)
    order = np.lexsort((np.arange(nl), -rem))
    out = base.copy()
    out[order[:short]] += 1
    return out


# ----------------------------------------------------------------------------
# fixed-depth baselines on the same planes
# ----------------------------------------------------------------------------

def sparq_depth(q_basis: np.ndarray, r: int) -> np.ndarray:
    """SparQ's channel choice as a depth vector: depth 4 on r channels, 0 elsewhere.

    [Fathom §2, SparQ] each query picks the r channels of largest |q_j|; under
    grouped-query attention the public rule first sums |q| over the query
    heads that share the KV head, so one set of r channels is read per KV
    head, at full (4-bit) depth.  Reading: the sum runs in fp32, heads in
    ascending order; equal sums go to the lower channel index.
    """
    q = np.asarray(q_basis, dtype=np.float32)
    acc = np.zeros(q.shape[1], dtype=np.float32)
    for h in range(q.shape[0]):
        acc = (acc + np.abs(q[h])).astype(np.float32)
    nd = q.shape[1]
    take = min(max(int(r), 0), nd)
    order = np.lexsort((np.arange(nd), -acc.astype(np.float64)))
    depth = np.zeros(nd, dtype=np.uint8)
    depth[order[:take]] = PLANES
    return depth


def double_sparsity_channels(mean_abs_q: np.ndarray, mean_abs_k: np.ndarray, c: int) -> np.ndarray:
    """Double Sparsity's static channel set of one KV head, ascending.

    [Fathom §2, Double Sparsity] c channels chosen offline per head from
    calibration statistics: the product of the mean |q| and the mean |k| of
    each channel.  Reading: the c largest products (fp64), equal products to
    the lower channel index.
    """
    score = np.asarray(mean_abs_q, dtype=np.float64) * np.asarray(mean_abs_k, dtype=np.float64)
    nd = score.shape[0]
    order = np.lexsort((np.arange(nd), -score))
    return np.sort(order[: min(max(int(c), 0), nd)])


def channel_set_depth(channels, nd: int = D) -> np.ndarray:
    """Depth 4 on the given channels (Double Sparsity reads its c channels at
    4 bits [Fathom §2]), 0 elsewhere."""
    depth = np.zeros(nd, dtype=np.uint8)
    depth[np.asarray(channels, dtype=np.int64)] = PLANES
    return depth


def uniform_depth(t: int, nd: int = D) -> np.ndarray:
    """Every channel at depth t; t = 2 is the 2-bit thumbnail scan, which
    reads the top two planes of all channels [Fathom §2, thumbnail scan]."""
    return np.full(nd, min(max(int(t), 0), PLANES), dtype=np.uint8)


# ----------------------------------------------------------------------------
# key scan
# ----------------------------------------------------------------------------

def scan_scores(q_basis: np.ndarray, depth: np.ndarray, planes: np.ndarray,
                scales: np.ndarray, n: int, chunk_blocks: int = 2048):
    """Approximate scores of every key of the complete blocks, in fp64.

    [Fathom §1, §3.2] each key is reconstructed from the first t_j planes of
    every channel (the block's fp16 scale times the prefix cell midpoint) and
    dotted with the query: s_hat[h, i] = sum_j q_hj * s_bj * m_ij.
    Returns ``(scores, l1)`` of shape (G, nb * 64): ``l1`` is
    sum_j |q_hj * s_bj * m_ij|, the scale of the rounding tolerance.
    """
    q = np.asarray(q_basis, dtype=np.float64)
    nb = n // BLOCK
    scores = np.zeros((q.shape[0], nb * BLOCK), dtype=np.float64)
    l1 = np.zeros_like(scores)
    for b0 in range(0, nb, chunk_blocks):
        blocks = np.arange(b0, min(nb, b0 + chunk_blocks))
        vals = np.zeros((len(blocks) * BLOCK, q.shape[1]), dtype=np.float64)
        for j in range(q.shape[1]):
            t = int(depth[j])
            if t == 0:
                continue
            m = prefix_values(codes_from_planes(planes, t, j, blocks), t)
            s = np.repeat(scales[j, blocks].astype(np.float64), BLOCK)
            vals[:, j] = s * m
        sl = slice(b0 * BLOCK, (b0 + len(blocks)) * BLOCK)
        scores[:, sl] = q @ vals.T
        l1[:, sl] = np.abs(q) @ np.abs(vals).T
    return scores, l1


# ----------------------------------------------------------------------------
# top-k selection
# ----------------------------------------------------------------------------

def kept_tail(n: int) -> int:
    """Number of always-kept trailing tokens.

    [Fathom §2] the last 32 tokens are always kept.  Reading for an open
    trailing block (n not a multiple of 64): its tokens have no planes yet,
    so all of them are kept too -- W = max(32, n mod 64).
    """
    return max(LAST_KEPT, n % BLOCK)


def select_topk(scores: np.ndarray, n: int, k: int) -> np.ndarray:
    """Per query head: always-kept tokens plus the best remaining scores.

    [Fathom §2, Top-k decoding] the first 4 and the last W tokens are always
    kept; the other k - 4 - W are the highest-scoring keys, chosen for each
    query head on its own (no group summing).  Equal scores go to the lower
    token index.  If n <= k every token is kept.  Output: int64 array
    (G, min(n, k)), ascending.
    """
    g = scores.shape[0]
    if n <= k:
        return np.tile(np.arange(n, dtype=np.int64), (g, 1))
    w = kept_tail(n)
    fixed = np.concatenate([np.arange(FIRST_KEPT), np.arange(n - w, n)])
    rest = k - len(fixed)
    if rest < 0 or n - w < FIRST_KEPT:
        raise ValueError("k does not cover the always-kept tokens")
    cand = np.arange(FIRST_KEPT, n - w)
    out = np.zeros((g, k), dtype=np.int64)
    for h in range(g):
        order = np.lexsort((cand, -scores[h, cand]))
        out[h] = np.sort(np.concatenate([fixed, cand[order[:rest]]]))
    return out


# ----------------------------------------------------------------------------
# exact attention over the selected keys
# ----------------------------------------------------------------------------

def attend(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, idx: np.ndarray,
           scale: float) -> np.ndarray:
    """Softmax attention of each query head over its own selected rows, fp64.

    [Fathom §2] methods are judged by exact attention restricted to their
    selected set: softmax(q K^T * scale) over S_h, then the weighted sum of
    the V rows.  ``idx`` entries < 0 are padding and ignored; a head with no
    selected row (an empty sequence) outputs zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros((q.shape[0], v_rows.shape[1]), dtype=np.float64)
    for h in range(q.shape[0]):
        sel = idx[h][idx[h] >= 0]
        if len(sel) == 0:
            continue
        logits = (k_rows[sel].astype(np.float64) @ q[h]) * scale
        p = np.exp(logits - logits.max())
        p /= p.sum()
        out[h] = p @ v_rows[sel].astype(np.float64)
    return out


def dense_attention(q, k_rows, v_rows, scale):
    """Full softmax attention over every row (the k = n special case)."""
    n = k_rows.shape[0]
    idx = np.tile(np.arange(n), (np.asarray(q).shape[0], 1))
    return attend(q, k_rows, v_rows, idx, scale)


# ----------------------------------------------------------------------------
# rotated (KLT) basis
# ----------------------------------------------------------------------------

def rotate_basis(rot: np.ndarray, x: np.ndarray) -> np.ndarray:
    """z = R^T x for every row of x, fp64 running sum in d order, then fp32.

    [Fathom §1 contributions] models without QK normalisation are scanned in
    a KLT basis.  Reading: the encoder and the query both use z = R^T x with
    the per-(layer, head) orthogonal R; each product of two fp32/bf16 values
    is exact in fp64 and is added in channel order d = 0 .. D-1.
    """
    r = np.asarray(rot, dtype=np.float64)
    xx = np.asarray(x, dtype=np.float64)
    acc = np.zeros((xx.shape[0], r.shape[1]), dtype=np.float64)
    for d in range(r.shape[0]):
        acc = acc + xx[:, d:d + 1] * r[d:d + 1, :]
    return acc.astype(np.float32)


# ----------------------------------------------------------------------------
# one decode step of one (sequence, layer, KV head) unit
# ----------------------------------------------------------------------------

def decode_unit(q: np.ndarray, chan_var: np.ndarray, k_rows: np.ndarray,
                v_rows: np.ndarray, n: int, budget: int, k: int, scale: float,
                rot: np.ndarray | None = None, planes=None, scales=None):
    """encode -> allocate -> scan -> select -> attend for one unit.

    ``q`` (G, D) float32 (bf16 values), ``k_rows`` / ``v_rows`` (n, D)
    float32 values of the stored rows.  Returns a dict of every stage.
    """
    enc_in = k_rows[:n] if rot is None else rotate_basis(rot, k_rows[:n])
    if planes is None:
        planes, scales = encode_unit(enc_in)
    qb = np.asarray(q, dtype=np.float32) if rot is None else rotate_basis(rot, q)
    depth = alloc_depth(qb, chan_var, budget)
    scores, l1 = scan_scores(qb, depth, planes, scales, n)
    full = np.zeros((qb.shape[0], n), dtype=np.float64)
    full[:, : scores.shape[1]] = scores
    idx = select_topk(full, n, k)
    out = attend(q, k_rows, v_rows, idx, scale)
    return dict(planes=planes, scales=scales, q_basis=qb, depth=depth,
                scores=scores, l1=l1, idx=idx, out=out)


# ----------------------------------------------------------------------------
# byte accounting
# ----------------------------------------------------------------------------

def scan_bits_per_token(depth: np.ndarray) -> float:
    """Bits one key costs the scan at depths t.

    [Fathom §1, §2] counts are per token, per KV head, per layer; a fp16
    scale per 64-token block costs 16 / 64 = 0.25 bit for every channel that
    is read at all.
    """
    t = np.asarray(depth, dtype=np.int64)
    return float(t.sum()) + 0.25 * float((t > 0).sum())


def scan_bytes_unit(depth: np.ndarray, n: int) -> float:
    """Algorithmic bytes of one unit's scan over n tokens: planes + scales."""
    t = np.asarray(depth, dtype=np.int64)
    nb = n // BLOCK
    return float(t.sum()) * nb * 8.0 + float((t > 0).sum()) * nb * 2.0


# ----------------------------------------------------------------------------
# value-side depths (ReadKV stage 2)
# ----------------------------------------------------------------------------

def encode_values(v_rows: np.ndarray):
    """Per-token value planes and scales.

    [ReadKV §5.3] value precision is chosen per token, every channel of a
    token sharing one depth; [ReadKV §6.1] new tokens are appended as
    progressive planes.  Reading on this storage: each value row is coded
    like a key block turned on its side -- one fp16 scale per token,
    s_i = fp16_rne(max_j |v_ij| / 8) (saturating), and the same symmetric
    4-bit code c_ij = clip(floor(v_ij / s_i), -8, 7) + 8 with the exact floor.
    Plane p of a token holds bit 3 - p of its 128 codes: channel j is bit
    j % 8 of byte j // 8.  Every token is coded as soon as it arrives (no
    block to wait for).  Returns ``planes`` uint8 [n][4][D / 8] and
    ``scales`` float16 [n].
    """
    v = np.asarray(v_rows, dtype=np.float32)
    s = block_scales(v.T)                      # the row maxima
    c = quantize_codes(v.T, s).T               # [n][D]
    planes = np.zeros((v.shape[0], PLANES, v.shape[1] // 8), dtype=np.uint8)
    for p in range(PLANES):
        bit = ((c >> (PLANES - 1 - p)) & 1).astype(np.uint8)
        planes[:, p, :] = np.packbits(bit, axis=1, bitorder="little")
    return planes, s


def value_prefix_rows(vplanes: np.ndarray, vscales: np.ndarray, rows, depth) -> np.ndarray:
    """Value rows rebuilt from the first t_i planes of each token, fp64.

    The t-plane prefix of a code is its t-bit quantizer cell, rebuilt at the
    cell midpoint (as for keys, Fathom §1 observation 2) times the token's
    scale; depth 0 reads nothing and rebuilds 0, the mean of the symmetric
    code.  Returns [len(rows)][D].
    """
    nd = vplanes.shape[2] * 8
    out = np.zeros((len(rows), nd), dtype=np.float64)
    for r, (i, t) in enumerate(zip(rows, depth)):
        t = int(t)
        if t == 0:
            continue
        pre = np.zeros(nd, dtype=np.int64)
        for p in range(t):
            pre = pre * 2 + np.unpackbits(vplanes[i, p], bitorder="little").astype(np.int64)
        out[r] = float(vscales[i]) * prefix_values(pre, t)
    return out


def value_gains(weights: np.ndarray, vscales: np.ndarray) -> np.ndarray:
    """w_i = a_i * s_i^2 in fp32 (s_i^2 is exact, one rounding for the product).

    [ReadKV §5.3, §5.4] a_i is token i's importance, the sum over the query
    heads sharing the KV head of its squared attention probabilities (every
    head weighted 1).  The predicted error of rebuilding the token from t
    planes is proportional to s_i^2 4^-t (the uniform cell of width
    16 s_i 2^-t has mean squared error (16 s_i 2^-t)^2 / 12 per channel, and
    the depth-0 rebuild of a value spread over the whole range errs by the
    same formula at t = 0).  Reading: the token's own scale is the
    standardised unit of this storage, so it enters the gain squared.
    """
    s = np.asarray(vscales, dtype=np.float16).astype(np.float32)
    return (np.asarray(weights, dtype=np.float32) * (s * s)).astype(np.float32)


def _fill_rows(w: np.ndarray, budget: int) -> np.ndarray:
    """Token depths from gains w (fp32 or fp64, values in that precision)."""
    n = w.shape[0]
    i = np.repeat(np.arange(n), PLANES)
    t = np.tile(np.arange(PLANES), n)
    v = (w[i] * w.dtype.type(0.25) ** t.astype(w.dtype)).astype(w.dtype)
    order = np.lexsort((t, i, -v.astype(np.float64)))
    order = order[v[order] > 0]                # no plane without a positive gain
    take = order[: max(int(budget), 0)]
    depth = np.zeros(n, dtype=np.int64)
    np.add.at(depth, i[take], 1)
    return depth.astype(np.uint8)


def alloc_value_depth(weights: np.ndarray, vscales: np.ndarray, budget: int) -> np.ndarray:
    """Per-token value depths from importances a_i (fp32) and scales s_i.

    [ReadKV §5.4] the greedy allocator grants one plane at a time to the
    object whose next plane lowers the predicted error the most, until the
    budget is spent or no grant helps.  The next plane of token i at depth t
    lowers a_i s_i^2 4^-t by 3/4 of itself, so the grants are the candidates
    (i, t) of largest value w_i 4^-t (fp32), taken in value order while the
    value is positive; equal values go to the lower token, then the lower
    plane.  Rows are in token order.  Returns uint8 depths.
    """
    return _fill_rows(value_gains(weights, vscales), budget)


def attend_values(q: np.ndarray, k_rows: np.ndarray, vplanes: np.ndarray,
                  vscales: np.ndarray, idx: np.ndarray, scale: float, v_budget: int):
    """Attention over each head's selected rows with value rows read at
    per-token depths, fp64.

    [Fathom §2] each head's softmax is over its own selected set, from exact
    keys; [ReadKV §5.3] the probabilities then fix the value depths: the rows
    of the union of the heads' sets (token order) get importances
    a_i = sum_h p_hi^2 (p_hi = 0 for a head that did not select i), the
    budget of v_budget planes is allocated as in alloc_value_depth (values
    w_i 4^-t in fp64 here), and o_h = sum_i p_hi v_hat_i with v_hat_i the
    t_i-plane rebuild.  ``idx`` entries < 0 are padding.
    Returns a dict with out [G][D], union rows, depth, p [G][union], a.
    """
    q64 = np.asarray(q, dtype=np.float64)
    g = q64.shape[0]
    sel = [idx[h][idx[h] >= 0] for h in range(g)]
    union = np.unique(np.concatenate(sel)) if g else np.zeros(0, dtype=np.int64)
    union = union.astype(np.int64)
    pos = {int(tok): r for r, tok in enumerate(union)}
    p = np.zeros((g, len(union)), dtype=np.float64)
    for h in range(g):
        if len(sel[h]) == 0:
            continue
        logits = (k_rows[sel[h]].astype(np.float64) @ q64[h]) * scale
        e = np.exp(logits - logits.max())
        for tok, val in zip(sel[h], e / e.sum()):
            p[h, pos[int(tok)]] = val
    a = (p * p).sum(axis=0)
    s = np.asarray(vscales, dtype=np.float16)[union].astype(np.float64)
    depth = _fill_rows(a * s * s, v_budget)
    vhat = value_prefix_rows(vplanes, vscales, union, depth)
    out = p @ vhat if len(union) else np.zeros((g, vplanes.shape[2] * 8))
    return dict(out=out, union=union, depth=depth, p=p, a=a)


def value_bytes(depth: np.ndarray) -> float:
    """Algorithmic bytes of reading value rows at depths t_i: 16 bytes per
    plane (128 channels) plus the 2-byte scale of every row read at all."""
    t = np.asarray(depth, dtype=np.int64)
    return float(t.sum()) * 16.0 + float((t > 0).sum()) * 2.0
