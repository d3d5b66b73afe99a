/*
 * bpk.h -- C ABI of the MI355X (gfx950) bit-plane key-cache decode library.
 *
 * Top-k sparse decode attention over a 4-bit key cache stored as bit planes:
 * a query chooses how many planes of each key channel to read (reverse
 * water-filling of a plane budget), scans every key at those depths to rank
 * it, and runs exact softmax attention only over each query head's winners.
 *
 * Sources (the Fathom page, a translation of arXiv 2609.17652, and the
 * ReadKV explainer page), cited per entry point below by section.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer is a DEVICE pointer owned by the caller, except where marked
 *   HOST.  The library allocates nothing, keeps no state between calls and
 *   never synchronises the host; every call is enqueued on `stream`
 *   (a hipStream_t passed as void*, NULL = the null stream).  Outputs are valid
 *   once the stream has reached the call.
 * - A *unit* is one (sequence s, layer l, KV head h).  Cache arrays (rows,
 *   planes, scales, chan_var) cover every unit: [S][L][H]..., unit index
 *   (s * L + l) * H + h.  Entry points that take a layer range [l0, l1) work
 *   on the units of every sequence and of those layers, and their per-call
 *   arrays (q, q_basis, depth, scores, idx, out) cover only those:
 *   [S][l1 - l0][H]..., unit index (s * (l1 - l0) + (l - l0)) * H + h.
 * - Return value: BPK_OK (0) or a negative BPK_E* code.  All arguments are
 *   validated before anything is enqueued, so a call that fails with
 *   BPK_EINVAL / BPK_EUNSUPPORTED / BPK_EWORKSPACE / BPK_ECAPACITY has no
 *   effect.  bpk_last_error() returns a thread-local message for the last
 *   failing call of the calling thread.  No C++ exception crosses the ABI.
 * - Supported shapes: head_dim == 128, group (query heads per KV head) in
 *   {1, 2, 4, 8}, 1 <= num_seqs <= 64, capacity a positive multiple of 64.
 */
#ifndef BPK_H
#define BPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BPK_HEAD_DIM 128 /* channels per KV head */
#define BPK_BLOCK 64     /* tokens per quantisation block (Fathom §3.2) */
#define BPK_PLANES 4     /* bits per key code (Fathom §3.2) */
#define BPK_MAX_SEQS 64
#define BPK_MAX_K 4096   /* largest top-k per query head */
#define BPK_MAX_SELECTED 8192 /* largest group * k */
/* words per plane row and scales per scale row of a cache of `cap` tokens */
#define BPK_BLOCK_STRIDE(cap) ((((cap) / BPK_BLOCK) + 7) / 8 * 8)

enum bpk_status {
  BPK_OK = 0,
  BPK_EINVAL = -1,       /* null pointer, bad range, k or budget out of range */
  BPK_EUNSUPPORTED = -2, /* shape outside the supported set */
  BPK_EWORKSPACE = -3,   /* workspace missing or smaller than bpk_workspace_bytes */
  BPK_ECAPACITY = -4,    /* an append would pass the cache capacity */
  BPK_EHIP = -5          /* a HIP launch failed; the message names the error */
};

enum bpk_dtype { BPK_F32 = 0, BPK_BF16 = 1 };

enum bpk_op {
  BPK_OP_SELECT = 3,
  BPK_OP_ATTEND = 4,
  BPK_OP_DECODE = 5,
  BPK_OP_POOLED = 6,
  BPK_OP_ATTEND_V = 7,
  BPK_OP_DECODE_V = 8
};

/*
 * The cache: storage shared by every entry point.  All arrays are
 * caller-allocated device memory except n_tokens (HOST).
 *
 * k_rows   [S][L][H][capacity][128]  key rows, fp32 or bf16 (k_dtype).
 * v_rows   [S][L][H][capacity][128]  value rows, bf16 bit patterns.
 * planes   [S][L][H][128][4][NBS] uint64, NBS = BPK_BLOCK_STRIDE(capacity) (the
 *          capacity in blocks rounded up to a multiple of 8, so that every row
 *          starts 64-byte aligned; words past capacity/64 are never written,
 *          may be loaded by whole-row reads, and never change a result).
 *          Word (j, p, b) holds bit p
 *          (p = 0 is the most significant bit, i.e. the sign) of the 4-bit
 *          codes of channel j over the 64 tokens of block b; bit i of the word
 *          belongs to token 64 b + i.  Channel-major, so the first t planes of
 *          a channel are contiguous (Fathom §3.2).
 * scales   [S][L][H][128][NBS] fp16 bit patterns, one per (channel,
 *          block): the block's max |k| divided by 8 (Fathom §3.2).
 * chan_var [S][L][H][128] fp32: the variance of each key channel in the scan
 *          basis, used by the depth rule (Fathom §1, observation 1).
 * rot      NULL for the raw channel basis, or [L][H][128][128] fp32 row-major
 *          orthogonal R per (layer, head): keys and queries are scanned in the
 *          basis z = R^T x (the KLT basis of Fathom §1, contributions).
 * n_tokens HOST [S]: tokens present in each sequence, including the tokens of
 *          an open (incomplete) trailing block, which have rows but no planes.
 * v_planes NULL, or [S][L][H][capacity][4][16] uint8: value planes for the
 *          value-depth entry points (ReadKV §5.3: every channel of a token
 *          shares one depth; §6.1: progressive planes).  Each token's value
 *          row is coded with one scale and the same 4-bit symmetric code as
 *          the keys; the 16 bytes of plane p hold bit 3 - p of its 128 codes,
 *          channel j in bit j % 8 of byte j / 8.  A token's 64 bytes are
 *          contiguous, so reading it at depth t reads its first 16 t bytes.
 * v_scales NULL, or [S][L][H][capacity] fp16 bit patterns: per token, its
 *          max |v| divided by 8 (round to nearest even, saturated at 65504).
 *          v_planes and v_scales are both set or both NULL.
 */
typedef struct bpk_cache {
  int32_t num_seqs;
  int32_t num_layers;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t group;
  int32_t k_dtype;
  int64_t capacity;
  const int64_t* n_tokens; /* HOST */
  void* k_rows;
  uint16_t* v_rows;
  uint64_t* planes;
  uint16_t* scales;
  const float* chan_var;
  const float* rot;
  uint8_t* v_planes;
  uint16_t* v_scales;
} bpk_cache_t;

/*
 * Append n_new tokens to sequence `seq` of every (layer, KV head) and encode
 * the 64-token blocks the append completes (Fathom §3.2; planes are
 * append-only and never re-encoded, ReadKV §6.1).
 *
 * k_new [L][H][n_new][128] in the cache's k_dtype, v_new [L][H][n_new][128]
 * bf16: copied to rows n_tokens[seq] .. n_tokens[seq] + n_new - 1.  If both
 * are NULL the rows are taken to be in place already.  Each completed block
 * gets, per channel j, the scale s = fp16_rne(max|k| / 8) (saturated at
 * 65504) and the codes c = clip(floor(k / s), -8, 7) + 8 with the exact real
 * floor (c = 8 when s = 0), packed into the four plane words.  With rot set,
 * k is first mapped to z = R^T k (fp64 sum over d ascending, rounded to fp32).
 * With v_planes set, every appended token's value row is coded at once
 * (there is no block to wait for): s = fp16_rne(max_j |v_j| / 8) and the
 * same codes, written as the token's four planes.
 * The caller advances n_tokens[seq] by n_new afterwards.
 * Errors: BPK_EINVAL (seq out of range, n_new < 0, only one of k_new / v_new
 * given), BPK_ECAPACITY (n_tokens[seq] + n_new > capacity).
 */
int bpk_encode_append(const bpk_cache_t* cache, int32_t seq, const void* k_new,
                      const uint16_t* v_new, int64_t n_new, void* stream);

/*
 * Per-query depth allocation (Fathom §1 observation 1 and §3; ReadKV §5.2,
 * §5.4): one wavefront per unit.
 *
 * q [S][nl][H][G][128] bf16 (nl = l1 - l0).  Writes q_basis [S][nl][H][G][128]
 * fp32 (the query in the scan basis: q itself, or R^T q with rot set) and
 * depth [S][nl][H][128] uint8.  g_j = chan_var_j * sum_h q_hj^2 (fp32, h ascending);
 * the budget of min(budget_planes, 512) planes goes to the (channel, plane)
 * candidates of largest value g_j * 4^-t, ties to the lower channel then the
 * lower plane; depth_j = number of channel j's candidates taken.
 * Errors: BPK_EINVAL (bad layer range, budget_planes < 0, null pointer).
 */
int bpk_alloc_depth(const bpk_cache_t* cache, const uint16_t* q, int32_t l0, int32_t l1,
                    int32_t budget_planes, uint8_t* depth, float* q_basis, void* stream);

/* Depth rules of bpk_fixed_depth: the fixed-depth scans the Fathom page
 * compares its per-query depths against (§2), run on the same planes. */
enum bpk_depth_rule {
  BPK_DEPTH_WATERFILL = 0, /* bpk_alloc_depth's rule (not accepted by bpk_fixed_depth) */
  BPK_DEPTH_SPARQ = 1,     /* param r: the r channels of largest sum_h |q_hj| at depth 4 */
  BPK_DEPTH_CHANNELS = 2,  /* param c: a static set of c channels at depth 4 (Double Sparsity) */
  BPK_DEPTH_UNIFORM = 3    /* param t: every channel at depth t (t = 2: the 2-bit thumbnail) */
};

/*
 * Fixed-depth baselines (Fathom §2, "SparQ", "Double Sparsity", thumbnail
 * scan), written in the form bpk_alloc_depth writes, so that bpk_scan_scores
 * and bpk_decode_step_depth run them on the same planes:
 * - BPK_DEPTH_SPARQ, param r in [0, 128]: s_j = sum_h |q_hj| over the group's
 *   query heads (fp32, heads ascending, in the scan basis); the r largest
 *   (equal sums: lower channel first) get depth 4, the others 0.
 * - BPK_DEPTH_CHANNELS, param c in [0, 128]: channels, DEVICE [L][H][c] uint8,
 *   the channel indices of each (layer, KV head), chosen offline; those get
 *   depth 4, the others 0 (indices >= 128 are ignored).
 * - BPK_DEPTH_UNIFORM, param t in [0, 4]: every channel gets depth t.
 * q, q_basis and depth as in bpk_alloc_depth (q_basis is written for every
 * rule).  channels is only read by BPK_DEPTH_CHANNELS (may be NULL otherwise).
 * Errors: BPK_EINVAL (bad rule, param out of range, NULL pointer).
 */
int bpk_fixed_depth(const bpk_cache_t* cache, const uint16_t* q, int32_t l0, int32_t l1,
                    int32_t rule, int32_t param, const uint8_t* channels, uint8_t* depth,
                    float* q_basis, void* stream);

/*
 * Per-layer budget calibration (Fathom §3 names it as optional; the rule is
 * not on the page, so this is a reading): a calibration query is water-filled
 * over every unit of layers [l0, l1) at once, the budget of units *
 * budget_planes planes going to the most valuable (unit, channel, plane)
 * candidates g_uj 4^-t (g as in bpk_alloc_depth; equal values to the lower
 * unit, channel, plane).  bpk_pooled_planes writes the planes each unit gets,
 * plane_counts [S][nl][H] int32 (DEVICE).  ws: bpk_workspace_bytes(..,
 * BPK_OP_POOLED, ..) bytes (k ignored).  One workgroup: a calibration call,
 * not a decode-path call.
 * bpk_layer_budgets turns the counts of n_queries calibration queries,
 * [n_queries][S][nl][H] int32 (DEVICE), into per-layer budgets [nl] int32
 * (DEVICE): a layer's budget is the mean count of its units, rounded by
 * largest remainder (ties to the lower layer) so that the budgets sum to
 * nl * budget_planes.  Decoding then calls bpk_decode_step per layer with
 * its budget.  Errors: BPK_EINVAL (NULL pointers, budget_planes < 0,
 * n_queries < 1, more than 256 layers), BPK_EWORKSPACE.
 */
int bpk_pooled_planes(const bpk_cache_t* cache, const uint16_t* q, int32_t l0, int32_t l1,
                      int32_t budget_planes, int32_t* plane_counts, void* ws, size_t ws_bytes,
                      void* stream);
int bpk_layer_budgets(const bpk_cache_t* cache, const int32_t* plane_counts, int32_t n_queries,
                      int32_t l0, int32_t l1, int32_t budget_planes, int32_t* layer_budgets,
                      void* stream);
/*
 * bpk_alloc_depth with a budget per layer: layer_budgets [nl] int32 (DEVICE,
 * for instance from bpk_layer_budgets; values below 0 count as 0); the units
 * of layer l0 + i get min(layer_budgets[i], 512) planes.  Decoding all layers
 * at their budgets in one call: this, then bpk_decode_step_depth.
 * Errors: BPK_EINVAL (NULL pointer, bad layer range).
 */
int bpk_alloc_depth_layers(const bpk_cache_t* cache, const uint16_t* q, int32_t l0, int32_t l1,
                           const int32_t* layer_budgets, uint8_t* depth, float* q_basis,
                           void* stream);

/*
 * Key scan (Fathom §1, §3.2): approximate scores of every token of every
 * complete block, reading only planes p < depth_j of each channel and the
 * scales of channels with depth_j >= 1:
 *   score[h][i] = sum_j q_basis_hj * s_bj * m_ij,
 *   m_ij = (prefix_ij + 1/2) * 2^(4 - t_j) - 8   (t_j >= 1), 0 (t_j = 0),
 * where prefix_ij is the t_j-bit prefix of the token's code.
 * q_basis and depth as written by bpk_alloc_depth.
 * scores [S][nl][H][G][capacity] fp32; entries at or past 64 * floor(n/64) are
 * not written.  Errors: BPK_EINVAL.
 */
int bpk_scan_scores(const bpk_cache_t* cache, const float* q_basis, const uint8_t* depth,
                    int32_t l0, int32_t l1, float* scores, void* stream);

/*
 * Per-query-head top-k (Fathom §2, "Top-k decoding"): the first 4 and the
 * last W tokens are always kept, W = max(32, n mod 64) (the open trailing
 * block has no planes, so it is kept whole); the other k - 4 - W are the
 * highest scores among tokens [4, n - W), equal scores to the lower index.
 * If n <= k all n tokens are kept.  scores as written by bpk_scan_scores.
 * idx [S][nl][H][G][k] int32: the min(n, k)
 * selected token indices in ascending order, then -1 padding.
 * ws may be NULL (needs 0 bytes).
 * Errors: BPK_EINVAL (k < 1, k > BPK_MAX_K, or n > k with k < 4 + W).
 */
int bpk_select_topk(const bpk_cache_t* cache, const float* scores, int32_t l0, int32_t l1,
                    int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Exact attention over each query head's selected rows (Fathom §1, §2): the
 * union of the G heads' index sets is fetched once per unit, then for each
 * head h, out_h = sum_i softmax_i(softmax_scale * q_h . K_i) V_i over its own
 * set, accumulated in fp32 from the bf16 (or fp32) rows.  q is bf16 in the
 * model basis, [S][nl][H][G][128]; idx as written by
 * bpk_select_topk (entries outside [0, n) are skipped, so -1 padding is
 * harmless); out [S][nl][H][G][128] fp32 (zero for a head with no rows).
 * ws: at least bpk_workspace_bytes(cache, BPK_OP_ATTEND, l0, l1, k) bytes.
 * Errors: BPK_EINVAL, BPK_EWORKSPACE.
 */
int bpk_sparse_attend(const bpk_cache_t* cache, const uint16_t* q, const int32_t* idx,
                      int32_t l0, int32_t l1, int32_t k, float softmax_scale, float* out,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step over layers [l0, l1) of every sequence: alloc_depth ->
 * scan_scores -> select_topk -> sparse_attend, all enqueued on `stream`,
 * the cost model of Fathom §3.1 (Eq. 1) without the weight term.
 * q [S][nl][H][G][128] bf16, out [S][nl][H][G][128] fp32.
 * depth_out ([S][nl][H][128]) and idx_out ([S][nl][H][G][k]) are optional
 * (NULL: kept in the workspace).  ws: at least
 * bpk_workspace_bytes(cache, BPK_OP_DECODE, l0, l1, k) bytes.
 * Errors: those of the four stages, BPK_EWORKSPACE.
 */
int bpk_decode_step(const bpk_cache_t* cache, const uint16_t* q, int32_t l0, int32_t l1,
                    int32_t budget_planes, int32_t k, float softmax_scale, float* out,
                    uint8_t* depth_out, int32_t* idx_out, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * bpk_decode_step on depths the caller gives (for instance from
 * bpk_fixed_depth) instead of its own allocation: scan -> select -> attend
 * exactly as bpk_decode_step does after bpk_alloc_depth.  q_basis
 * [S][nl][H][G][128] fp32 and depth [S][nl][H][128] uint8 as bpk_alloc_depth
 * or bpk_fixed_depth writes them; q bf16 for the attention; the other
 * arguments, the workspace (bpk_workspace_bytes(.., BPK_OP_DECODE, ..)) and
 * the errors as bpk_decode_step.  max_rows: 0 when not known, else a bound on
 * the plane rows every unit reads (the sum of its depths; the rules of
 * bpk_fixed_depth read at most 4 r, 4 c and 128 t rows, bpk_alloc_depth_layers
 * exactly the layer's budget).  The library cannot see the depths from the
 * host, so without a bound it launches every scan variant and most of their
 * workgroups only read the depths and leave; with a bound of at most 128 it
 * launches only the variant that holds that many rows.  A unit reading more
 * rows than a given bound is not scanned: its selection and output are then
 * undefined (it finds no candidates and is redone by the fallback, which
 * picks among the unit's own tokens, so every row the attention reads is a
 * token of the unit).  BPK_EINVAL for max_rows < 0.
 */
int bpk_decode_step_depth(const bpk_cache_t* cache, const uint16_t* q, const float* q_basis,
                          const uint8_t* depth, int32_t max_rows, int32_t l0, int32_t l1,
                          int32_t k, float softmax_scale, float* out, int32_t* idx_out, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * bpk_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * bpk_decode_step; the workspace is instead a scratch array inside the
 * library, BPK_NOALLOC_SCRATCH_BYTES on each GPU, held until the process ends
 * (its address is looked up once per device, on the first call with that
 * device current).  The call allocates nothing.
 * - It runs on the current device, which must be the device of `stream` and
 *   of the cache.
 * - Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents: calls that overlap on one GPU (other streams, other threads)
 *   race and must be serialised by the caller.
 * Errors: those of bpk_decode_step; BPK_EWORKSPACE when
 * bpk_workspace_bytes(cache, BPK_OP_DECODE, l0, l1, k) exceeds
 * BPK_NOALLOC_SCRATCH_BYTES (use bpk_decode_step with a workspace instead).
 */
#define BPK_NOALLOC_SCRATCH_BYTES (32u << 20)
int bpk_decode_step_noalloc(const bpk_cache_t* cache, const uint16_t* q, int32_t l0, int32_t l1,
                            int32_t budget_planes, int32_t k, float softmax_scale, float* out,
                            uint8_t* depth_out, int32_t* idx_out, void* stream);

/*
 * Diagnostic of the fused selection inside bpk_decode_step (k <= 1024): that
 * step takes a sampled score threshold, keeps the tokens at or above it, and
 * picks the top-k among those; a unit whose kept tokens are too few (or
 * overflow their buffers) is redone by a full scan and radix select, with the
 * same result.  This call writes to *count (a DEVICE int32) how many units
 * of the last bpk_decode_step that used `ws` with the same cache, layer range
 * and k were redone that way (0 for k > 1024, which never takes the fused
 * path).  Enqueued on `stream` after that step.
 * Errors: BPK_EINVAL, BPK_EWORKSPACE.
 */
int bpk_decode_fallback_units(const bpk_cache_t* cache, int32_t l0, int32_t l1, int32_t k,
                              const void* ws, size_t ws_bytes, int32_t* count, void* stream);

/*
 * Value-side depths (ReadKV §5.3, §5.4) from given importances: for each
 * unit, rows[u][0 .. n_rows[u]) are tokens of its sequence and
 * weights[u][r] their importances a_r (fp32, finite and >= 0; anything else
 * counts as 0).  The gain of row r is w_r = a_r * s_r^2 (fp32, s_r the
 * token's value scale) and its t-th plane is worth w_r * 4^-t (fp32); the
 * v_budget planes go to the candidates (r, t) of largest positive value,
 * equal values to the lower row, then the lower plane, and no plane goes to
 * a candidate worth 0.  Writes depth[u][r] = planes granted to row r for
 * r < row_ld (0 past n_rows[u]).  Pass the rows in token order for the
 * lower-token tie rule.  A token outside [0, n_tokens) gets no plane.
 * rows, weights, depth: [S][nl][H][row_ld]; n_rows: [S][nl][H] int32
 * (device), clamped to [0, row_ld].
 * Errors: BPK_EINVAL (NULL pointer, v_budget < 0, row_ld outside
 * [1, BPK_MAX_SELECTED], no value planes in the cache).
 */
int bpk_value_depth(const bpk_cache_t* cache, int32_t l0, int32_t l1, const int32_t* rows,
                    const int32_t* n_rows, int32_t row_ld, const float* weights,
                    int32_t v_budget, uint8_t* depth, void* stream);

/*
 * Sparse attention with the value rows read at per-token depths (Fathom §2
 * for the selection and the per-head softmax from exact keys; ReadKV §5.3
 * for the value stage).  Per unit: the union of the G heads' selected rows
 * (token order), each head's softmax p_h over its own rows, importances
 * a_r = sum_h p_hr^2 (p_hr = 0 where head h did not select r), depths as
 * bpk_value_depth with budget v_budget, and
 * out_h = sum_r p_hr v_hat_r, v_hat_r the row rebuilt from its first t_r
 * value planes (cell midpoints times the token's scale; 0 at depth 0).
 * q, idx, out and the errors as bpk_sparse_attend; union_out
 * ([S][nl][H][G * k] int32: the union's tokens in order, -1 past its end)
 * and v_depth_out ([S][nl][H][G * k] uint8: each union row's depth, 0 past
 * the end) are optional.  ws: bpk_workspace_bytes(.., BPK_OP_ATTEND_V, ..).
 * The probabilities are fp32 (expf), so a depth can differ from an exact
 * computation's only where two plane values are within rounding of each
 * other.  Errors as bpk_sparse_attend, and BPK_EINVAL for v_budget < 0 or
 * no value planes.
 */
int bpk_sparse_attend_v(const bpk_cache_t* cache, const uint16_t* q, const int32_t* idx,
                        int32_t l0, int32_t l1, int32_t k, float softmax_scale,
                        int32_t v_budget, float* out, int32_t* union_out,
                        uint8_t* v_depth_out, void* ws, size_t ws_bytes, void* stream);

/*
 * bpk_decode_step with bpk_sparse_attend_v as its attention stage: alloc ->
 * scan -> select -> attention with value depths.  Arguments as
 * bpk_decode_step, plus v_budget, union_out and v_depth_out as
 * bpk_sparse_attend_v; ws: bpk_workspace_bytes(.., BPK_OP_DECODE_V, ..).
 */
int bpk_decode_step_v(const bpk_cache_t* cache, const uint16_t* q, int32_t l0, int32_t l1,
                      int32_t budget_planes, int32_t k, float softmax_scale, int32_t v_budget,
                      float* out, uint8_t* depth_out, int32_t* idx_out, int32_t* union_out,
                      uint8_t* v_depth_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Workspace bytes an entry point needs for layers [l0, l1) and top-k k
 * (op = BPK_OP_SELECT, BPK_OP_ATTEND, BPK_OP_DECODE, BPK_OP_POOLED,
 * BPK_OP_ATTEND_V or BPK_OP_DECODE_V).  Returns 0 for an invalid cache or op.
 */
size_t bpk_workspace_bytes(const bpk_cache_t* cache, int32_t op, int32_t l0, int32_t l1,
                           int32_t k);

/* Message of the calling thread's last failing call ("" if none). */
const char* bpk_last_error(void);

/* The stages of bpk_decode_step that stage tracing times. */
enum bpk_stage {
  BPK_STAGE_ALLOC = 0,     /* depth allocation */
  BPK_STAGE_SAMPLE = 1,    /* sampled scan (fused selection) */
  BPK_STAGE_THRESHOLD = 2, /* per-head candidate thresholds (fused selection) */
  BPK_STAGE_SCAN = 3,      /* the key scan over every complete block */
  BPK_STAGE_SELECT = 4,    /* top-k (exact, among the candidates when fused) */
  BPK_STAGE_FALLBACK = 5,  /* full scan and select of flagged units (fused selection) */
  BPK_STAGE_ATTEND = 6,    /* union-gather attention */
  BPK_STAGE_COUNT = 7
};

/*
 * Stage tracing, a profiling aid that changes no result.  While it is on for
 * the calling thread, each bpk_decode_step call of that thread records a HIP
 * event before and after every stage on the call's stream (the stages a call
 * skips get none).  bpk_trace_read waits for the recorded events, writes
 * to ms[BPK_STAGE_COUNT] the milliseconds of each stage summed over the
 * recorded calls and to *calls their number, and with reset != 0 forgets them.
 * bpk_trace_enable(0) also forgets them.  The events are created by the
 * library and kept for reuse until the thread ends.
 * Errors: BPK_EINVAL (NULL ms or calls), BPK_EHIP (an event call failed).
 */
int bpk_trace_enable(int32_t on);
int bpk_trace_read(double* ms, int64_t* calls, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* BPK_H */
