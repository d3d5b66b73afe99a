// C ABI of the library: argument validation, workspace carving and launch
// sequencing.  Every check runs before the first launch, so a call that
// returns a validation error has enqueued nothing.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "bpk_internal.h"

// Scratch memory of bpk_decode_step_noalloc: one copy per GPU, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[BPK_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BPK_OK;
  return fail(BPK_EHIP, "%s: %s", what, hipGetErrorString(e));
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- stage tracing: per thread, event pairs around the stages of
// decode_step, read back and summed by bpk_trace_read ----
struct TraceRecord {
  int stage;
  hipEvent_t start, stop;
};
struct TraceState {
  bool on = false;
  std::vector<hipEvent_t> pool;  // events created so far, reused after a reset
  size_t used = 0;
  std::vector<TraceRecord> records;
  long long calls = 0;
  ~TraceState() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};
thread_local TraceState g_trace;

hipEvent_t trace_event() {
  if (g_trace.used == g_trace.pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_trace.pool.push_back(e);
  }
  return g_trace.pool[g_trace.used++];
}

// Records the events around one stage when tracing is on; a failing event
// call turns tracing off for the rest of the call (results are unaffected).
class StageTimer {
 public:
  StageTimer(int stage, hipStream_t st, bool traced) : st_(st) {
    if (!traced || !g_trace.on) return;
    rec_.stage = stage;
    rec_.start = trace_event();
    rec_.stop = trace_event();
    if (rec_.start && rec_.stop && hipEventRecord(rec_.start, st_) == hipSuccess) active_ = true;
  }
  ~StageTimer() {
    if (active_ && hipEventRecord(rec_.stop, st_) == hipSuccess) g_trace.records.push_back(rec_);
  }

 private:
  hipStream_t st_;
  TraceRecord rec_{};
  bool active_ = false;
};

// Checks shared by every entry point; fills the geometry of layers [l0, l1).
int check_cache(const bpk_cache_t* c, int l0, int l1, bpk::Geom* g) {
  if (!c) return fail(BPK_EINVAL, "cache is NULL");
  if (c->head_dim != BPK_HEAD_DIM)
    return fail(BPK_EUNSUPPORTED, "head_dim %d unsupported (only %d)", c->head_dim, BPK_HEAD_DIM);
  if (c->group != 1 && c->group != 2 && c->group != 4 && c->group != 8)
    return fail(BPK_EUNSUPPORTED, "group %d unsupported (1, 2, 4 or 8)", c->group);
  if (c->num_seqs < 1 || c->num_seqs > BPK_MAX_SEQS)
    return fail(BPK_EUNSUPPORTED, "num_seqs %d outside [1, %d]", c->num_seqs, BPK_MAX_SEQS);
  if (c->num_layers < 1 || c->num_kv_heads < 1)
    return fail(BPK_EINVAL, "num_layers and num_kv_heads must be >= 1");
  if ((long long)c->num_layers * c->num_kv_heads > 65535)
    return fail(BPK_EUNSUPPORTED, "num_layers * num_kv_heads > 65535");
  if (c->capacity <= 0 || c->capacity % BPK_BLOCK != 0 || c->capacity > (1ll << 28))
    return fail(BPK_EUNSUPPORTED, "capacity %lld must be a positive multiple of 64, <= 2^28",
                (long long)c->capacity);
  if (c->k_dtype != BPK_F32 && c->k_dtype != BPK_BF16)
    return fail(BPK_EINVAL, "k_dtype %d invalid", c->k_dtype);
  if (!c->n_tokens) return fail(BPK_EINVAL, "n_tokens is NULL");
  if (!c->k_rows || !c->v_rows || !c->planes || !c->scales || !c->chan_var)
    return fail(BPK_EINVAL, "cache array pointer is NULL");
  if ((c->v_planes == nullptr) != (c->v_scales == nullptr))
    return fail(BPK_EINVAL, "v_planes and v_scales must both be set or both be NULL");
  for (int s = 0; s < c->num_seqs; ++s)
    if (c->n_tokens[s] < 0 || c->n_tokens[s] > c->capacity)
      return fail(BPK_EINVAL, "n_tokens[%d] = %lld outside [0, capacity]", s,
                  (long long)c->n_tokens[s]);
  if (l0 < 0 || l1 > c->num_layers || l0 >= l1)
    return fail(BPK_EINVAL, "layer range [%d, %d) invalid for %d layers", l0, l1, c->num_layers);
  const long long units = (long long)c->num_seqs * (l1 - l0) * c->num_kv_heads;
  if (units > 65535) return fail(BPK_EUNSUPPORTED, "more than 65535 units in one call");
  g->S = c->num_seqs;
  g->L = c->num_layers;
  g->H = c->num_kv_heads;
  g->G = c->group;
  g->l0 = l0;
  g->nl = l1 - l0;
  g->cap = c->capacity;
  for (int s = 0; s < BPK_MAX_SEQS; ++s) g->n[s] = s < c->num_seqs ? c->n_tokens[s] : 0;
  return BPK_OK;
}

int check_k(const bpk_cache_t* c, int k) {
  if (k < 1 || k > BPK_MAX_K) return fail(BPK_EINVAL, "k = %d outside [1, %d]", k, BPK_MAX_K);
  if ((long long)k * c->group > BPK_MAX_SELECTED)
    return fail(BPK_EUNSUPPORTED, "group * k = %lld > %d", (long long)k * c->group,
                BPK_MAX_SELECTED);
  for (int s = 0; s < c->num_seqs; ++s) {
    const long long n = c->n_tokens[s];
    const long long w = (n % BPK_BLOCK) > 32 ? (n % BPK_BLOCK) : 32;
    if (n > k && k < 4 + w)
      return fail(BPK_EINVAL, "k = %d does not cover the %lld always-kept tokens of sequence %d",
                  k, 4 + w, s);
  }
  return BPK_OK;
}

// decode_step's workspace.  Sizes follow the capacity, not the current token
// counts, so one workspace serves every step of a growing cache.
struct DecodeWs {
  size_t q_basis, depth, scores, idx, attend;
  size_t sample, thresh, count, cval, cidx, flag;  // fused selection
  long long sample_ld, regions;
  size_t total;
};

// With `values` the attention region fits the value-depth attention.
DecodeWs decode_ws(const bpk::Geom& g, int k, bool values = false) {
  DecodeWs w;
  const size_t units = (size_t)g.units();
  const size_t uh = units * g.G;
  const long long groups = (g.nbcap() + bpk::SAMPLE_STRIDE - 1) / bpk::SAMPLE_STRIDE;
  w.sample_ld = groups * bpk::SAMPLE_GROUP * bpk::BLK;
  // candidate regions of 16 blocks (a scan workgroup of wb blocks takes wb / 16
  // of them); the capacity rounded up to the largest span fits every span
  w.regions = (g.nbcap() + bpk::SCAN_MAX_WG_BLOCKS - 1) / bpk::SCAN_MAX_WG_BLOCKS *
              (bpk::SCAN_MAX_WG_BLOCKS / bpk::SCAN_MIN_WG_BLOCKS);
  const size_t slots = uh * (size_t)w.regions * bpk::CAND_SLOTS;
  size_t off = 0;
  w.q_basis = off; off += align256(uh * bpk::D * sizeof(float));
  w.depth = off;   off += align256(units * bpk::D);
  w.scores = off;  off += align256(uh * (size_t)g.cap * sizeof(float));
  w.idx = off;     off += align256(uh * (size_t)k * sizeof(int32_t));
  w.attend = off;
  off += align256(values ? bpk::attend_v_ws_bytes(g, k) : bpk::attend_ws_bytes(g, k));
  w.sample = off;  off += align256(uh * (size_t)w.sample_ld * sizeof(uint16_t));
  w.thresh = off;  off += align256(uh * sizeof(uint32_t));
  w.count = off;   off += align256(uh * (size_t)w.regions * bpk::CAND_PARTS * sizeof(int32_t));
  w.cval = off;    off += align256(slots * sizeof(float));
  w.cidx = off;    off += align256(slots * sizeof(int32_t));
  w.flag = off;    off += align256(units * sizeof(int32_t));
  w.total = off;
  return w;
}

// bpk_pooled_planes' workspace: q in the scan basis, depths (unused), gains
size_t pooled_ws(const bpk::Geom& g) {
  const size_t units = (size_t)g.units();
  return align256(units * g.G * bpk::D * sizeof(float)) + align256(units * bpk::D) +
         align256(units * bpk::D * sizeof(float));
}

}  // namespace

extern "C" {

const char* bpk_last_error(void) { return g_err.c_str(); }

size_t bpk_workspace_bytes(const bpk_cache_t* c, int32_t op, int32_t l0, int32_t l1, int32_t k) {
  bpk::Geom g;
  if (check_cache(c, l0, l1, &g) != BPK_OK) return 0;
  if (k < 1 || k > BPK_MAX_K) return 0;
  switch (op) {
    case BPK_OP_SELECT: return 0;
    case BPK_OP_ATTEND: return bpk::attend_ws_bytes(g, k);
    case BPK_OP_DECODE: return decode_ws(g, k).total;
    case BPK_OP_POOLED: return pooled_ws(g);
    case BPK_OP_ATTEND_V: return bpk::attend_v_ws_bytes(g, k);
    case BPK_OP_DECODE_V: return decode_ws(g, k, true).total;
    default: return 0;
  }
}

int bpk_encode_append(const bpk_cache_t* c, int32_t seq, const void* k_new, const uint16_t* v_new,
                      int64_t n_new, void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, 0, c ? c->num_layers : 1, &g);
  if (rc) return rc;
  if (seq < 0 || seq >= c->num_seqs) return fail(BPK_EINVAL, "seq %d out of range", seq);
  if (n_new < 0) return fail(BPK_EINVAL, "n_new < 0");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(BPK_EINVAL, "k_new and v_new must both be given or both be NULL");
  const long long n0 = c->n_tokens[seq];
  if (n0 + n_new > c->capacity)
    return fail(BPK_ECAPACITY, "append of %lld tokens to %lld passes capacity %lld",
                (long long)n_new, n0, (long long)c->capacity);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (k_new) {
    rc = hip_status(bpk::launch_append_rows(g, seq, c->k_dtype, k_new, v_new, n0, n_new, c->k_rows,
                                            c->v_rows, st),
                    "append rows");
    if (rc) return rc;
  }
  const long long b0 = n0 / BPK_BLOCK, b1 = (n0 + n_new) / BPK_BLOCK;
  rc = hip_status(bpk::launch_encode(g, seq, c->k_dtype, c->k_rows, c->rot, c->planes, c->scales,
                                     b0, b1 - b0, st),
                  "encode");
  if (rc || !c->v_planes) return rc;
  return hip_status(bpk::launch_vencode(g, seq, c->v_rows, c->v_planes, c->v_scales, n0, n_new, st),
                    "encode values");
}

int bpk_alloc_depth(const bpk_cache_t* c, const uint16_t* q, int32_t l0, int32_t l1,
                    int32_t budget_planes, uint8_t* depth, float* q_basis, void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!q || !depth || !q_basis) return fail(BPK_EINVAL, "q, depth and q_basis must be non-NULL");
  if (budget_planes < 0) return fail(BPK_EINVAL, "budget_planes < 0");
  return hip_status(bpk::launch_alloc(g, q, c->chan_var, c->rot, budget_planes, depth, q_basis,
                                      static_cast<hipStream_t>(stream)),
                    "alloc_depth");
}

int bpk_fixed_depth(const bpk_cache_t* c, const uint16_t* q, int32_t l0, int32_t l1,
                    int32_t rule, int32_t param, const uint8_t* channels, uint8_t* depth,
                    float* q_basis, void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!q || !depth || !q_basis) return fail(BPK_EINVAL, "q, depth and q_basis must be non-NULL");
  switch (rule) {
    case BPK_DEPTH_SPARQ:
    case BPK_DEPTH_CHANNELS:
      if (param < 0 || param > bpk::D)
        return fail(BPK_EINVAL, "param %d outside [0, %d]", param, bpk::D);
      if (rule == BPK_DEPTH_CHANNELS && !channels && param > 0)
        return fail(BPK_EINVAL, "channels must be non-NULL");
      break;
    case BPK_DEPTH_UNIFORM:
      if (param < 0 || param > bpk::NP)
        return fail(BPK_EINVAL, "depth %d outside [0, %d]", param, bpk::NP);
      break;
    default:
      return fail(BPK_EINVAL, "depth rule %d invalid", rule);
  }
  return hip_status(bpk::launch_alloc(g, q, c->chan_var, c->rot, param, depth, q_basis,
                                      static_cast<hipStream_t>(stream), rule, channels),
                    "fixed_depth");
}

int bpk_pooled_planes(const bpk_cache_t* c, const uint16_t* q, int32_t l0, int32_t l1,
                      int32_t budget_planes, int32_t* plane_counts, void* ws, size_t ws_bytes,
                      void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!q || !plane_counts) return fail(BPK_EINVAL, "q and plane_counts must be non-NULL");
  if (budget_planes < 0) return fail(BPK_EINVAL, "budget_planes < 0");
  const size_t need = pooled_ws(g);
  if (!ws || ws_bytes < need)
    return fail(BPK_EWORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  char* base = static_cast<char*>(ws);
  const size_t units = (size_t)g.units();
  float* qb = reinterpret_cast<float*>(base);
  uint8_t* depth = reinterpret_cast<uint8_t*>(base + align256(units * g.G * bpk::D * sizeof(float)));
  float* gains = reinterpret_cast<float*>(base + align256(units * g.G * bpk::D * sizeof(float)) +
                                          align256(units * bpk::D));
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the gains of every unit (an allocation with no budget writes them)
  rc = hip_status(bpk::launch_alloc(g, q, c->chan_var, c->rot, 0, depth, qb, st,
                                    BPK_DEPTH_WATERFILL, nullptr, gains),
                  "pooled_planes/gains");
  if (rc) return rc;
  return hip_status(bpk::launch_pooled(g, gains, budget_planes, plane_counts, st),
                    "pooled_planes");
}

int bpk_alloc_depth_layers(const bpk_cache_t* c, const uint16_t* q, int32_t l0, int32_t l1,
                           const int32_t* layer_budgets, uint8_t* depth, float* q_basis,
                           void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!q || !layer_budgets || !depth || !q_basis)
    return fail(BPK_EINVAL, "q, layer_budgets, depth and q_basis must be non-NULL");
  return hip_status(bpk::launch_alloc(g, q, c->chan_var, c->rot, 0, depth, q_basis,
                                      static_cast<hipStream_t>(stream), BPK_DEPTH_WATERFILL,
                                      nullptr, nullptr, layer_budgets),
                    "alloc_depth_layers");
}

int bpk_layer_budgets(const bpk_cache_t* c, const int32_t* plane_counts, int32_t n_queries,
                      int32_t l0, int32_t l1, int32_t budget_planes, int32_t* layer_budgets,
                      void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!plane_counts || !layer_budgets)
    return fail(BPK_EINVAL, "plane_counts and layer_budgets must be non-NULL");
  if (n_queries < 1) return fail(BPK_EINVAL, "n_queries < 1");
  if (budget_planes < 0) return fail(BPK_EINVAL, "budget_planes < 0");
  if (g.nl > 256) return fail(BPK_EINVAL, "more than 256 layers in one call");
  return hip_status(bpk::launch_layer_budgets(g, plane_counts, n_queries, budget_planes,
                                              layer_budgets, static_cast<hipStream_t>(stream)),
                    "layer_budgets");
}

int bpk_scan_scores(const bpk_cache_t* c, const float* q_basis, const uint8_t* depth, int32_t l0,
                    int32_t l1, float* scores, void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!q_basis || !depth || !scores)
    return fail(BPK_EINVAL, "q_basis, depth and scores must be non-NULL");
  return hip_status(bpk::launch_scan(g, q_basis, depth, c->planes, c->scales, scores, -1,
                                     static_cast<hipStream_t>(stream)),
                    "scan_scores");
}

int bpk_select_topk(const bpk_cache_t* c, const float* scores, int32_t l0, int32_t l1, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!scores || !idx) return fail(BPK_EINVAL, "scores and idx must be non-NULL");
  rc = check_k(c, k);
  if (rc) return rc;
  return hip_status(bpk::launch_topk(g, scores, k, idx, static_cast<hipStream_t>(stream)),
                    "select_topk");
}

int bpk_sparse_attend(const bpk_cache_t* c, const uint16_t* q, const int32_t* idx, int32_t l0,
                      int32_t l1, int32_t k, float softmax_scale, float* out, void* ws,
                      size_t ws_bytes, void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!q || !idx || !out) return fail(BPK_EINVAL, "q, idx and out must be non-NULL");
  rc = check_k(c, k);
  if (rc) return rc;
  const size_t need = bpk::attend_ws_bytes(g, k);
  if (!ws || ws_bytes < need)
    return fail(BPK_EWORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  return hip_status(bpk::launch_attend(g, c->k_dtype, c->k_rows, c->v_rows, q, idx, k,
                                       softmax_scale, out, ws, static_cast<hipStream_t>(stream)),
                    "sparse_attend");
}

int bpk_value_depth(const bpk_cache_t* c, int32_t l0, int32_t l1, const int32_t* rows,
                    const int32_t* n_rows, int32_t row_ld, const float* weights,
                    int32_t v_budget, uint8_t* depth, void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!c->v_planes) return fail(BPK_EINVAL, "the cache has no value planes");
  if (!rows || !n_rows || !weights || !depth)
    return fail(BPK_EINVAL, "rows, n_rows, weights and depth must be non-NULL");
  if (row_ld < 1 || row_ld > BPK_MAX_SELECTED)
    return fail(BPK_EINVAL, "row_ld %d outside [1, %d]", row_ld, BPK_MAX_SELECTED);
  if (v_budget < 0) return fail(BPK_EINVAL, "v_budget < 0");
  return hip_status(bpk::launch_value_depth(g, rows, n_rows, row_ld, weights, c->v_scales,
                                            v_budget, depth, static_cast<hipStream_t>(stream)),
                    "value_depth");
}

int bpk_sparse_attend_v(const bpk_cache_t* c, const uint16_t* q, const int32_t* idx, int32_t l0,
                        int32_t l1, int32_t k, float softmax_scale, int32_t v_budget, float* out,
                        int32_t* union_out, uint8_t* v_depth_out, void* ws, size_t ws_bytes,
                        void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!q || !idx || !out) return fail(BPK_EINVAL, "q, idx and out must be non-NULL");
  if (!c->v_planes) return fail(BPK_EINVAL, "the cache has no value planes");
  if (v_budget < 0) return fail(BPK_EINVAL, "v_budget < 0");
  rc = check_k(c, k);
  if (rc) return rc;
  const size_t need = bpk::attend_v_ws_bytes(g, k);
  if (!ws || ws_bytes < need)
    return fail(BPK_EWORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  return hip_status(bpk::launch_attend_v(g, c->k_dtype, c->k_rows, c->v_planes, c->v_scales, q,
                                         idx, k, softmax_scale, v_budget, out, union_out,
                                         v_depth_out, ws, false, static_cast<hipStream_t>(stream)),
                    "sparse_attend_v");
}

}  // extern "C"

namespace {

// The decode step on a workspace the caller has checked (ws holds at least
// decode_ws(g, k).total bytes); `traced` lets stage tracing record events.
// With depth_in and qb_in given, the allocation is skipped and those are scanned.
int decode_step_impl(const bpk_cache_t* c, const bpk::Geom& g, const uint16_t* q,
                     int32_t budget_planes, int32_t k, float softmax_scale, float* out,
                     uint8_t* depth_out, int32_t* idx_out, char* base, bool traced,
                     hipStream_t st, const uint8_t* depth_in = nullptr,
                     const float* qb_in = nullptr, int v_budget = -1,
                     int32_t* union_out = nullptr, uint8_t* vdepth_out = nullptr,
                     int rows_bound = 0) {
  const DecodeWs w = decode_ws(g, k, v_budget >= 0);
  const bool given = depth_in != nullptr;
  float* q_basis = given ? const_cast<float*>(qb_in) : reinterpret_cast<float*>(base + w.q_basis);
  uint8_t* depth = given ? const_cast<uint8_t*>(depth_in)
                         : depth_out ? depth_out : reinterpret_cast<uint8_t*>(base + w.depth);
  float* scores = reinterpret_cast<float*>(base + w.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + w.idx);
  int rc = BPK_OK;
  // alloc_depth hands out exactly min(P, 4D) planes per unit; given depths:
  // the caller's bound when it fits the fast scan (every unit at most that
  // many rows), else not known on the host
  const int rows = given ? (rows_bound > 0 && rows_bound <= bpk::SCAN_FAST_ROWS ? rows_bound : -1)
                         : budget_planes < 4 * bpk::D ? budget_planes : 4 * bpk::D;
  if (traced && g_trace.on) ++g_trace.calls;
  auto timer = [&](int stage) { return StageTimer(stage, st, traced); };
  if (!given) {
    auto t = timer(BPK_STAGE_ALLOC);
    rc = hip_status(bpk::launch_alloc(g, q, c->chan_var, c->rot, budget_planes, depth, q_basis, st),
                    "decode_step/alloc");
  }
  if (rc) return rc;
  const bool values = v_budget >= 0;
  char* att_ws = base + w.attend;
  // the union arrays of the attention workspace
  const bpk::UnionBufs ub = bpk::union_bufs(g, k, att_ws);
  bool union_ready = false;  // the selection merged every unflagged unit's lists
  if (k <= bpk::FUSED_MAX_K) {
    // sampled threshold -> scan keeping candidates -> exact top-k among them;
    // flagged units (too few candidates, or too many) are redone unfused
    bpk::CandBufs cb;
    cb.sample = reinterpret_cast<uint16_t*>(base + w.sample);
    cb.sample_ld = w.sample_ld;
    cb.thresh = reinterpret_cast<uint32_t*>(base + w.thresh);
    cb.wg_blocks = bpk::scan_wg_blocks(g);
    cb.part_slots = bpk::CAND_PART_SLOTS * cb.wg_blocks / bpk::SCAN_MIN_WG_BLOCKS;
    cb.regions = w.regions;
    cb.count = reinterpret_cast<int32_t*>(base + w.count);
    cb.val = reinterpret_cast<float*>(base + w.cval);
    cb.idx = reinterpret_cast<int32_t*>(base + w.cidx);
    cb.flag = reinterpret_cast<int32_t*>(base + w.flag);
    {
      auto t = timer(BPK_STAGE_SAMPLE);
      rc = hip_status(
          bpk::launch_scan_sample(g, q_basis, depth, c->planes, c->scales, cb, rows, st),
          "decode_step/sample scan");
    }
    if (rc) return rc;
    {
      auto t = timer(BPK_STAGE_THRESHOLD);
      rc = hip_status(bpk::launch_threshold(g, k, cb, st), "decode_step/threshold");
    }
    if (rc) return rc;
    {
      auto t = timer(BPK_STAGE_SCAN);
      // with the caller's bound, a unit above it is skipped by the scan: its
      // counts start at zero, so that it has no candidates and is redone
      if (given && rows > 0)
        rc = hip_status(bpk::launch_zero_counts(g, cb, st), "decode_step/counts");
      if (!rc)
        rc = hip_status(
            bpk::launch_scan_cand(g, q_basis, depth, c->planes, c->scales, k, cb, rows, st),
            "decode_step/scan");
    }
    if (rc) return rc;
    {
      auto t = timer(BPK_STAGE_SELECT);
      rc = hip_status(bpk::launch_cand_select(g, k, cb, idx, &ub, &union_ready, st),
                      "decode_step/select");
    }
    if (rc) return rc;
    {
      auto t = timer(BPK_STAGE_FALLBACK);
      rc = hip_status(bpk::launch_scan_flagged(g, q_basis, depth, c->planes, c->scales, scores,
                                               cb.flag, rows, st),
                      "decode_step/fallback scan");
      if (!rc)  // (and the flagged units' union when the selection merged the others')
        rc = hip_status(bpk::launch_topk_flagged(g, scores, k, idx, cb.flag,
                                                 union_ready ? &ub : nullptr, st),
                        "decode_step/fallback select");
    }
    if (rc) return rc;
  } else {
    {
      auto t = timer(BPK_STAGE_SCAN);
      rc = hip_status(bpk::launch_scan(g, q_basis, depth, c->planes, c->scales, scores, rows, st),
                      "decode_step/scan");
    }
    if (rc) return rc;
    {
      auto t = timer(BPK_STAGE_SELECT);
      rc = hip_status(bpk::launch_topk(g, scores, k, idx, st), "decode_step/select");
    }
    if (rc) return rc;
  }
  auto t = timer(BPK_STAGE_ATTEND);
  if (values)
    return hip_status(bpk::launch_attend_v(g, c->k_dtype, c->k_rows, c->v_planes, c->v_scales, q,
                                           idx, k, softmax_scale, v_budget, out, union_out,
                                           vdepth_out, att_ws, union_ready, st),
                      "decode_step/attend_v");
  if (union_ready)
    return hip_status(bpk::launch_attend_rows(g, c->k_dtype, c->k_rows, c->v_rows, q, k,
                                              softmax_scale, out, att_ws, st),
                      "decode_step/attend");
  return hip_status(bpk::launch_attend(g, c->k_dtype, c->k_rows, c->v_rows, q, idx, k,
                                       softmax_scale, out, att_ws, st),
                    "decode_step/attend");
}

// Checks shared by the two decode entry points.
int check_decode(const bpk_cache_t* c, int32_t l0, int32_t l1, const uint16_t* q,
                 int32_t budget_planes, int32_t k, const float* out, bpk::Geom* g) {
  int rc = check_cache(c, l0, l1, g);
  if (rc) return rc;
  if (!q || !out) return fail(BPK_EINVAL, "q and out must be non-NULL");
  if (budget_planes < 0) return fail(BPK_EINVAL, "budget_planes < 0");
  return check_k(c, k);
}

// Device address of this device's scratch array (looked up once per device).
int scratch_address(char** out) {
  static std::mutex mu;
  static void* addr[256] = {};
  int dev = -1;
  int rc = hip_status(hipGetDevice(&dev), "decode_step_noalloc/hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= 256) return fail(BPK_EUNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                    "decode_step_noalloc/hipGetSymbolAddress");
    if (rc) return rc;
    addr[dev] = p;
  }
  *out = static_cast<char*>(addr[dev]);
  return BPK_OK;
}

}  // namespace

extern "C" {

int bpk_decode_step(const bpk_cache_t* c, const uint16_t* q, int32_t l0, int32_t l1,
                    int32_t budget_planes, int32_t k, float softmax_scale, float* out,
                    uint8_t* depth_out, int32_t* idx_out, void* ws, size_t ws_bytes,
                    void* stream) {
  bpk::Geom g;
  int rc = check_decode(c, l0, l1, q, budget_planes, k, out, &g);
  if (rc) return rc;
  const size_t need = decode_ws(g, k).total;
  if (!ws || ws_bytes < need)
    return fail(BPK_EWORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  return decode_step_impl(c, g, q, budget_planes, k, softmax_scale, out, depth_out, idx_out,
                          static_cast<char*>(ws), true, static_cast<hipStream_t>(stream));
}

int bpk_decode_step_v(const bpk_cache_t* c, const uint16_t* q, int32_t l0, int32_t l1,
                      int32_t budget_planes, int32_t k, float softmax_scale, int32_t v_budget,
                      float* out, uint8_t* depth_out, int32_t* idx_out, int32_t* union_out,
                      uint8_t* v_depth_out, void* ws, size_t ws_bytes, void* stream) {
  bpk::Geom g;
  int rc = check_decode(c, l0, l1, q, budget_planes, k, out, &g);
  if (rc) return rc;
  if (!c->v_planes) return fail(BPK_EINVAL, "the cache has no value planes");
  if (v_budget < 0) return fail(BPK_EINVAL, "v_budget < 0");
  const size_t need = decode_ws(g, k, true).total;
  if (!ws || ws_bytes < need)
    return fail(BPK_EWORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  return decode_step_impl(c, g, q, budget_planes, k, softmax_scale, out, depth_out, idx_out,
                          static_cast<char*>(ws), true, static_cast<hipStream_t>(stream), nullptr,
                          nullptr, v_budget, union_out, v_depth_out);
}

int bpk_decode_step_depth(const bpk_cache_t* c, const uint16_t* q, const float* q_basis,
                          const uint8_t* depth, int32_t max_rows, int32_t l0, int32_t l1,
                          int32_t k, float softmax_scale, float* out, int32_t* idx_out, void* ws,
                          size_t ws_bytes, void* stream) {
  bpk::Geom g;
  int rc = check_decode(c, l0, l1, q, 0, k, out, &g);
  if (rc) return rc;
  if (!q_basis || !depth) return fail(BPK_EINVAL, "q_basis and depth must be non-NULL");
  if (max_rows < 0) return fail(BPK_EINVAL, "max_rows < 0");
  const size_t need = decode_ws(g, k).total;
  if (!ws || ws_bytes < need)
    return fail(BPK_EWORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  return decode_step_impl(c, g, q, 0, k, softmax_scale, out, nullptr, idx_out,
                          static_cast<char*>(ws), true, static_cast<hipStream_t>(stream), depth,
                          q_basis, -1, nullptr, nullptr, max_rows);
}

int bpk_decode_step_noalloc(const bpk_cache_t* c, const uint16_t* q, int32_t l0, int32_t l1,
                            int32_t budget_planes, int32_t k, float softmax_scale, float* out,
                            uint8_t* depth_out, int32_t* idx_out, void* stream) {
  bpk::Geom g;
  int rc = check_decode(c, l0, l1, q, budget_planes, k, out, &g);
  if (rc) return rc;
  const size_t need = decode_ws(g, k).total;
  if (need > (size_t)BPK_NOALLOC_SCRATCH_BYTES)
    return fail(BPK_EWORKSPACE,
                "this call needs %zu bytes of scratch; the allocation-free decode step holds "
                "%zu (use bpk_decode_step with a workspace)",
                need, (size_t)BPK_NOALLOC_SCRATCH_BYTES);
  char* base = nullptr;
  rc = scratch_address(&base);
  if (rc) return rc;
  return decode_step_impl(c, g, q, budget_planes, k, softmax_scale, out, depth_out, idx_out, base,
                          false, static_cast<hipStream_t>(stream));
}

int bpk_decode_fallback_units(const bpk_cache_t* c, int32_t l0, int32_t l1, int32_t k,
                              const void* ws, size_t ws_bytes, int32_t* count, void* stream) {
  bpk::Geom g;
  int rc = check_cache(c, l0, l1, &g);
  if (rc) return rc;
  if (!count) return fail(BPK_EINVAL, "count must be non-NULL");
  rc = check_k(c, k);
  if (rc) return rc;
  const DecodeWs w = decode_ws(g, k);
  if (!ws || ws_bytes < w.total)
    return fail(BPK_EWORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, w.total);
  const int32_t* flag =
      reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + w.flag);
  // the unfused path (k > FUSED_MAX_K) flags nothing: count no unit
  const int units = k > bpk::FUSED_MAX_K ? 0 : g.units();
  return hip_status(bpk::launch_count_flags(units, flag, count, static_cast<hipStream_t>(stream)),
                    "decode_fallback_units");
}

int bpk_trace_enable(int32_t on) {
  g_trace.on = on != 0;
  if (!g_trace.on) {
    g_trace.records.clear();
    g_trace.used = 0;
    g_trace.calls = 0;
  }
  return BPK_OK;
}

int bpk_trace_read(double* ms, int64_t* calls, int32_t reset) {
  if (!ms || !calls) return fail(BPK_EINVAL, "ms and calls must be non-NULL");
  for (int i = 0; i < BPK_STAGE_COUNT; ++i) ms[i] = 0.0;
  for (const TraceRecord& r : g_trace.records) {
    float t = 0.f;
    int rc = hip_status(hipEventSynchronize(r.stop), "trace_read");
    if (!rc) rc = hip_status(hipEventElapsedTime(&t, r.start, r.stop), "trace_read");
    if (rc) return rc;
    ms[r.stage] += t;
  }
  *calls = g_trace.calls;
  if (reset) {
    g_trace.records.clear();
    g_trace.used = 0;
    g_trace.calls = 0;
  }
  return BPK_OK;
}

}  // extern "C"
