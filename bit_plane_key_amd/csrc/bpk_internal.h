// Internal declarations shared by the library's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bpk.h"

namespace bpk {

constexpr int D = BPK_HEAD_DIM;
constexpr int BLK = BPK_BLOCK;
constexpr int NP = BPK_PLANES;

// Geometry of the units a launch covers: every sequence, layers [l0, l0 + nl),
// every KV head.  Local unit u -> (s, l, h) with h fastest.
struct Geom {
  int S, L, H, G;
  int l0, nl;
  long long cap;  // tokens per sequence (multiple of 64)
  long long n[BPK_MAX_SEQS];

  __host__ __device__ int units() const { return S * nl * H; }
  __host__ __device__ int seq_of(int u) const { return u / (H * nl); }
  // global unit index (s * L + l) * H + h of local unit u
  __host__ __device__ long long global_unit(int u) const {
    int h = u % H;
    int l = l0 + (u / H) % nl;
    int s = u / (H * nl);
    return ((long long)s * L + l) * H + h;
  }
  // words per plane row (and fp16 scales per scale row): the capacity in
  // blocks rounded up to a multiple of 8, so every row starts 64-byte aligned
  __host__ __device__ long long nbcap() const { return BPK_BLOCK_STRIDE(cap); }
};

// ---- launchers (each returns hipGetLastError() of its launches) ----
hipError_t launch_encode(const Geom& g, int seq, int k_dtype, const void* k_rows,
                         const float* rot, uint64_t* planes, uint16_t* scales, long long b0,
                         long long nblocks, hipStream_t st);

hipError_t launch_append_rows(const Geom& g, int seq, int k_dtype, const void* k_new,
                              const uint16_t* v_new, long long n0, long long n_new, void* k_rows,
                              uint16_t* v_rows, hipStream_t st);

// depth allocation (rule BPK_DEPTH_WATERFILL, budget = planes) or a fixed
// baseline depth rule (budget = its parameter, channels its channel lists)
hipError_t launch_alloc(const Geom& g, const uint16_t* q, const float* chan_var, const float* rot,
                        int budget, uint8_t* depth, float* q_basis, hipStream_t st,
                        int rule = BPK_DEPTH_WATERFILL, const uint8_t* channels = nullptr,
                        float* gains = nullptr, const int32_t* layer_budget = nullptr);
// per-layer budget calibration: pooled plane counts of every unit, and the
// per-layer budgets of counts from several queries
hipError_t launch_pooled(const Geom& g, const float* gains, int budget, int32_t* counts,
                         hipStream_t st);
hipError_t launch_layer_budgets(const Geom& g, const int32_t* counts, int queries, int budget,
                                int32_t* out, hipStream_t st);

// Every scan launcher takes `rows`, the number of plane rows every unit of
// the call reads (min(P, 4D) after alloc_depth), or -1 when it is not known:
// units reading at most SCAN_FAST_ROWS rows go to the fast kernel, the others
// to the wide one, and with -1 both are launched and each skips the other's
// units.
constexpr int SCAN_FAST_ROWS = 128;
hipError_t launch_scan(const Geom& g, const float* q_basis, const uint8_t* depth,
                       const uint64_t* planes, const uint16_t* scales, float* scores, int rows,
                       hipStream_t st);

hipError_t launch_topk(const Geom& g, const float* scores, int k, int32_t* idx, hipStream_t st);

// ---- decode_step's fused selection ----
// A sampled scan (the first 64 blocks of every 4096) sets per (unit, query
// head) a score threshold expected to pass about 2 (k - 4 - W) tokens; the full
// scan then keeps only the tokens at or above it, and the exact top-k is taken
// among those.  Each scan workgroup of wg_blocks blocks owns a region of
// CAND_SLOTS * wg_blocks / SCAN_MIN_WG_BLOCKS slots per head (a unit's regions
// together always hold about 8 slots per block; no global atomics), in one
// part per wavefront; a unit whose candidates are too few, overflow a part or
// exceed CAND_CAP in all is flagged and redone by a full scan and radix
// select.
constexpr int SAMPLE_STRIDE = 4096;  // blocks from one sampled group to the next
constexpr int SAMPLE_GROUP = 64;     // blocks per sampled group
constexpr int CAND_SLOTS = 128;      // candidate slots per (16 scanned blocks, head)
constexpr int CAND_PARTS = 4;        // parts of a region, one per scan wavefront, counted apart
constexpr int CAND_PART_SLOTS = CAND_SLOTS / CAND_PARTS;
constexpr int CAND_CAP = 4096;       // candidates the exact selection takes per head
constexpr int FUSED_MAX_K = 1024;    // larger k take the unfused path
constexpr int SCAN_MIN_WG_BLOCKS = 16;

struct CandBufs {
  uint16_t* sample;     // [units][G][sample_ld] upper halves of the sampled scores' order keys
  long long sample_ld;  // sample_groups * SAMPLE_GROUP * 64
  uint32_t* thresh;     // [units][G] order key of the threshold
  int wg_blocks;        // blocks per workgroup of the candidate scan
  int part_slots;       // CAND_PART_SLOTS * wg_blocks / SCAN_MIN_WG_BLOCKS
  long long regions;    // per (unit, head): regions of 16 blocks the buffers hold
  int32_t* count;       // [units][G][regions][CAND_PARTS]: workgroup x, part p at x * CAND_PARTS + p
  float* val;           // [units][G][regions * CAND_SLOTS]: workgroup x, part p from (x * CAND_PARTS + p) * part_slots
  int32_t* idx;         // the same
  int32_t* flag;        // [units] 1 = redo this unit unfused
};

// blocks per workgroup of a scan over g: 16, doubled up to SCAN_MAX_WG_BLOCKS
// while the launch keeps at least 2048 workgroups (each workgroup's set-up is
// then spread over up to 1024 blocks), and further while a unit would have
// more than 1024 workgroups (the candidate selection indexes at most 4096
// region parts, four per workgroup, per head)
constexpr int SCAN_MAX_WG_BLOCKS = 1024;
inline int scan_wg_blocks(const Geom& g) {
  long long maxnb = 0;
  for (int s = 0; s < g.S; ++s) maxnb = g.n[s] / BPK_BLOCK > maxnb ? g.n[s] / BPK_BLOCK : maxnb;
  const long long total = maxnb * g.units();
  int wb = SCAN_MIN_WG_BLOCKS;
  while (wb < SCAN_MAX_WG_BLOCKS && (total / (2 * wb) >= 2048 || maxnb > 1024ll * wb)) wb *= 2;
  return wb;
}

// largest number of sampled groups over the sequences of g
__host__ __device__ inline long long sample_groups(const Geom& g) {
  long long m = 0;
  for (int s = 0; s < g.S; ++s) {
    const long long ns = (g.n[s] / BPK_BLOCK + SAMPLE_STRIDE - 1) / SAMPLE_STRIDE;
    m = ns > m ? ns : m;
  }
  return m;
}

hipError_t launch_scan_sample(const Geom& g, const float* q_basis, const uint8_t* depth,
                              const uint64_t* planes, const uint16_t* scales, const CandBufs& cb,
                              int rows, hipStream_t st);
hipError_t launch_threshold(const Geom& g, int k, const CandBufs& cb, hipStream_t st);
// the candidate part counts set to zero (a scan that may skip units writes
// none for them)
hipError_t launch_zero_counts(const Geom& g, const CandBufs& cb, hipStream_t st);
hipError_t launch_scan_cand(const Geom& g, const float* q_basis, const uint8_t* depth,
                            const uint64_t* planes, const uint16_t* scales, int k,
                            const CandBufs& cb, int rows, hipStream_t st);
// The union of a unit's G lists of k selected rows, written by union_kernel
// (attend.hip) or merged by the selection's workgroup itself: uidx [unit][G k]
// ascending rows, umask [unit][G k] the heads holding each row, ucount [unit].
struct UnionBufs {
  int32_t* uidx;
  uint8_t* umask;
  int32_t* ucount;
};
// the union arrays at the start of an attention workspace (launch_attend's
// and the value-depth attention's begin alike)
UnionBufs union_bufs(const Geom& g, int k, void* ws);
// largest LDS of a selection workgroup that also merges its unit's lists
constexpr size_t CAND_FUSED_LDS = 65536;
// exact top-k among the candidates; with un, also the union of every
// unflagged unit (when its lists and merge fit CAND_FUSED_LDS; the return's
// *fused says whether they did)
hipError_t launch_cand_select(const Geom& g, int k, const CandBufs& cb, int32_t* idx,
                              const UnionBufs* un, bool* fused, hipStream_t st);
// full scan and radix select of the flagged units only
hipError_t launch_scan_flagged(const Geom& g, const float* q_basis, const uint8_t* depth,
                               const uint64_t* planes, const uint16_t* scales, float* scores,
                               const int32_t* flag, int rows, hipStream_t st);
// (with un, also the union of each flagged unit's lists)
hipError_t launch_topk_flagged(const Geom& g, const float* scores, int k, int32_t* idx,
                               const int32_t* flag, const UnionBufs* un, hipStream_t st);
// the number of set flags among flag[0 .. units), into *count (device)
hipError_t launch_count_flags(int units, const int32_t* flag, int32_t* count, hipStream_t st);

size_t attend_ws_bytes(const Geom& g, int k);
hipError_t launch_attend(const Geom& g, int k_dtype, const void* k_rows, const uint16_t* v_rows,
                         const uint16_t* q, const int32_t* idx, int k, float scale, float* out,
                         void* ws, hipStream_t st);
// the union stage alone, into ub
hipError_t launch_union(const Geom& g, const int32_t* idx, int k, const UnionBufs& ub,
                        hipStream_t st);
// launch_attend after its union stage (the workspace already holds the union)
hipError_t launch_attend_rows(const Geom& g, int k_dtype, const void* k_rows,
                              const uint16_t* v_rows, const uint16_t* q, int k, float scale,
                              float* out, void* ws, hipStream_t st);

// union of the heads' selections and, per split of 256 union rows, the
// softmax terms e_hr = exp(l_hr - m_h) ([unit][G][G * k], 0 where head h did
// not select row r) and the split's (m_h, sum_r e_hr) ([unit][split][G][2]),
// as the first half of launch_attend; uidx / umask / ucount as its union stage
constexpr int ATT_SPLIT_ROWS = 256;
// (and each union row's value scale, as fp32 [unit][G * k])
// (union_ready: uidx / umask / ucount already hold the union, idx is not read)
hipError_t launch_union_logits(const Geom& g, int k_dtype, const void* k_rows, const uint16_t* q,
                               const int32_t* idx, int k, float scale, int32_t* uidx,
                               uint8_t* umask, int32_t* ucount, float* e, float* stats,
                               const uint16_t* vscales, float* vsc, bool union_ready,
                               hipStream_t st);

// ---- value-side depths (values.hip) ----
// code the value rows of tokens [n0, n0 + n_new) of sequence seq
hipError_t launch_vencode(const Geom& g, int seq, const uint16_t* v_rows, uint8_t* vplanes,
                          uint16_t* vscales, long long n0, long long n_new, hipStream_t st);
size_t attend_v_ws_bytes(const Geom& g, int k);
// (union_ready: the workspace's union arrays already hold the union of idx)
hipError_t launch_attend_v(const Geom& g, int k_dtype, const void* k_rows, const uint8_t* vplanes,
                           const uint16_t* vscales, const uint16_t* q, const int32_t* idx, int k,
                           float scale, int v_budget, float* out, int32_t* union_out,
                           uint8_t* vdepth_out, void* ws, bool union_ready, hipStream_t st);
hipError_t launch_value_depth(const Geom& g, const int32_t* rows, const int32_t* n_rows,
                              int row_ld, const float* weights, const uint16_t* vscales,
                              int v_budget, uint8_t* depth, hipStream_t st);

// ---- small device helpers ----
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Code of one value: clip(floor(v / s), -8, 7) + 8 with the exact real floor.
// m * s and (m + 1) * s are exact in fp32 (|m| < 2^5, s has 11 significant
// bits), so the correction removes any rounding of the quotient.
__device__ __forceinline__ uint32_t quant_code(float v, float s) {
  if (s == 0.f) return 8u;
  float m = floorf(v / s);
  if (m * s > v)
    m -= 1.f;
  else if ((m + 1.f) * s <= v)
    m += 1.f;
  m = fminf(fmaxf(m, -8.f), 7.f);
  return (uint32_t)((int)m + 8);
}

// fp16 scale of a maximum magnitude: amax / 8 rounded to nearest even,
// saturated at 65504 (amax / 8 is exact in fp32)
__device__ __forceinline__ _Float16 scale_of_max(float amax) {
  _Float16 hs = (_Float16)(amax * 0.125f);
  if (__builtin_isinf((float)hs)) hs = (_Float16)65504.0f;
  return hs;
}

// monotone map float -> uint32 (larger float, larger key); -0 is mapped to +0
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// always-kept tail of a sequence of n tokens: the last 32, or the whole open
// block when it holds more
__host__ __device__ inline long long kept_tail(long long n) {
  return (n % BPK_BLOCK) > 32 ? (n % BPK_BLOCK) : 32;
}

}  // namespace bpk
