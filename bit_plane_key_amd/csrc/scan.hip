// Prefix-plane key scan (Fathom §1, §3.2): approximate scores of every key of
// every complete block, reading only planes p < t_j of each read channel and
// the fp16 block scales of those channels.  This file holds the kernel for
// units that read at most SCAN_FAST_ROWS plane rows (budgets up to 128
// planes) and the launchers; scan_wide.hip holds the kernel for the others.
//
// Arithmetic.  The t-bit prefix value of a 4-bit code is
//   m = sum_{p<t} 2^(3-p) b_p + 2^(3-t) - 8 = sum_{p<t} 2^(3-p) (b_p - 1/2)
// (plane 0 = most significant bit), so with one row r = (j, p) per read plane
// and the weight w_r = q_hj s_bj 2^(3-p):
//   s_hat = sum_j q_hj s_bj m_ij = sum_r w_r (b_r - 1/2) = S - C/2,
//   S = sum_r w_r b_r,  C = sum_r w_r.
// The weights of one 16-block step and head are put in a common fixed-point
// frame, X_r = round(w_r 2^E) (to nearest, ties to even), with E chosen so
// that |X_r| < 2^29, and each X_r is split into four balanced signed bytes
// (one fp64 fma: w_r 2^E is exact in fp64).  S and C are then exact integer
// contractions of int8 digits with 0/1 bits, and the score is
// s_hat = (2 S - C) 2^-(E+1).  E comes from max_j |q_hj| 8 smax_j over the
// step (smax_j = the largest scale of channel j in the step); a block whose own
// largest weight may be more than 4x smaller (tested on the channel that sets
// the frame) gets a frame of its own, so every block's largest weight is at
// least 2^26 units.  Frames depend only on the step's blocks, so scores are
// bit-identical in every launch mode.
//
// Error bound.  Rounding X_r moves the score by at most sum_r |X_r - w_r 2^E|
// |b_r - 1/2| <= R/4 units of 2^-E, the fp32 assembly of 2 S - C by at most
// 4 units plus 2^-23 of the score.  A token's L1 mass sum_j |q_hj s_bj m_ij|
// is at least the largest weight / 16 (|m| >= 2^(3-t) >= 1/2), so at least
// 2^22 units, and the error is below (R/4 + 4) 2^-22 + 2^-23 <= 1e-5 of the L1
// mass for every R <= 128 (the 1e-4 tolerance holds with a factor of 10).
//
// The candidate test (decode_step's fused selection) is a cheap superset of
// "written score >= theta": it drops the two low digit rows of S and C (at
// most 3 R (2^15 + 2^7) units of 2 S - C) and compares the high halves with a
// per-(head, block) integer threshold (cand_tau).  Passing tokens are appended
// with their exact scores; the selection keeps only those at or above theta.
//
// Mapping onto gfx950 (fast kernel):
// * A workgroup (4 wavefronts, two per CU) owns a range of blocks of one unit
//   and walks it in steps of 16 blocks, with one barrier per step.  Each
//   thread prefetches its share of the step's plane words (coalesced 128-byte
//   reads of every read row; buffer loads at offsets fixed per thread, rows
//   past the last read one out of range so that they read zeros) two steps
//   ahead and the fp16 scales three steps ahead, in registers; at the top of a
//   step they go to LDS (planes double-, scales triple-buffered), and after the
//   barrier wavefront w computes the frames of head w for the next step.
// * Wavefront w then takes blocks 4w .. 4w+3 one at a time: it writes the
//   block's X digits (4 bytes per (row, head)) into its own LDS records and
//   contracts them with the plane bits on the matrix cores,
//   v_mfma_i32_16x16x64_i8 (a 32-row remainder as the same product with
//   zero A bytes in the upper half of each K group).  Both
//   operands come from LDS through the transposing read ds_read_b64_tr_b8:
//   the B bytes are the raw plane words, each byte holding 8 tokens of one
//   row, and one AND per 4 bytes keeps bit 2c + (n / 8) of column n, so the
//   four matrices c = 0..3 give the 64 tokens of the block, token
//   8 (n % 8) + 2c + n / 8 in column n, scaled by 2^(2c + n / 8) (by -2^7 for
//   bit 7: the int8 byte 0x80 is -128).  A fifth product with all-one bytes
//   gives C.
// * Lane l ends with the four digit sums of head 4 hg + l / 16 for its
//   token; the candidate test combines the two high ones, and one branch per
//   block skips the appends when no lane passes.
#include "scan_common.h"

namespace bpk {
namespace {

constexpr int NB = 4;                 // blocks per wavefront per step
static_assert(SCAN_THREADS / 64 == CAND_PARTS, "one candidate part per wavefront");
constexpr int GB = SCAN_GB;           // blocks per step
constexpr int PSTRIDE = 136;          // LDS bytes per plane row: 16 words + 8 bytes of padding
constexpr int SCS = 20;               // LDS fp16 slots per read channel: 16 blocks + 4 of padding
constexpr int RM_SMALL = 96;          // row capacity of the three-workgroups-per-CU variant
constexpr long long FAST_MAX_CAP = 1ll << 25;   // one unit's planes fit a 32-bit buffer offset
constexpr int FLAGGED_SPAN = 4096;              // blocks per workgroup of a flagged-units scan
constexpr uint32_t OUT_OF_RANGE = 0x80000000u;  // a buffer offset past every unit's planes
constexpr int RSRC_WORD3 = 0x00020000;          // raw (untyped) buffer, 32-bit data format

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LDS of a workgroup whose unit reads at most RM plane rows (and so at most
// RM channels)
template <int HG, int RM>
struct FastSmem {
  static constexpr int GP = 4 * HG;               // heads, padded to whole MFMA row groups
  alignas(16) uint8_t planes[2][RM * PSTRIDE];    // per step parity: [row][block] words
  alignas(16) uint8_t atab[4][RM][16 * HG];       // per wavefront: [row] X digits, 4 bytes a head
  alignas(16) uint8_t azero[16][16 * HG];         // zero A rows (upper K groups of a 32-row pass)
  alignas(16) uint16_t sc[3][RM][SCS];            // per step mod 3: fp16 scales [read channel][block]
  float smax[3][RM];                              // per step mod 3: largest scale of a read channel
  float q[GP][D];                                 // the unit's query heads (0 beyond G)
  int tlo[2][GP][GB];                             // per step parity: cand_tau + 1 of (head, block)
  int ex[2][GP][GB];                              // per step parity: frame exponent of (head, block)
  int exh[2][GP];                                 // per step parity: frame exponent of the step
  int own[2][GP];                                 // per step parity: a block of the head has its own frame
  int wsum[2];                                    // plan: (rows, read channels) of channels 0-63, 64-127
  uint8_t rowc[RM];                               // read channel of each plane row
  uint8_t rowp[RM];                               // plane of each plane row
  uint8_t chj[RM];                                // channel of each read channel
  int ccount[GP];                                 // candidates of this workgroup per head
  int wcount[4][GP];                              // candidates of each wavefront's part, per head
  float qa8[GP][128];                             // |q_hj| 8 of read channel c (0 past the read ones)
  float theta[GP];                                // candidate threshold of each head
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           RSRC_WORD3);
}

template <int G, int MODE, int RM>
__global__ __launch_bounds__(SCAN_THREADS, G == 8 ? 1 : (RM <= RM_SMALL ? 3 : 2)) void scan_fast_kernel(
    ScanArgs a) {
  constexpr int HG = (G + 3) / 4;
  using SM = FastSmem<HG, RM>;
  constexpr int GP = SM::GP;
  constexpr int NPAIR = GP / 2;           // head pairs of a row (8-byte record halves)
  constexpr int RPP = 64 / NPAIR;         // rows per builder pass
  __shared__ __attribute__((aligned(16))) SM sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int u = blockIdx.y;
  const long long gu = a.g.global_unit(u);
  const long long n = a.g.n[a.g.seq_of(u)];
  const long long nb = n / BLK;
  if constexpr (MODE == SCAN_FULL) {
    if (a.unit_flag && a.unit_flag[u] == 0) return;
  }
  if constexpr (MODE == SCAN_CAND) {
    if (n <= a.k) return;  // everything is selected
  }
  const long long span = MODE == SCAN_SAMPLE ? SAMPLE_GROUP : a.wg_blocks;
  const long long wb0 = (long long)blockIdx.x * (MODE == SCAN_SAMPLE ? SAMPLE_STRIDE : a.wg_blocks);
  if (wb0 >= nb) return;
  const long long wb1 = (wb0 + span) < nb ? (wb0 + span) : nb;
  const long long nbcap = a.g.nbcap();
  const long long cand_hi = n - kept_tail(n);  // candidates are tokens [4, cand_hi)

  // ---- where a score goes ----
  auto region = [&](int h) {
    return ((long long)u * G + h) * a.regions * CAND_SLOTS +
           (long long)blockIdx.x * CAND_PARTS * a.part_slots;
  };
  auto store = [&](long long tok, int h, float s) {  // FULL / SAMPLE
    const long long uh = (long long)u * G + h;
    if constexpr (MODE == SCAN_FULL) {
      a.out[uh * a.out_ld + tok] = s;
    } else {
      a.sample[uh * a.out_ld + (long long)blockIdx.x * (SAMPLE_GROUP * BLK) + (tok - wb0 * BLK)] =
          (uint16_t)(order_key(s) >> 16);
    }
  };
  // (only where nothing is read) the workgroup's candidates fill each head's
  // region front to back through an LDS counter
  auto append = [&](long long tok, int h, float s) {
    if (tok < 4 || tok >= cand_hi) return;
    const int off = atomicAdd(&sm.ccount[h], 1);
    if (off < CAND_PARTS * a.part_slots) {
      a.cand_val[region(h) + off] = s;
      a.cand_idx[region(h) + off] = (int32_t)tok;
    }
  };
  auto store_counts = [&]() {
    if constexpr (MODE == SCAN_CAND) {
      __syncthreads();
      if (tid < G)
        contiguous_part_counts(
            a.cand_count + (((long long)u * G + tid) * a.regions + blockIdx.x) * CAND_PARTS,
            sm.ccount[tid], a.part_slots);
    }
  };

  // ---- plan: plane rows channel by channel (j ascending, p ascending) ----
  // inclusive prefix sums of (depth, read flag) over the channels, held by
  // wavefronts 0 and 1; the unit's row count comes first so that a unit of
  // another launch leaves at once
  int tj = 0;
  if (tid < D) {
    tj = a.depth[(long long)u * D + tid];
    tj = tj > NP ? NP : tj;
  }
  int pre = tid < D ? (tj | ((tj > 0) << 16)) : 0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(pre, off);
    if (lane >= off) pre += o;
  }
  if (lane == 63 && wave < 2) sm.wsum[wave] = pre;
  __syncthreads();
  const int tot = sm.wsum[0] + sm.wsum[1];
  const int R = tot & 0xFFFF;
  const int CR = tot >> 16;                  // read channels
  if (R > RM || R <= a.rows_above) return;   // another launch's unit (uniform)
  if (wave == 1) pre += sm.wsum[0];
  if (MODE == SCAN_CAND && tid < GP) sm.ccount[tid] = 0;
  if (MODE == SCAN_CAND && tid < 4 * GP) (&sm.wcount[0][0])[tid] = 0;
  if (tid < 4 * 16 * HG) reinterpret_cast<uint32_t*>(&sm.azero[0][0])[tid] = 0u;
  for (int i = tid; i < GP * D; i += SCAN_THREADS) {
    const int h = i / D;
    sm.q[h][i % D] = h < G ? a.q_basis[((long long)u * G + h) * D + i % D] : 0.f;
  }
  if (tid < 2 * GP * GB) {  // padding heads never pass
    const int h = (tid / GB) % GP;
    if (h >= G) sm.tlo[tid / (GP * GB)][h][tid % GB] = (1 << 24) + 1;
  }
  if (tid < D && tj > 0) {
    const int r0 = (pre & 0xFFFF) - tj;
    const int c = (pre >> 16) - 1;
    sm.chj[c] = (uint8_t)tid;
    for (int p = 0; p < tj; ++p) {
      sm.rowc[r0 + p] = (uint8_t)c;
      sm.rowp[r0 + p] = (uint8_t)p;
    }
  }
  __syncthreads();

  if (R == 0) {  // nothing is read: every score is 0
    float theta[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
      theta[h] = MODE == SCAN_CAND ? key_to_float(a.thresh[(long long)u * G + h]) : 0.f;
    // (wb1 - wb0) * 64 is a multiple of 64: each wavefront's lanes run the same trips
    for (long long e = tid; e < (wb1 - wb0) * BLK; e += SCAN_THREADS) {
      const long long tok = wb0 * BLK + e;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if constexpr (MODE == SCAN_CAND) {
          if (0.f >= theta[h]) append(tok, h, 0.f);
        } else {
          store(tok, h, 0.f);
        }
      }
    }
    store_counts();
    return;
  }

  const int nsteps = (int)((wb1 - wb0 + GB - 1) / GB);
  const int rpt = (R + 31) / 32;  // 32-row pieces of the K passes (A is zero beyond R)
  auto step_g0 = [&](int i) { return wb0 + (long long)i * GB; };
  auto step_blocks = [&](int i) {
    const long long r = wb1 - step_g0(i);
    return r < GB ? (int)r : GB;
  };
  const long long g0_last = step_g0(nsteps - 1);
  // the unit's planes and scales; a step's loads use a buffer based at its
  // first block (steps past the range re-read the last one, never used)
  const long long unit_words = (long long)D * NP * nbcap;
  const uint64_t* ubase = a.planes + gu * unit_words;
  const uint16_t* sbase = a.scales + gu * (long long)D * nbcap;
  auto step_first = [&](int i) { return step_g0(i) < g0_last ? step_g0(i) : g0_last; };
  auto plane_rsrc = [&](int i) {
    const long long f = step_first(i);
    return make_rsrc(ubase + f, (uint32_t)((unit_words - f) * 8));
  };
  auto scale_rsrc = [&](int i) {
    const long long f = step_first(i);
    return make_rsrc(sbase + f, (uint32_t)(((long long)D * nbcap - f) * 2));
  };

  // ---- scales: thread t loads read channel t / 2, blocks 8 (t % 2) .. +7 ----
  const int sc_c = tid >> 1, sc_h = tid & 1;
  const bool svalid = sc_c < CR;
  const long long srow = svalid ? (long long)sm.chj[sc_c] * nbcap : 0;
  // byte offsets; in the last step clamped to the row's stride (the words
  // past the step's blocks are never used)
  uint32_t soff = OUT_OF_RANGE, soff_last = OUT_OF_RANGE;
  if (svalid) {
    soff = (uint32_t)((srow + 8 * sc_h) * 2);
    const long long w = (g0_last + 8 * sc_h) < nbcap - 8 ? (g0_last + 8 * sc_h) : nbcap - 8;
    soff_last = (uint32_t)((srow + w - g0_last) * 2);
  }
  u32x4 sw;  // scales of the next step to write
  auto issue_scales = [&](int i) {
    const auto rs = scale_rsrc(i);
    sw = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(i >= nsteps - 1 ? soff_last : soff), 0, 0);
  };
  auto write_scales = [&](int i) {  // scales of step i and their per-channel max
    const int b3 = i % 3;
    // fp16 bits of non-negative values order like the values; only the step's blocks count
    u16x2 mv = {0, 0};
    if (step_blocks(i) == GB) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        // the word goes through a scalar first: a bit cast of the vector
        // element itself compiled to a read of element 0 for every x
        const uint32_t w = sw[x];
        mv = __builtin_elementwise_max(mv, __builtin_bit_cast(u16x2, w));
      }
    } else {
      const int nv = step_blocks(i) - 8 * sc_h;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t keep = (2 * x < nv ? 0xFFFFu : 0u) | (2 * x + 1 < nv ? 0xFFFF0000u : 0u);
        mv = __builtin_elementwise_max(mv, __builtin_bit_cast(u16x2, sw[x] & keep));
      }
    }
    uint32_t m = mv.x > mv.y ? mv.x : mv.y;
    const uint32_t mo = lane_xor1(m);
    m = mo > m ? mo : m;
    if (svalid) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(&sm.sc[b3][sc_c][8 * sc_h]);  // 8-byte aligned
      *reinterpret_cast<uint2*>(dst) = make_uint2(sw.x, sw.y);
      *reinterpret_cast<uint2*>(dst + 2) = make_uint2(sw.z, sw.w);
      if (sc_h == 0) sm.smax[b3][sc_c] = half_bits_to_f32((uint16_t)m);
    }
  };

  // Frames of a step: one wavefront computes them for every head: 16-lane row
  // r takes head 4 k + r, and lane b of the row takes block b of the step and
  // the read channels 8 b .. 8 b + 7; the thresholds of the heads and |q_hj| 8
  // of every head and read channel go to LDS once (seen by the frames after
  // the prologue's barrier).
  if (tid < FastSmem<HG, RM>::GP)
    sm.theta[tid] = (MODE == SCAN_CAND && tid < G) ? key_to_float(a.thresh[(long long)u * G + tid]) : 0.f;
  for (int e = tid; e < FastSmem<HG, RM>::GP * 128; e += SCAN_THREADS) {
    const int h = e >> 7, c = e & 127;
    sm.qa8[h][c] = (h < G && c < CR) ? fabsf(sm.q[h][sm.chj[c]]) * 8.f : 0.f;
  }

  // the frame of (head h, block blk): E of the step (from the largest key,
  // value bits and read channel, over the head's read channels), the block's
  // own exponent, and the candidate test threshold
  auto frame_write = [&](int par, int b3, int gblk, int h, int blk, uint32_t key, float theta,
                         bool& own) {
    // an upper bound of the largest |q| 8 smax, and the channel that reaches it
    const float best = key ? __uint_as_float((key & 0xFFFFFF00u) + 0x100u) : 0.f;
    const int cs = (int)(key & 0xFFu);
    const int E = frame_exp(best, FRAME_BITS);
    int eb = E;
    own = false;
    if (blk < gblk && best > 0.f) {
      // the block's own largest weight is at least a quarter of the frame's
      // if the channel that sets the frame keeps a quarter of its step max
      if (4.f * half_bits_to_f32(sm.sc[b3][cs][blk]) < sm.smax[b3][cs]) {
        // the block's largest weight, over the read channels (|q| 8 from
        // qa8, zero past CR; 8 channels' reads in flight at a time)
        float mb = 0.f;
        for (int c0 = 0; c0 < CR; c0 += 8) {
#pragma unroll
          for (int c = c0; c < c0 + 8; ++c)
            mb = fmaxf(mb, sm.qa8[h][c] * half_bits_to_f32(sm.sc[b3][c < RM ? c : 0][blk]));
        }
        eb = frame_exp(mb, FRAME_BITS);
        own = eb != E;
      }
    }
    if (h < G && blk < GB) {
      sm.ex[par][h][blk] = eb;
      if constexpr (MODE == SCAN_CAND) sm.tlo[par][h][blk] = cand_tau(theta, eb, R) + 1;
    }
    return E;
  };

  // ---- frames of step i, by the calling wavefront for every head; every
  // lane of the wavefront must be active ----
  auto compute_frame = [&](int i) {
    const int par = i & 1, b3 = i % 3, gblk = step_blocks(i);
    const int frow = lane >> 4, fblk = lane & 15;
#pragma unroll
    for (int k = 0; k < HG; ++k) {
      const int h = 4 * k + frow;  // heads past G compute zeros and write nothing
      uint32_t key = 0;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int c = 8 * fblk + m;
        const float v = sm.qa8[h][c] * (c < CR ? sm.smax[b3][c] : 0.f);
        const uint32_t kk = v > 0.f ? (__float_as_uint(v) & 0xFFFFFF00u) | (uint32_t)c : 0u;
        key = kk > key ? kk : key;
      }
      key = row_max_u32_dpp(key);
      bool own;
      const int E = frame_write(par, b3, gblk, h, fblk, key, sm.theta[h], own);
      const uint64_t ob = __ballot(own);
      if (h < G && fblk == 0) {
        sm.exh[par][h] = E;
        sm.own[par][h] = ((ob >> (16 * frow)) & 0xFFFFull) != 0ull;
      }
    }
  };

  // ---- the main loop, specialised on the K passes: RPT 32-row pieces, that
  // is RPT / 2 passes of 64 rows and, for odd RPT, one of 32 ----
  auto main_loop = [&](auto RPTC) {
    constexpr int RPT = decltype(RPTC)::value;
    constexpr int N64 = RPT / 2;
    constexpr bool HAS32 = (RPT & 1) != 0;
    constexpr int NPASS = 32 * RPT / RPP;  // builder passes
    constexpr int PL = RPT;                // 16-byte plane loads per thread and step

    // ---- plane loads: slot k covers row (tid + 256 k) / 8, words
    // 2 ((tid + 256 k) % 8), +1 of the step; rows >= R read zeros ----
    uint32_t poff[PL], poff_last[PL];  // byte offsets; in the last step clamped to the capacity
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const int e = tid + k * SCAN_THREADS, r = e >> 3, part = 2 * (e & 7);
      poff[k] = poff_last[k] = OUT_OF_RANGE;
      if (r < R) {
        const long long row = ((long long)sm.chj[sm.rowc[r]] * NP + sm.rowp[r]) * nbcap;
        poff[k] = (uint32_t)((row + part) * 8);
        const long long w = (g0_last + part) < nbcap - 2 ? (g0_last + part) : nbcap - 2;
        poff_last[k] = (uint32_t)((row + w - g0_last) * 8);
      }
    }
    u32x4 pw[PL];  // plane words of the next step to write
    auto issue_planes = [&](int i) {
      const auto rs = plane_rsrc(i);
      const bool last = i >= nsteps - 1;
#pragma unroll
      for (int k = 0; k < PL; ++k)
        pw[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(last ? poff_last[k] : poff[k]), 0, 0);
    };
    auto write_planes = [&](int i) {  // rows are 8-byte aligned
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const int e = tid + k * SCAN_THREADS;
        uint8_t* dst = &sm.planes[i & 1][(e >> 3) * PSTRIDE + 16 * (e & 7)];
        *reinterpret_cast<uint2*>(dst) = make_uint2(pw[k].x, pw[k].y);
        *reinterpret_cast<uint2*>(dst + 8) = make_uint2(pw[k].z, pw[k].w);
      }
    };

    // builder items: pass m covers row RPP m + lane / NPAIR and heads
    // 2 (lane % NPAIR), +1; rows >= R have zero weights, hence zero digits
    const int prow = lane / NPAIR, ppair = lane % NPAIR;
    // q_hj 2^(3-p+E_h) of the item's row and heads in the current step's frames
    // (exact power-of-two rescalings from step to step; the frame exponents
    // they are in are fexp)
    double fqe[NPASS][2];
    int fexp[2] = {0, 0};
    int soffm[NPASS];     // the item's row's scales in sc[.]: read channel * SCS
#pragma unroll
    for (int m = 0; m < NPASS; ++m) {
      const int r = m * RPP + prow;
      soffm[m] = (r < R ? sm.rowc[r] : 0) * SCS;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int h = 2 * ppair + x;
        fqe[m][x] = (r < R && h < G) ? ldexp((double)sm.q[h][sm.chj[sm.rowc[r]]], 3 - sm.rowp[r]) : 0.0;
      }
    }

    // MFMA operand addressing: lane l is column / A-row l % 16 of K-group l / 16;
    // a transposing read takes, in each 16-lane group, row r0 + (l % 16) / 2
    const int kg = lane >> 4, s16 = lane & 15;
    const int rsub = s16 >> 1, ahalf = 8 * (s16 & 1), hb = s16 >> 3;
    uint32_t bmask[4];  // product c keeps bit bp = 2c + hb of each byte in column n
#pragma unroll
    for (int c = 0; c < 4; ++c) bmask[c] = 0x01010101u << (2 * c + hb);
    const int neg3 = hb ? -1 : 0;  // lanes whose c = 3 column keeps bit 7 (v = -128)
    const i32x4 ones4 = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const i32x4 zero4 = {0, 0, 0, 0};
    // a register pair whose contents never matter: it only meets zero A bytes
    auto junk2 = []() {
      i32x2 v;
      asm volatile("" : "=v"(v));
      return v;
    };

    // fp16 scale of block b (0..3) of the wavefront's four, from a pass's 8 bytes
    auto scale_of = [](const u32x2& v, int b) {
      const uint32_t w = b < 2 ? v.x : v.y;
      return __builtin_bit_cast(_Float16, (uint16_t)((b & 1) ? (w >> 16) : w));
    };
    // A records of the wavefront's block b
    auto build = [&](int b, const double (&fqe)[NPASS][2], const u32x2 (&scl)[NPASS]) {
      uint8_t* rec = &sm.atab[wave][prow][8 * ppair];
#pragma unroll
      for (int m = 0; m < NPASS; ++m) {
        const double sv = (double)(float)scale_of(scl[m], b);
        *reinterpret_cast<uint2*>(rec + m * RPP * (16 * HG)) =
            make_uint2(x_digits4(fqe[m][0], sv), x_digits4(fqe[m][1], sv));
      }
    };
    // the same for a step where some (head, block) has a frame of its own
    auto build_own = [&](int par, int wb, int b, const double (&fqe)[NPASS][2],
                         const u32x2 (&scl)[NPASS], const int (&exh2)[2]) {
      double g[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int h = 2 * ppair + x;
        g[x] = h < G ? ldexp(1.0, sm.ex[par][h][wb + b] - exh2[x]) : 0.0;
      }
      uint8_t* rec = &sm.atab[wave][prow][8 * ppair];
#pragma unroll
      for (int m = 0; m < NPASS; ++m) {
        const double sv = (double)(float)scale_of(scl[m], b);
        *reinterpret_cast<uint2*>(rec + m * RPP * (16 * HG)) =
            make_uint2(x_digits4(fqe[m][0] * g[0], sv), x_digits4(fqe[m][1] * g[1], sv));
      }
    };
    // operands of block blk (planes pl, the wavefront's A records), read from LDS
    // ahead of their products
    struct Ops {
      i32x4 b[N64 ? N64 : 1];
      i32x4 a[N64 ? N64 : 1][HG];
      i32x2 b32;
      i32x4 a32[HG];  // 32 rows in the lower half of each K group, zeros above
    };
    auto fetch = [&](const uint8_t* pl, int blk, Ops& o) {
      const uint8_t* at = &sm.atab[wave][0][0];
#pragma unroll
      for (int kp = 0; kp < N64; ++kp) {
        const int r0 = 64 * kp + 16 * kg + rsub;
        const i32x2 b0 = tr8(pl + r0 * PSTRIDE + 8 * blk);
        const i32x2 b1 = tr8(pl + (r0 + 8) * PSTRIDE + 8 * blk);
        o.b[kp] = i32x4{b0.x, b0.y, b1.x, b1.y};
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const i32x2 a0 = tr8(at + r0 * (16 * HG) + 16 * hg + ahalf);
          const i32x2 a1 = tr8(at + (r0 + 8) * (16 * HG) + 16 * hg + ahalf);
          o.a[kp][hg] = i32x4{a0.x, a0.y, a1.x, a1.y};
        }
      }
      if constexpr (HAS32) {
        const int r0 = 64 * N64 + 8 * kg + rsub;
        o.b32 = tr8(pl + r0 * PSTRIDE + 8 * blk);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const i32x2 a0 = tr8(at + r0 * (16 * HG) + 16 * hg + ahalf);
          const i32x2 a1 = tr8(&sm.azero[rsub][16 * hg + ahalf]);
          o.a32[hg] = i32x4{a0.x, a0.y, a1.x, a1.y};
        }
      }
    };
    auto mask4 = [](const i32x4& v, uint32_t m) {
      const int mi = (int)m;
      return i32x4{v.x & mi, v.y & mi, v.z & mi, v.w & mi};
    };
    // digit sums of a block from its operands
    auto contract = [&](const Ops& o, i32x4 (&acc)[HG][4], i32x4 (&accc)[HG]) {
#pragma unroll
      for (int kp = 0; kp < N64; ++kp) {
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[hg][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(o.a[kp][hg], mask4(o.b[kp], bmask[c]),
                                                               kp ? acc[hg][c] : zero4, 0, 0, 0);
          accc[hg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(o.a[kp][hg], ones4, kp ? accc[hg] : zero4, 0, 0, 0);
        }
      }
      if constexpr (HAS32) {
        // the 32-row remainder as a K = 64 product whose A bytes are zero in
        // the upper half of each lane (the K = 32 form's result latency is not
        // reliably waited for); B's upper half is left as it is
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const i32x4& av = o.a32[hg];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int m = (int)bmask[c];
            const i32x2 j = junk2();
            acc[hg][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, i32x4{o.b32.x & m, o.b32.y & m, j.x, j.y},
                                                               N64 ? acc[hg][c] : zero4, 0, 0, 0);
          }
          accc[hg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, ones4, N64 ? accc[hg] : zero4, 0, 0, 0);
        }
      }
    };
    // exact score of column c of product c
    auto exact_score = [&](const i32x4& d, const i32x4& dc, int c, int eb) {
      return score4(d, dc, 2 * c + hb, c == 3 && hb, eb);
    };
    // scores of block blk: lane <-> (head 4 hg + l / 16, column l % 16)
    // candidates: wavefront w fills part w of each head's region, its slots
    // handed out by its own LDS counter per head (sm.wcount[w][h]; the count
    // may pass the part's size, which the selection flags).  Offsets within
    // the unit's buffers fit 32 bits (capacity <= FAST_MAX_CAP).
    const uint32_t cand_bytes = MODE == SCAN_CAND ? (uint32_t)(G * a.regions * CAND_SLOTS * 4) : 0u;
    const auto cval_rsrc =
        make_rsrc(MODE == SCAN_CAND ? a.cand_val + (long long)u * G * a.regions * CAND_SLOTS : a.out, cand_bytes);
    const auto cidx_rsrc =
        make_rsrc(MODE == SCAN_CAND ? (const void*)(a.cand_idx + (long long)u * G * a.regions * CAND_SLOTS)
                                    : (const void*)a.out,
                  cand_bytes);
    // head h's slots start at h * head_ld, this wavefront's part at part_off
    const int head_ld = (int)(a.regions * CAND_SLOTS);
    const int part_off = (int)(blockIdx.x * CAND_PARTS + wave) * a.part_slots;
    auto scores = [&](int par, long long g0, int blk, const i32x4 (&acc)[HG][4], const i32x4 (&accc)[HG],
                      const int (&tl)[HG], const int (&exb)[HG]) {
      const long long tok0 = (g0 + blk) * BLK + 8 * (s16 & 7) + hb;
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const int h = 4 * hg + kg;
        const i32x4 dc = accc[hg];
        if constexpr (MODE == SCAN_CAND) {
          // 2 P' - C_hi >= tau  <=>  P' >= kap = ceil((tau + C_hi) / 2), with
          // P = v P' the raw high digit sums: P >= kap 2^bp, or for v = -128
          // (c = 3, bit 7) -P >= kap 2^7, i.e. ~P >= kap 2^7 - 1
          const int kap = (tl[hg] + (dc.w * 256 + dc.z)) >> 1;  // tl = tau + 1
          const uint32_t kh = (uint32_t)kap << hb;
          bool pass[4];
          int p[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const i32x4 d = acc[hg][c];
            p[c] = d.w * 256 + d.z;
            const int th = (int)((kh << (2 * c)) + (uint32_t)(c == 3 ? neg3 : 0));
            pass[c] = (c == 3 ? (p[c] ^ neg3) : p[c]) >= th;
          }
          if (__ballot(pass[0] || pass[1] || pass[2] || pass[3]) != 0ull) {
            // tokens outside [4, cand_hi) are never candidates: only the unit's
            // first block and its last ones hold such tokens
            if ((g0 + blk) == 0 || (g0 + blk + 1) * BLK > cand_hi) {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const long long tok = tok0 + 2 * c;
                pass[c] = pass[c] && tok >= 4 && tok < cand_hi;
              }
            }
            // exact score: T_hi = 2 P' - C_hi, T_lo = 2 S_lo - C_lo (units of
            // 2^16 and 1), with P' = P / v and S_lo = (2^8 D1 + D0) / v; the
            // raw sums are multiples of 2^bp and, for R <= 128, within 2^29
            const int nchi = -(dc.w * 256 + dc.z);
            const int nclo = -(dc.y * 256 + dc.x);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              if (pass[c]) {
                const int slot = atomicAdd(&sm.wcount[wave][h], 1);
                if (slot < a.part_slots) {
                  const int bp = 2 * c + hb;
                  const i32x4 d = acc[hg][c];
                  int ph = p[c] >> bp;
                  int pl = (d.y * 256 + d.x) >> bp;
                  if (c == 3) {  // v = -128 on the lanes with hb = 1
                    ph = (ph ^ neg3) - neg3;
                    pl = (pl ^ neg3) - neg3;
                  }
                  const float th = (float)(2 * ph + nchi), tlo = (float)(2 * pl + nclo);
                  const float sc = ldexpf(__builtin_fmaf(th, 65536.f, tlo), -(exb[hg] + 1));
                  const int off = (h * head_ld + part_off + slot) * 4;
                  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), cval_rsrc, off, 0, 0);
                  __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(tok0 + 2 * c), cidx_rsrc, off, 0, 0);
                }
              }
            }
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (h < G) store(tok0 + 2 * c, h, exact_score(acc[hg][c], dc, c, exb[hg]));
        }
      }
    };

    // ---- one step: the wavefront's blocks ----
    auto blocks = [&](int i) {
      const int par = i & 1, b3 = i % 3;
      const long long g0 = step_g0(i);
      const int wb = NB * wave;
      const int nblk = step_blocks(i) - wb;  // blocks of this wavefront (uniform)
      if (nblk <= 0) return;
      // the rows' weights in this step's frames, and the rows' scales of the
      // wavefront's four blocks
      u32x2 scl[NPASS];
      int exh2[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) exh2[x] = 2 * ppair + x < G ? sm.exh[par][2 * ppair + x] : 0;
#pragma unroll
      for (int m = 0; m < NPASS; ++m) {
#pragma unroll
        for (int x = 0; x < 2; ++x) fqe[m][x] = ldexp(fqe[m][x], exh2[x] - fexp[x]);
        scl[m] = *reinterpret_cast<const u32x2*>(&sm.sc[b3][0][0] + soffm[m] + wb);
      }
      fexp[0] = exh2[0];
      fexp[1] = exh2[1];
      bool own_any = false;
#pragma unroll
      for (int h = 0; h < G; ++h) own_any |= sm.own[par][h] != 0;
      const uint8_t* pl = &sm.planes[par][0];

      // the candidate thresholds of the four blocks for the lane's heads
      int4 tl4[HG];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        if constexpr (MODE == SCAN_CAND) tl4[hg] = *reinterpret_cast<const int4*>(&sm.tlo[par][4 * hg + kg][wb]);
        else tl4[hg] = int4{0, 0, 0, 0};
      }
      // and their frame exponents (heads past G: never used)
      int4 ex4[HG];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) ex4[hg] = *reinterpret_cast<const int4*>(&sm.ex[par][4 * hg + kg][wb]);
      auto pick = [](const int4& v, int b) { return b == 0 ? v.x : b == 1 ? v.y : b == 2 ? v.z : v.w; };
      auto tl_of = [&](int b, int (&tl)[HG], int (&exb)[HG]) {
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          tl[hg] = pick(tl4[hg], b);
          exb[hg] = pick(ex4[hg], b);
        }
      };
      // per block b: score b, then read the operands of b + 1 (its digits
      // were written one block earlier) and issue its products, then write
      // the digits of b + 2 over those of b + 1 (the reads come first: LDS
      // operations of a wavefront complete in order).  A transposing read
      // returns into its registers asynchronously, so the operands are only
      // replaced once the products that read them have completed (the scores
      // of b waited for them).  COMMON: all four blocks present and no block
      // with a frame of its own (the loop then has no run-time test).
      auto run = [&](auto COMMON) {
        constexpr bool common = decltype(COMMON)::value;
        auto bld = [&](int b) {
          if (!common && own_any) build_own(par, wb, b, fqe, scl, exh2);
          else build(b, fqe, scl);
        };
        auto has = [&](int b) { return common ? b < NB : b < nblk; };
        i32x4 acc[HG][4];
        i32x4 accc[HG];
        Ops ops;
        bld(0);
        fetch(pl, wb, ops);
        contract(ops, acc, accc);
        if (has(1)) bld(1);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (!has(b)) break;
          int tl[HG], exb[HG];
          tl_of(b, tl, exb);
          scores(par, g0, wb + b, acc, accc, tl, exb);
          if (has(b + 1)) {
            fetch(pl, wb + b + 1, ops);
            contract(ops, acc, accc);
          }
          if (has(b + 2)) bld(b + 2);
        }
      };
      if (nblk >= NB && !own_any) run(std::true_type{});
      else run(std::false_type{});
    };

    // ---- prologue: scales of steps 0 and 1, planes of step 0, frames of
    // step 0; the loads are issued in the loop's order (planes of i, then
    // scales of i + 1) ----
    issue_scales(0);
    issue_planes(0);
    write_scales(0);
    issue_scales(1);
    __syncthreads();
    if (wave == 0) compute_frame(0);

    // ---- steps: the loads of step i + 1 (planes) and i + 2 (scales) are in
    // flight while step i is computed ----
    for (int i = 0; i < nsteps; ++i) {
      write_planes(i);
      if (i + 1 < nsteps) write_scales(i + 1);
      __syncthreads();  // planes of i, scales of i + 1 and frames of i are in LDS
      issue_planes(i + 1);
      issue_scales(i + 2);
      if (i + 1 < nsteps && wave == ((i + 1) & 3)) compute_frame(i + 1);  // by turns
      blocks(i);
    }
    if constexpr (MODE == SCAN_CAND) {
      // the counters of this wavefront's part (its own LDS atomics completed
      // in order before this read)
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const int h = 4 * hg + kg;
        if (s16 == 0 && h < G)
          a.cand_count[(((long long)u * G + h) * a.regions + blockIdx.x) * CAND_PARTS + wave] =
              sm.wcount[wave][h];
      }
    }
  };
  switch (rpt) {  // rpt <= RM / 32
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 3: main_loop(std::integral_constant<int, 3>{}); break;
    default:
      if constexpr (RM > RM_SMALL) main_loop(std::integral_constant<int, 4>{});
      break;
  }
}

// rows: the plane rows every unit reads (-1: not known, any up to
// SCAN_FAST_ROWS); up to RM_SMALL rows take the variant with the smaller LDS
// footprint (three workgroups per CU).  Not known: both variants are launched
// and each takes its own units.
template <int G, int MODE>
hipError_t launch_fast(const ScanArgs& a0, int rows, hipStream_t st) {
  ScanArgs a = a0;
  a.rows_above = -1;
  long long maxnb = 0;
  for (int s = 0; s < a.g.S; ++s) maxnb = a.g.n[s] / BLK > maxnb ? a.g.n[s] / BLK : maxnb;
  if (maxnb == 0 || a.g.units() == 0) return hipSuccess;
  dim3 grid;
  if (MODE == SCAN_SAMPLE) {
    a.wg_blocks = SAMPLE_GROUP;
    grid = dim3((unsigned)sample_groups(a.g), (unsigned)a.g.units());
  } else {
    int wb = scan_wg_blocks(a.g);
    // the decode step's fallback scan usually finds no unit flagged: larger
    // spans mean fewer workgroups that only read a flag and leave (a flagged
    // unit of 2^20 tokens is then rescored by 4 workgroups)
    if (MODE == SCAN_FULL && a.unit_flag && wb < FLAGGED_SPAN) wb = FLAGGED_SPAN;
    a.wg_blocks = wb;
    grid = dim3((unsigned)((maxnb + wb - 1) / wb), (unsigned)a.g.units());
  }
  if (rows <= RM_SMALL) {  // known and small, or not known: the small variant first
    scan_fast_kernel<G, MODE, RM_SMALL><<<grid, SCAN_THREADS, 0, st>>>(a);
    if (rows >= 0) return hipGetLastError();
    a.rows_above = RM_SMALL;  // not known: the large variant takes the rest
  }
  scan_fast_kernel<G, MODE, SCAN_FAST_ROWS><<<grid, SCAN_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch_fast(const ScanArgs& a, int rows, hipStream_t st) {
  switch (a.g.G) {
    case 1: return launch_fast<1, MODE>(a, rows, st);
    case 2: return launch_fast<2, MODE>(a, rows, st);
    case 4: return launch_fast<4, MODE>(a, rows, st);
    case 8: return launch_fast<8, MODE>(a, rows, st);
    default: return hipErrorInvalidValue;
  }
}

// rows >= 0: every unit reads that many rows, one kernel; rows < 0: both,
// the wide one with fewer, larger workgroups (its workgroups of fast units
// only read the depths and leave).  Capacities past FAST_MAX_CAP take the wide
// kernel for every unit.
template <int MODE>
hipError_t dispatch(const ScanArgs& a, int rows, hipStream_t st) {
  if (a.g.cap > FAST_MAX_CAP) {
    ScanArgs w = a;
    w.all_rows = 1;
    return launch_scan_wide(w, MODE, 0, st);
  }
  if (rows >= 0 && rows <= SCAN_FAST_ROWS) return dispatch_fast<MODE>(a, rows, st);
  if (rows > SCAN_FAST_ROWS) return launch_scan_wide(a, MODE, 0, st);
  const hipError_t e = dispatch_fast<MODE>(a, -1, st);
  if (e != hipSuccess) return e;
  return launch_scan_wide(a, MODE, MODE == SCAN_FULL ? SCAN_WIDE_SPAN : 0, st);
}

ScanArgs base_args(const Geom& g, const float* q_basis, const uint8_t* depth,
                   const uint64_t* planes, const uint16_t* scales) {
  ScanArgs a{};
  a.g = g;
  a.q_basis = q_basis;
  a.depth = depth;
  a.planes = planes;
  a.scales = scales;
  return a;
}

}  // namespace

hipError_t launch_scan(const Geom& g, const float* q_basis, const uint8_t* depth,
                       const uint64_t* planes, const uint16_t* scales, float* scores, int rows,
                       hipStream_t st) {
  ScanArgs a = base_args(g, q_basis, depth, planes, scales);
  a.out = scores;
  a.out_ld = g.cap;
  return dispatch<SCAN_FULL>(a, rows, st);
}

hipError_t launch_scan_flagged(const Geom& g, const float* q_basis, const uint8_t* depth,
                               const uint64_t* planes, const uint16_t* scales, float* scores,
                               const int32_t* flag, int rows, hipStream_t st) {
  ScanArgs a = base_args(g, q_basis, depth, planes, scales);
  a.out = scores;
  a.out_ld = g.cap;
  a.unit_flag = flag;
  return dispatch<SCAN_FULL>(a, rows, st);
}

hipError_t launch_scan_sample(const Geom& g, const float* q_basis, const uint8_t* depth,
                              const uint64_t* planes, const uint16_t* scales, const CandBufs& cb,
                              int rows, hipStream_t st) {
  ScanArgs a = base_args(g, q_basis, depth, planes, scales);
  a.sample = cb.sample;
  a.out_ld = cb.sample_ld;
  return dispatch<SCAN_SAMPLE>(a, rows, st);
}

hipError_t launch_scan_cand(const Geom& g, const float* q_basis, const uint8_t* depth,
                            const uint64_t* planes, const uint16_t* scales, int k,
                            const CandBufs& cb, int rows, hipStream_t st) {
  ScanArgs a = base_args(g, q_basis, depth, planes, scales);
  a.k = k;
  a.thresh = cb.thresh;
  a.regions = cb.regions;
  a.part_slots = cb.part_slots;
  a.cand_count = cb.count;
  a.cand_val = cb.val;
  a.cand_idx = cb.idx;
  return dispatch<SCAN_CAND>(a, rows, st);
}

}  // namespace bpk
