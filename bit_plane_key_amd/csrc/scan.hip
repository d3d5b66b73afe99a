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
// frame, X_r = round(w_r 2^E), with E chosen so that sum_r |X_r| < 2^29, and
// each X_r (|X_r| < 2^23) is split into three balanced signed bytes.  S and C
// are then exact integer contractions of int8 digits with 0/1 bits, and the
// score is s_hat = (2 S - C) 2^-(E+1).  The only rounding is that of X_r (half
// a unit), far below the 1e-4 tolerance relative to the score's own L1 mass
// as long as the frame is within a few bits of each block's largest weight.
// E comes from max_j |q_hj| 8 smax_j over the step (smax_j = the largest scale
// of channel j in the step); a block whose own largest weight may be more
// than 4x smaller (tested on the channel that sets the frame) gets a frame of
// its own.  Frames depend only on the step's blocks, so scores are
// bit-identical in every launch mode.
//
// Mapping onto gfx950 (fast kernel):
// * A workgroup (4 wavefronts, two per CU) owns a range of blocks of one unit
//   and walks it in steps of 16 blocks, with one barrier per step.  Each
//   thread prefetches its share of the step's plane words (coalesced 128-byte
//   reads of every read row) two steps ahead and the fp16 scales three steps
//   ahead, in registers; at the top of a step they go to LDS (planes double-,
//   scales triple-buffered), and after the barrier wavefront w computes the
//   frames of head w for the next step.
// * Wavefront w then takes blocks 4w .. 4w+3 one at a time: it writes the
//   block's X digits (4 bytes per (row, head)) into its own LDS records and
//   contracts them with the plane bits on the matrix cores,
//   v_mfma_i32_16x16x64_i8 (and _16x16x32_i8 for a 32-row remainder).  Both
//   operands come from LDS through the transposing read ds_read_b64_tr_b8:
//   the B bytes are the raw plane words, each byte holding 8 tokens of one
//   row, and one AND per 4 bytes keeps bit 2c + (n / 8) of column n, so the
//   four matrices c = 0..3 give the 64 tokens of the block, token
//   8 (n % 8) + 2c + n / 8 in column n, scaled by 2^(2c + n / 8) (by -2^7 for
//   bit 7: the int8 byte 0x80 is -128).  A fifth product with all-one bytes
//   gives C.
// * Lane l ends with the digit sums of head 4 hg + l / 16 for its token and
//   recombines them with shifts into the int32 S; the candidate test compares
//   (float)(2 S - C) with threshold 2^(E+1), the same value the score is
//   written from.
#include "scan_common.h"

namespace bpk {
namespace {

constexpr int NB = 4;                 // blocks per wavefront per step
constexpr int GB = SCAN_GB;           // blocks per step
constexpr int RMAX = SCAN_FAST_ROWS;  // plane rows at most
constexpr int CMAX = D;               // read channels at most
constexpr int PSTRIDE = 144;          // LDS bytes per plane row: 16 words + 16 bytes of padding
constexpr int PL = RMAX * 8 / SCAN_THREADS;  // 16-byte plane loads per thread and step

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <int HG>
struct FastSmem {
  static constexpr int GP = 4 * HG;               // heads, padded to whole MFMA row groups
  alignas(16) uint8_t planes[2][RMAX * PSTRIDE];  // per step parity: [row][block] words
  alignas(16) uint8_t atab[4][2][RMAX][16 * HG];  // per wavefront, two blocks: [row] X digits, 4 bytes a head
  alignas(16) uint16_t sc[3][CMAX][GB];           // per step mod 3: fp16 scales [read channel][block]
  float smax[3][CMAX];                            // per step mod 3: largest scale of a read channel
  float q[GP][D];                                 // the unit's query heads (0 beyond G)
  float thp[2][GP][GB];                           // per step parity: threshold 2^(E+1) of (head, block)
  int ex[2][GP][GB];                              // per step parity: frame exponent of (head, block)
  int exh[2][GP];                                 // per step parity: frame exponent of the step
  int own[2][GP];                                 // per step parity: a block of the head has its own frame
  int scan_buf[D];                                // plan: prefix sums of (depth, read flag)
  uint8_t rowc[RMAX];                             // read channel of each plane row
  uint8_t rowp[RMAX];                             // plane of each plane row
  uint8_t chj[CMAX];                              // channel of each read channel
  int ccount[GP];                                 // candidates of this workgroup per head
};

// theta 2^(E+1) for the test (float)T >= it, T an integer: values of
// magnitude below 1 (including an underflow to 0) are replaced by +-1/2, which
// decides every integer the same way
__device__ __forceinline__ float scaled_threshold(float theta, int e) {
  float t = ldexpf(theta, e + 1);
  if (theta != 0.f && fabsf(t) < 1.f) t = theta > 0.f ? 0.5f : -0.5f;
  return t;
}

template <int G, int MODE, bool VEC>
__global__ __launch_bounds__(SCAN_THREADS, G == 8 ? 1 : 2) void scan_fast_kernel(ScanArgs a) {
  constexpr int HG = (G + 3) / 4;
  using SM = FastSmem<HG>;
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
    return (((long long)u * G + h) * a.regions + blockIdx.x) * CAND_SLOTS;
  };
  auto store = [&](long long tok, int h, float s) {  // FULL / SAMPLE
    const long long uh = (long long)u * G + h;
    if constexpr (MODE == SCAN_FULL) {
      a.out[uh * a.out_ld + tok] = s;
    } else {
      a.out[uh * a.out_ld + (long long)blockIdx.x * (SAMPLE_GROUP * BLK) + (tok - wb0 * BLK)] = s;
    }
  };
  auto append = [&](long long tok, int h, float s) {  // CAND, a lane whose test passed
    if (tok < 4 || tok >= cand_hi) return;
    const int off = atomicAdd(&sm.ccount[h], 1);
    if (off < CAND_SLOTS) {
      a.cand_val[region(h) + off] = s;
      a.cand_idx[region(h) + off] = (int32_t)tok;
    }
  };
  auto store_counts = [&]() {
    if constexpr (MODE == SCAN_CAND) {
      __syncthreads();
      if (tid < G) a.cand_count[((long long)u * G + tid) * a.regions + blockIdx.x] = sm.ccount[tid];
    }
  };

  // ---- plan: plane rows channel by channel (j ascending, p ascending) ----
  int tj = 0;
  if (MODE == SCAN_CAND && tid < GP) sm.ccount[tid] = 0;
  if (tid < D) {
    tj = a.depth[(long long)u * D + tid];
    tj = tj > NP ? NP : tj;
    sm.scan_buf[tid] = tj | ((tj > 0) << 16);
  }
  for (int i = tid; i < GP * D; i += SCAN_THREADS) {
    const int h = i / D;
    sm.q[h][i % D] = h < G ? a.q_basis[((long long)u * G + h) * D + i % D] : 0.f;
  }
  __syncthreads();
  for (int off = 1; off < D; off <<= 1) {
    int v = 0;
    if (tid < D && tid >= off) v = sm.scan_buf[tid - off];
    __syncthreads();
    if (tid < D) sm.scan_buf[tid] += v;
    __syncthreads();
  }
  const int R = sm.scan_buf[D - 1] & 0xFFFF;
  const int CR = sm.scan_buf[D - 1] >> 16;  // read channels
  if (R > RMAX) return;                      // the wide kernel's unit (uniform)
  if (tid < D && tj > 0) {
    const int r0 = (sm.scan_buf[tid] & 0xFFFF) - tj;
    const int c = (sm.scan_buf[tid] >> 16) - 1;
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

  // frame size: |X| < 2^lx and R 2^lx <= 2^29
  int lx = 29;
  for (int r = R - 1; r > 0; r >>= 1) --lx;  // 29 - ceil(log2 R)
  lx = lx > 22 ? 22 : lx;
  const int nsteps = (int)((wb1 - wb0 + GB - 1) / GB);
  const int rpt = (R + 31) / 32;  // 32-row pieces of the K passes (A is zero beyond R)
  auto step_g0 = [&](int i) { return wb0 + (long long)i * GB; };
  auto step_blocks = [&](int i) {
    const long long r = wb1 - step_g0(i);
    return r < GB ? (int)r : GB;
  };

  // ---- per-thread load slots ----
  // planes: slot k covers row (tid + 256 k) / 8, words 2 ((tid + 256 k) % 8), +1
  // of the step; scales: read channel tid / 2, blocks 8 (tid % 2) .. +7.  With
  // VEC (capacity / 64 a multiple of 8: every plane row 16-byte aligned, every
  // scale row too) each thread issues the same loads at every step, with no
  // branch: rows >= R read row 0, words past the capacity re-read the last
  // ones, steps past the range re-read the last step (duplicates the caches
  // serve, never used).  The compiler can then wait for the oldest step's loads
  // alone, and two steps stay in flight.
  const uint64_t* prow[PL];  // the slot's plane row (row 0 for rows >= R)
  int ppart[PL];
  bool pvalid[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k) {
    const int e = tid + k * SCAN_THREADS, r = e >> 3, rr = r < R ? r : 0;
    prow[k] = a.planes + ((uint64_t)(gu * D + sm.chj[sm.rowc[rr]]) * NP + sm.rowp[rr]) * nbcap;
    ppart[k] = 2 * (e & 7);
    pvalid[k] = r < R;
  }
  const int sc_c = tid >> 1, sc_h = tid & 1;
  const uint16_t* srow = a.scales + (uint64_t)(gu * D + sm.chj[sc_c < CR ? sc_c : 0]) * nbcap;
  const bool svalid = sc_c < CR;
  const long long g0_last = step_g0(nsteps - 1);

  u32x4 pw[2][PL];  // plane words of the steps of parity 0 / 1
  u32x4 sw[2];      // scales of the steps of parity 0 / 1
  auto issue_planes = [&](int i, auto P) {
    constexpr int p = decltype(P)::value;
    if constexpr (VEC) {
      const long long g0 = step_g0(i) < g0_last ? step_g0(i) : g0_last;
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        const long long w = (g0 + ppart[k]) < nbcap - 2 ? (g0 + ppart[k]) : nbcap - 2;
        pw[p][k] = *reinterpret_cast<const u32x4_a8*>(prow[k] + w);
      }
    } else {
      if (i >= nsteps) return;
      const long long g0 = step_g0(i);
      const int gblk = step_blocks(i);
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        pw[p][k] = u32x4{0u, 0u, 0u, 0u};
        if (pvalid[k]) {
          const uint64_t* src = prow[k] + g0 + ppart[k];
          if (ppart[k] + 1 < gblk) {
            pw[p][k] = *reinterpret_cast<const u32x4_a8*>(src);
          } else if (ppart[k] < gblk) {
            const uint64_t w0 = src[0];
            pw[p][k] = u32x4{(uint32_t)w0, (uint32_t)(w0 >> 32), 0u, 0u};
          }
        }
      }
    }
  };
  auto issue_scales = [&](int i, auto P) {
    constexpr int p = decltype(P)::value;
    if constexpr (VEC) {
      const long long g0 = step_g0(i) < g0_last ? step_g0(i) : g0_last;
      const long long w = (g0 + 8 * sc_h) < nbcap - 8 ? (g0 + 8 * sc_h) : nbcap - 8;
      sw[p] = *reinterpret_cast<const u32x4*>(srow + w);
    } else {
      if (i >= nsteps) return;
      sw[p] = u32x4{0u, 0u, 0u, 0u};
      if (!svalid) return;
      const uint16_t* src = srow + step_g0(i) + 8 * sc_h;
      const int gblk = step_blocks(i) - 8 * sc_h;
      uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if (b < gblk) v[b >> 1] |= (uint32_t)src[b] << (16 * (b & 1));
      sw[p] = u32x4{v[0], v[1], v[2], v[3]};
    }
  };
  auto write_planes = [&](int i, auto P) {  // rows >= R: row 0's words, never used (A is zero there)
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const int e = tid + k * SCAN_THREADS;
      *reinterpret_cast<u32x4*>(&sm.planes[i & 1][(e >> 3) * PSTRIDE + 16 * (e & 7)]) = pw[p][k];
    }
  };
  auto write_scales = [&](int i, auto P) {  // scales of step i and their per-channel max
    constexpr int p = decltype(P)::value;
    const int b3 = i % 3;
    // the blocks of the step only; fp16 bits of non-negative values order like the values
    const int nv = step_blocks(i) - 8 * sc_h;
    u16x2 mv = {0, 0};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t keep = (2 * x < nv ? 0xFFFFu : 0u) | (2 * x + 1 < nv ? 0xFFFF0000u : 0u);
      mv = __builtin_elementwise_max(mv, __builtin_bit_cast(u16x2, sw[p][x] & keep));
    }
    uint32_t m = mv.x > mv.y ? mv.x : mv.y;
    const uint32_t mo = (uint32_t)__shfl_xor((int)m, 1);
    m = mo > m ? mo : m;
    if (svalid) {
      *reinterpret_cast<u32x4*>(&sm.sc[b3][sc_c][8 * sc_h]) = sw[p];
      if (sc_h == 0) sm.smax[b3][sc_c] = half_bits_to_f32((uint16_t)m);
    }
  };

  // the thresholds of this wavefront's heads (w, w + 4), read once
  float theta_k[HG];
#pragma unroll
  for (int k = 0; k < HG; ++k) {
    const int h = wave + 4 * k;
    theta_k[k] = (MODE == SCAN_CAND && h < G) ? key_to_float(a.thresh[(long long)u * G + h]) : 0.f;
  }

  // ---- frames of step i: wavefront w handles heads w, w + 4 ----
  auto compute_frame = [&](int i) {
    const int par = i & 1, b3 = i % 3, gblk = step_blocks(i);
#pragma unroll
    for (int k = 0; k < HG; ++k) {
      const int h = wave + 4 * k;
      if (h >= G) continue;  // wavefront-uniform
      uint32_t key = 0;
      for (int c = lane; c < CR; c += 64) {
        const float v = fabsf(sm.q[h][sm.chj[c]]) * 8.f * sm.smax[b3][c];
        const uint32_t kk = (__float_as_uint(v) & 0xFFFFFF00u) | (uint32_t)c;
        key = kk > key ? kk : key;
      }
      key = wave_max_u32(key);
      // an upper bound of the largest |q| 8 smax, and the channel that reaches it
      const float best = key ? __uint_as_float((key & 0xFFFFFF00u) + 0x100u) : 0.f;
      const int cs = (int)(key & 0xFFu);
      const int E = frame_exp(best, lx);
      int eb = E;
      bool own = false;
      if (lane < gblk && best > 0.f) {
        // the block's own largest weight is at least a quarter of the frame's
        // if the channel that sets the frame keeps a quarter of its step max
        if (4.f * half_bits_to_f32(sm.sc[b3][cs][lane]) < sm.smax[b3][cs]) {
          float mb = 0.f;
          for (int c = 0; c < CR; ++c)
            mb = fmaxf(mb, fabsf(sm.q[h][sm.chj[c]]) * 8.f * half_bits_to_f32(sm.sc[b3][c][lane]));
          eb = frame_exp(mb, lx);
          own = eb != E;
        }
      }
      if (lane < GB) {
        sm.ex[par][h][lane] = eb;
        if constexpr (MODE == SCAN_CAND)
          sm.thp[par][h][lane] = scaled_threshold(theta_k[k], eb);
      }
      const bool any_own = __ballot(own) != 0ull;
      if (lane == 0) {
        sm.exh[par][h] = E;
        sm.own[par][h] = any_own;
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

    // builder items: pass m covers row RPP m + lane / NPAIR and heads
    // 2 (lane % NPAIR), +1; rows >= R have zero weights, hence zero digits
    const int prow = lane / NPAIR, ppair = lane % NPAIR;
    float fq0[NPASS][2];  // q_hj 2^(3-p) of the item's row and heads
    int soff[NPASS];      // the item's row's scales in sc[.]: read channel * GB
#pragma unroll
    for (int m = 0; m < NPASS; ++m) {
      const int r = m * RPP + prow;
      soff[m] = (r < R ? sm.rowc[r] : 0) * GB;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int h = 2 * ppair + x;
        fq0[m][x] = (r < R && h < G) ? ldexpf(sm.q[h][sm.chj[sm.rowc[r]]], 3 - sm.rowp[r]) : 0.f;
      }
    }

    // MFMA operand addressing: lane l is column / A-row l % 16 of K-group l / 16;
    // a transposing read takes, in each 16-lane group, row r0 + (l % 16) / 2
    const int kg = lane >> 4, s16 = lane & 15;
    const int rsub = s16 >> 1, ahalf = 8 * (s16 & 1);
    uint32_t bmask[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bmask[c] = 0x01010101u << (2 * c + (s16 >> 3));
    const uint32_t neg7 = (s16 >> 3) ? 0xFFFFFFFFu : 0u;  // lanes whose c = 3 column keeps bit 7
    const i32x4 ones4 = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const long ones2 = 0x0101010101010101l;
    const i32x4 zero4 = {0, 0, 0, 0};

    // A records of block blk into buffer buf
    auto build = [&](int b3, int blk, int buf, const float (&fqe)[NPASS][2]) {
      const uint16_t* scb = &sm.sc[b3][0][0] + blk;
      uint8_t* rec = &sm.atab[wave][buf][prow][8 * ppair];
#pragma unroll
      for (int m = 0; m < NPASS; ++m) {
        const float sv = half_bits_to_f32(scb[soff[m]]);
        const uint32_t x0 = (uint32_t)__builtin_fmaf(fqe[m][0], sv, DIGIT_BIAS) ^ 0x808080u;
        const uint32_t x1 = (uint32_t)__builtin_fmaf(fqe[m][1], sv, DIGIT_BIAS) ^ 0x808080u;
        *reinterpret_cast<uint2*>(rec + m * RPP * (16 * HG)) = make_uint2(x0, x1);
      }
    };
    // the same for a step where some (head, block) has a frame of its own
    auto build_own = [&](int par, int b3, int blk, int buf, const float (&fqe)[NPASS][2],
                         const int (&exh2)[2]) {
      float g[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int h = 2 * ppair + x;
        g[x] = h < G ? ldexpf(1.f, sm.ex[par][h][blk] - exh2[x]) : 0.f;
      }
      const uint16_t* scb = &sm.sc[b3][0][0] + blk;
      uint8_t* rec = &sm.atab[wave][buf][prow][8 * ppair];
#pragma unroll
      for (int m = 0; m < NPASS; ++m) {
        const float sv = half_bits_to_f32(scb[soff[m]]);
        const uint32_t x0 = (uint32_t)__builtin_fmaf(fqe[m][0] * g[0], sv, DIGIT_BIAS) ^ 0x808080u;
        const uint32_t x1 = (uint32_t)__builtin_fmaf(fqe[m][1] * g[1], sv, DIGIT_BIAS) ^ 0x808080u;
        *reinterpret_cast<uint2*>(rec + m * RPP * (16 * HG)) = make_uint2(x0, x1);
      }
    };
    // digit sums of block blk (planes pl, A records of buffer buf)
    auto contract = [&](const uint8_t* pl, int blk, int buf, i32x4 (&acc)[HG][4], i32x4 (&accc)[HG]) {
      const uint8_t* at = &sm.atab[wave][buf][0][0];
#pragma unroll
      for (int kp = 0; kp < N64; ++kp) {
        const int r0 = 64 * kp + 16 * kg + rsub;
        const i32x2 b0 = tr8(pl + r0 * PSTRIDE + 8 * blk);
        const i32x2 b1 = tr8(pl + (r0 + 8) * PSTRIDE + 8 * blk);
        const i32x4 bv = {b0.x, b0.y, b1.x, b1.y};
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const i32x2 a0 = tr8(at + r0 * (16 * HG) + 16 * hg + ahalf);
          const i32x2 a1 = tr8(at + (r0 + 8) * (16 * HG) + 16 * hg + ahalf);
          const i32x4 av = {a0.x, a0.y, a1.x, a1.y};
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[hg][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv & (int)bmask[c],
                                                               kp ? acc[hg][c] : zero4, 0, 0, 0);
          accc[hg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, ones4, kp ? accc[hg] : zero4, 0, 0, 0);
        }
      }
      if constexpr (HAS32) {
        const int r0 = 64 * N64 + 8 * kg + rsub;
        const i32x2 b0 = tr8(pl + r0 * PSTRIDE + 8 * blk);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const long av = __builtin_bit_cast(long, tr8(at + r0 * (16 * HG) + 16 * hg + ahalf));
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[hg][c] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                av, __builtin_bit_cast(long, b0 & (int)bmask[c]), N64 ? acc[hg][c] : zero4, 0, 0, 0);
          accc[hg] = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, ones2, N64 ? accc[hg] : zero4, 0, 0, 0);
        }
      }
    };
    // scores of block blk: lane <-> (head 4 hg + l / 16, column l % 16)
    auto scores = [&](int par, long long g0, int blk, const i32x4 (&acc)[HG][4], const i32x4 (&accc)[HG]) {
      const long long tok0 = (g0 + blk) * BLK + 8 * (s16 & 7) + (s16 >> 3);
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const int h = 4 * hg + kg;
        const int hh = h < G ? h : 0;
        const i32x4 dc = accc[hg];
        const uint32_t cc = ((uint32_t)dc.z << 16) + ((uint32_t)dc.y << 8) + (uint32_t)dc.x;  // C
        const int eb = sm.ex[par][hh][blk];
        float thr = 0.f;
        if constexpr (MODE == SCAN_CAND) thr = sm.thp[par][hh][blk];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int bp = 2 * c + (s16 >> 3);
          const i32x4 d = acc[hg][c];
          // S = sum_r X_r b_r (the digit sums are multiples of 2^bp); T = 2 S - C
          const uint32_t sS = ((uint32_t)d.z << (16 - bp)) + ((uint32_t)d.y << (8 - bp)) +
                              (uint32_t)(d.x >> bp);
          uint32_t s2 = 2u * sS;
          if (c == 3) s2 = (s2 ^ neg7) - neg7;  // bit 7 kept as the int8 byte 0x80 = -128
          const float tf = (float)(int)(s2 - cc);
          const long long tok = tok0 + 2 * c;
          if constexpr (MODE == SCAN_CAND) {
            const bool pass = h < G && tf >= thr;
            if (__ballot(pass) != 0ull && pass) append(tok, h, ldexpf(tf, -(eb + 1)));
          } else {
            if (h < G) store(tok, h, ldexpf(tf, -(eb + 1)));
          }
        }
      }
    };

    // ---- one step: the wavefront's blocks, building block b + 1 while the
    // matrix cores work on block b ----
    auto blocks = [&](int i) {
      const int par = i & 1, b3 = i % 3;
      const long long g0 = step_g0(i);
      const int wb = NB * wave;
      const int nblk = step_blocks(i) - wb;  // blocks of this wavefront (uniform)
      if (nblk <= 0) return;
      // the rows' weights in this step's frames
      float fqe[NPASS][2];
      int exh2[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) exh2[x] = 2 * ppair + x < G ? sm.exh[par][2 * ppair + x] : 0;
#pragma unroll
      for (int m = 0; m < NPASS; ++m)
#pragma unroll
        for (int x = 0; x < 2; ++x) fqe[m][x] = ldexpf(fq0[m][x], exh2[x]);
      bool own_any = false;
#pragma unroll
      for (int h = 0; h < G; ++h) own_any |= sm.own[par][h] != 0;
      const uint8_t* pl = &sm.planes[par][0];

      if (own_any) build_own(par, b3, wb, 0, fqe, exh2);
      else build(b3, wb, 0, fqe);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b >= nblk) break;
        i32x4 acc[HG][4];
        i32x4 accc[HG];
        contract(pl, wb + b, b & 1, acc, accc);
        if (b + 1 < nblk) {
          if (own_any) build_own(par, b3, wb + b + 1, (b + 1) & 1, fqe, exh2);
          else build(b3, wb + b + 1, (b + 1) & 1, fqe);
        }
        scores(par, g0, wb + b, acc, accc);
      }
    };

    // ---- prologue: loads of steps 0 and 1, scales and frames of step 0 ----
    constexpr std::integral_constant<int, 0> P0{};
    constexpr std::integral_constant<int, 1> P1{};
    issue_planes(0, P0);
    issue_planes(1, P1);
    issue_scales(0, P0);
    issue_scales(1, P1);
    write_scales(0, P0);
    issue_scales(2, P0);
    __syncthreads();
    compute_frame(0);

    // ---- steps (two per trip, so that the prefetch registers are static) ----
    auto step = [&](int i, auto P, auto Q) {  // P = i % 2, Q = (i + 1) % 2
      write_planes(i, P);
      if (i + 1 < nsteps) write_scales(i + 1, Q);
      __syncthreads();  // planes of i, scales of i + 1 and frames of i are in LDS
      issue_planes(i + 2, P);
      issue_scales(i + 3, Q);
      if (i + 1 < nsteps) compute_frame(i + 1);
      blocks(i);
    };
    for (int i = 0; i < nsteps; i += 2) {
      step(i, P0, P1);
      if (i + 1 < nsteps) step(i + 1, P1, P0);
    }
  };
  switch (rpt) {
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    case 2: main_loop(std::integral_constant<int, 2>{}); break;
    case 3: main_loop(std::integral_constant<int, 3>{}); break;
    default: main_loop(std::integral_constant<int, 4>{}); break;
  }
  store_counts();
}

template <int G, int MODE>
hipError_t launch_fast(const ScanArgs& a0, hipStream_t st) {
  ScanArgs a = a0;
  long long maxnb = 0;
  for (int s = 0; s < a.g.S; ++s) maxnb = a.g.n[s] / BLK > maxnb ? a.g.n[s] / BLK : maxnb;
  if (maxnb == 0 || a.g.units() == 0) return hipSuccess;
  dim3 grid;
  if (MODE == SCAN_SAMPLE) {
    a.wg_blocks = SAMPLE_GROUP;
    grid = dim3((unsigned)sample_groups(a.g), (unsigned)a.g.units());
  } else {
    const int wb = scan_wg_blocks(a.g);
    a.wg_blocks = wb;
    grid = dim3((unsigned)((maxnb + wb - 1) / wb), (unsigned)a.g.units());
  }
  if (a.g.nbcap() % 8 == 0)
    scan_fast_kernel<G, MODE, true><<<grid, SCAN_THREADS, 0, st>>>(a);
  else
    scan_fast_kernel<G, MODE, false><<<grid, SCAN_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch_fast(const ScanArgs& a, hipStream_t st) {
  switch (a.g.G) {
    case 1: return launch_fast<1, MODE>(a, st);
    case 2: return launch_fast<2, MODE>(a, st);
    case 4: return launch_fast<4, MODE>(a, st);
    case 8: return launch_fast<8, MODE>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// rows >= 0: every unit reads that many rows, one kernel; rows < 0: both,
// the wide one with fewer, larger workgroups (its workgroups of fast units
// only read the depths and leave)
template <int MODE>
hipError_t dispatch(const ScanArgs& a, int rows, hipStream_t st) {
  if (rows >= 0 && rows <= SCAN_FAST_ROWS) return dispatch_fast<MODE>(a, st);
  if (rows > SCAN_FAST_ROWS) return launch_scan_wide(a, MODE, 0, st);
  const hipError_t e = dispatch_fast<MODE>(a, st);
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
  a.out = cb.sample;
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
  a.cand_count = cb.count;
  a.cand_val = cb.val;
  a.cand_idx = cb.idx;
  return dispatch<SCAN_CAND>(a, rows, st);
}

}  // namespace bpk
