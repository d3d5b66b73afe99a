// Prefix-plane key scan (Fathom §1, §3.2), wide kernel: the units that read
// more than SCAN_FAST_ROWS plane rows (budgets above 128 planes).  Same
// arithmetic as the fast kernel in scan.hip, but the rows are cut into
// segments that are staged one after the other, with the accumulators of a
// wavefront's four blocks kept across segments.
//
// Arithmetic.  The t-bit prefix value of a 4-bit code is
//   m = sum_{p<t} 2^(3-p) b_p + 2^(3-t) - 8 = sum_{p<t} 2^(3-p) (b_p - 1/2)
// (plane 0 = most significant bit), so with one row r = (j, p) per read plane
// and the weight w_r = q_hj s_bj 2^(3-p):
//   s_hat = sum_j q_hj s_bj m_ij = sum_r w_r (b_r - 1/2) = S - C/2,
//   S = sum_r w_r b_r,  C = sum_r w_r.
// The weights of one 16-block step and head are put in a common fixed-point
// frame, X_r = round(w_r 2^E) with |X_r| < 2^29, each split into four balanced
// signed bytes, and the score is s_hat = (2 S - C) 2^-(E+1), with the frames,
// digits, error bound and candidate test of the fast kernel (scan.hip; the
// shared pieces are in scan_common.h).  For R <= 512 rows the rounding error
// stays below (R/4 + 4) 2^-22 + 2^-23 <= 4e-5 of the token's L1 mass.
//
// Mapping onto gfx950:
// * A workgroup (4 wavefronts) owns a range of blocks of one unit and walks
//   it in steps of 16 blocks; the plane rows (channel by channel) are cut into
//   segments of 128 rows (64 when G = 8) so the LDS footprint is fixed.  Per
//   (step, segment) task the workgroup stages the 16 words of each row in LDS
//   (coalesced 128-byte reads, issued one task ahead) and builds, per (block,
//   row), the 16-byte record of the digits of the G heads' X.
// * Wavefront w contracts blocks 4w .. 4w+3 on the matrix cores with
//   v_mfma_i32_16x16x64_i8 (a 32-row remainder with zero upper bytes).  The
//   A operand (row m = 4h + digit, K = plane rows) and the B operand (K =
//   plane rows, column = token) both come from LDS through the transposing
//   read ds_read_b64_tr_b8: the B bytes are the raw plane words, each byte
//   holding 8 tokens of one row, and one AND per 4 bytes keeps bit
//   2c + (n / 8) of column n, so the four matrices c = 0..3 give the 64
//   tokens of the block, token 8 (n % 8) + 2c + n / 8 in column n, each
//   scaled by 2^(2c + n / 8) (by -2^7 for bit 7: the int8 byte 0x80 is
//   -128).  A fifth product with all-one bytes gives C.
// * Lane l ends with the four digit sums of head 4 hg + l / 16 for its token;
//   in the candidate mode the two high ones are tested against the
//   per-(head, block) threshold and passing tokens get their exact scores.
#include "scan_common.h"

namespace bpk {
namespace {

constexpr int NB = 4;        // blocks per wavefront per step
constexpr int GB = SCAN_GB;  // blocks per step
constexpr int CMAX = D;      // read channels at most
constexpr int PSTRIDE = 144; // LDS bytes per plane row: 16 words + 16 bytes of padding

template <int HG>
struct ScanSmem {
  static constexpr int SEG = HG == 1 ? 128 : 64;  // plane rows per segment
  static constexpr int GP = 4 * HG;               // heads, padded to whole MFMA row groups
  alignas(16) uint8_t planes[SEG * PSTRIDE];      // [row][block] words of one task
  alignas(16) uint8_t atab[GB][SEG][16 * HG];     // [block][row] X digits: 4 bytes per head
  alignas(16) float fqe[2][SEG][GP];              // per task parity: q_hj 2^(3-p+E_h) of each row
  alignas(16) uint16_t sc[2][CMAX][GB];           // per step parity: fp16 scales [read channel][block]
  float smax[2][CMAX];                            // per step parity: largest scale of a read channel
  float q[GP][D];                                 // the unit's query heads (0 beyond G)
  int ex[2][GP][GB];                              // per step parity: frame exponent of (head, block)
  int ith[2][GP][GB];                             // per step parity: cand_tau + 1 of (head, block)
  int exh[2][GP];                                 // per step parity: frame exponent of the step
  int own[2][GP];                                 // per step parity: some block has a frame of its own
  int scan_buf[D];                                // plan: prefix sums of (depth, read flag)
  uint8_t rowc[NP * D];                           // read channel of each plane row
  uint8_t rowp[NP * D];                           // plane of each plane row
  uint8_t chj[CMAX];                              // channel of each read channel
  int ccount[GP];                                 // candidates of this workgroup per head
};

template <int G, int MODE>
__global__ __launch_bounds__(SCAN_THREADS, G == 8 ? 1 : 2) void scan_wide_kernel(ScanArgs a) {
  constexpr int HG = (G + 3) / 4;
  using SM = ScanSmem<HG>;
  constexpr int SEG = SM::SEG;
  constexpr int GP = SM::GP;
  constexpr int PL = SEG * 8 / SCAN_THREADS;  // 16-byte plane loads per thread and task
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

  // ---- where a score goes (every lane of the wavefront calls emit) ----
  float theta[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h)
    theta[h] = (MODE == SCAN_CAND && h < G) ? key_to_float(a.thresh[(long long)u * G + h])
                                            : -__builtin_inff();
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
  auto append = [&](long long tok, int h, float s) {  // CAND, lanes whose test passed
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
  if (!a.all_rows && R <= SCAN_FAST_ROWS) return;  // the fast kernel's unit (uniform)
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

  const int nseg = (R + SEG - 1) / SEG;
  const int nsteps = (int)((wb1 - wb0 + GB - 1) / GB);
  const int ntask = nsteps * nseg;
  auto step_g0 = [&](int i) { return wb0 + (long long)i * GB; };
  auto step_blocks = [&](int i) {
    const long long r = wb1 - step_g0(i);
    return r < GB ? (int)r : GB;
  };
  auto seg_rows = [&](int s) { return (R - s * SEG) < SEG ? (R - s * SEG) : SEG; };

  // ---- loads (global -> registers; written to LDS at the top of a task) ----
  u32x4 pw[PL];        // plane words: row e / 8 of the segment, words 2 (e % 8), +1
  u32x4 sw;            // scales: read channel tid / 2, blocks 8 (tid % 2) .. +7
  auto issue_planes = [&](int task) {
    const int i = task / nseg, s = task % nseg;
    const long long g0 = step_g0(i);
    const int gblk = step_blocks(i);
    const int rs = seg_rows(s);
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const int e = tid + k * SCAN_THREADS;
      const int rr = e >> 3, part = e & 7;
      pw[k] = u32x4{0u, 0u, 0u, 0u};
      if (rr < rs) {
        const int r = s * SEG + rr;
        const uint64_t* src =
            a.planes + ((uint64_t)(gu * D + sm.chj[sm.rowc[r]]) * NP + sm.rowp[r]) * nbcap + g0 + 2 * part;
        if (2 * part + 1 < gblk) {
          pw[k] = *reinterpret_cast<const u32x4*>(src);
        } else if (2 * part < gblk) {
          const uint64_t w0 = src[0];
          pw[k] = u32x4{(uint32_t)w0, (uint32_t)(w0 >> 32), 0u, 0u};
        }
      }
    }
  };
  auto issue_scales = [&](int i) {
    sw = u32x4{0u, 0u, 0u, 0u};
    const int c = tid >> 1, hf = tid & 1;
    if (i >= nsteps || c >= CR) return;
    const long long g0 = step_g0(i) + 8 * hf;
    const int gblk = step_blocks(i) - 8 * hf;
    const uint16_t* src = a.scales + (uint64_t)(gu * D + sm.chj[c]) * nbcap + g0;
    if (gblk >= 8) {
      sw = *reinterpret_cast<const u32x4*>(src);
    } else {
      uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if (b < gblk) v[b >> 1] |= (uint32_t)src[b] << (16 * (b & 1));
      sw = u32x4{v[0], v[1], v[2], v[3]};
    }
  };
  auto write_planes = [&](int task) {
    (void)task;
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const int e = tid + k * SCAN_THREADS;
      *reinterpret_cast<u32x4*>(&sm.planes[(e >> 3) * PSTRIDE + 16 * (e & 7)]) = pw[k];
    }
  };
  auto write_scales = [&](int i) {  // scales of step i (loaded by issue_scales(i))
    const int c = tid >> 1, hf = tid & 1, par = i & 1;
    float m = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      m = fmaxf(m, half_bits_to_f32((uint16_t)(sw[b] & 0xFFFF)));
      m = fmaxf(m, half_bits_to_f32((uint16_t)(sw[b] >> 16)));
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    if (c < CR) {
      *reinterpret_cast<u32x4*>(&sm.sc[par][c][8 * hf]) = sw;
      if (hf == 0) sm.smax[par][c] = m;
    }
  };

  // ---- frames of step i (wavefront w handles heads w, w + 4) ----
  auto compute_frame = [&](int i) {
    const int par = i & 1, gblk = step_blocks(i);
#pragma unroll
    for (int k = 0; k < HG; ++k) {
      const int h = wave + 4 * k;
      if (h >= G) continue;  // wavefront-uniform
      float best = 0.f;
      uint32_t bkey = 0;
      for (int c = lane; c < CR; c += 64) {
        const float v = fabsf(sm.q[h][sm.chj[c]]) * 8.f * sm.smax[par][c];
        best = fmaxf(best, v);
        const uint32_t key = (__float_as_uint(v) & 0xFFFFFF00u) | (uint32_t)c;
        bkey = key > bkey ? key : bkey;
      }
      best = wave_max(best);
      bkey = wave_max_u32(bkey);
      const int cs = (int)(bkey & 0xFFu);
      const int E = frame_exp(best, FRAME_BITS);
      int eb = E;
      bool own = false;
      if (lane < GB && lane < gblk && best > 0.f) {
        // the block's own largest weight is at least a quarter of the frame's
        // if the channel that sets the frame keeps a quarter of its step max
        if (4.f * half_bits_to_f32(sm.sc[par][cs][lane]) < sm.smax[par][cs]) {
          float mb = 0.f;
          for (int c = 0; c < CR; ++c)
            mb = fmaxf(mb, fabsf(sm.q[h][sm.chj[c]]) * 8.f * half_bits_to_f32(sm.sc[par][c][lane]));
          eb = frame_exp(mb, FRAME_BITS);
          own = eb != E;
        }
      }
      if (lane < GB) {
        sm.ex[par][h][lane] = eb;
        sm.ith[par][h][lane] =
            MODE == SCAN_CAND ? cand_tau(key_to_float(a.thresh[(long long)u * G + h]), eb, R) + 1 : 0;
      }
      const bool any_own = __ballot(own) != 0ull;
      if (lane == 0) {
        sm.exh[par][h] = E;
        sm.own[par][h] = any_own;
      }
    }
  };
  // q_hj 2^(3-p+E_h) of the rows of task (i, s), into fqe[tp] (0 beyond the
  // segment's rows and for heads >= G); wavefront w handles heads w, w + 4
  auto fill_fqe = [&](int task, int tp) {
    const int i = task / nseg, s = task % nseg;
    const int rs = seg_rows(s);
#pragma unroll
    for (int k = 0; k < HG; ++k) {
      const int h = wave + 4 * k;
      const int E = h < G ? sm.exh[i & 1][h] : 0;
      for (int rr = lane; rr < SEG; rr += 64) {
        float v = 0.f;
        if (h < G && rr < rs) {
          const int r = s * SEG + rr;
          v = ldexpf(sm.q[h][sm.chj[sm.rowc[r]]], 3 - sm.rowp[r] + E);
        }
        sm.fqe[tp][rr][h] = v;
      }
    }
  };

  // ---- prologue: scales and frames of step 0, fqe of task 0 (the loop's
  // first barrier publishes them) ----
  issue_scales(0);
  write_scales(0);
  __syncthreads();
  issue_planes(0);
  issue_scales(1);
  compute_frame(0);
  fill_fqe(0, 0);

  // MFMA operand addressing: lane l is column / A-row l % 16 of K-group l / 16;
  // a transposing read takes, in each 16-lane group, row r0 + (l % 16) / 2
  const int kg = lane >> 4, s16 = lane & 15;
  const int rsub = s16 >> 1, ahalf = 8 * (s16 & 1);
  uint32_t bmask[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) bmask[c] = 0x01010101u << (2 * c + (s16 >> 3));
  const int neg3 = (s16 >> 3) ? -1 : 0;  // lanes whose c = 3 column keeps bit 7 (v = -128)
  const i32x4 ones4 = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const i32x4 ones2x = {0x01010101, 0x01010101, 0, 0};

  i32x4 acc[NB][HG][4];
  i32x4 accc[NB][HG];

  for (int task = 0; task < ntask; ++task) {
    const int i = task / nseg, s = task % nseg;
    const int par = i & 1, tp = task & 1;
    const long long g0 = step_g0(i);
    const int gblk = step_blocks(i);
    const int rs = seg_rows(s);
    int n64 = rs >> 6, rem = rs & 63;
    if (rem > 32) {
      ++n64;
      rem = 0;
    }
    const bool has32 = rem > 0;
    const int rp = 64 * n64 + (has32 ? 32 : 0);  // rows with A records (zero beyond rs)

    // ---- the previous task's planes and A records are no longer read: this
    // task's plane words, and the next step's scales, into LDS ----
    __syncthreads();
    write_planes(task);
    if (s == 0 && i + 1 < nsteps) write_scales(i + 1);

    // ---- A records: X digits of (block, row) for every head ----
    const bool own_any = [&]() {
      bool o = false;
#pragma unroll
      for (int h = 0; h < G; ++h) o |= sm.own[par][h] != 0;
      return o;
    }();
    // thread -> block tid / 16, rows tid % 16 + 16 k (rp is a multiple of 32)
    for (int rr = tid & 15, b = tid >> 4; rr < rp; rr += 16) {
      u32x4 rec[HG];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) rec[hg] = u32x4{0u, 0u, 0u, 0u};
      if (b < gblk && rr < rs) {
        const float sv = half_bits_to_f32(sm.sc[par][sm.rowc[s * SEG + rr]][b]);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const float4 f = *reinterpret_cast<const float4*>(&sm.fqe[tp][rr][4 * hg]);
          float fv[4] = {f.x, f.y, f.z, f.w};
          if (own_any) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const int h = 4 * hg + x;
              if (h < G) fv[x] = ldexpf(fv[x], sm.ex[par][h][b] - sm.exh[par][h]);
            }
          }
#pragma unroll
          for (int x = 0; x < 4; ++x) rec[hg][x] = x_digits4((double)fv[x], (double)sv);
        }
      }
#pragma unroll
      for (int hg = 0; hg < HG; ++hg)
        *reinterpret_cast<u32x4*>(&sm.atab[b][rr][16 * hg]) = rec[hg];
    }
    __syncthreads();  // planes, A records and the next step's scales are in LDS
    if (task + 1 < ntask) {
      issue_planes(task + 1);
      const int i1 = (task + 1) / nseg;
      if (i1 != i) issue_scales(i1 + 1);
      // what the next task needs: the next step's frames (from its scales,
      // written above) and its rows' q 2^(3-p+E); each wavefront fills the
      // heads whose frames it computed
      if (i1 != i) compute_frame(i1);
      fill_fqe(task + 1, tp ^ 1);
    }

    // ---- contraction: wavefront takes blocks 4 wave .. 4 wave + 3 of the step ----
    const int wb = NB * wave;
    if (s == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          accc[b][hg] = i32x4{0, 0, 0, 0};
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[b][hg][c] = i32x4{0, 0, 0, 0};
        }
    }
    if (wb < gblk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int blk = wb + b;
        if (blk >= gblk) break;
        for (int kp = 0; kp < n64; ++kp) {
          const int r0 = 64 * kp + 16 * kg + rsub;
          const i32x2 b0 = tr8(&sm.planes[r0 * PSTRIDE + 8 * blk]);
          const i32x2 b1 = tr8(&sm.planes[(r0 + 8) * PSTRIDE + 8 * blk]);
          const i32x4 bv = {b0.x, b0.y, b1.x, b1.y};
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            const i32x2 a0 = tr8(&sm.atab[blk][r0][16 * hg + ahalf]);
            const i32x2 a1 = tr8(&sm.atab[blk][r0 + 8][16 * hg + ahalf]);
            const i32x4 av = {a0.x, a0.y, a1.x, a1.y};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const i32x4 m = bv & (int)bmask[c];
              acc[b][hg][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, m, acc[b][hg][c], 0, 0, 0);
            }
            accc[b][hg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, ones4, accc[b][hg], 0, 0, 0);
          }
        }
        if (has32) {
          const int r0 = 64 * n64 + 8 * kg + rsub;
          const i32x2 b0 = tr8(&sm.planes[r0 * PSTRIDE + 8 * blk]);
          // as a K = 64 product with zero upper bytes (the K = 32 form's result
          // latency is not reliably waited for)
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            const i32x2 a0 = tr8(&sm.atab[blk][r0][16 * hg + ahalf]);
            const i32x4 av = {a0.x, a0.y, 0, 0};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const i32x2 m = b0 & (int)bmask[c];
              acc[b][hg][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, i32x4{m.x, m.y, 0, 0},
                                                                     acc[b][hg][c], 0, 0, 0);
            }
            accc[b][hg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, ones2x, accc[b][hg], 0, 0, 0);
          }
        }
      }
    }

    // ---- epilogue after the last segment: lane <-> (head 4 hg + l / 16, column l % 16) ----
    if (s == nseg - 1 && wb < gblk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int blk = wb + b;
        if (blk >= gblk) break;
        const long long tok0 = (g0 + blk) * BLK + 8 * (s16 & 7) + (s16 >> 3);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const int h = 4 * hg + kg;
          const i32x4 dc = accc[b][hg];
          const int eb = sm.ex[par][h < G ? h : 0][blk];
          // the candidate test of scan.hip: P >= kap 2^bp (~P >= kap 2^7 - 1 for bit 7)
          const int kap = MODE == SCAN_CAND && h < G
                              ? (sm.ith[par][h][blk] + (dc.w * 256 + dc.z)) >> 1
                              : 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int bp = 2 * c + (s16 >> 3);
            const i32x4 d = acc[b][hg][c];
            const long long tok = tok0 + 2 * c;
            if constexpr (MODE == SCAN_CAND) {
              const int p = d.w * 256 + d.z;
              const int th = (int)(((uint32_t)kap << bp) + (uint32_t)(c == 3 ? neg3 : 0));
              const bool pass = h < G && (c == 3 ? (p ^ neg3) : p) >= th;
              // the test's margin for the dropped low digits grows with the
              // rows read; a passing token is kept only if its written score
              // reaches theta (the candidates are then exactly those tokens)
              if (__ballot(pass) != 0ull && pass) {
                const float sc = score4(d, dc, bp, c == 3 && neg3 != 0, eb);
                if (sc >= theta[h]) append(tok, h, sc);
              }
            } else {
              if (h < G) store(tok, h, score4(d, dc, bp, c == 3 && neg3 != 0, eb));
            }
          }
        }
      }
    }
  }
  store_counts();
}

template <int G, int MODE>
hipError_t launch_gm(const ScanArgs& a0, int span, hipStream_t st) {
  ScanArgs a = a0;
  long long maxnb = 0;
  for (int s = 0; s < a.g.S; ++s) maxnb = a.g.n[s] / BLK > maxnb ? a.g.n[s] / BLK : maxnb;
  if (maxnb == 0 || a.g.units() == 0) return hipSuccess;
  dim3 grid;
  if (MODE == SCAN_SAMPLE) {
    a.wg_blocks = SAMPLE_GROUP;
    grid = dim3((unsigned)sample_groups(a.g), (unsigned)a.g.units());
  } else {
    const int wb = span > 0 ? span : scan_wg_blocks(a.g);
    a.wg_blocks = wb;
    grid = dim3((unsigned)((maxnb + wb - 1) / wb), (unsigned)a.g.units());
  }
  scan_wide_kernel<G, MODE><<<grid, SCAN_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(const ScanArgs& a, int span, hipStream_t st) {
  switch (a.g.G) {
    case 1: return launch_gm<1, MODE>(a, span, st);
    case 2: return launch_gm<2, MODE>(a, span, st);
    case 4: return launch_gm<4, MODE>(a, span, st);
    case 8: return launch_gm<8, MODE>(a, span, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_scan_wide(const ScanArgs& a, int mode, int span, hipStream_t st) {
  switch (mode) {
    case SCAN_FULL: return dispatch<SCAN_FULL>(a, span, st);
    case SCAN_SAMPLE: return dispatch<SCAN_SAMPLE>(a, span, st);
    case SCAN_CAND: return dispatch<SCAN_CAND>(a, span, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bpk
