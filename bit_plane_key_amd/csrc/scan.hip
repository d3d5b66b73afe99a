// Prefix-plane key scan (Fathom §1, §3.2): approximate scores of every key of
// every complete block, reading only planes p < t_j of each read channel and
// the fp16 block scales of those channels.
//
// The t-bit prefix value of a 4-bit code is m = (c' + 1/2) 2^(4-t) - 8, with
// c' = sum_{p<t} b_p 2^(t-1-p) read from planes 0 .. t-1 (plane 0 = most
// significant bit).  Since sum_{p<t} 2^(2-p) = 8 - 2^(3-t), the same value is
// a signed binary expansion:
//   m = sum_{p<t} 2^(2-p) B_p,   B_p = 2 b_p - 1 in {-1, +1},
// so with one "row" per read plane (j, p) and A_{h,(j,p)} = q_hj s_bj 2^(2-p):
//   s_hat = sum_j q_hj s_bj m_ij = sum_rows A_{h,r} B_{r,i},
// a contraction over rows of +-1 bits with no constant term.
//
// Mapping onto gfx950:
// * A workgroup (4 wavefronts) owns a range of blocks of one unit and walks it
//   in steps of 16 blocks.  The read planes are listed channel by channel,
//   padded to whole 8-row chunks (padding rows have A = 0) and cut into
//   segments of 64 rows, so the LDS footprint is fixed whatever the depths.
//   Per (step, segment) the workgroup stages into LDS, with coalesced global
//   reads: the plane words, interleaved in pairs of rows at a 16-bit stride
//   (dword (pair, g, block) = 16 tokens of row 2q in its low half and of row
//   2q+1 in its high half), and A split into bf16 hi + lo parts per (block,
//   chunk, head): each thread takes (row, block) items, multiplying the row's
//   -q_hj 2^(2-p) (tabled once per workgroup) by the block scale it loaded.
//   The global loads of the next (step, segment) are in flight while the
//   current one is scored.
// * Wavefront w scores blocks 4w .. 4w+3 of the step, lane i <-> token i.  One
//   16-byte LDS read gives a row pair's dword for the four blocks; a funnel
//   rotation by a per-lane constant moves the lane's two bits to the bf16 sign
//   positions, and one and-or makes the pair (-B, -B) = (+-1.0, +-1.0) (A is
//   negated to match): two VALU operations per two planes of a token.
// * The G-head contraction runs on the matrix cores: v_mfma_f32_16x16x32_bf16
//   with B = the lane's 8 rows of the chunk and A block-diagonal over the four
//   16-lane token groups (row 4g + h of A is nonzero only in token group g's
//   k-range), so D row 4g + h, column n is head h's partial score of token
//   16g + n and each lane ends with the G scores of its own token.  The hi + lo
//   split keeps each term within ~2^-17 of its exact value.
#include "bpk_internal.h"

namespace bpk {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float floatx2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

constexpr int SCAN_THREADS = 256;
constexpr int SCAN_WAVES = SCAN_THREADS / 64;
constexpr int NB = 4;                       // blocks per wavefront per step
constexpr int GB = NB * SCAN_WAVES;         // blocks per workgroup step
constexpr int SEG_ROWS = 64;                // plane rows staged per segment
constexpr int SEG_PAIRS = SEG_ROWS / 2;
constexpr int SEG_CHUNKS = SEG_ROWS / 8;    // 8-row chunks (one MFMA k-range each)
constexpr int MAX_ROWS = NP * D;
constexpr int SC_PER = SEG_ROWS * GB / SCAN_THREADS;  // (row, block) items per thread
static_assert(SCAN_MIN_WG_BLOCKS == GB, "a workgroup takes whole steps");
static_assert(SAMPLE_GROUP % GB == 0 && SAMPLE_STRIDE % SAMPLE_GROUP == 0, "sample plan");
static_assert(SEG_PAIRS * (GB / 2) == SCAN_THREADS, "one (row pair, block pair) per thread");
static_assert(SCAN_THREADS % GB == 0 && SEG_ROWS % (SCAN_THREADS / GB) == 0, "row items");

// bf16 pair (-1)^(bit 15 of x) * 1.0, (-1)^(bit 31 of x) * 1.0.  Written out
// because the and-or form needs its two constants in registers (a VOP3
// instruction takes no literal here); mask is wave-uniform, one a register.
__device__ __forceinline__ uint32_t sign_pair(uint32_t x, uint32_t mask, uint32_t one) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(one));
  return r;
}

// What a launch does with the scores it computes:
// * SCAN_FULL writes every score ([unit][G][cap]);
// * SCAN_SAMPLE scores only the first SAMPLE_GROUP blocks of every
//   SAMPLE_STRIDE (one workgroup per sampled group) into [unit][G][sample_ld];
// * SCAN_CAND appends (score, token) of the tokens of [4, n - W) whose score
//   is at or above the head's threshold to the workgroup's candidate region
//   of that head (slots handed out by an LDS counter; the count, which may
//   pass the region's size, is stored at the end).
// A block's scores are computed by the same instructions in every mode, so
// they are bit-identical across modes and workgroup sizes.
enum ScanMode { SCAN_FULL = 0, SCAN_SAMPLE = 1, SCAN_CAND = 2 };

struct ScanArgs {
  Geom g;
  const float* __restrict__ q_basis;
  const uint8_t* __restrict__ depth;
  const uint64_t* __restrict__ planes;
  const uint16_t* __restrict__ scales;
  float* __restrict__ out;          // scores (FULL) or sampled scores (SAMPLE)
  long long out_ld;                 // per (unit, head) row length of out
  int wg_blocks;                    // blocks per workgroup (multiple of GB)
  int k;                            // top-k (CAND: units with n <= k are skipped)
  const int32_t* __restrict__ unit_flag;  // FULL: if set, only units with flag != 0
  const uint32_t* __restrict__ thresh;    // CAND: [unit][G] order keys
  long long regions;                      // CAND: region stride per (unit, head)
  int32_t* __restrict__ cand_count;       // CAND: [unit][G][regions]
  float* __restrict__ cand_val;           // CAND: [unit][G][regions][CAND_SLOTS]
  int32_t* __restrict__ cand_idx;         // CAND: [unit][G][regions][CAND_SLOTS]
};

// Appends (s, tok) of the lanes with pred to a candidate region; all 64 lanes
// of the wavefront take part.  One LDS atomic per wavefront reserves the
// slots; the count keeps growing past the region's size so that overflow is
// seen.
__device__ __forceinline__ void cand_append(bool pred, float s, long long tok, int* count,
                                            float* val, int32_t* idx, int lane) {
  const unsigned long long m = __ballot(pred);
  if (m == 0ull) return;
  const int leader = __ffsll(m) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(count, __popcll(m));
  base = __shfl(base, leader);
  const int off = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  if (pred && off < CAND_SLOTS) {
    val[off] = s;
    idx[off] = (int32_t)tok;
  }
}

// (x0, x1) -> bf16 hi parts (round to nearest even) and bf16 lo parts of the
// exact fp32 residuals, each packed low = x0, high = x1
__device__ __forceinline__ void split2(float x0, float x1, uint32_t* hi, uint32_t* lo) {
  const floatx2 x = {x0, x1};
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  const floatx2 r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xFFFF0000u)};
  *hi = h;
  *lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

// 128-bit LDS accesses must be 16-byte aligned (misaligned ones stall)
template <int G>
struct ScanSmem {
  static constexpr int HG = (G + 3) / 4;  // head groups of 4 (MFMA rows)
  int scan_buf[D];                 // plan: prefix sums of the depths
  uint8_t row_j[MAX_ROWS];         // channel of each plane row
  uint8_t row_p[MAX_ROWS];         // plane of each plane row
  alignas(16) float fq[MAX_ROWS][G];  // -q_hj 2^(2-p) of each row (0 for padding rows)
  alignas(16) uint32_t words[SEG_PAIRS][4][GB];  // [row pair][token group][block]
  // A hi/lo per block: [chunk][hg][part][h][row] bf16, each block's table
  // padded by 16 bytes so that the 16 blocks of a staging write land in
  // different LDS banks
  static constexpr int ASTRIDE = SEG_CHUNKS * HG * 2 * 4 * 8 + 8;
  alignas(16) uint16_t atab[GB][ASTRIDE];
  alignas(16) uint32_t zero4[4];   // the A operand of lanes off the block diagonal
  int ccount[G];                   // candidates of this workgroup per head
};

template <int G, int MODE>
__global__ __launch_bounds__(SCAN_THREADS) void scan_kernel(ScanArgs a) {
  using SM = ScanSmem<G>;
  constexpr int HG = SM::HG;
  // offset of the 8 rows of (chunk k, head group hg, part, head h) in a block's A table
  auto a_index = [](int k, int hg, int part, int h) { return (((k * HG + hg) * 2 + part) * 4 + h) * 8; };
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

  // where the score of (token, head) goes
  const long long cand_hi = n - kept_tail(n);  // candidates are tokens [4, cand_hi)
  uint32_t tkey[G];
#pragma unroll
  for (int h = 0; h < G; ++h) tkey[h] = MODE == SCAN_CAND ? a.thresh[(long long)u * G + h] : 0u;
  auto emit = [&](long long tok, int h, float s) {  // every lane of the wavefront calls it
    const long long uh = (long long)u * G + h;
    if constexpr (MODE == SCAN_FULL) {
      a.out[uh * a.out_ld + tok] = s;
    } else if constexpr (MODE == SCAN_SAMPLE) {
      a.out[uh * a.out_ld + (long long)blockIdx.x * (SAMPLE_GROUP * BLK) + (tok - wb0 * BLK)] = s;
    } else {
      const bool pred = tok >= 4 && tok < cand_hi && order_key(s) >= tkey[h];
      const long long reg = (uh * a.regions + blockIdx.x) * CAND_SLOTS;
      cand_append(pred, s, tok, &sm.ccount[h], a.cand_val + reg, a.cand_idx + reg,
                  threadIdx.x & 63);
    }
  };
  // the region's count, once every wavefront has appended
  auto store_counts = [&]() {
    if constexpr (MODE == SCAN_CAND) {
      __syncthreads();
      if (threadIdx.x < G)
        a.cand_count[((long long)u * G + threadIdx.x) * a.regions + blockIdx.x] =
            sm.ccount[threadIdx.x];
    }
  };

  // ---- plan: plane rows channel by channel (j ascending, p ascending) ----
  int tj = 0;
  if (MODE == SCAN_CAND && tid < G) sm.ccount[tid] = 0;
  if (tid < 4) sm.zero4[tid] = 0u;
  if (tid < D) {
    tj = a.depth[(long long)u * D + tid];
    tj = tj > NP ? NP : tj;
    sm.scan_buf[tid] = tj;
  }
  __syncthreads();
  for (int off = 1; off < D; off <<= 1) {
    int v = 0;
    if (tid < D && tid >= off) v = sm.scan_buf[tid - off];
    __syncthreads();
    if (tid < D) sm.scan_buf[tid] += v;
    __syncthreads();
  }
  const int R = sm.scan_buf[D - 1];
  const int Rp = (R + 7) & ~7;                      // whole 8-row chunks
  const int nseg = (Rp + SEG_ROWS - 1) / SEG_ROWS;
  if (tid < D && tj > 0) {
    const int r0 = sm.scan_buf[tid] - tj;
    float qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = a.q_basis[((long long)u * G + h) * D + tid];
    float f = -4.f;
    for (int p = 0; p < tj; ++p, f *= 0.5f) {
      sm.row_j[r0 + p] = (uint8_t)tid;
      sm.row_p[r0 + p] = (uint8_t)p;
#pragma unroll
      for (int h = 0; h < G; ++h) sm.fq[r0 + p][h] = qv[h] * f;
    }
  }
  if (tid < Rp - R) {
#pragma unroll
    for (int h = 0; h < G; ++h) sm.fq[R + tid][h] = 0.f;
  }
  __syncthreads();

  // A-operand ownership: lane l holds row 4*(l/16) + (l%4) of a head group,
  // in k-group l/16, only when (l%16)/4 == l/16 (block-diagonal).
  const bool a_active = ((lane & 15) >> 2) == (lane >> 4) && (lane & 3) < (G < 4 ? G : 4);
  const int a_hh = lane & 3;
  const int grp = lane >> 4;                        // token group of the lane
  const uint32_t rot = (uint32_t)(((lane & 15) + 17) & 31);  // bit (lane%16) -> bit 15
  const uint32_t smask = __builtin_amdgcn_readfirstlane(0x80008000u);
  const uint32_t vone = 0x3F803F80u;
  const int wb = NB * wave;

  // ---- tasks = (16-block step, segment); the loads of task i+1 are in flight
  // while task i is scored ----
  const int nsteps = (int)((wb1 - wb0 + GB - 1) / GB);
  const int ntask = nsteps * nseg;
  const int sb = tid % GB;                 // block of this thread's (row, block) items
  const int pr = tid / (GB / 2), bp = 2 * (tid % (GB / 2));  // row pair, first block
  uint64_t w[2][2];                        // [row of the pair][block]
  float sv[SC_PER];                        // scales of rows tid/16 + 16 i, block sb
  auto issue_loads = [&](int task) {
    const long long g0 = wb0 + (long long)(task / nseg) * GB;
    const int sg = task % nseg;
    const int gblk = (wb1 - g0) < GB ? (int)(wb1 - g0) : GB;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = sg * SEG_ROWS + 2 * pr + q;
      w[q][0] = 0;
      w[q][1] = 0;
      if (r < R) {
        const uint64_t* src = a.planes +
                              ((uint64_t)(gu * D + sm.row_j[r]) * NP + sm.row_p[r]) * nbcap + g0 + bp;
        if (bp + 1 < gblk) {  // rows are 8-byte aligned only
          w[q][0] = src[0];
          w[q][1] = src[1];
        } else if (bp < gblk) {
          w[q][0] = src[0];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < SC_PER; ++i) {
      const int r = sg * SEG_ROWS + tid / GB + i * (SCAN_THREADS / GB);
      sv[i] = 0.f;
      if (r < R && sb < gblk)
        sv[i] = (float)__builtin_bit_cast(
            _Float16, a.scales[(uint64_t)(gu * D + sm.row_j[r]) * nbcap + g0 + sb]);
    }
  };

  if (nseg == 0) {  // nothing is read: every score is 0
    // (wb1 - wb0) * 64 is a multiple of 64: each wavefront's lanes run the same trips
    for (long long e = tid; e < (wb1 - wb0) * BLK; e += SCAN_THREADS)
#pragma unroll
      for (int h = 0; h < G; ++h) emit(wb0 * BLK + e, h, 0.f);
    store_counts();
    return;
  }
  floatx4 acc[NB][HG];
  issue_loads(0);
  for (int task = 0; task < ntask; ++task) {
    const long long g0 = wb0 + (long long)(task / nseg) * GB;
    const int sg = task % nseg;
    const int gblk = (wb1 - g0) < GB ? (int)(wb1 - g0) : GB;
    const int seg_r0 = sg * SEG_ROWS;
    const int nck = ((Rp - seg_r0) < SEG_ROWS ? (Rp - seg_r0) : SEG_ROWS) >> 3;
    if (sg == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) acc[b][hg] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();  // the previous task's tables are no longer read

    // ---- plane words -> LDS: row pairs interleaved at 16 bits ----
    if (2 * pr < nck * 8) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const uint32_t sel = (gq & 1) ? 0x07060302u : 0x05040100u;
        uint32_t d[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const uint32_t x0 = (uint32_t)(w[0][bb] >> (32 * (gq >> 1)));
          const uint32_t x1 = (uint32_t)(w[1][bb] >> (32 * (gq >> 1)));
          d[bb] = __builtin_amdgcn_perm(x1, x0, sel);
        }
        *reinterpret_cast<uint2*>(&sm.words[pr][gq][bp]) = make_uint2(d[0], d[1]);
      }
    }
    // ---- A = -q_hj 2^(2-p) s_bj, bf16 hi + lo, per (row, block); padding rows 0 ----
#pragma unroll
    for (int i = 0; i < SC_PER; ++i) {
      const int lr = tid / GB + i * (SCAN_THREADS / GB);
      if (lr < nck * 8) {
        const int k = lr >> 3, i8 = lr & 7;
        const float* fr = sm.fq[seg_r0 + lr];
#pragma unroll
        for (int h0 = 0; h0 < G; h0 += 2) {
          const float x0 = fr[h0] * sv[i];
          const float x1 = h0 + 1 < G ? fr[h0 + 1] * sv[i] : 0.f;
          uint32_t hi, lo;
          split2(x0, x1, &hi, &lo);
          sm.atab[sb][a_index(k, h0 >> 2, 0, h0 & 3) + i8] = (uint16_t)hi;
          sm.atab[sb][a_index(k, h0 >> 2, 1, h0 & 3) + i8] = (uint16_t)lo;
          if (h0 + 1 < G) {
            sm.atab[sb][a_index(k, (h0 + 1) >> 2, 0, (h0 + 1) & 3) + i8] = (uint16_t)(hi >> 16);
            sm.atab[sb][a_index(k, (h0 + 1) >> 2, 1, (h0 + 1) & 3) + i8] = (uint16_t)(lo >> 16);
          }
        }
      }
    }
    __syncthreads();
    if (task + 1 < ntask) issue_loads(task + 1);  // in flight during the scoring below

    // ---- score the segment: wavefront takes blocks wb .. wb+3 of the step ----
    if (wb < gblk) {
      for (int k = 0; k < nck; ++k) {
        uint4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = *reinterpret_cast<const uint4*>(&sm.words[4 * k + q][grp][wb]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          uint32_t bw[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x = b == 0 ? v[q].x : b == 1 ? v[q].y : b == 2 ? v[q].z : v[q].w;
            // the lane's bits of rows 2q and 2q+1 at the sign bits of a bf16 pair
            bw[q] = sign_pair(__builtin_amdgcn_alignbit(x, x, rot), smask, vone);
          }
          bf16x8 bv;
          __builtin_memcpy(&bv, bw, 16);
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            const uint16_t* ap = a_active ? &sm.atab[wb + b][a_index(k, hg, 0, a_hh)]
                                          : reinterpret_cast<const uint16_t*>(sm.zero4);
            const uint16_t* aq = a_active ? ap + 4 * 8 : ap;
            const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(ap);
            const bf16x8 alo = *reinterpret_cast<const bf16x8*>(aq);
            acc[b][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, acc[b][hg], 0, 0, 0);
            acc[b][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, acc[b][hg], 0, 0, 0);
          }
        }
      }
    }

    // ---- epilogue after the last segment: lane <-> token, acc row r <-> head 4*hg + r ----
    if (sg == nseg - 1 && wb < gblk) {
      const int nblk = (gblk - wb) < NB ? (gblk - wb) : NB;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b >= nblk) break;
        const long long tok = (g0 + wb + b) * BLK + lane;
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int h = 4 * hg + r;
            if (h < G) emit(tok, h, acc[b][hg][r]);
          }
      }
    }
  }
  store_counts();
}

template <int G, int MODE>
hipError_t launch_gm(const ScanArgs& a0, hipStream_t st) {
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
  scan_kernel<G, MODE><<<grid, SCAN_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(const ScanArgs& a, hipStream_t st) {
  switch (a.g.G) {
    case 1: return launch_gm<1, MODE>(a, st);
    case 2: return launch_gm<2, MODE>(a, st);
    case 4: return launch_gm<4, MODE>(a, st);
    case 8: return launch_gm<8, MODE>(a, st);
    default: return hipErrorInvalidValue;
  }
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
                       const uint64_t* planes, const uint16_t* scales, float* scores,
                       hipStream_t st) {
  ScanArgs a = base_args(g, q_basis, depth, planes, scales);
  a.out = scores;
  a.out_ld = g.cap;
  return dispatch<SCAN_FULL>(a, st);
}

hipError_t launch_scan_flagged(const Geom& g, const float* q_basis, const uint8_t* depth,
                               const uint64_t* planes, const uint16_t* scales, float* scores,
                               const int32_t* flag, hipStream_t st) {
  ScanArgs a = base_args(g, q_basis, depth, planes, scales);
  a.out = scores;
  a.out_ld = g.cap;
  a.unit_flag = flag;
  return dispatch<SCAN_FULL>(a, st);
}

hipError_t launch_scan_sample(const Geom& g, const float* q_basis, const uint8_t* depth,
                              const uint64_t* planes, const uint16_t* scales, const CandBufs& cb,
                              hipStream_t st) {
  ScanArgs a = base_args(g, q_basis, depth, planes, scales);
  a.out = cb.sample;
  a.out_ld = cb.sample_ld;
  return dispatch<SCAN_SAMPLE>(a, st);
}

hipError_t launch_scan_cand(const Geom& g, const float* q_basis, const uint8_t* depth,
                            const uint64_t* planes, const uint16_t* scales, int k,
                            const CandBufs& cb, hipStream_t st) {
  ScanArgs a = base_args(g, q_basis, depth, planes, scales);
  a.k = k;
  a.thresh = cb.thresh;
  a.regions = cb.regions;
  a.cand_count = cb.count;
  a.cand_val = cb.val;
  a.cand_idx = cb.idx;
  return dispatch<SCAN_CAND>(a, st);
}

}  // namespace bpk
