// Prefix-plane key scan (Fathom §1, §3.2): approximate scores of every key of
// every complete block, reading only planes p < t_j of each read channel and
// the fp16 block scales of those channels.
//
// Per unit the score of token i for query head h is
//   s_hat = sum_j q_hj s_bj m_ij,  m = (c' + 1/2) 2^(4-t) - 8 = z 2^(4-t) + 2^(3-t)
// with c' the t-bit prefix code and z = c' - 2^(t-1) in [-8, 7].  Writing
// A_hj = q_hj s_bj 2^(4-t_j) gives s_hat = sum_j A_hj z_ij + sum_j A_hj / 2.
//
// Mapping onto gfx950:
// * A workgroup (4 wavefronts) owns a range of blocks of one unit and walks it
//   in steps of 16 blocks.  The read channels are cut into segments of whole
//   8-channel chunks holding at most 128 plane rows, so the LDS footprint is
//   fixed (~36 KB) whatever the depth vector.  Per (step, segment) the
//   workgroup stages into LDS, with coalesced reads, the segment's plane words
//   (rows of 16 consecutive blocks, split into 32-bit halves, the sign plane
//   complemented) and, per (block, channel, head), A_hj split into bf16 hi + lo
//   parts plus per-wavefront partial sums of the per-(block, head) constant.
//   Every global load of a (step, segment) is issued before the first is
//   used, and several resident workgroups per CU overlap one step's loads
//   with another's arithmetic.
// * Read channels are ordered deepest first, so an 8-channel chunk nearly
//   always has one depth and its Horner loop runs without per-channel
//   branches (a bit-field width of 0 idles a shallower channel).
// * Wavefront w scores blocks 4w .. 4w+3 of the step, lane i <-> token i.  For
//   a read channel a lane reads its half-word of each plane for the four
//   blocks with one 16-byte LDS read per plane and assembles z by a Horner
//   chain of bit-field extracts (a signed extract of the complemented sign
//   bit gives b0 - 1).
// * The G-head contraction runs on the matrix cores: v_mfma_f32_16x16x32_bf16
//   with B = 8 channels' z values of the lane's token (exact in bf16) and A
//   block-diagonal over the four 16-lane token groups (row 4g + h of A is
//   nonzero only in token group g's k-range), so D row 4g + h, column n is
//   head h's partial score of token 16g + n and each lane ends with the G
//   scores of its own token.  The hi + lo split of A keeps each term within
//   ~2^-17 of its exact value.
#include "bpk_internal.h"

namespace bpk {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

constexpr int SCAN_THREADS = 256;
constexpr int SCAN_WAVES = SCAN_THREADS / 64;
constexpr int NB = 4;                 // blocks per wavefront per step
constexpr int GB = NB * SCAN_WAVES;   // blocks per workgroup step
constexpr int SEG_ROWS = 128;         // plane rows staged per segment
constexpr int SEG_CHUNKS = 8;         // 8-channel chunks per segment
constexpr int MAX_SEGS = D / 8;       // one chunk per segment at worst
static_assert(SCAN_MIN_WG_BLOCKS == GB, "a workgroup takes whole steps");
static_assert(SAMPLE_GROUP % GB == 0 && SAMPLE_STRIDE % SAMPLE_GROUP == 0, "sample plan");

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

__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// z = c' - 2^(t-1) of the 8 channels of a chunk for the wavefront's 4 blocks.
// `base` is the lane's half-word of block 0 in plane row 0; row r is 2*GB
// dwords further.  All reads of a plane level are issued before they are
// used; a channel shallower than the level gets bit-field width 0 (no shift,
// no bit), a padding slot (t = 0) width 0 throughout (z = 0).
template <int TMAX>
__device__ __forceinline__ void chunk_codes(const uint32_t* base, const int rr[8], const int tc[8],
                                            int bitpos, int z[8][NB]) {
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    const uint32_t* row = base + rr[cc] * (2 * GB);
    const uint4 w0 = *reinterpret_cast<const uint4*>(row);
    const int wd0 = (int)((0u - (uint32_t)tc[cc]) >> 31);  // 1 if t > 0
    // plane 0 is stored complemented: a signed extract gives b0 - 1
    z[cc][0] = __builtin_amdgcn_sbfe(w0.x, bitpos, wd0);
    z[cc][1] = __builtin_amdgcn_sbfe(w0.y, bitpos, wd0);
    z[cc][2] = __builtin_amdgcn_sbfe(w0.z, bitpos, wd0);
    z[cc][3] = __builtin_amdgcn_sbfe(w0.w, bitpos, wd0);
#pragma unroll
    for (int p = 1; p < TMAX; ++p) {
      const uint4 w = *reinterpret_cast<const uint4*>(row + p * (2 * GB));
      const int wd = (int)(((uint32_t)p - (uint32_t)tc[cc]) >> 31);  // 1 if t > p
      z[cc][0] = (z[cc][0] << wd) | __builtin_amdgcn_ubfe(w.x, bitpos, wd);
      z[cc][1] = (z[cc][1] << wd) | __builtin_amdgcn_ubfe(w.y, bitpos, wd);
      z[cc][2] = (z[cc][2] << wd) | __builtin_amdgcn_ubfe(w.z, bitpos, wd);
      z[cc][3] = (z[cc][3] << wd) | __builtin_amdgcn_ubfe(w.w, bitpos, wd);
    }
  }
}

// 128-bit LDS accesses must be 16-byte aligned (misaligned ones stall)
template <int G>
struct ScanSmem {
  static constexpr int HG = (G + 3) / 4;  // head groups of 4 (MFMA rows)
  int scan_buf[D];
  uint8_t sel_j[D];
  uint8_t sel_t[D];                // depth of read channel c (0 past the last)
  uint16_t sel_pb[D];              // first plane row of read channel c
  int counts[4];                   // read channels, planes, segments
  int seg_c[MAX_SEGS + 1];         // first read channel of each segment
  uint64_t chan_sc[D];             // offset of the scales of read channel c; its plane 0
                                   // starts at word 4 * chan_sc[c] (planes [D][4][nbcap])
  uint8_t row_c[NP * D];           // plane row -> read channel
  uint8_t row_p[NP * D];           // plane row -> plane
  alignas(16) float qc[D * G];     // q_hj * 2^(4 - t_j) of read channel c
  alignas(16) uint32_t words[SEG_ROWS + 4][2][GB];  // [row][half][block] (+4 rows of slack)
  // A hi/lo per block: [chunk][hg][part][h][ch] bf16, rows padded by 16 bytes so
  // that the 16 blocks of a staging write land in different LDS banks
  static constexpr int ASTRIDE = SEG_CHUNKS * HG * 2 * 4 * 8 + 8;
  alignas(16) uint16_t atab[GB][ASTRIDE];
  alignas(16) float cpart[SCAN_WAVES][GB][G];  // per-wavefront partial sums of A / 2
  int ccount[G];                               // candidates of this workgroup per head
};

template <int G, int MODE>
__global__ __launch_bounds__(SCAN_THREADS) __attribute__((amdgpu_waves_per_eu(4, 8)))
void scan_kernel(ScanArgs a) {
  using SM = ScanSmem<G>;
  constexpr int HG = SM::HG;
  // offset of the 8 channels of (chunk k, head group hg, part, head h) in a block's A row
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

  // ---- plan: the read channels (t_j >= 1) sorted by depth, deepest first (j
  // ascending within a depth), so an 8-channel chunk is almost always of one
  // depth.  scan_buf packs four 8-bit counters, one per depth.
  int tj = 0;
  if (MODE == SCAN_CAND && tid < G) sm.ccount[tid] = 0;
  if (tid < D) {
    sm.sel_t[tid] = 0;
    tj = a.depth[(long long)u * D + tid];
    tj = tj > NP ? NP : tj;
    sm.scan_buf[tid] = tj > 0 ? 1 << (8 * (tj - 1)) : 0;
  }
  __syncthreads();
  for (int off = 1; off < D; off <<= 1) {
    int v = 0;
    if (tid < D && tid >= off) v = sm.scan_buf[tid - off];
    __syncthreads();
    if (tid < D) sm.scan_buf[tid] += v;
    __syncthreads();
  }
  const int tot = sm.scan_buf[D - 1];
  const int n4 = (tot >> 24) & 0xFF, n3 = (tot >> 16) & 0xFF, n2 = (tot >> 8) & 0xFF,
            n1 = tot & 0xFF;
  if (tid < D && tj > 0) {
    const int k = ((sm.scan_buf[tid] >> (8 * (tj - 1))) & 0xFF) - 1;  // rank within its depth
    const int cbase = tj == 4 ? 0 : tj == 3 ? n4 : tj == 2 ? n4 + n3 : n4 + n3 + n2;
    const int rbase0 = tj == 4 ? 0 : tj == 3 ? 4 * n4 : tj == 2 ? 4 * n4 + 3 * n3
                                                               : 4 * n4 + 3 * n3 + 2 * n2;
    const int c = cbase + k;
    const int pb = rbase0 + k * tj;
    sm.sel_j[c] = (uint8_t)tid;
    sm.sel_t[c] = (uint8_t)tj;
    sm.sel_pb[c] = (uint16_t)pb;
    sm.chan_sc[c] = (uint64_t)(gu * D + tid) * (uint64_t)nbcap;
    for (int p = 0; p < tj; ++p) {
      sm.row_c[pb + p] = (uint8_t)c;
      sm.row_p[pb + p] = (uint8_t)p;
    }
    const float w = (float)(1 << (NP - tj));
#pragma unroll
    for (int h = 0; h < G; ++h)
      sm.qc[c * G + h] = a.q_basis[((long long)u * G + h) * D + tid] * w;
  }
  __syncthreads();
  if (tid == 0) {
    // segments: whole chunks, at most SEG_CHUNKS chunks and SEG_ROWS rows
    const int C = n4 + n3 + n2 + n1;
    const int P = 4 * n4 + 3 * n3 + 2 * n2 + n1;
    int ns = 0, c = 0;
    while (c < C) {
      sm.seg_c[ns++] = c;
      int rows = 0, chunks = 0;
      while (c < C && chunks < SEG_CHUNKS) {
        const int ce = (c + 8) < C ? (c + 8) : C;
        const int r = (int)sm.sel_pb[ce - 1] + sm.sel_t[ce - 1] - sm.sel_pb[c];
        if (chunks > 0 && rows + r > SEG_ROWS) break;
        rows += r;
        c = ce;
        ++chunks;
      }
    }
    sm.seg_c[ns] = C;
    sm.counts[0] = C;
    sm.counts[1] = P;
    sm.counts[2] = ns;
  }
  __syncthreads();
  const int C = sm.counts[0];
  const int nseg = sm.counts[2];

  // A-operand ownership: lane l holds row 4*(l/16) + (l%4) of a head group,
  // in k-group l/16, only when (l%16)/4 == l/16 (block-diagonal).
  const bool a_active = ((lane & 15) >> 2) == (lane >> 4) && (lane & 3) < (G < 4 ? G : 4);
  const int a_hh = lane & 3;
  const int half = lane >> 5, bitpos = lane & 31;
  const int wb = NB * wave;

  // ---- tasks = (16-block step, segment); the loads of task i+1 are in flight
  // while task i is scored ----
  const int nsteps = (int)((wb1 - wb0 + GB - 1) / GB);
  const int ntask = nsteps * nseg;
  constexpr int PER = SEG_ROWS * (GB / 2) / SCAN_THREADS;   // word pairs per thread
  constexpr int PERS = SEG_CHUNKS * 8 * GB / SCAN_THREADS;  // scales per thread
  const int sb = tid % GB;  // block of this thread's scales (same for every i)
  uint64_t w[PER][2];
  float sv[PERS];
  auto issue_loads = [&](int task) {
    const long long g0 = wb0 + (long long)(task / nseg) * GB;
    const int sg = task % nseg;
    const int gblk = (wb1 - g0) < GB ? (int)(wb1 - g0) : GB;
    const int cs0 = sm.seg_c[sg], cs1 = sm.seg_c[sg + 1];
    const int rbase = sm.sel_pb[cs0];
    const int nrows = (int)sm.sel_pb[cs1 - 1] + sm.sel_t[cs1 - 1] - rbase;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * SCAN_THREADS;
      const int rr = e / (GB / 2), b2 = 2 * (e % (GB / 2));
      w[i][0] = 0;
      w[i][1] = 0;
      if (rr < nrows) {
        const int r = rbase + rr;
        const int c = sm.row_c[r], p = sm.row_p[r];
        const uint64_t* src = a.planes + NP * sm.chan_sc[c] + (uint64_t)p * nbcap + g0 + b2;
        if (b2 + 1 < gblk) {  // rows are 8-byte aligned only
          w[i][0] = src[0];
          w[i][1] = src[1];
        } else if (b2 < gblk) {
          w[i][0] = src[0];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < PERS; ++i) {
      const int c = cs0 + (tid + i * SCAN_THREADS) / GB;
      sv[i] = 0.f;
      if (c < cs1 && sb < gblk)
        sv[i] = (float)__builtin_bit_cast(_Float16, a.scales[sm.chan_sc[c] + g0 + sb]);
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
  bf16x8 ahi, alo;  // A operand (hi, lo parts); zero on the block-diagonal's idle lanes
  {
    const uint32_t z4[4] = {0u, 0u, 0u, 0u};
    __builtin_memcpy(&ahi, z4, 16);
    __builtin_memcpy(&alo, z4, 16);
  }
  issue_loads(0);
  for (int task = 0; task < ntask; ++task) {
    const long long g0 = wb0 + (long long)(task / nseg) * GB;
    const int sg = task % nseg;
    const int gblk = (wb1 - g0) < GB ? (int)(wb1 - g0) : GB;
    if (sg == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) acc[b][hg] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    {
      const int cs0 = sm.seg_c[sg], cs1 = sm.seg_c[sg + 1];
      const int rbase = sm.sel_pb[cs0];
      const int nrows = (int)sm.sel_pb[cs1 - 1] + sm.sel_t[cs1 - 1] - rbase;
      const int nck = (cs1 - cs0 + 7) >> 3;
      __syncthreads();  // the previous task's tables are no longer read

      // ---- words -> LDS (the sign plane complemented) ----
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = tid + i * SCAN_THREADS;
        const int rr = e / (GB / 2), b2 = 2 * (e % (GB / 2));
        if (rr < nrows) {
          if (sm.row_p[rbase + rr] == 0) {
            w[i][0] = ~w[i][0];
            w[i][1] = ~w[i][1];
          }
          *reinterpret_cast<uint2*>(&sm.words[rr][0][b2]) =
              make_uint2((uint32_t)w[i][0], (uint32_t)w[i][1]);
          *reinterpret_cast<uint2*>(&sm.words[rr][1][b2]) =
              make_uint2((uint32_t)(w[i][0] >> 32), (uint32_t)(w[i][1] >> 32));
        }
      }
      // ---- A = q_hj s_bj 2^(4-t_j) as bf16 hi + lo, partial sums of A / 2 ----
      float part[G];
#pragma unroll
      for (int h = 0; h < G; ++h) part[h] = 0.f;
#pragma unroll
      for (int i = 0; i < PERS; ++i) {
        const int cl = (tid + i * SCAN_THREADS) / GB;
        if (cl < nck * 8) {
          const int c = cs0 + cl;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float x = c < cs1 ? sm.qc[c * G + h] * sv[i] : 0.f;
            part[h] += 0.5f * x;
            const uint16_t hi = bf16_rne_bits(x);
            const uint16_t lo = bf16_rne_bits(x - __uint_as_float((uint32_t)hi << 16));
            sm.atab[sb][a_index(cl >> 3, h >> 2, 0, h & 3) + (cl & 7)] = hi;
            sm.atab[sb][a_index(cl >> 3, h >> 2, 1, h & 3) + (cl & 7)] = lo;
          }
        }
      }
      // lanes l, l+16, l+32, l+48 share a block: fixed-order reduction
#pragma unroll
      for (int h = 0; h < G; ++h) {
        part[h] += __shfl_xor(part[h], 16);
        part[h] += __shfl_xor(part[h], 32);
      }
      if (lane < GB) {
#pragma unroll
        for (int h = 0; h < G; ++h) sm.cpart[wave][lane][h] = part[h];
      }
      __syncthreads();
      if (task + 1 < ntask) issue_loads(task + 1);  // in flight during the scoring below

      // ---- score the segment: wavefront takes blocks wb .. wb+3 of the step ----
      if (wb < gblk) {
        // the constant sum_j A_hj / 2 enters the accumulator of (token, head 4hg + r)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int hg = 0; hg < HG; ++hg)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int h = 4 * hg + r;
              if (h < G) {
                float cs = 0.f;
#pragma unroll
                for (int ww = 0; ww < SCAN_WAVES; ++ww) cs += sm.cpart[ww][wb + b][h];
                acc[b][hg][r] += cs;
              }
            }

        for (int kl = 0; kl < nck; ++kl) {
          const int cb = cs0 + 8 * kl;
          // the chunk's depths and first rows, wave-uniform
          const uint32_t t03 = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(&sm.sel_t[cb]));
          const uint32_t t47 = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(&sm.sel_t[cb + 4]));
          uint32_t pbw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pbw[i] = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(&sm.sel_pb[cb + 2 * i]));
          // chunk channels are sorted by depth: channel 0 is the deepest
          const int tmax = (int)(t03 & 0xFFu);
          int tc[8], rr[8], z[8][NB];
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            tc[cc] = (int)(((cc < 4 ? t03 : t47) >> (8 * (cc & 3))) & 0xFFu);
            // a padding slot (t = 0) reads row 0 of the segment with width 0: z = 0
            rr[cc] = tc[cc] > 0 ? (int)((pbw[cc >> 1] >> (16 * (cc & 1))) & 0xFFFFu) - rbase : 0;
          }
          switch (tmax) {
            case 1: chunk_codes<1>(&sm.words[0][half][wb], rr, tc, bitpos, z); break;
            case 2: chunk_codes<2>(&sm.words[0][half][wb], rr, tc, bitpos, z); break;
            case 3: chunk_codes<3>(&sm.words[0][half][wb], rr, tc, bitpos, z); break;
            default: chunk_codes<4>(&sm.words[0][half][wb], rr, tc, bitpos, z); break;
          }
          // bf16 pairs of z (exact): the high halves of their fp32 values
          uint32_t bw[NB][4];
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int cp = 0; cp < 4; ++cp)
              bw[b][cp] = __builtin_amdgcn_perm(__float_as_uint((float)z[2 * cp + 1][b]),
                                                __float_as_uint((float)z[2 * cp][b]), 0x07060302u);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            bf16x8 bv;
            __builtin_memcpy(&bv, bw[b], 16);
#pragma unroll
            for (int hg = 0; hg < HG; ++hg) {
              // inactive lanes keep the zeros they were given once
              if (a_active) {
                ahi = *reinterpret_cast<const bf16x8*>(&sm.atab[wb + b][a_index(kl, hg, 0, a_hh)]);
                alo = *reinterpret_cast<const bf16x8*>(&sm.atab[wb + b][a_index(kl, hg, 1, a_hh)]);
              }
              acc[b][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, acc[b][hg], 0, 0, 0);
              acc[b][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, acc[b][hg], 0, 0, 0);
            }
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
