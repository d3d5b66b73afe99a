// Prefix-plane key scan (Fathom §1, §3.2): approximate scores of every key of
// every complete block, reading only planes p < t_j of each channel and the
// block scales of the channels that are read at all.
//
// Work split: one workgroup (4 wavefronts) per (unit, chunk of CB blocks).
// The workgroup stages, in LDS, the compacted list of read channels, the
// chunk's plane words (each (channel, plane) row of CB words is one contiguous
// CB*8-byte read) and, per (block, channel, head), the coefficient
// q_hj * s_bj * 2^(4-t_j) plus a per-(block, head) constant.  Then each
// wavefront scores whole 64-token blocks, lane i <-> token i: the prefix code
// of a channel is assembled from bit i of its plane words (Horner), converted
// to fp32 and accumulated into G per-head scores:
//   score_h = sum_j coef_bjh * prefix_ij + const_bh,
//   const_bh = sum_j q_hj s_bj (2^(3-t_j) - 8) = sum_j coef_bjh (1/2 - 2^(t_j-1)),
// which is sum_j q_hj s_bj ((prefix_ij + 1/2) 2^(4-t_j) - 8) regrouped.
#include "bpk_internal.h"

namespace bpk {
namespace {

struct ScanArgs {
  Geom g;
  const float* q_basis;
  const uint8_t* depth;
  const uint64_t* planes;
  const uint16_t* scales;
  float* scores;
};

constexpr int SCAN_THREADS = 256;
constexpr int SCAN_WAVES = SCAN_THREADS / 64;

template <int G, int CB>
struct ScanSmem {
  uint64_t words[NP * D][CB];   // staged plane words, row r = (channel c, plane p)
  float coef[CB][D][G];         // q_hj * s_bj * 2^(4 - t_j) of read channel c
  float cst[CB][G];
  int scan_buf[D];
  uint8_t sel_j[D];
  uint8_t sel_t[D];
  uint16_t sel_pb[D];           // first staged row of read channel c
  uint8_t row_c[NP * D];        // staged row -> read channel
  uint8_t row_p[NP * D];        // staged row -> plane
  int n_read, n_rows;
};

template <int G, int CB>
__global__ __launch_bounds__(SCAN_THREADS) void scan_kernel(ScanArgs a) {
  __shared__ ScanSmem<G, CB> sm;
  const int u = blockIdx.y;
  const long long gu = a.g.global_unit(u);
  const long long n = a.g.n[a.g.seq_of(u)];
  const long long nb = n / BLK;
  const long long blk0 = (long long)blockIdx.x * CB;
  if (blk0 >= nb) return;
  const int nblk = (int)((nb - blk0) < CB ? (nb - blk0) : CB);
  const long long nbcap = a.g.nbcap();
  const int tid = threadIdx.x;

  // 1. compact the read channels (t_j >= 1) and number their plane rows
  int tj = 0, flag = 0;
  if (tid < D) {
    tj = a.depth[(long long)u * D + tid];
    tj = tj > NP ? NP : tj;
    flag = tj > 0;
    sm.scan_buf[tid] = (flag << 16) | tj;  // two counters in one int
  }
  __syncthreads();
  for (int off = 1; off < D; off <<= 1) {  // inclusive Hillis-Steele scan
    int v = 0;
    if (tid < D && tid >= off) v = sm.scan_buf[tid - off];
    __syncthreads();
    if (tid < D) sm.scan_buf[tid] += v;
    __syncthreads();
  }
  if (tid < D && flag) {
    const int incl = sm.scan_buf[tid];
    const int c = (incl >> 16) - 1;
    const int pb = (incl & 0xffff) - tj;
    sm.sel_j[c] = (uint8_t)tid;
    sm.sel_t[c] = (uint8_t)tj;
    sm.sel_pb[c] = (uint16_t)pb;
    for (int p = 0; p < tj; ++p) {
      sm.row_c[pb + p] = (uint8_t)c;
      sm.row_p[pb + p] = (uint8_t)p;
    }
  }
  if (tid == D - 1) {
    sm.n_read = sm.scan_buf[tid] >> 16;
    sm.n_rows = sm.scan_buf[tid] & 0xffff;
  }
  __syncthreads();
  const int n_read = sm.n_read;
  const int n_rows = sm.n_rows;

  // 2. stage plane words: row r of channel sel_j[c], plane p, blocks blk0..
  for (int e = tid; e < n_rows * CB; e += SCAN_THREADS) {
    const int r = e / CB, b = e % CB;
    uint64_t w = 0;
    if (b < nblk) {
      const int j = sm.sel_j[sm.row_c[r]];
      w = a.planes[((gu * D + j) * NP + sm.row_p[r]) * nbcap + blk0 + b];
    }
    sm.words[r][b] = w;
  }
  // 3. per-(block, read channel, head) coefficients
  const float* qb = a.q_basis + (long long)u * G * D;
  for (int e = tid; e < n_read * CB; e += SCAN_THREADS) {
    const int c = e / CB, b = e % CB;
    const int j = sm.sel_j[c], t = sm.sel_t[c];
    float s = 0.f;
    if (b < nblk) s = (float)__builtin_bit_cast(_Float16, a.scales[(gu * D + j) * nbcap + blk0 + b]);
    const float w = s * (float)(1 << (NP - t));
#pragma unroll
    for (int h = 0; h < G; ++h) sm.coef[b][c][h] = qb[h * D + j] * w;
  }
  __syncthreads();
  if (tid < CB * G) {
    // q_hj s_bj (2^(3-t) - 8) = coef_bjh * (1/2 - 2^(t-1))
    const int b = tid / G, h = tid % G;
    float acc = 0.f;
    for (int c = 0; c < n_read; ++c)
      acc = fmaf(sm.coef[b][c][h], 0.5f - (float)(1 << (sm.sel_t[c] - 1)), acc);
    sm.cst[b][h] = acc;
  }
  __syncthreads();

  // 4. score: wavefront w takes blocks w, w + 4, ...; lane <-> token
  const int wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, bitpos = lane & 31;
  float* out = a.scores + (long long)u * G * a.g.cap;
  for (int b = wave; b < nblk; b += SCAN_WAVES) {
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = sm.cst[b][h];
    for (int c = 0; c < n_read; ++c) {
      const int t = sm.sel_t[c], pb = sm.sel_pb[c];
      uint32_t code = 0;
      for (int p = 0; p < t; ++p) {
        const uint32_t wh = reinterpret_cast<const uint32_t*>(&sm.words[pb + p][b])[half];
        code = (code << 1) | ((wh >> bitpos) & 1u);
      }
      const float fc = (float)code;
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = fmaf(sm.coef[b][c][h], fc, acc[h]);
    }
    const long long tok = (blk0 + b) * BLK + lane;
#pragma unroll
    for (int h = 0; h < G; ++h) out[h * a.g.cap + tok] = acc[h];
  }
}

template <int G, int CB>
void launch_gc(const ScanArgs& a, hipStream_t st) {
  long long maxnb = 0;
  for (int s = 0; s < a.g.S; ++s) maxnb = a.g.n[s] / BLK > maxnb ? a.g.n[s] / BLK : maxnb;
  if (maxnb == 0) return;
  dim3 grid((unsigned)((maxnb + CB - 1) / CB), (unsigned)a.g.units());
  scan_kernel<G, CB><<<grid, SCAN_THREADS, 0, st>>>(a);
}

}  // namespace

hipError_t launch_scan(const Geom& g, const float* q_basis, const uint8_t* depth,
                       const uint64_t* planes, const uint16_t* scales, float* scores,
                       hipStream_t st) {
  ScanArgs a{g, q_basis, depth, planes, scales, scores};
  switch (g.G) {
    case 1: launch_gc<1, 8>(a, st); break;
    case 2: launch_gc<2, 8>(a, st); break;
    case 4: launch_gc<4, 8>(a, st); break;
    case 8: launch_gc<8, 4>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bpk
