// Per-query-head top-k (Fathom §2, "Top-k decoding"): the first 4 and the last
// W tokens are kept, W = max(32, n mod 64); the other k - 4 - W are the largest
// scores among tokens [4, n - W), equal scores to the lower index.
//
// One workgroup of 1024 threads per (unit, query head).  A radix select over
// order-preserving 32-bit keys (3 digit passes of 11/11/10 bits, histograms in
// LDS) finds the exact key K* of the (k - 4 - W)-th largest score and how many
// keys equal to K* must be taken; if fewer than all of them, a second radix
// select over the complemented token index picks the lowest indices among the
// ties.  The winners are collected into LDS, sorted ascending with a bitonic
// network and written out.
//
// decode_step's fused selection adds two kernels:
// * threshold_reg_kernel (threshold_kernel, on the radix machinery, for
//   samples over 16384 scores): per (unit, head), the r-th largest of the
//   sampled scores of candidate tokens, with r chosen so that about
//   2 (k - 4 - W) tokens of the whole range are expected at or above it (plus
//   8 for the sampling noise of small r).  The sample holds the upper 16 bits
//   of each score's order key, so the threshold is that score with its low
//   16 key bits cleared: at most 2^-7 of it below the sampled score (never
//   above), a few more candidates and never fewer;
// * cand_select_kernel: one workgroup per unit; for each query head one
//   wavefront takes the exact top (k - 4 - W) of the candidates (every token
//   at or above the threshold, and possibly a few just below it, so the
//   k - 4 - W largest of the whole range are among them whenever at least
//   that many are at or above it) by a bit-by-bit counting search over its
//   register-resident keys, and sorts the winners by index.  A head with too
//   few candidates at or above the threshold, or more than the buffers hold,
//   flags its unit for the full scan and radix select.  Otherwise the
//   workgroup also merges the unit's G lists into the union of rows that the
//   attention reads (the union stage of attend.hip, for the flagged units
//   only, runs after their full selection).
#include <limits.h>

#include <type_traits>

#include "bpk_internal.h"
#include "union_common.h"

namespace bpk {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_BINS = 2048;

struct TopkArgs {
  Geom g;
  const float* scores;
  int k;
  int32_t* idx;
  const int32_t* unit_flag;  // if set, only units with flag != 0
};

struct TkSmem {
  uint32_t hist[TK_BINS];
  int scan[TK_THREADS];
  int32_t buf[BPK_MAX_K];
  int digit, rem, cnt;
};

// Exclusive prefix sum of one value per thread over the workgroup.
__device__ int block_excl_scan(TkSmem& sm, int v) {
  const int tid = threadIdx.x;
  sm.scan[tid] = v;
  __syncthreads();
  for (int off = 1; off < TK_THREADS; off <<= 1) {
    int x = tid >= off ? sm.scan[tid - off] : 0;
    __syncthreads();
    sm.scan[tid] += x;
    __syncthreads();
  }
  const int incl = sm.scan[tid];
  __syncthreads();
  return incl - v;
}

// Radix select: among elements i in [lo, hi) with pred(i), find the want-th
// largest key (want >= 1, and at least want such elements exist).  Returns
// the key; *taken_eq = how many elements equal to it are among the top want;
// *count_eq = how many elements equal it.
template <typename KeyFn, typename PredFn>
__device__ uint32_t radix_select(TkSmem& sm, long long lo, long long hi, int want, KeyFn keyf,
                                 PredFn pred, int* taken_eq, int* count_eq) {
  const int tid = threadIdx.x;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  uint32_t prefix = 0, mask = 0;
  int rem = want, last_count = 0;
#pragma unroll
  for (int ps = 0; ps < 3; ++ps) {
    const int sh = shifts[ps];
    const uint32_t nbins = 1u << widths[ps];
    for (int b = tid; b < TK_BINS; b += TK_THREADS) sm.hist[b] = 0;
    __syncthreads();
    for (long long i = lo + tid; i < hi; i += TK_THREADS) {
      if (!pred(i)) continue;
      const uint32_t key = keyf(i);
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> sh) & (nbins - 1)], 1u);
    }
    __syncthreads();
    // thread t owns bins nbins-1-2t and nbins-2-2t (descending key order)
    int own = 0;
    for (int q = 0; q < 2; ++q) {
      const int b = (int)nbins - 1 - 2 * tid - q;
      if (b >= 0) own += (int)sm.hist[b];
    }
    int run = block_excl_scan(sm, own);
    for (int q = 0; q < 2; ++q) {
      const int b = (int)nbins - 1 - 2 * tid - q;
      if (b < 0) break;
      const int c = (int)sm.hist[b];
      if (run < rem && run + c >= rem) {
        sm.digit = b;
        sm.rem = rem - run;
        sm.cnt = c;
      }
      run += c;
    }
    __syncthreads();
    prefix |= (uint32_t)sm.digit << sh;
    mask |= (nbins - 1) << sh;
    rem = sm.rem;
    last_count = sm.cnt;
    __syncthreads();
  }
  *taken_eq = rem;
  *count_eq = last_count;
  return prefix;
}

// Sorts buf[0..k) ascending (a bitonic network, INT_MAX padding up to a power
// of two; buf holds at least that many entries) and writes it to out.
__device__ void sort_and_write(int32_t* buf, int k, int32_t* out) {
  const int tid = threadIdx.x;
  int m = 1;
  while (m < k) m <<= 1;
  for (int i = k + tid; i < m; i += TK_THREADS) buf[i] = INT_MAX;
  __syncthreads();
  for (int size = 2; size <= m; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < m / 2; i += TK_THREADS) {
        const int lo_i = 2 * i - (i & (stride - 1));
        const int hi_i = lo_i + stride;
        const bool up = ((lo_i & size) == 0);
        const int32_t x = buf[lo_i], y = buf[hi_i];
        if ((x > y) == up) {
          buf[lo_i] = y;
          buf[hi_i] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += TK_THREADS) out[i] = buf[i];
}

// the top-k of query head h of unit u, by the TK_THREADS threads of a
// workgroup (every thread calls it)
__device__ __forceinline__ void topk_head(TkSmem& sm, const TopkArgs& a, int u, int h) {
  const int G = a.g.G;
  const long long n = a.g.n[a.g.seq_of(u)];
  const int k = a.k;
  const int tid = threadIdx.x;
  int32_t* out = a.idx + ((long long)u * G + h) * k;
  if (n <= k) {
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  const long long w = kept_tail(n);
  const long long lo = 4, hi = n - w;
  const int want = k - 4 - (int)w;
  const float* sc = a.scores + ((long long)u * G + h) * a.g.cap;
  auto keyf = [&](long long i) { return order_key(sc[i]); };
  auto all = [](long long) { return true; };

  uint32_t kstar = 0;
  int take_eq = 0, count_eq = 0;
  long long idx_limit = LLONG_MAX;
  if (want > 0) {
    kstar = radix_select(sm, lo, hi, want, keyf, all, &take_eq, &count_eq);
    if (take_eq < count_eq) {
      // lowest token indices among the ties: largest complemented index
      auto ckey = [&](long long i) { return ~(uint32_t)i; };
      auto tie = [&](long long i) { return order_key(sc[i]) == kstar; };
      int t2, c2;
      const uint32_t k2 = radix_select(sm, lo, hi, take_eq, ckey, tie, &t2, &c2);
      idx_limit = (long long)(~k2);
    }
  }
  __syncthreads();
  if (tid == 0) sm.cnt = 0;
  __syncthreads();
  // always-kept tokens
  for (long long i = tid; i < 4; i += TK_THREADS) sm.buf[atomicAdd(&sm.cnt, 1)] = (int32_t)i;
  for (long long i = hi + tid; i < n; i += TK_THREADS) sm.buf[atomicAdd(&sm.cnt, 1)] = (int32_t)i;
  if (want > 0) {
    for (long long i = lo + tid; i < hi; i += TK_THREADS) {
      const uint32_t key = order_key(sc[i]);
      if (key > kstar || (key == kstar && i <= idx_limit))
        sm.buf[atomicAdd(&sm.cnt, 1)] = (int32_t)i;
    }
  }
  __syncthreads();
  sort_and_write(sm.buf, k, out);
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
  __shared__ TkSmem sm;
  topk_head(sm, a, blockIdx.x / a.g.G, blockIdx.x % a.g.G);
}

// decode_step's fallback: one workgroup per unit whose flag is set takes the
// top-k of its heads in turn and then, with un.uidx, the union of the lists
// it wrote (union_of_lists; the workgroup's own global writes, ordered by
// its barriers)
__global__ __launch_bounds__(TK_THREADS) void topk_unit_kernel(TopkArgs a, UnionBufs un) {
  __shared__ TkSmem sm;
  const int u = blockIdx.x;
  if (a.unit_flag[u] == 0) return;
  const int G = a.g.G;
  for (int h = 0; h < G; ++h) {
    topk_head(sm, a, u, h);
    __syncthreads();
  }
  if (!un.uidx) return;
  const long long sel = (long long)G * a.k;
  union_of_lists(a.idx + u * sel, G, a.k, a.g.n[a.g.seq_of(u)], un.uidx + u * sel,
                 un.umask + u * sel, un.ucount + u);
}

// maximum over the wavefront: DPP inside each 16-lane row (quad_perm xor 1,
// xor 2, row_half_mirror, row_mirror), then the four rows' results read out;
// every lane must be active
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  auto mx = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return mx(mx((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
            mx((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// sum over the wavefront: DPP inside each 16-lane row (quad_perm xor 1, xor
// 2, row_half_mirror, row_mirror), then the four rows' sums read out; every
// lane must be active
__device__ __forceinline__ int wave_sum_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// bits at and below the highest set bit of x (0 for x == 0), by smearing
// (no leading-zero count and no select on x == 0, both of which have
// compiled to scalar code testing the wrong condition)
__device__ __forceinline__ uint32_t low_mask(uint32_t x) {
  x |= x >> 1;
  x |= x >> 2;
  x |= x >> 4;
  x |= x >> 8;
  x |= x >> 16;
  return x;
}

struct ThreshArgs {
  Geom g;
  int k;
  CandBufs cb;
};

__global__ __launch_bounds__(TK_THREADS) void threshold_kernel(ThreshArgs a) {
  __shared__ TkSmem sm;
  const int G = a.g.G;
  const int u = blockIdx.x / G, h = blockIdx.x % G;
  const long long uh = (long long)u * G + h;
  const int tid = threadIdx.x;
  const long long n = a.g.n[a.g.seq_of(u)];
  const long long w = kept_tail(n);
  const long long hi = n - w;
  const long long want = (long long)a.k - 4 - w;
  uint32_t tkey = 0xFFFFFFFFu;  // nothing is a candidate
  if (n > a.k && want > 0) {
    // sample position i = (group gi, offset j) holds token gi * SAMPLE_STRIDE * 64 + j
    const long long nb = n / BLK;
    const long long ngr = (nb + SAMPLE_STRIDE - 1) / SAMPLE_STRIDE;
    const long long gtok = (long long)SAMPLE_STRIDE * BLK, glen = (long long)SAMPLE_GROUP * BLK;
    auto tok_of = [&](long long i) { return (i / glen) * gtok + i % glen; };
    auto valid = [&](long long i) {
      const long long t = tok_of(i);
      return t >= 4 && t < hi;
    };
    // candidate tokens that were sampled
    long long m = 0;
    for (long long gi = 0; gi < ngr; ++gi) {
      const long long t0 = gi * gtok, t1 = t0 + glen;
      const long long x0 = t0 > 4 ? t0 : 4, x1 = t1 < hi ? t1 : hi;
      m += x1 > x0 ? x1 - x0 : 0;
    }
    const long long nc = hi - 4;
    const long long r = (2 * want * m + nc - 1) / nc + 8;
    if (r > m) {
      tkey = 0;  // the sample is too small to cut anything: all are candidates
    } else {
      const uint16_t* sc = a.cb.sample + uh * a.cb.sample_ld;
      auto keyf = [&](long long i) { return (uint32_t)sc[i] << 16; };
      int t_eq, c_eq;
      tkey = radix_select(sm, 0, ngr * glen, (int)r, keyf, valid, &t_eq, &c_eq);
    }
  }
  if (tid == 0) {
    a.cb.thresh[uh] = tkey;
    if (h == 0) a.cb.flag[u] = 0;
  }
}

// The same threshold with the sample in registers (NPT keys a thread, the
// sample of every head of the launch at most 256 * NPT): T, the largest key
// with at least r valid keys >= T.  When r <= 64, each wavefront first takes
// the r-th largest of its lanes' largest keys: r keys of that wavefront alone
// are at or above it, so it is at most T, and so is the largest of the four.
// The keys at or above that bound (a few r) are compacted into LDS and T is
// found bit by bit from the top over them alone, four a lane in registers.
// Otherwise (r > 64, or more than TH_CAP keys pass the bound, as when r is
// close to 64) every bit is probed over all keys, each count reduced over the
// wavefronts through LDS (two slots, so one barrier a probe).
constexpr int TH_THREADS = 256;
constexpr int TH_CAP = 256;  // compacted keys searched in registers (4 a lane)

template <int NPT>
__global__ __launch_bounds__(TH_THREADS) void threshold_reg_kernel(ThreshArgs a) {
  __shared__ int part[2][TH_THREADS / 64];
  __shared__ uint32_t bound[TH_THREADS / 64];
  __shared__ uint32_t near[TH_CAP];
  __shared__ int nnear;
  const int G = a.g.G;
  const int u = blockIdx.x / G, h = blockIdx.x % G;
  const long long uh = (long long)u * G + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long n = a.g.n[a.g.seq_of(u)];
  const long long w = kept_tail(n);
  const long long hi = n - w;
  const long long want = (long long)a.k - 4 - w;
  uint32_t tkey = 0xFFFFFFFFu;  // nothing is a candidate
  if (n > a.k && want > 0) {
    const long long nb = n / BLK;
    const long long ngr = (nb + SAMPLE_STRIDE - 1) / SAMPLE_STRIDE;
    const long long gtok = (long long)SAMPLE_STRIDE * BLK, glen = (long long)SAMPLE_GROUP * BLK;
    long long m = 0;
    for (long long gi = 0; gi < ngr; ++gi) {
      const long long t0 = gi * gtok, t1 = t0 + glen;
      const long long x0 = t0 > 4 ? t0 : 4, x1 = t1 < hi ? t1 : hi;
      m += x1 > x0 ? x1 - x0 : 0;
    }
    const long long nc = hi - 4;
    const long long r = (2 * want * m + nc - 1) / nc + 8;
    if (r > m) {
      tkey = 0;  // the sample is too small to cut anything: all are candidates
    } else {
      // sample position i = (group gi, offset j) holds token gi * SAMPLE_STRIDE * 64 + j;
      // invalid positions hold key 0, below every probe
      // (16-byte loads: thread t takes positions 8 (q * TH_THREADS + t) .. + 7;
      // rows and len are multiples of 8; a key is its stored upper half)
      const uint4* sc = reinterpret_cast<const uint4*>(a.cb.sample + uh * a.cb.sample_ld);
      const long long len = ngr * glen;
      uint4 w8[NPT / 8];
#pragma unroll
      for (int q = 0; q < NPT / 8; ++q) {
        const long long i8 = (long long)q * TH_THREADS + tid;
        w8[q] = sc[8 * i8 < len ? i8 : 0];
      }
      uint32_t key[NPT];
      uint32_t mx = 0u;
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        const long long i = 8 * ((long long)(q / 8) * TH_THREADS + tid) + q % 8;
        const long long t = (i / glen) * gtok + i % glen;
        const uint4 v = w8[q / 8];
        const uint32_t w = (q % 8) / 2 == 0 ? v.x : (q % 8) / 2 == 1 ? v.y : (q % 8) / 2 == 2 ? v.z : v.w;
        const uint32_t k16 = (q % 2) ? (w & 0xFFFF0000u) : (w << 16);
        key[q] = (i < len && t >= 4 && t < hi) ? k16 : 0u;
        mx = key[q] > mx ? key[q] : mx;
      }
      if (tid == 0) nnear = 0;
      int slot = 0;
      // keys >= t over the workgroup
      auto block_count = [&](uint32_t t) {
        int c = 0;
#pragma unroll
        for (int q = 0; q < NPT; ++q) {
          c += __popcll(__ballot(key[q] >= t));
          // a few masks live at a time (the compiler would otherwise hold
          // them all in scalar registers)
          if (q % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        }
        if (lane == 0) part[slot][wave] = c;
        __syncthreads();
        int tot = 0;
#pragma unroll
        for (int x = 0; x < TH_THREADS / 64; ++x) tot += part[slot][x];
        slot ^= 1;
        return tot;
      };
      // the lower bound (0 when r > 64: no cut)
      uint32_t lw = 0u;
      if (r <= 64) {  // (keys have 16 significant bits)
        for (int b = 31; b >= 16; --b) {
          const uint32_t t = lw | (1u << b);
          if (__popcll(__ballot(mx >= t)) >= r) lw = t;
        }
      }
      if (lane == 0) bound[wave] = lw;
      __syncthreads();
      uint32_t L = 0u;
#pragma unroll
      for (int x = 0; x < TH_THREADS / 64; ++x) L = bound[x] > L ? bound[x] : L;
      uint32_t T = 0u;
      if (L != 0u) {
        // the keys at or above the bound
#pragma unroll
        for (int q = 0; q < NPT; ++q) {
          const bool nr = key[q] >= L;
          const uint64_t mk = __ballot(nr);
          if (mk != 0ull) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&nnear, __popcll(mk));
            base = __shfl(base, 0);
            const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                       (uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
            if (nr && pos < TH_CAP) near[pos] = key[q];
          }
        }
        __syncthreads();
      }
      const int nn = nnear;
      if (L != 0u && nn <= TH_CAP) {
        // every wavefront finishes the same search over the compacted keys,
        // four a lane in registers (0 past nn, below every probe); T >= L,
        // so the bits above the highest one where L and the largest compacted
        // key differ are L's
        uint32_t nk[4];
        uint32_t hk = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = lane + 64 * j;
          nk[j] = i < nn ? near[i] : 0u;
          hk = nk[j] > hk ? nk[j] : hk;
        }
        hk = wave_max_dpp(hk);
        const uint32_t low = low_mask(L ^ hk);
        T = L & ~low;
        for (int b = __popc(low) - 1; b >= 16; --b) {
          const uint32_t t = T | (1u << b);
          int c = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) c += __popcll(__ballot(nk[j] >= t));
          if (c >= r) T = t;
        }
      } else {
        for (int b = 31; b >= 16; --b) {
          const uint32_t t = T | (1u << b);
          if (block_count(t) >= r) T = t;
        }
      }
      tkey = T;
    }
  }
  if (tid == 0) {
    a.cb.thresh[uh] = tkey;
    if (h == 0) a.cb.flag[u] = 0;
  }
}

// The same threshold with one wavefront per (unit, head), four heads per
// workgroup and no workgroup barrier, for samples of at most 64 * NPT keys
// (NPT keys a lane): the lane maxima's r-th largest bounds T from below when
// r <= 64, the keys at or above the bound are compacted into the wavefront's
// LDS area and searched bit by bit, four a lane; otherwise every bit is
// probed over all keys.
template <int NPT>
__global__ __launch_bounds__(256) void threshold_wave_kernel(ThreshArgs a) {
  __shared__ uint32_t near[4][TH_CAP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = a.g.G;
  const long long uh = (long long)blockIdx.x * 4 + wave;
  if (uh >= (long long)a.g.units() * G) return;  // (no barrier follows)
  const int u = (int)(uh / G), h = (int)(uh % G);
  const long long n = a.g.n[a.g.seq_of(u)];
  const long long w = kept_tail(n);
  const long long hi = n - w;
  const long long want = (long long)a.k - 4 - w;
  uint32_t tkey = 0xFFFFFFFFu;  // nothing is a candidate
  if (n > a.k && want > 0) {
    const long long nb = n / BLK;
    const long long ngr = (nb + SAMPLE_STRIDE - 1) / SAMPLE_STRIDE;
    const long long gtok = (long long)SAMPLE_STRIDE * BLK, glen = (long long)SAMPLE_GROUP * BLK;
    long long m = 0;
    for (long long gi = 0; gi < ngr; ++gi) {
      const long long t0 = gi * gtok, t1 = t0 + glen;
      const long long x0 = t0 > 4 ? t0 : 4, x1 = t1 < hi ? t1 : hi;
      m += x1 > x0 ? x1 - x0 : 0;
    }
    const long long nc = hi - 4;
    const long long r = (2 * want * m + nc - 1) / nc + 8;
    if (r > m) {
      tkey = 0;  // the sample is too small to cut anything: all are candidates
    } else {
      // 16-byte loads: lane l takes positions 8 (q * 64 + l) .. + 7 (rows and
      // len are multiples of 8; a key is its stored upper half)
      const uint4* sc = reinterpret_cast<const uint4*>(a.cb.sample + uh * a.cb.sample_ld);
      const long long len = ngr * glen;
      uint4 w8[NPT / 8];
#pragma unroll
      for (int q = 0; q < NPT / 8; ++q) {
        const long long i8 = (long long)q * 64 + lane;
        w8[q] = sc[8 * i8 < len ? i8 : 0];
      }
      uint32_t key[NPT];
      uint32_t mx = 0u;
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        const long long i = 8 * ((long long)(q / 8) * 64 + lane) + q % 8;
        const long long t = (i / glen) * gtok + i % glen;
        const uint4 v = w8[q / 8];
        const uint32_t wd = (q % 8) / 2 == 0 ? v.x : (q % 8) / 2 == 1 ? v.y : (q % 8) / 2 == 2 ? v.z : v.w;
        const uint32_t k16 = (q % 2) ? (wd & 0xFFFF0000u) : (wd << 16);
        key[q] = (i < len && t >= 4 && t < hi) ? k16 : 0u;
        mx = key[q] > mx ? key[q] : mx;
      }
      // the lower bound (0 when r > 64: no cut); keys have 16 significant bits
      uint32_t L = 0u;
      if (r <= 64) {
        for (int b = 31; b >= 16; --b) {
          const uint32_t t = L | (1u << b);
          if (__popcll(__ballot(mx >= t)) >= r) L = t;
        }
      }
      uint32_t T = 0u;
      int nn = TH_CAP + 1;
      if (L != 0u) {
        // the keys at or above the bound, compacted in key order of the lanes
        int base = 0;
#pragma unroll
        for (int q = 0; q < NPT; ++q) {
          const bool nr = key[q] >= L;
          const uint64_t mk = __ballot(nr);
          const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
          if (nr && pos < TH_CAP) near[wave][pos] = key[q];
          base += __popcll(mk);
        }
        nn = base;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (L != 0u && nn <= TH_CAP) {
        // four compacted keys a lane (0 past nn, below every probe); T >= L,
        // so the bits above the highest one where L and the largest compacted
        // key differ are L's
        uint32_t nk[4];
        uint32_t hk = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = lane + 64 * j;
          nk[j] = i < nn ? near[wave][i] : 0u;
          hk = nk[j] > hk ? nk[j] : hk;
        }
        hk = wave_max_dpp(hk);
        const uint32_t low = low_mask(L ^ hk);
        T = L & ~low;
        for (int b = __popc(low) - 1; b >= 16; --b) {
          const uint32_t t = T | (1u << b);
          int c = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) c += __popcll(__ballot(nk[j] >= t));
          if (c >= r) T = t;
        }
      } else {
        for (int b = 31; b >= 16; --b) {
          const uint32_t t = T | (1u << b);
          int c = 0;
#pragma unroll
          for (int q = 0; q < NPT; ++q) c += key[q] >= t ? 1 : 0;
          if (wave_sum_dpp(c) >= r) T = t;
        }
      }
      tkey = T;
    }
  }
  if (lane == 0) {
    a.cb.thresh[uh] = tkey;
    if (h == 0) a.cb.flag[u] = 0;
  }
}

constexpr int CAND_MAX_PARTS = 4096;  // region parts per head the selection indexes (more: flagged)
static_assert(CAND_CAP < 65536, "16-bit part prefixes");
static_assert(8 * (int)sizeof(int) * (CAND_MAX_PARTS / 2 > FUSED_MAX_K ? CAND_MAX_PARTS / 2 : FUSED_MAX_K) <=
                  65536,
              "eight heads' areas fit 64 KiB of LDS");
constexpr int CS_NPL = CAND_CAP / 64;  // candidates per lane
constexpr int CS_WPL = FUSED_MAX_K / 64;  // winners per lane in the index sort
static_assert(CAND_CAP % 64 == 0 && FUSED_MAX_K % 64 == 0, "whole wavefront rows");
static_assert(FUSED_MAX_K <= 16 * 64, "the union merge takes at most 16 entries a lane");

struct CandArgs {
  Geom g;
  int k;
  CandBufs cb;
  int32_t* idx;
  int lds_ints;    // LDS ints per wavefront: the 16-bit part prefix, then the winners and the head's list
  UnionBufs un;    // the unit's union rows (when fuse_union)
  int fuse_union;  // 1: the workgroup also merges its unit's lists (unflagged units)
};

// number of lanes of candidate rows r < NPL with pred(r): per-lane counts in
// two registers (no scalar chain per row), then one wavefront sum; rows are
// taken in groups of CS_GROUP, a group wholly at or past total skipped
constexpr int CS_GROUP = 16;
template <int NPL, typename Pred>
__device__ __forceinline__ int wave_count(int total, Pred pred) {
  int c0 = 0, c1 = 0;
#pragma unroll
  for (int g = 0; g < NPL; g += CS_GROUP) {
    if (g * 64 < total) {
  #pragma unroll
      for (int r = g; r < g + CS_GROUP; r += 2) {
        c0 += pred(r) ? 1 : 0;
        c1 += pred(r + 1) ? 1 : 0;
      }
    }
  }
  return wave_sum_dpp(c0 + c1);
}

// Sorts the wavefront's 64 * NE values ascending (lane-major: element
// lane * NE + r in x[r]) with a bitonic network: exchanges inside a lane for
// strides below NE, across lanes by shuffles above.
template <int NE>
__device__ __forceinline__ void wave_bitonic_sort(int32_t (&x)[NE], int lane) {
#pragma unroll
  for (int k = 2; k <= 64 * NE; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < NE) {
#pragma unroll
        for (int r = 0; r < NE; ++r) {
          if (r & j) continue;
          const bool asc = k < NE ? ((r & k) == 0) : (((lane * NE) & k) == 0);
          const int32_t a = x[r], b = x[r | j];
          const int32_t lo = a < b ? a : b, hi = a < b ? b : a;
          x[r] = asc ? lo : hi;
          x[r | j] = asc ? hi : lo;
        }
      } else {
        const int d = j / NE;
        const bool keep_min = ((lane & d) == 0) == (((lane * NE) & k) == 0);
#pragma unroll
        for (int r = 0; r < NE; ++r) {
          const int32_t y = __shfl_xor(x[r], d);
          x[r] = keep_min ? (x[r] < y ? x[r] : y) : (x[r] < y ? y : x[r]);
        }
      }
    }
  }
}

// the want winners in lds sorted ascending and written to out, and as union
// keys (token << 3 | head) to list (which may alias lds: every value is read
// before any is written) (NE a lane)
template <int NE>
__device__ __forceinline__ void sort_winners(const int* lds, int want, int lane, int32_t* out,
                                             uint32_t* list, int h) {
  int32_t x[NE];
#pragma unroll
  for (int r = 0; r < NE; ++r) {
    const int e = lane * NE + r;
    x[r] = e < want ? lds[e] : INT_MAX;
  }
  wave_bitonic_sort<NE>(x, lane);
#pragma unroll
  for (int r = 0; r < NE; ++r) {
    const int e = lane * NE + r;
    if (e < want) {
      out[e] = x[r];
      list[e] = ((uint32_t)x[r] << 3) | (uint32_t)h;
    }
  }
}

// One wavefront: the exact top-k of query head h of unit u from its
// candidates (at most CAND_CAP, CS_NPL a lane in registers), gathered through
// the prefix of the region part counts; the key K* of the (k - 4 - W)-th
// largest is found bit by bit from the top (the largest T with at least want
// keys >= T), the lowest token indices among keys equal to K* likewise when
// not all of them are taken; the winners are compacted in LDS, sorted by
// token index and written between the first 4 and the last W tokens.  The
// head's list also goes to list[0, k) as union keys (token << 3 | h; padding
// past n is ~0).  Returns true when the unit has to be redone unfused (its
// flag is then set and nothing is written).
__device__ __forceinline__ bool select_head(const CandArgs& a, int u, int h, int lane, int* lds,
                                            uint32_t* list) {
  const int G = a.g.G;
  const long long uh = (long long)u * G + h;
  const int k = a.k;
  const long long n = a.g.n[a.g.seq_of(u)];
  int32_t* out = a.idx + uh * k;
  if (n <= k) {
    for (int i = lane; i < k; i += 64) {
      out[i] = i < n ? i : -1;
      list[i] = i < n ? ((uint32_t)i << 3) | (uint32_t)h : 0xFFFFFFFFu;
    }
    return false;
  }
  const long long w = kept_tail(n);
  const long long hi = n - w;
  const int want = k - 4 - (int)w;
  auto flag = [&]() {
    if (lane == 0) a.cb.flag[u] = 1;
    return true;
  };
  if (want > 0) {
    const long long R = (n / BLK + a.cb.wg_blocks - 1) / a.cb.wg_blocks;
    const int nparts = (int)(R * CAND_PARTS);
    if (nparts > CAND_MAX_PARTS || nparts > 2 * a.lds_ints) return flag();
    // the part counts, then their prefix, as 16-bit values over the wave's
    // area (a unit is only taken when its total is at most CAND_CAP < 2^16)
    uint16_t* pre = reinterpret_cast<uint16_t*>(lds);
    // exclusive prefix of the part counts ([region][part], in order): lane l
    // takes parts [l * cpl, (l + 1) * cpl), loads them all, then writes
    // their prefix after a scan of the lane sums
    const int32_t* cnt = a.cb.count + uh * a.cb.regions * CAND_PARTS;
    const int ps = a.cb.part_slots;
    const int cpl = (nparts + 63) / 64;
    const int x0 = lane * cpl;
    int sum = 0;
    bool over = false;
#pragma unroll 8
    for (int i = 0; i < cpl; ++i) {
      const int x = x0 + i;
      if (x < nparts) {
        const int c = cnt[x];
        pre[x] = (uint16_t)c;
        sum += c;
        over |= c > ps || c < 0;  // (a part no scan wrote, for a unit it skipped)
      }
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int carry = __shfl(incl, 63);
    int run = incl - sum;
    for (int i = 0; i < cpl; ++i) {
      const int x = x0 + i;
      if (x < nparts) {
        const int c = pre[x];
        pre[x] = (uint16_t)run;
        run += c;
      }
    }
    const int total = carry;
    if (__ballot(over) != 0ull || total < want || total > CAND_CAP) return flag();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // candidate j = r * 64 + lane: its part is the last with prefix <= j
    // (prefix 0 of part 0 is <= every j), found by halving [0, nparts) the
    // same number of times for every row (the reads of a step issued
    // together; rows of a group wholly past total are skipped)
    int part[CS_NPL];
#pragma unroll
    for (int r = 0; r < CS_NPL; ++r) part[r] = 0;
    for (int m = nparts; m > 1;) {
      const int half = m >> 1;
#pragma unroll
      for (int g = 0; g < CS_NPL; g += CS_GROUP) {
        if (g * 64 < total) {
  #pragma unroll
          for (int r = g; r < g + CS_GROUP; ++r)
            part[r] = (int)pre[part[r] + half - 1] <= r * 64 + lane ? part[r] + half : part[r];
        }
      }
      m -= half;
    }
    // part[r] parts are known to start at or below j, and part[r] itself is
    // the one left to test: the last part with prefix <= j
#pragma unroll
    for (int g = 0; g < CS_NPL; g += CS_GROUP) {
      if (g * 64 < total) {
  #pragma unroll
        for (int r = g; r < g + CS_GROUP; ++r)
          part[r] = (int)pre[part[r]] <= r * 64 + lane ? part[r] : part[r] - 1;
      }
    }
    // (order key, token index); padding (past total) is (0, INT_MAX), and no
    // token index is INT_MAX
    const float* v = a.cb.val + uh * a.cb.regions * CAND_SLOTS;  // part x at x * ps
    const int32_t* ix = a.cb.idx + uh * a.cb.regions * CAND_SLOTS;
    uint32_t key[CS_NPL];
    int32_t id[CS_NPL];
#pragma unroll
    for (int r = 0; r < CS_NPL; ++r) {
      key[r] = 0u;
      id[r] = INT_MAX;
    }
    // every load issued before any is used (invalid lanes read slot 0), the
    // scores' bits straight into key
#pragma unroll
    for (int g = 0; g < CS_NPL; g += CS_GROUP) {
      if (g * 64 < total) {
  #pragma unroll
        for (int r = g; r < g + CS_GROUP; ++r) {
          const int j = r * 64 + lane;
          const long long e = j < total ? (long long)part[r] * ps + (j - pre[part[r]]) : 0;
          key[r] = __float_as_uint(v[e]);
          id[r] = ix[e];
        }
      }
    }
#pragma unroll
    for (int g = 0; g < CS_NPL; g += CS_GROUP) {
      if (g * 64 < total) {
  #pragma unroll
        for (int r = g; r < g + CS_GROUP; ++r) {
          const bool ok = r * 64 + lane < total;
          key[r] = ok ? order_key(__uint_as_float(key[r])) : 0u;
          id[r] = ok ? id[r] : INT_MAX;
        }
      }
    }
    // the scan's test may also pass tokens a little below the threshold: only
    // those at or above it count towards want
    const uint32_t tkey = a.cb.thresh[uh];
    const int ge =
        wave_count<CS_NPL>(total, [&](int r) { return id[r] != INT_MAX && key[r] >= tkey; });
    if (ge < want) return flag();
    // K*: the largest T with at least want keys >= T.  tkey <= K* <= the
    // largest key, so K* has their common top bits and the probes start below
    // them (padding keys are 0 and every probed T is at least 1).
    uint32_t mx = 0u;
#pragma unroll
    for (int r = 0; r < CS_NPL; ++r) mx = key[r] > mx ? key[r] : mx;
    mx = wave_max_dpp(mx);
    const uint32_t low = low_mask(tkey ^ mx);
    uint32_t T = tkey & ~low;
    // The free bits of K*, 8 a pass from the top (the last pass the rest):
    // keys with T's bits above the digit are counted by the digit's value in
    // 256 LDS bins over the spent part prefix, and the digit is the largest
    // D with (keys above) + (keys in bins >= D) >= want.  That count never
    // drops below want at D = 0 (it is then the count of keys >= T), and the
    // keys above stay fewer than want, so D exists and no empty bin is taken.
    // Padding keys are 0: they can only land in bin 0 of a pass whose upper
    // bits are all 0, and never decide D (a real key is at least 1, so is K*).
    int above = 0, eq = 0;  // keys above T, and equal to it, after the passes
    int* hist = lds;
    const int nfree = __popc(low);
    for (int nb = nfree; nb > 0;) {
      const int d = nb < 8 ? nb : 8;
      const int sh = nb - d;
      const uint32_t hm = sh + d >= 32 ? 0u : ~0u << (sh + d);
      const uint32_t tb = T & hm;
      const uint32_t dm = (1u << d) - 1u;
#pragma unroll
      for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
#pragma unroll
      for (int g = 0; g < CS_NPL; g += CS_GROUP) {
        if (g * 64 < total) {
  #pragma unroll
          for (int r = g; r < g + CS_GROUP; ++r)
            if ((key[r] & hm) == tb) atomicAdd(&hist[(key[r] >> sh) & dm], 1);
        }
      }
      // suffix sums over the bins, lane l holding bins 4l .. 4l + 3
      int hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[i] = hist[4 * lane + i];
      const int s3 = hb[3], s2 = s3 + hb[2], s1 = s2 + hb[1], s0 = s1 + hb[0];
      int v = s0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_down(v, off);
        if (lane + off < 64) v += y;
      }
      const int base_cnt = above + v - s0;  // keys above, and in higher lanes' bins
      int best = -1;
      if (base_cnt + s0 >= want) best = 4 * lane;
      if (base_cnt + s1 >= want) best = 4 * lane + 1;
      if (base_cnt + s2 >= want) best = 4 * lane + 2;
      if (base_cnt + s3 >= want) best = 4 * lane + 3;
      const int D = (int)wave_max_dpp((uint32_t)(best + 1)) - 1;
      int gt = 0, at = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gt += 4 * lane + i > D ? hb[i] : 0;
        at += 4 * lane + i == D ? hb[i] : 0;
      }
      above += wave_sum_dpp(gt);
      eq = wave_sum_dpp(at);
      T = tb | ((uint32_t)D << sh);
      nb -= d;
    }
    if (nfree == 0) {  // every candidate key at or above the threshold is tkey
      above = wave_count<CS_NPL>(total, [&](int r) { return key[r] > T; });
      eq = wave_count<CS_NPL>(total, [&](int r) { return key[r] == T; });
    }
    // the winners: the keys above K*, and the lowest-index keys equal to it
    // (rem >= 1 of them)
    const int rem = want - above;
    int32_t imax = INT_MAX;  // ties taken: index <= imax
    if (eq > rem) {
      // the rem-th lowest tie index: the largest I with fewer than rem tie
      // indices below it
      int32_t I = 0;
      for (int b = 30; b >= 0; --b) {
        const int32_t t = I | (1 << b);
        if (wave_count<CS_NPL>(total, [&](int r) { return key[r] == T && id[r] < t; }) < rem) I = t;
      }
      imax = I;
    }
    // compacted into LDS over the spent part prefix
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int base = 0;
#pragma unroll
    for (int g = 0; g < CS_NPL; g += CS_GROUP) {
      if (g * 64 < total) {
  #pragma unroll
        for (int r = g; r < g + CS_GROUP; ++r) {
          const bool w_ = key[r] > T || (key[r] == T && id[r] <= imax);
          const uint64_t m = __ballot(w_);
          const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (w_) lds[pos] = id[r];
          base += __popcll(m);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (want <= 64 * (CS_WPL / 2))
      sort_winners<CS_WPL / 2>(lds, want, lane, out + 4, list + 4, h);
    else
      sort_winners<CS_WPL>(lds, want, lane, out + 4, list + 4, h);
  }
  const int nk = want > 0 ? want : 0;
  if (lane < 4 && lane < k) {
    out[lane] = lane;
    list[lane] = ((uint32_t)lane << 3) | (uint32_t)h;
  }
  for (long long i = lane; 4 + nk + i < k; i += 64) {
    out[4 + nk + i] = (int32_t)(hi + i);
    list[4 + nk + i] = ((uint32_t)(hi + i) << 3) | (uint32_t)h;
  }
  return false;
}

// One workgroup per unit, wavefront h for query head h (select_head).  With
// fuse_union, once no head of the unit was flagged, the workgroup merges the
// G strictly ascending lists (position of an entry = its index in its list
// plus the entries below it in every other list), collapses runs of one token
// into a union row with a G-bit head mask and writes the rows, masks and
// row count as union_kernel does.
// (WPE: wavefronts per SIMD the registers allow; three caps them at 168,
// which costs each wavefront some speed but fits 50 % more workgroups)
template <int G, int WPE>
__global__ __launch_bounds__(G * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void cand_select_kernel(CandArgs a) {
  extern __shared__ int cs_lds[];
  const int tid = threadIdx.x, lane = tid & 63, h = tid >> 6;
  const int u = blockIdx.x;
  const int k = a.k;
  int* lds = cs_lds + h * a.lds_ints;
  auto list_of = [&](int b) { return reinterpret_cast<uint32_t*>(cs_lds + b * a.lds_ints); };
  const bool flagged = select_head(a, u, h, lane, lds, list_of(h));
  if (__syncthreads_or(flagged) || !a.fuse_union) return;

  constexpr int NT = G * 64;
  const int sel = G * k;
  const long long n = a.g.n[a.g.seq_of(u)];
  const int nv = n < k ? (int)n : k;  // valid entries of every list
  uint32_t* merged = reinterpret_cast<uint32_t*>(cs_lds + G * a.lds_ints);
  uint32_t* masks = merged + sel;  // one byte per union row
  int* wsum = reinterpret_cast<int*>(masks + (sel + 3) / 4);
  for (int e = tid; e < (sel + 3) / 4; e += NT) masks[e] = 0u;
  // wavefront h brings the entries of list h, lane l entries l + 64 j (at
  // most nv / 64 <= k / 64 a lane); a thread then owns at most as many
  // merged positions
  auto run = [&](auto EC) {
    constexpr int E = decltype(EC)::value;
    uint32_t x[E];
    bool ok[E];
    int p[E];  // entries below x[j] in its own list: its index
    const uint32_t* own = list_of(h);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = lane + 64 * j;
      ok[j] = i < nv;
      x[j] = own[i < nv ? i : 0];
      p[j] = i;
    }
    merge_by_rank<E>(list_of, [&](int) { return nv; }, G, x, ok, p, h, merged);
    write_union<E>(merged, G * nv, masks, wsum, a.un.uidx + (long long)u * sel,
                   a.un.umask + (long long)u * sel, a.un.ucount + u, tid, NT);
  };
  if (k <= 256) run(std::integral_constant<int, 4>{});
  else if (k <= 512) run(std::integral_constant<int, 8>{});
  else run(std::integral_constant<int, 16>{});
}

// number of units whose flag is set, into *count (one workgroup; every
// thread reaches the reduction)
__global__ __launch_bounds__(256) void count_flags_kernel(const int32_t* flag, int units,
                                                          int32_t* count) {
  __shared__ int part[4];
  int c = 0;
  for (int u = threadIdx.x; u < units; u += 256) c += flag[u] != 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) *count = part[0] + part[1] + part[2] + part[3];
}

}  // namespace

// the candidate part counts the selection reads (every workgroup of every
// unit and head) set to zero
__global__ __launch_bounds__(256) void zero_counts_kernel(int32_t* count, long long regions,
                                                          int parts, long long total) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256)
    count[(e / parts) * regions * CAND_PARTS + e % parts] = 0;
}

hipError_t launch_zero_counts(const Geom& g, const CandBufs& cb, hipStream_t st) {
  long long maxnb = 0;
  for (int s = 0; s < g.S; ++s) maxnb = g.n[s] / BLK > maxnb ? g.n[s] / BLK : maxnb;
  const int parts = (int)((maxnb + cb.wg_blocks - 1) / cb.wg_blocks) * CAND_PARTS;
  const long long total = (long long)g.units() * g.G * parts;
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 255) / 256 < 1024 ? (total + 255) / 256 : 1024;
  zero_counts_kernel<<<(unsigned)blocks, 256, 0, st>>>(cb.count, cb.regions, parts, total);
  return hipGetLastError();
}

hipError_t launch_count_flags(int units, const int32_t* flag, int32_t* count, hipStream_t st) {
  count_flags_kernel<<<1, 256, 0, st>>>(flag, units, count);
  return hipGetLastError();
}

hipError_t launch_topk(const Geom& g, const float* scores, int k, int32_t* idx, hipStream_t st) {
  TopkArgs a{g, scores, k, idx, nullptr};
  const long long blocks = (long long)g.units() * g.G;
  if (blocks == 0) return hipSuccess;
  topk_kernel<<<(unsigned)blocks, TK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk_flagged(const Geom& g, const float* scores, int k, int32_t* idx,
                               const int32_t* flag, const UnionBufs* un, hipStream_t st) {
  TopkArgs a{g, scores, k, idx, flag};
  if (g.units() == 0) return hipSuccess;
  topk_unit_kernel<<<(unsigned)g.units(), TK_THREADS, 0, st>>>(a, un ? *un : UnionBufs{});
  return hipGetLastError();
}

hipError_t launch_threshold(const Geom& g, int k, const CandBufs& cb, hipStream_t st) {
  ThreshArgs a{g, k, cb};
  const long long blocks = (long long)g.units() * g.G;
  if (blocks == 0) return hipSuccess;
  const long long len = sample_groups(g) * SAMPLE_GROUP * BLK;
  if (len <= 64 * 64)
    threshold_wave_kernel<64><<<(unsigned)((blocks + 3) / 4), 256, 0, st>>>(a);
  else if (len <= 64 * TH_THREADS)
    threshold_reg_kernel<64><<<(unsigned)blocks, TH_THREADS, 0, st>>>(a);
  else
    threshold_kernel<<<(unsigned)blocks, TK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_cand_select(const Geom& g, int k, const CandBufs& cb, int32_t* idx,
                              const UnionBufs* un, bool* fused, hipStream_t st) {
  if (fused) *fused = false;
  if (g.units() == 0) return hipSuccess;
  long long maxnb = 0;
  for (int s = 0; s < g.S; ++s) maxnb = g.n[s] / BLK > maxnb ? g.n[s] / BLK : maxnb;
  const long long parts = (maxnb + cb.wg_blocks - 1) / cb.wg_blocks * CAND_PARTS;
  // per head: the part prefix (16 bits a part) or the k <= FUSED_MAX_K
  // winners and list (32 bits an entry); at most 8 KiB a head
  int lds_ints = (int)((parts < CAND_MAX_PARTS ? parts : CAND_MAX_PARTS) + 1) / 2;
  lds_ints = lds_ints > FUSED_MAX_K ? lds_ints : FUSED_MAX_K;
  const size_t sel = (size_t)g.G * k;
  const size_t lists = (size_t)lds_ints * sizeof(int) * g.G;
  const size_t merge = sel * sizeof(uint32_t) + (sel + 3) / 4 * sizeof(uint32_t) + g.G * sizeof(int);
  CandArgs a{g, k, cb, idx, lds_ints, un ? *un : UnionBufs{}, 0};
  // the merge's LDS is only taken while the workgroup stays small
  a.fuse_union = un != nullptr && lists + merge <= CAND_FUSED_LDS;
  if (fused) *fused = a.fuse_union != 0;
  const size_t lds = lists + (a.fuse_union ? merge : 0);
  // units beyond what two wavefronts per SIMD hold at once (G of them per
  // workgroup, 4 SIMDs on each of 256 CUs) take the three-wavefront variant
  const bool many = (long long)g.units() * g.G > 2LL * 4 * 256;
  switch (g.G) {
    case 1:
      if (many) cand_select_kernel<1, 3><<<g.units(), 64, lds, st>>>(a);
      else cand_select_kernel<1, 2><<<g.units(), 64, lds, st>>>(a);
      break;
    case 2:
      if (many) cand_select_kernel<2, 3><<<g.units(), 128, lds, st>>>(a);
      else cand_select_kernel<2, 2><<<g.units(), 128, lds, st>>>(a);
      break;
    case 4:
      if (many) cand_select_kernel<4, 3><<<g.units(), 256, lds, st>>>(a);
      else cand_select_kernel<4, 2><<<g.units(), 256, lds, st>>>(a);
      break;
    case 8: cand_select_kernel<8, 2><<<g.units(), 512, lds, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bpk
