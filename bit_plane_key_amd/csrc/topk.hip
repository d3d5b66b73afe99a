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
// decode_step's fused selection adds two kernels on the same machinery:
// * threshold_kernel: per (unit, head), the r-th largest of the sampled
//   scores of candidate tokens, with r chosen so that about 2 (k - 4 - W)
//   tokens of the whole range are expected at or above it (plus 8 for the
//   sampling noise of small r);
// * cand_select_kernel: per (unit, head), the exact top (k - 4 - W) of the
//   candidates (every token at or above the threshold, and possibly a few just
//   below it, so the k - 4 - W largest of the whole range are among them
//   whenever at least that many are at or above it), by a bitonic sort of
//   (score key, complemented index) pairs.  A head with too few candidates at
//   or above the threshold, or more than the buffer holds, flags its unit for
//   the full scan and radix select.
#include <limits.h>

#include "bpk_internal.h"

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

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
  __shared__ TkSmem sm;
  const int G = a.g.G;
  const int u = blockIdx.x / G, h = blockIdx.x % G;
  if (a.unit_flag && a.unit_flag[u] == 0) return;
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
      const float* sc = a.cb.sample + uh * a.cb.sample_ld;
      auto keyf = [&](long long i) { return order_key(sc[i]); };
      int t_eq, c_eq;
      tkey = radix_select(sm, 0, ngr * glen, (int)r, keyf, valid, &t_eq, &c_eq);
    }
  }
  if (tid == 0) {
    a.cb.thresh[uh] = tkey;
    if (h == 0) a.cb.flag[u] = 0;
  }
}

struct CandSmem {
  uint64_t key[CAND_CAP];
  int32_t buf[BPK_MAX_K];
  int total, over, fill, ge;
};

struct CandArgs {
  Geom g;
  int k;
  CandBufs cb;
  int32_t* idx;
};

__global__ __launch_bounds__(TK_THREADS) void cand_select_kernel(CandArgs a) {
  __shared__ CandSmem sm;
  const int G = a.g.G;
  const int u = blockIdx.x / G, h = blockIdx.x % G;
  const long long uh = (long long)u * G + h;
  const int tid = threadIdx.x;
  const int k = a.k;
  const long long n = a.g.n[a.g.seq_of(u)];
  int32_t* out = a.idx + uh * k;
  if (n <= k) {
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  const long long w = kept_tail(n);
  const long long hi = n - w;
  const int want = k - 4 - (int)w;
  int nk = 0;
  if (want > 0) {
    // the candidate regions of this unit's scan workgroups
    const long long R = (n / BLK + a.cb.wg_blocks - 1) / a.cb.wg_blocks;
    const int32_t* cnt = a.cb.count + uh * a.cb.regions * CAND_PARTS;  // [region][part]
    if (tid == 0) {
      sm.total = 0;
      sm.over = 0;
      sm.fill = 0;
      sm.ge = 0;
    }
    __syncthreads();
    int tot = 0, over = 0;
    const int ps = a.cb.part_slots;
    for (long long x = tid; x < R * CAND_PARTS; x += TK_THREADS) {
      const int c = cnt[x];
      tot += c;
      over |= c > ps;
    }
    if (tot) atomicAdd(&sm.total, tot);
    if (over) atomicOr(&sm.over, 1);
    __syncthreads();
    const int total = sm.total;
    if (sm.over || total < want || total > CAND_CAP) {
      if (tid == 0) a.cb.flag[u] = 1;
      return;
    }
    // (score key, complemented index) in descending order = score down, index
    // up; the scan's test may also pass tokens a little below the threshold,
    // so only those at or above it count towards want
    const uint32_t tkey = a.cb.thresh[uh];
    const float* v = a.cb.val + uh * a.cb.regions * CAND_SLOTS;  // part x at x * ps
    const int32_t* ix = a.cb.idx + uh * a.cb.regions * CAND_SLOTS;
    int ge = 0;
    for (long long x = tid; x < R * CAND_PARTS; x += TK_THREADS) {  // one region part a thread
      const int c = cnt[x];
      const int pos0 = c ? atomicAdd(&sm.fill, c) : 0;
      for (int i = 0; i < c; ++i) {
        const long long e = x * ps + i;
        const uint32_t key = order_key(v[e]);
        ge += key >= tkey;
        sm.key[pos0 + i] = ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)ix[e]);
      }
    }
    if (ge) atomicAdd(&sm.ge, ge);
    __syncthreads();
    if (sm.ge < want) {
      if (tid == 0) a.cb.flag[u] = 1;
      return;
    }
    int m = 1;
    while (m < total) m <<= 1;
    for (int i = total + tid; i < m; i += TK_THREADS) sm.key[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= m; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < m / 2; i += TK_THREADS) {
          const int lo_i = 2 * i - (i & (stride - 1));
          const int hi_i = lo_i + stride;
          const bool down = ((lo_i & size) == 0);
          const uint64_t x = sm.key[lo_i], y = sm.key[hi_i];
          if ((x < y) == down) {
            sm.key[lo_i] = y;
            sm.key[hi_i] = x;
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < want; i += TK_THREADS)
      sm.buf[i] = (int32_t)(~(uint32_t)(sm.key[i] & 0xFFFFFFFFull));
    nk = want;
  }
  for (int i = tid; i < 4; i += TK_THREADS) sm.buf[nk + i] = i;
  for (long long i = tid; i < w; i += TK_THREADS) sm.buf[nk + 4 + i] = (int32_t)(hi + i);
  __syncthreads();
  sort_and_write(sm.buf, k, out);
}

}  // namespace

hipError_t launch_topk(const Geom& g, const float* scores, int k, int32_t* idx, hipStream_t st) {
  TopkArgs a{g, scores, k, idx, nullptr};
  const long long blocks = (long long)g.units() * g.G;
  if (blocks == 0) return hipSuccess;
  topk_kernel<<<(unsigned)blocks, TK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk_flagged(const Geom& g, const float* scores, int k, int32_t* idx,
                               const int32_t* flag, hipStream_t st) {
  TopkArgs a{g, scores, k, idx, flag};
  const long long blocks = (long long)g.units() * g.G;
  if (blocks == 0) return hipSuccess;
  topk_kernel<<<(unsigned)blocks, TK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_threshold(const Geom& g, int k, const CandBufs& cb, hipStream_t st) {
  ThreshArgs a{g, k, cb};
  const long long blocks = (long long)g.units() * g.G;
  if (blocks == 0) return hipSuccess;
  threshold_kernel<<<(unsigned)blocks, TK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_cand_select(const Geom& g, int k, const CandBufs& cb, int32_t* idx,
                              hipStream_t st) {
  CandArgs a{g, k, cb, idx};
  const long long blocks = (long long)g.units() * g.G;
  if (blocks == 0) return hipSuccess;
  cand_select_kernel<<<(unsigned)blocks, TK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace bpk
