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
};

// monotone map float -> uint32 (larger float, larger key); -0 is mapped to +0
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
  __shared__ TkSmem sm;
  const int G = a.g.G;
  const int u = blockIdx.x / G, h = blockIdx.x % G;
  const long long n = a.g.n[a.g.seq_of(u)];
  const int k = a.k;
  const int tid = threadIdx.x;
  int32_t* out = a.idx + ((long long)u * G + h) * k;
  if (n <= k) {
    for (int i = tid; i < k; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  const long long w = (n % BLK) > 32 ? (n % BLK) : 32;
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
  // bitonic sort of buf[0..k) ascending (padding INT_MAX up to a power of two)
  int m = 1;
  while (m < k) m <<= 1;
  for (int i = k + tid; i < m; i += TK_THREADS) sm.buf[i] = INT_MAX;
  __syncthreads();
  for (int size = 2; size <= m; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < m / 2; i += TK_THREADS) {
        const int lo_i = 2 * i - (i & (stride - 1));
        const int hi_i = lo_i + stride;
        const bool up = ((lo_i & size) == 0);
        const int32_t x = sm.buf[lo_i], y = sm.buf[hi_i];
        if ((x > y) == up) {
          sm.buf[lo_i] = y;
          sm.buf[hi_i] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += TK_THREADS) out[i] = sm.buf[i];
}

}  // namespace

hipError_t launch_topk(const Geom& g, const float* scores, int k, int32_t* idx, hipStream_t st) {
  TopkArgs a{g, scores, k, idx};
  const long long blocks = (long long)g.units() * g.G;
  if (blocks == 0) return hipSuccess;
  topk_kernel<<<(unsigned)blocks, TK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace bpk
