// The union of a unit's G selected lists (Fathom §1: the rows a KV head reads
// are the union of its query heads' winners), shared by the selection
// workgroup (topk.hip) and union_kernel (attend.hip).  Not part of the ABI.
#pragma once

#include "bpk_internal.h"

namespace bpk {

// Merge by rank of G strictly ascending lists of keys (token << 3 | list
// index, so no key repeats): list b holds len_of(b) <= L keys from
// list_of(b); merged[0, sum of the lengths) ascending.  The calling thread
// brings E entries x[j] (ok[j]: a real entry); an entry's position is the
// number of entries below it over all lists (in its own list, its index),
// each found by a lower-bound search in every list but `skip`, whose counts
// the caller has put in p (skip = -1: none).  The searches halve the range
// the same number of times for every entry (ceil(log2 len) steps, each read
// inside the list, the result selected), so the E reads of a step are issued
// together.  Every thread calls it; it ends with a barrier.
template <int E, typename ListFn, typename LenFn>
__device__ __forceinline__ void merge_by_rank(ListFn list_of, LenFn len_of, int G,
                                              const uint32_t (&x)[E], const bool (&ok)[E],
                                              int (&p)[E], int skip, uint32_t* merged) {
  for (int b = 0; b < G; ++b) {
    const uint32_t* l = list_of(b);
    const int len = len_of(b);
    if (len == 0 || b == skip) continue;
    int base[E];
#pragma unroll
    for (int j = 0; j < E; ++j) base[j] = 0;
    // the entries [0, base) are below x; the count is in [base, base + m]
    for (int m = len; m > 1;) {
      const int half = m >> 1;
#pragma unroll
      for (int j = 0; j < E; ++j) base[j] = l[base[j] + half - 1] < x[j] ? base[j] + half : base[j];
      m -= half;
    }
#pragma unroll
    for (int j = 0; j < E; ++j) p[j] += base[j] + (l[base[j]] < x[j] ? 1 : 0);
  }
#pragma unroll
  for (int j = 0; j < E; ++j)
    if (ok[j]) merged[p[j]] = x[j];
  __syncthreads();
}

// Runs of one token in the ascending keys merged[0, tot) collapse to union
// rows: uidx[r] = the row's token, umask[r] = the bits of the lists holding
// it, *ucount = the number of rows.  Thread tid of nt owns the positions
// [tid per, (tid + 1) per), per = ceil(tot / nt) <= P.  masks: LDS of at least
// ceil(tot / 4) words, zero on entry (and ordered before this call by a
// barrier); wsum: nt / 64 ints of LDS.  Every thread calls it.
template <int P>
__device__ __forceinline__ void write_union(const uint32_t* merged, int tot, uint32_t* masks,
                                            int* wsum, int32_t* uidx, uint8_t* umask,
                                            int32_t* ucount, int tid, int nt) {
  const int lane = tid & 63, wv = tid >> 6;
  if (tot == 0) {
    if (tid == 0) *ucount = 0;
    return;
  }
  const int per = (tot + nt - 1) / nt;
  const int e0 = tid * per;
  // v[j] = merged[e0 - 1 + j] (reads clamped into the keys); position e
  // starts a run when e == 0 or its token differs from that of e - 1
  uint32_t v[P + 1];
#pragma unroll
  for (int j = 0; j <= P; ++j) {
    const int e = e0 - 1 + j;
    v[j] = merged[e < 0 ? 0 : (e < tot ? e : tot - 1)];
  }
  auto starts = [&](int j) { return e0 - 1 + j == 0 || (v[j - 1] >> 3) != (v[j] >> 3); };
  int own = 0;
#pragma unroll
  for (int j = 1; j <= P; ++j)
    if (j <= per && e0 - 1 + j < tot && starts(j)) ++own;
  int incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int x = 0; x < nt / 64; ++x) {
    const int t = wsum[x];
    before += x < wv ? t : 0;
    total += t;
  }
  int pos = before + incl - own - 1;  // union position of the current run
#pragma unroll
  for (int j = 1; j <= P; ++j) {
    if (j <= per && e0 - 1 + j < tot) {
      const uint32_t key = v[j];
      if (starts(j)) {
        ++pos;
        uidx[pos] = (int32_t)(key >> 3);
      }
      atomicOr(&masks[pos >> 2], (1u << (key & 7u)) << (8 * (pos & 3)));
    }
  }
  __syncthreads();
  for (int e = tid; e < total; e += nt) umask[e] = (uint8_t)(masks[e >> 2] >> (8 * (e & 3)));
  if (tid == 0) *ucount = total;
}

constexpr int UNION_THREADS = 1024;

// The union of one unit's G lists of k indices src[0, G k) (entries outside
// [0, n) are padding), by the UNION_THREADS threads of a workgroup: lists
// that are strictly ascending with their padding at the end (as the top-k
// selections write them) are merged by rank, any other input is sorted whole
// (bitonic network); uidx / umask / *ucount as write_union.  Every thread
// calls it.
__device__ __forceinline__ void union_of_lists(const int32_t* src, int G, int k, long long n,
                                               int32_t* uidx, uint8_t* umask, int32_t* ucount) {
  static_assert(BPK_MAX_SELECTED <= 8 * UNION_THREADS, "eight entries a thread");
  __shared__ uint32_t keys[BPK_MAX_SELECTED];
  __shared__ uint32_t merged[BPK_MAX_SELECTED];
  __shared__ uint32_t masks[BPK_MAX_SELECTED / 4];  // one byte per union row
  __shared__ int lens[8];
  __shared__ int wsum[UNION_THREADS / 64];
  __shared__ int nval;
  const int tid = threadIdx.x;
  if (tid == 0) nval = 0;
  const int sel = G * k;
  int m = 1;
  while (m < sel) m <<= 1;
  int nvalid = 0;
  for (int e = tid; e < m; e += UNION_THREADS) {
    uint32_t key = 0xFFFFFFFFu;
    if (e < sel) {
      const int32_t t = src[e];
      // entries outside [0, n) are padding (never a row read out of range)
      if (t >= 0 && t < n) key = ((uint32_t)t << 3) | (uint32_t)(e / k);
    }
    keys[e] = key;
    nvalid += key != 0xFFFFFFFFu;
  }
  for (int e = tid; e < (sel + 3) / 4; e += UNION_THREADS) masks[e] = 0;
  __syncthreads();
  bool bad = false;
  for (int e = tid; e < sel; e += UNION_THREADS) {
    if ((e + 1) % k == 0) continue;
    const uint32_t x = keys[e], y = keys[e + 1];
    bad |= !(x < y || (x == 0xFFFFFFFFu && y == 0xFFFFFFFFu));
  }
  if (tid < G) {  // list tid's entries before its first padding one
    int lo = 0, hi = k;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (keys[tid * k + mid] != 0xFFFFFFFFu) lo = mid + 1;
      else hi = mid;
    }
    lens[tid] = lo;
  }
  atomicAdd(&nval, nvalid);
  const bool sorted = !__syncthreads_or(bad);
  const int tot = nval;  // valid entries over all lists
  if (sorted) {
    // thread tid brings the entries tid + j UNION_THREADS of the G lists
    uint32_t x[8];
    bool ok[8];
    int p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = tid + j * UNION_THREADS;
      const int b = e < sel ? e / k : 0;
      ok[j] = e < sel && e - b * k < lens[b];
      x[j] = keys[e < sel ? e : 0];
      p[j] = 0;
    }
    merge_by_rank<8>([&](int b) { return keys + b * k; }, [&](int b) { return lens[b]; }, G, x,
                     ok, p, -1, merged);
    write_union<8>(merged, tot, masks, wsum, uidx, umask, ucount, tid, UNION_THREADS);
    return;
  }
  for (int size = 2; size <= m; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < m / 2; i += UNION_THREADS) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const uint32_t x = keys[lo], y = keys[hi];
        if ((x > y) == up) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  write_union<8>(keys, tot, masks, wsum, uidx, umask, ucount, tid, UNION_THREADS);
}

}  // namespace bpk
