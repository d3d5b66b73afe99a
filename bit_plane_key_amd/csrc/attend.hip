// Exact attention over the selected rows, fetched once per KV head as the union
// of its query heads' winners (Fathom §1: at most G*k rows per KV head;
// Fathom §2: each head's output is softmax attention over its own set).
//
// 1. union_kernel (one workgroup per unit): the G sorted index lists are
//    merged with a bitonic sort of (token << 3 | head) keys in LDS, runs of
//    equal tokens collapse to one union row carrying a G-bit head mask.
// 2. attend_kernel (one workgroup per (split of ATT_ROWS union rows, unit)):
//    thread r loads union row r of K once and forms the logits of the heads in
//    its mask; per-head max and exp-sum over the split; then the split's V rows
//    are read once (a wavefront reads one 256-byte row per step, lane <-> two
//    channels) and accumulated for every head with its weights.  The split
//    writes (max, sum, unnormalised output) per head.
// 3. combine_kernel: log-sum-exp merge of the splits per (unit, head).
#include <limits.h>

#include "bpk_internal.h"

namespace bpk {
namespace {

constexpr int UNION_THREADS = 1024;
constexpr int ATT_ROWS = 256;
constexpr int ATT_THREADS = 256;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t uidx, umask, ucount, part, total;
  int nsplit;
};

WsLayout ws_layout(const Geom& g, int k) {
  WsLayout w;
  const size_t units = (size_t)g.units();
  const size_t sel = (size_t)g.G * k;
  w.nsplit = (int)((sel + ATT_ROWS - 1) / ATT_ROWS);
  size_t off = 0;
  w.uidx = off;   off += align256(units * sel * sizeof(int32_t));
  w.umask = off;  off += align256(units * sel);
  w.ucount = off; off += align256(units * sizeof(int32_t));
  w.part = off;   off += align256(units * (size_t)w.nsplit * g.G * (D + 2) * sizeof(float));
  w.total = off;
  return w;
}

struct UnionArgs {
  Geom g;
  const int32_t* idx;
  int k;
  int32_t* uidx;
  uint8_t* umask;
  int32_t* ucount;
};

__global__ __launch_bounds__(UNION_THREADS) void union_kernel(UnionArgs a) {
  __shared__ uint32_t keys[BPK_MAX_SELECTED];
  __shared__ int scan[UNION_THREADS];
  __shared__ uint32_t masks[BPK_MAX_SELECTED / 4];  // one byte per union row
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  const int G = a.g.G;
  const int sel = G * a.k;
  int m = 1;
  while (m < sel) m <<= 1;
  const int32_t* src = a.idx + (long long)u * sel;
  const long long n = a.g.n[a.g.seq_of(u)];
  for (int e = tid; e < m; e += UNION_THREADS) {
    uint32_t key = 0xFFFFFFFFu;
    if (e < sel) {
      const int32_t t = src[e];
      // entries outside [0, n) are padding (never a row read out of range)
      if (t >= 0 && t < n) key = ((uint32_t)t << 3) | (uint32_t)(e / a.k);
    }
    keys[e] = key;
  }
  for (int e = tid; e < BPK_MAX_SELECTED / 4; e += UNION_THREADS) masks[e] = 0;
  __syncthreads();
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
  // thread t owns a contiguous run of `per` sorted positions
  const int per = (m + UNION_THREADS - 1) / UNION_THREADS;
  const int e0 = tid * per;
  int own = 0;
  for (int e = e0; e < e0 + per && e < m; ++e) {
    const uint32_t key = keys[e];
    if (key != 0xFFFFFFFFu && (e == 0 || (keys[e - 1] >> 3) != (key >> 3))) ++own;
  }
  scan[tid] = own;
  __syncthreads();
  for (int off = 1; off < UNION_THREADS; off <<= 1) {
    const int x = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += x;
    __syncthreads();
  }
  int pos = scan[tid] - own - 1;  // union position of the current run
  for (int e = e0; e < e0 + per && e < m; ++e) {
    const uint32_t key = keys[e];
    if (key == 0xFFFFFFFFu) break;
    if (e == 0 || (keys[e - 1] >> 3) != (key >> 3)) {
      ++pos;
      a.uidx[(long long)u * sel + pos] = (int32_t)(key >> 3);
    }
    atomicOr(&masks[pos >> 2], (1u << (key & 7u)) << (8 * (pos & 3)));
  }
  __syncthreads();
  const int total = scan[UNION_THREADS - 1];
  for (int e = tid; e < total; e += UNION_THREADS)
    a.umask[(long long)u * sel + e] = (uint8_t)(masks[e >> 2] >> (8 * (e & 3)));
  if (tid == 0) a.ucount[u] = total;
}

struct AttArgs {
  Geom g;
  const void* k_rows;
  const uint16_t* v_rows;
  const uint16_t* q;
  int k;
  float scale;
  const int32_t* uidx;
  const uint8_t* umask;
  const int32_t* ucount;
  float* part;
  int nsplit;
};

template <int G, bool F32>
__global__ __launch_bounds__(ATT_THREADS) void attend_kernel(AttArgs a) {
  __shared__ float sq[G][D];
  __shared__ float p[G][ATT_ROWS];
  __shared__ int32_t rows[ATT_ROWS];
  __shared__ float red[ATT_THREADS / 64][G];
  __shared__ float oacc[4][G][D];
  const int tid = threadIdx.x;
  const int split = blockIdx.x, u = blockIdx.y;
  const long long gu = a.g.global_unit(u);
  const long long sel = (long long)G * a.k;
  const int count = a.ucount[u];
  const int r0 = split * ATT_ROWS;
  const int nr = count - r0 < ATT_ROWS ? (count - r0 > 0 ? count - r0 : 0) : ATT_ROWS;
  float* part = a.part + (((long long)u * a.nsplit + split) * G) * (D + 2);

  for (int e = tid; e < G * D; e += ATT_THREADS) sq[e / D][e % D] = bf16_to_f32(a.q[(long long)u * G * D + e]);
  // logits of union row tid for the heads in its mask
  int mask = 0;
  long long row = 0;
  if (tid < nr) {
    row = a.uidx[(long long)u * sel + r0 + tid];
    mask = a.umask[(long long)u * sel + r0 + tid];
  }
  rows[tid] = (int32_t)row;
  __syncthreads();
  float lg[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lg[h] = 0.f;
  if (mask) {
    const long long base = (gu * a.g.cap + row) * D;
    if constexpr (F32) {
      const float4* kr = reinterpret_cast<const float4*>(static_cast<const float*>(a.k_rows) + base);
      for (int c = 0; c < D / 4; ++c) {
        const float4 v = kr[c];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          lg[h] = fmaf(sq[h][4 * c], v.x, lg[h]);
          lg[h] = fmaf(sq[h][4 * c + 1], v.y, lg[h]);
          lg[h] = fmaf(sq[h][4 * c + 2], v.z, lg[h]);
          lg[h] = fmaf(sq[h][4 * c + 3], v.w, lg[h]);
        }
      }
    } else {
      const uint4* kr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_rows) + base);
      for (int c = 0; c < D / 8; ++c) {
        const uint4 v = kr[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(w[e] << 16);
          const float hi = __uint_as_float(w[e] & 0xFFFF0000u);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            lg[h] = fmaf(sq[h][8 * c + 2 * e], lo, lg[h]);
            lg[h] = fmaf(sq[h][8 * c + 2 * e + 1], hi, lg[h]);
          }
        }
      }
    }
  }
  // per-head max over the split
  const int wave = tid >> 6, lane = tid & 63;
  float mx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = ((mask >> h) & 1) ? lg[h] * a.scale : -INFINITY;
    lg[h] = v;
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane == 0) red[wave][h] = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = red[0][h];
    for (int w = 1; w < ATT_THREADS / 64; ++w) v = fmaxf(v, red[w][h]);
    mx[h] = v;
  }
  __syncthreads();
  float sum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float e = (lg[h] == -INFINITY) ? 0.f : expf(lg[h] - mx[h]);
    p[h][tid] = e;
    float v = e;
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[wave][h] = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = 0.f;
    for (int w = 0; w < ATT_THREADS / 64; ++w) v += red[w][h];
    sum[h] = v;
  }
  // V: wavefront `wave` takes rows wave, wave + 4, ...; lane owns channels 2*lane, 2*lane+1
  float o[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) o[h][0] = o[h][1] = 0.f;
  for (int r = wave; r < nr; r += ATT_THREADS / 64) {
    const uint32_t v2 =
        reinterpret_cast<const uint32_t*>(a.v_rows + (gu * a.g.cap + rows[r]) * D)[lane];
    const float v0 = __uint_as_float(v2 << 16), v1 = __uint_as_float(v2 & 0xFFFF0000u);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w = p[h][r];
      o[h][0] = fmaf(w, v0, o[h][0]);
      o[h][1] = fmaf(w, v1, o[h][1]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    oacc[wave][h][2 * lane] = o[h][0];
    oacc[wave][h][2 * lane + 1] = o[h][1];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += ATT_THREADS) {
    const int h = e / D, d = e % D;
    float v = 0.f;
    for (int w = 0; w < ATT_THREADS / 64; ++w) v += oacc[w][h][d];
    part[h * (D + 2) + 2 + d] = v;
  }
  if (tid < G) {
    part[tid * (D + 2)] = mx[tid];
    part[tid * (D + 2) + 1] = sum[tid];
  }
}

template <int G>
__global__ __launch_bounds__(G * D) void combine_kernel(const Geom g, const float* part, int nsplit,
                                                       float* out) {
  const int u = blockIdx.x;
  const int h = threadIdx.x / D, d = threadIdx.x % D;
  const float* pp = part + ((long long)u * nsplit * G + h) * (D + 2);
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, pp[(long long)s * G * (D + 2)]);
  float l = 0.f, o = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float* q = pp + (long long)s * G * (D + 2);
      if (q[0] == -INFINITY) continue;
      const float f = expf(q[0] - m);
      l = fmaf(q[1], f, l);
      o = fmaf(q[2 + d], f, o);
    }
  }
  out[((long long)u * G + h) * D + d] = l > 0.f ? o / l : 0.f;
}

template <int G>
void launch_att_g(const AttArgs& a, int k_dtype, float* out, hipStream_t st) {
  dim3 grid((unsigned)a.nsplit, (unsigned)a.g.units());
  if (k_dtype == BPK_F32)
    attend_kernel<G, true><<<grid, ATT_THREADS, 0, st>>>(a);
  else
    attend_kernel<G, false><<<grid, ATT_THREADS, 0, st>>>(a);
  combine_kernel<G><<<a.g.units(), G * D, 0, st>>>(a.g, a.part, a.nsplit, out);
}

}  // namespace

size_t attend_ws_bytes(const Geom& g, int k) { return ws_layout(g, k).total; }

hipError_t launch_attend(const Geom& g, int k_dtype, const void* k_rows, const uint16_t* v_rows,
                         const uint16_t* q, const int32_t* idx, int k, float scale, float* out,
                         void* ws, hipStream_t st) {
  if (g.units() == 0) return hipSuccess;
  const WsLayout w = ws_layout(g, k);
  char* base = static_cast<char*>(ws);
  int32_t* uidx = reinterpret_cast<int32_t*>(base + w.uidx);
  uint8_t* umask = reinterpret_cast<uint8_t*>(base + w.umask);
  int32_t* ucount = reinterpret_cast<int32_t*>(base + w.ucount);
  float* part = reinterpret_cast<float*>(base + w.part);
  UnionArgs ua{g, idx, k, uidx, umask, ucount};
  union_kernel<<<g.units(), UNION_THREADS, 0, st>>>(ua);
  AttArgs aa{g, k_rows, v_rows, q, k, scale, uidx, umask, ucount, part, w.nsplit};
  switch (g.G) {
    case 1: launch_att_g<1>(aa, k_dtype, out, st); break;
    case 2: launch_att_g<2>(aa, k_dtype, out, st); break;
    case 4: launch_att_g<4>(aa, k_dtype, out, st); break;
    case 8: launch_att_g<8>(aa, k_dtype, out, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bpk
