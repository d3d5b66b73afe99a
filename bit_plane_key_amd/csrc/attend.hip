// Exact attention over the selected rows, fetched once per KV head as the union
// of its query heads' winners (Fathom §1: at most G*k rows per KV head;
// Fathom §2: each head's output is softmax attention over its own set).
//
// 1. union_kernel (one workgroup per unit, union_of_lists): the G index
//    lists, as (token << 3 | head) keys in LDS, are merged by rank when each
//    is strictly ascending (as select_topk writes them) and sorted with a
//    bitonic network otherwise; runs of equal tokens collapse to one union row
//    carrying a G-bit head mask.  decode_step's selection workgroups merge
//    their own unit's lists the same way, and launch_attend_rows starts here
//    at 2.
// 2. attend_kernel (one workgroup per (split of ATT_ROWS union rows, unit)):
//    every K row of the split is read once, whole and coalesced (16 lanes of a
//    wavefront per row, 16 bytes a lane, all of a wavefront's loads in flight
//    together), the logits of the heads in its mask reduced across the 16
//    lanes; per-head max and exp-sum over the split; then the V rows are read
//    the same way and accumulated for every head with its weights.  The split
//    writes (max, sum, unnormalised output) per head.
// 3. combine_kernel: log-sum-exp merge of the splits per (unit, head).
// launch_union_logits runs 1 and 2 up to the split's softmax statistics for
// the value-depth attention (values.hip), and fetches each union row's value
// scale along with its key row.
#include <limits.h>

#include "bpk_internal.h"
#include "union_common.h"

namespace bpk {
namespace {

constexpr int ATT_ROWS = ATT_SPLIT_ROWS;
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
  const int u = blockIdx.x;
  const long long sel = (long long)a.g.G * a.k;
  union_of_lists(a.idx + u * sel, a.g.G, a.k, a.g.n[a.g.seq_of(u)], a.uidx + u * sel,
                 a.umask + u * sel, a.ucount + u);
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
  float* out;  // [unit][G][D] (not LG)
  float* e;       // LG launches: [unit][G][G * k] exp(logit - split max), by union position
  float* stats;   // LG launches: [unit][nsplit][G][2] split max and exp-sum
  const uint16_t* vscales;  // LG launches: the cache's value scales
  float* vsc;               // LG launches: [unit][G * k] each union row's value scale
};

// sum over the 16 lanes of a DPP row (every lane of the row gets it; the
// butterfly and mirrors add the same pairs in every lane, so the result is
// the same in all 16)
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// One workgroup per (split of ATT_ROWS union rows, unit).  Rows are read whole
// and coalesced: in each wavefront, lane l takes 16-byte chunk l % 16 (8
// channels) of row 4 it + l / 16 of the wavefront's 64, for it = 0..15, with
// all 16 loads in flight before the arithmetic.  With LG the kernel stops
// after the split's softmax statistics and writes, for the value-depth
// attention, e_hr = exp(l_hr - m_h) of every row (0 where head h did not
// select it) and the split's (m_h, sum_r e_hr).
template <int G, bool F32, bool LG>
__global__ __launch_bounds__(ATT_THREADS) void attend_kernel(AttArgs a) {
  constexpr int RPW = ATT_ROWS / (ATT_THREADS / 64);  // rows per wavefront (64)
  constexpr int IT = RPW / 4;                          // 4 rows per wavefront load
  __shared__ int32_t rows[ATT_ROWS];
  __shared__ int masks[ATT_ROWS];
  __shared__ float p[ATT_ROWS][G];                     // logits, then weights
  __shared__ float red[ATT_THREADS / 64][G];
  __shared__ float oacc[LG ? 1 : ATT_THREADS / 16][G][D];  // per 16-lane row group (not LG)
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, rs = lane >> 4, ch = lane & 15;
  const int split = blockIdx.x, u = blockIdx.y;
  const long long gu = a.g.global_unit(u);
  const long long sel = (long long)G * a.k;
  const int count = a.ucount[u];
  const int r0 = split * ATT_ROWS;
  const int nr = count - r0 < ATT_ROWS ? (count - r0 > 0 ? count - r0 : 0) : ATT_ROWS;
  float* part = a.part + (((long long)u * a.nsplit + split) * G) * (D + 2);
  if (nr == 0) {  // an empty split contributes nothing
    if (!LG && tid < G) part[tid * (D + 2)] = -INFINITY;
    return;
  }
  {
    int row = 0, mask = 0;  // rows past nr: token 0 of the unit (read, weight 0)
    if (tid < nr) {
      row = a.uidx[(long long)u * sel + r0 + tid];
      mask = a.umask[(long long)u * sel + r0 + tid];
    }
    rows[tid] = row;
    masks[tid] = mask;
  }
  // the lane's 8 channels of each query head
  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 qv = *reinterpret_cast<const uint4*>(a.q + ((long long)u * G + h) * D + 8 * ch);
    const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[h][2 * e] = __uint_as_float(w[e] << 16);
      qf[h][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
  __syncthreads();

  // ---- logits ----
  auto krow = [&](int r) { return (gu * a.g.cap + rows[r]) * D + 8 * ch; };
  float kf[IT][8];
  if constexpr (F32) {
    float4 kv[IT][2];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.k_rows) +
                                                          krow(RPW * wave + 4 * it + rs));
      kv[it][0] = src[0];
      kv[it][1] = src[1];
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      kf[it][0] = kv[it][0].x; kf[it][1] = kv[it][0].y; kf[it][2] = kv[it][0].z; kf[it][3] = kv[it][0].w;
      kf[it][4] = kv[it][1].x; kf[it][5] = kv[it][1].y; kf[it][6] = kv[it][1].z; kf[it][7] = kv[it][1].w;
    }
  } else {
    uint4 kv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it)
      kv[it] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_rows) +
                                               krow(RPW * wave + 4 * it + rs));
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint32_t w[4] = {kv[it].x, kv[it].y, kv[it].z, kv[it].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[it][2 * e] = __uint_as_float(w[e] << 16);
        kf[it][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  }
  // LG: the row's value scale, its load issued after the key rows' (stored
  // once the logits are done)
  uint16_t vs_bits = 0;
  if (LG && tid < nr) vs_bits = a.vscales[gu * a.g.cap + rows[tid]];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = RPW * wave + 4 * it + rs;
    const int mask = masks[r];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qf[h][e], kf[it][e], d);
      d = row16_sum(d);
      if (ch == 0) p[r][h] = ((mask >> h) & 1) ? d * a.scale : -INFINITY;
    }
  }
  // the V rows (same mapping), in flight during the softmax reductions
  uint4 vv[LG ? 1 : IT];
  if constexpr (!LG) {
#pragma unroll
    for (int it = 0; it < IT; ++it)
      vv[it] = *reinterpret_cast<const uint4*>(
          a.v_rows + (gu * a.g.cap + rows[RPW * wave + 4 * it + rs]) * D + 8 * ch);
  }
  __syncthreads();

  // ---- per-head max and exp-sum over the split (thread tid <-> row tid) ----
  float mx[G], sum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = p[tid][h];
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
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lg = p[tid][h];
    const float e = (lg == -INFINITY) ? 0.f : expf(lg - mx[h]);
    p[tid][h] = e;
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
  if constexpr (LG) {
    if (tid < nr) {
#pragma unroll
      for (int h = 0; h < G; ++h) a.e[((long long)u * G + h) * sel + r0 + tid] = p[tid][h];
      a.vsc[(long long)u * sel + r0 + tid] = (float)__builtin_bit_cast(_Float16, vs_bits);
    }
    if (tid < G) {
      float* st = a.stats + (((long long)u * a.nsplit + split) * G + tid) * 2;
      st[0] = mx[tid];
      st[1] = sum[tid];
    }
    return;
  }

  // ---- V (loaded above): the same row mapping; lane accumulates its 8
  // channels per head ----
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = RPW * wave + 4 * it + rs;
    const uint32_t w[4] = {vv[it].x, vv[it].y, vv[it].z, vv[it].w};
    float vf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vf[2 * e] = __uint_as_float(w[e] << 16);
      vf[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float wt = p[r][h];  // 0 for rows past nr and heads without the row
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = fmaf(wt, vf[e], o[h][e]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[4 * wave + rs][h][8 * ch + e] = o[h][e];
  __syncthreads();
  for (int e = tid; e < G * D; e += ATT_THREADS) {
    const int h = e / D, d = e % D;
    float v = 0.f;
    for (int gidx = 0; gidx < ATT_THREADS / 16; ++gidx) v += oacc[gidx][h][d];
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
void launch_att_g(const AttArgs& a, int k_dtype, hipStream_t st) {
  dim3 grid((unsigned)a.nsplit, (unsigned)a.g.units());
  if (a.e) {
    if (k_dtype == BPK_F32)
      attend_kernel<G, true, true><<<grid, ATT_THREADS, 0, st>>>(a);
    else
      attend_kernel<G, false, true><<<grid, ATT_THREADS, 0, st>>>(a);
    return;
  }
  if (k_dtype == BPK_F32)
    attend_kernel<G, true, false><<<grid, ATT_THREADS, 0, st>>>(a);
  else
    attend_kernel<G, false, false><<<grid, ATT_THREADS, 0, st>>>(a);
  combine_kernel<G><<<a.g.units(), G * D, 0, st>>>(a.g, a.part, a.nsplit, a.out);
}

hipError_t launch_att(const AttArgs& aa, int k_dtype, hipStream_t st) {
  switch (aa.g.G) {
    case 1: launch_att_g<1>(aa, k_dtype, st); break;
    case 2: launch_att_g<2>(aa, k_dtype, st); break;
    case 4: launch_att_g<4>(aa, k_dtype, st); break;
    case 8: launch_att_g<8>(aa, k_dtype, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t attend_ws_bytes(const Geom& g, int k) { return ws_layout(g, k).total; }

UnionBufs union_bufs(const Geom& g, int k, void* ws) {
  const WsLayout w = ws_layout(g, k);
  char* base = static_cast<char*>(ws);
  return UnionBufs{reinterpret_cast<int32_t*>(base + w.uidx), reinterpret_cast<uint8_t*>(base + w.umask),
                   reinterpret_cast<int32_t*>(base + w.ucount)};
}

hipError_t launch_union(const Geom& g, const int32_t* idx, int k, const UnionBufs& ub,
                        hipStream_t st) {
  if (g.units() == 0) return hipSuccess;
  UnionArgs ua{g, idx, k, ub.uidx, ub.umask, ub.ucount};
  union_kernel<<<g.units(), UNION_THREADS, 0, st>>>(ua);
  return hipGetLastError();
}

hipError_t launch_attend_rows(const Geom& g, int k_dtype, const void* k_rows,
                              const uint16_t* v_rows, const uint16_t* q, int k, float scale,
                              float* out, void* ws, hipStream_t st) {
  if (g.units() == 0) return hipSuccess;
  const WsLayout w = ws_layout(g, k);
  const UnionBufs ub = union_bufs(g, k, ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + w.part);
  AttArgs aa{g,    k_rows,   v_rows, q,       k,       scale,   ub.uidx, ub.umask, ub.ucount,
             part, w.nsplit, out,    nullptr, nullptr, nullptr, nullptr};
  return launch_att(aa, k_dtype, st);
}

hipError_t launch_attend(const Geom& g, int k_dtype, const void* k_rows, const uint16_t* v_rows,
                         const uint16_t* q, const int32_t* idx, int k, float scale, float* out,
                         void* ws, hipStream_t st) {
  hipError_t e = launch_union(g, idx, k, union_bufs(g, k, ws), st);
  if (e != hipSuccess) return e;
  return launch_attend_rows(g, k_dtype, k_rows, v_rows, q, k, scale, out, ws, st);
}

hipError_t launch_union_logits(const Geom& g, int k_dtype, const void* k_rows, const uint16_t* q,
                               const int32_t* idx, int k, float scale, int32_t* uidx,
                               uint8_t* umask, int32_t* ucount, float* e, float* stats,
                               const uint16_t* vscales, float* vsc, bool union_ready,
                               hipStream_t st) {
  if (g.units() == 0) return hipSuccess;
  if (!union_ready) {
    UnionArgs ua{g, idx, k, uidx, umask, ucount};
    union_kernel<<<g.units(), UNION_THREADS, 0, st>>>(ua);
  }
  const int nsplit = (int)(((long long)g.G * k + ATT_ROWS - 1) / ATT_ROWS);
  AttArgs aa{g,       k_rows, nullptr, q, k,     scale,   uidx, umask, ucount,
             nullptr, nsplit, nullptr, e, stats, vscales, vsc};
  return launch_att(aa, k_dtype, st);
}

}  // namespace bpk
