// Value-side depths (ReadKV §5.3, §5.4): value rows stored as per-token bit
// planes and read, once the attention probabilities are known, at a depth
// each token gets from them.
//
// vencode_kernel: 16 lanes per value row (8 channels each, one 16-byte load),
//   the row maximum by a DPP reduction inside the 16 lanes, then lane c writes
//   byte c (its 8 channels) of each of the row's four planes.
// Attention with value depths (launch_attend_v):
// 1. the union of the heads' rows, and per split of 256 union rows the
//    softmax terms e_hr = exp(l_hr - m_sh) and the split's (m_sh, sum e)
//    (attend.hip, launch_union_logits), with each union row's value scale;
// 2. vdepth_att_kernel, one workgroup per unit: the splits' statistics merged
//    into one factor per (split, head), so that p_hr = e_hr f_sh; importances
//    a_r = sum_h p_hr^2, gains w_r = a_r s_r^2, and the depth search (the
//    budget-th largest plane value w_r 4^-t by a radix select over the fp32
//    bit patterns, 8 bits a pass, then the planes equal to it handed out in
//    (row, plane) order);
// 3. vaccum_kernel, one workgroup per (split, unit): the rows' first t planes
//    read, the values rebuilt and accumulated with every head's probability;
// 4. vsum_kernel: the splits' partial outputs added in split order.
// vdepth_kernel runs the same depth search on given importances.
#include <float.h>

#include "bpk_internal.h"
#include "scan_common.h"

namespace bpk {
namespace {

constexpr int VENC_ROWS = 16;         // value rows per encode workgroup (4 per wavefront)
constexpr int VD_THREADS = 256;       // depth search from given importances: one workgroup per unit
constexpr int VD_PER = BPK_MAX_SELECTED / VD_THREADS;  // rows a thread owns at most (32)
constexpr int VD_SPLITS = BPK_MAX_SELECTED / ATT_SPLIT_ROWS;  // attention splits at most (32)
constexpr int VF_THREADS = 1024;      // the attention's depth search: one workgroup per unit
static_assert(BPK_MAX_SELECTED <= 8 * VF_THREADS, "at most 8 union rows a thread");
constexpr int VA_THREADS = 256;       // accumulation: one workgroup per split of union rows
constexpr int VREC = NP * D / 8;      // bytes of a token's four value planes (64)

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- encoding ----

struct VEncArgs {
  int L, H;
  long long cap;
  int seq;
  long long n0, n_new;
  const uint16_t* v_rows;
  uint8_t* vplanes;
  uint16_t* vscales;
};

// maximum over the 16 lanes of a DPP row, in every lane of the row (fmaxf, so
// a NaN loses to a number as in the key encoder)
__device__ __forceinline__ float row16_fmax(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

__global__ __launch_bounds__(64 * VENC_ROWS / 4) void vencode_kernel(VEncArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, rs = lane >> 4, ch = lane & 15;
  const long long i = a.n0 + (long long)blockIdx.x * VENC_ROWS + (tid >> 6) * 4 + rs;
  const int lh = blockIdx.y;
  const int l = lh / a.H, h = lh % a.H;
  const long long gu = ((long long)a.seq * a.L + l) * a.H + h;
  if (i >= a.n0 + a.n_new) return;  // the 16 lanes of a row leave together
  const long long row = gu * a.cap + i;
  const uint4 raw = *reinterpret_cast<const uint4*>(a.v_rows + row * D + 8 * ch);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  m = row16_fmax(m);
  const _Float16 hs = scale_of_max(m);
  const float s = (float)hs;
  uint32_t b0 = 0, b1 = 0, b2 = 0, b3 = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t c = quant_code(v[e], s);
    b0 |= ((c >> 3) & 1u) << e;
    b1 |= ((c >> 2) & 1u) << e;
    b2 |= ((c >> 1) & 1u) << e;
    b3 |= (c & 1u) << e;
  }
  uint8_t* dst = a.vplanes + row * VREC + ch;
  dst[0] = (uint8_t)b0;
  dst[16] = (uint8_t)b1;
  dst[32] = (uint8_t)b2;
  dst[48] = (uint8_t)b3;
  if (ch == 0) a.vscales[row] = __builtin_bit_cast(uint16_t, hs);
}

// ---- depth search ----

// sum over a wavefront, in every lane (all 64 lanes active)
__device__ __forceinline__ int wave_isum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// LDS of the depth search of NT threads: per-wavefront partial sums, double
// buffered (one barrier per sum: a buffer is written again only two sums
// later, after a barrier every reader of it has passed), the prefix scratch,
// two digit histograms and the chosen digit
template <int NT>
struct SearchLds {
  int sums[2][NT / 64][3];
  int pre[NT / 64];
  int hist[2][256];
  int sel[3];
};

// exclusive prefix sum over the workgroup in thread order
template <int NT>
__device__ __forceinline__ int block_prefix(int v, int* pre) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) pre[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += pre[w];
  return before + incl - v;
}

// The depths of the rows a workgroup of NT threads owns (thread t: rows
// NT j + t, j < PER).  key(j, t) is the value of plane t of row j as an fp32
// bit pattern (w 4^-t; 0: no positive gain).  T, the budget-th largest
// value, is found by a radix select over the bit patterns (positive floats
// order like their bits; bit 31 is clear): bits 30-23, 22-15, 14-7 and 6-0 in
// turn, each pass counting the keys that agree with the bits found so far by
// their next digit into LDS bins, one wavefront's suffix scan over the bins
// picking the digit.  Every plane above T is granted, and of those equal to
// T the first ones in (row, plane) order until the budget is spent.  Every
// thread of the workgroup calls this (it holds barriers).
template <int NT, int PER, class KeyF>
__device__ __forceinline__ void depth_search(const KeyF& key, int budget, int (&dep)[PER],
                                             SearchLds<NT>& lds) {
  constexpr int NW = NT / 64;
  static_assert(NT >= 256, "one thread per bin");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int buf = 0;
  auto sum1 = [&](int x) {
    x = wave_isum(x);
    if (lane == 0) lds.sums[buf][wave][0] = x;
    __syncthreads();
    x = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) x += lds.sums[buf][w][0];
    buf ^= 1;
    return x;
  };

  int npos = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j)
#pragma unroll
    for (int t = 0; t < NP; ++t) npos += key(j, t) != 0u;
  if (tid < 256) lds.hist[0][tid] = 0;
  const int total = sum1(npos);  // its barrier also orders the zeroing
  // T = 0: every positive plane (the budget covers them all); ~0: none
  uint32_t T = 0;
  int need = 0, eq_all = 0;
  if (budget == 0) {
    T = 0xFFFFFFFFu;
  } else if (total > budget) {
    uint32_t P = 0, M = 0;  // the bits found so far, and which they are
    int rem = budget;       // rank of T among the keys that agree with P
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int sh = pass == 3 ? 0 : 23 - 8 * pass;
      const uint32_t dm = pass == 3 ? 0x7Fu : 0xFFu;
      int* h = lds.hist[pass & 1];
      if (tid < 256) lds.hist[(pass + 1) & 1][tid] = 0;  // read two barriers ago, used next pass
#pragma unroll
      for (int j = 0; j < PER; ++j)
#pragma unroll
        for (int t = 0; t < NP; ++t) {
          const uint32_t x = key(j, t);
          if (x != 0u && (x & M) == P) atomicAdd(&h[(x >> sh) & dm], 1);
        }
      __syncthreads();
      if (wave == 0) {
        // lane l holds bins 4 l .. 4 l + 3; counts above a lane's bins, then
        // the lane whose bins hold the rem-th largest picks the digit
        const int4 b4 = *reinterpret_cast<const int4*>(&h[4 * lane]);
        const int ls = b4.x + b4.y + b4.z + b4.w;
        int incl = ls;  // keys in the bins of lanes >= l
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_down(incl, off);
          if (lane + off < 64) incl += y;
        }
        int c = incl - ls;
        if (c < rem && rem <= incl) {
          int k, bk;
          if (c + b4.w >= rem) {
            k = 3;
            bk = b4.w;
          } else {
            c += b4.w;
            if (c + b4.z >= rem) {
              k = 2;
              bk = b4.z;
            } else {
              c += b4.z;
              if (c + b4.y >= rem) {
                k = 1;
                bk = b4.y;
              } else {
                c += b4.y;
                k = 0;
                bk = b4.x;
              }
            }
          }
          lds.sel[0] = 4 * lane + k;
          lds.sel[1] = rem - c;
          lds.sel[2] = bk;
        }
      }
      __syncthreads();
      P |= (uint32_t)lds.sel[0] << sh;
      M |= dm << sh;
      rem = lds.sel[1];
      eq_all = lds.sel[2];
    }
    T = P;
    need = rem;  // the keys above T are budget - rem
  }
  const bool partial = T != 0u && T != 0xFFFFFFFFu;
  // more planes equal to T than needed (an exact tie): rank them in (row,
  // plane) order, that is chunk j, then thread, then plane
  const bool ranked = partial && eq_all > need;
  int base = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    int d = 0;
    if (ranked) {
      int eq = 0;
#pragma unroll
      for (int t = 0; t < NP; ++t) eq += key(j, t) == T;
      int rank = base + block_prefix<NT>(eq, lds.pre);
      base += sum1(eq);
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        const uint32_t x = key(j, t);
        if (x > T) {
          ++d;
        } else if (x == T) {
          d += rank < need;
          ++rank;
        }
      }
    } else if (T != 0xFFFFFFFFu) {
#pragma unroll
      for (int t = 0; t < NP; ++t) d += key(j, t) > T || (partial && key(j, t) == T);
    }
    dep[j] = d;
  }
}

// plane values w 4^-t of PER rows as fp32 bit patterns, kept in registers
// for up to 8 rows a thread and recomputed beyond
template <int PER>
struct PlaneKeys {
  static constexpr bool KEEP = PER <= 8;
  const float* w;
  uint32_t kb[KEEP ? PER : 1][NP];
  __device__ __forceinline__ static uint32_t make(float wv, int t) {
    constexpr float quarter[NP] = {1.f, 0.25f, 0.0625f, 0.015625f};
    const float v = wv * quarter[t];
    return v > 0.f ? __float_as_uint(v) : 0u;
  }
  __device__ __forceinline__ explicit PlaneKeys(const float (&wr)[PER]) : w(wr) {
    if constexpr (KEEP)
#pragma unroll
      for (int j = 0; j < PER; ++j)
#pragma unroll
        for (int t = 0; t < NP; ++t) kb[j][t] = make(wr[j], t);
  }
  __device__ __forceinline__ uint32_t operator()(int j, int t) const {
    if constexpr (KEEP) return kb[j][t];
    else return make(w[j], t);
  }
};

struct VDepthArgs {
  Geom g;
  long long ld;             // rows stride per unit
  const int32_t* count;     // [units] rows of each unit
  const int32_t* rows;      // [units][ld] token of each row
  const float* weights;     // [units][ld] importance of each row
  const uint16_t* vscales;
  int budget;
  uint8_t* depth;           // [units][ld]
};

// Depths from given importances: one workgroup of VD_THREADS per unit; gains
// w_r = a_r s_r^2 of the rows' tokens, then the depth search.  No branch
// around the loads: a row index past the count reads row 0 and a token
// outside [0, n) reads token 0, both masked afterwards.
template <int PER>
__global__ __launch_bounds__(VD_THREADS) void vdepth_kernel(VDepthArgs a) {
  __shared__ SearchLds<VD_THREADS> lds;
  const int tid = threadIdx.x, u = blockIdx.x;
  const long long gu = a.g.global_unit(u);
  const long long n = a.g.n[a.g.seq_of(u)];
  const long long ubase = (long long)u * a.ld;
  int count = a.count[u];
  count = count < 0 ? 0 : (count > a.ld ? (int)a.ld : count);

  float w[PER];
  int tok[PER];
  float wgt[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = j * VD_THREADS + tid;
    const long long rr = ubase + (r < count ? r : 0);
    tok[j] = a.rows[rr];
    wgt[j] = a.weights[rr];
  }
  constexpr int JB = PER < 8 ? PER : 8;  // rows per batch of the scale loads
#pragma unroll
  for (int j0 = 0; j0 < PER; j0 += JB) {
    uint32_t sbits[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int t = tok[j0 + jj];
      sbits[jj] = a.vscales[gu * a.g.cap + (t >= 0 && t < n ? t : 0)];
    }
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int j = j0 + jj;
      const int r = j * VD_THREADS + tid;
      const float s = half_bits_to_f32((uint16_t)sbits[jj]);
      const int t = tok[j];
      const float wt = wgt[j];
      const bool ok = r < count && t >= 0 && t < n && wt > 0.f && wt <= FLT_MAX;
      w[j] = ok ? wt * (s * s) : 0.f;
    }
  }
  const PlaneKeys<PER> key(w);
  int dep[PER];
  depth_search<VD_THREADS, PER>(key, a.budget, dep, lds);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = j * VD_THREADS + tid;
    if (r < a.ld) a.depth[ubase + r] = r < count ? (uint8_t)dep[j] : (uint8_t)0;
  }
}

// ---- the attention's depths ----

struct VAttDepthArgs {
  Geom g;
  long long ld;             // G * k: row stride per unit
  const int32_t* ucount;    // [units] union rows
  const int32_t* uidx;      // [units][ld] token of each union row
  const float* e;           // [units][G][ld] exp(l - split max)
  const float* stats;       // [units][nsplit][G][2] split max, exp-sum
  int nsplit;
  const float* vsc;         // [units][ld] value scale of each union row
  int budget;
  float* fac;               // [units][nsplit][G] exp(m_sh - M_h) / L_h, written
  uint8_t* depth;           // [units][ld], written
  uint8_t* depth_out;       // optional copy of depth
  int32_t* rows_out;        // optional copy of the union rows (-1 past the count)
};

// One workgroup of VF_THREADS per unit; thread t owns union rows
// VF_THREADS j + t.  The splits' softmax statistics merged into
// f_sh = exp(m_sh - M_h) / L_h (head h's max M_h and exp-sum L_h taken over
// the splits in order), so that p_hr = e_hr f_sh; importances
// a_r = sum_h p_hr^2, gains w_r = a_r s_r^2, and the depth search.
template <int G, int PER>
__global__ __launch_bounds__(VF_THREADS) void vdepth_att_kernel(VAttDepthArgs a) {
  constexpr int NT = VF_THREADS;
  __shared__ float smx[VD_SPLITS][G], ssm[VD_SPLITS][G], fs[VD_SPLITS][G];
  __shared__ float hM[G], hL[G];
  __shared__ SearchLds<NT> lds;
  const int tid = threadIdx.x, u = blockIdx.x;
  const long long ubase = (long long)u * a.ld;
  int count = a.ucount[u];
  count = count < 0 ? 0 : (count > a.ld ? (int)a.ld : count);

  // every load of the owned rows and of the splits' statistics first, none
  // waiting for the count (a row past the stride reads row 0; what lies past
  // the count is masked afterwards, and splits past the count are never used)
  float sc[PER];
  float ev[PER][G];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = j * NT + tid;
    const int rl = r < a.ld ? r : 0;
    sc[j] = a.vsc[ubase + rl];
#pragma unroll
    for (int h = 0; h < G; ++h) ev[j][h] = a.e[((long long)u * G + h) * a.ld + rl];
  }
  if (tid < a.nsplit * G) {
    const float* sp = a.stats + ((long long)u * a.nsplit * G + tid) * 2;
    smx[tid / G][tid % G] = sp[0];
    ssm[tid / G][tid % G] = sp[1];
  }
  const int ns = (count + ATT_SPLIT_ROWS - 1) / ATT_SPLIT_ROWS;
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY, L = 0.f;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, smx[sp][tid]);
    for (int sp = 0; sp < ns; ++sp) {
      const float m = smx[sp][tid];
      if (m != -INFINITY) L = fmaf(ssm[sp][tid], expf(m - M), L);
    }
    hM[tid] = M;
    hL[tid] = L;
  }
  __syncthreads();
  if (tid < ns * G) {
    const int sp = tid / G, h = tid % G;
    const float m = smx[sp][h], L = hL[h];
    const float f = (m == -INFINITY || !(L > 0.f)) ? 0.f : expf(m - hM[h]) / L;
    fs[sp][h] = f;
    a.fac[((long long)u * a.nsplit + sp) * G + h] = f;
  }
  __syncthreads();

  float w[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = j * NT + tid;
    const int rc = r < count ? r : 0;
    float acc = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = ev[j][h] * fs[rc / ATT_SPLIT_ROWS][h];
      acc = fmaf(p, p, acc);
    }
    w[j] = r < count ? acc * (sc[j] * sc[j]) : 0.f;
  }
  int dep[PER];
  {
    const PlaneKeys<PER> key(w);
    depth_search<NT, PER>(key, a.budget, dep, lds);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = j * NT + tid;
    if (r < a.ld) {
      const uint8_t dv = r < count ? (uint8_t)dep[j] : (uint8_t)0;
      a.depth[ubase + r] = dv;
      if (a.depth_out) a.depth_out[ubase + r] = dv;
      if (a.rows_out) a.rows_out[ubase + r] = r < count ? a.uidx[ubase + r] : -1;
    }
  }
}

// ---- accumulation ----

struct VAccArgs {
  Geom g;
  long long ld;  // G * k
  const int32_t* uidx;
  const int32_t* ucount;
  const float* e;        // [units][G][ld] exp(l - split max)
  const float* fac;      // [units][nsplit][G]
  const float* scale;    // [units][ld] value scale of each row
  const uint8_t* depth;  // [units][ld]
  const uint8_t* vplanes;
  float* part;           // [units][nsplit][G][D]
  int nsplit;
};

// One workgroup per (split of ATT_SPLIT_ROWS union rows, unit), the row
// mapping of the exact attention (16 lanes per row, 8 channels a lane): lane
// c loads dword c of the row's planes when its plane is read (all of a
// wavefront's loads in flight), a lane permute hands lane c byte c of every
// plane, a table spreads each plane byte's 8 bits into 8 bytes, and the 8
// channels are rebuilt as s (2^(3-t) - 8 + 8 b0 + 4 b1 + 2 b2 + b3) and
// accumulated with each head's p_hr = e_hr f_sh.  The four row groups of a
// wavefront, then the wavefronts, are summed in a fixed order.
template <int G>
__global__ __launch_bounds__(VA_THREADS) void vaccum_kernel(VAccArgs a) {
  constexpr int NW = VA_THREADS / 64;
  constexpr int RPW = ATT_SPLIT_ROWS / NW;  // rows per wavefront (64)
  constexpr int IT = RPW / 4;               // 4 rows per wavefront step
  static_assert(VA_THREADS == ATT_SPLIT_ROWS, "one thread per row of the split");
  __shared__ int32_t rows[ATT_SPLIT_ROWS];
  __shared__ int deps[ATT_SPLIT_ROWS];
  __shared__ float scl[ATT_SPLIT_ROWS];
  __shared__ float pr[ATT_SPLIT_ROWS][G];
  __shared__ uint2 spread[256];  // bit e of a byte -> byte e % 4 of word e / 4
  __shared__ float oacc[NW][G][D];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, rs = lane >> 4, ch = lane & 15;
  const int split = blockIdx.x, u = blockIdx.y;
  const long long gu = a.g.global_unit(u);
  const int count = a.ucount[u];
  const int r0 = split * ATT_SPLIT_ROWS;
  const int nr = count - r0 < ATT_SPLIT_ROWS ? (count - r0 > 0 ? count - r0 : 0) : ATT_SPLIT_ROWS;
  float* part = a.part + (((long long)u * a.nsplit + split) * G) * D;
  {
    const uint32_t b = (uint32_t)tid;  // 256 threads, one table entry each
    spread[tid] = make_uint2(((b & 15u) * 0x204081u) & 0x01010101u, ((b >> 4) * 0x204081u) & 0x01010101u);
    // the loads do not wait for the count: a row past the stride reads row
    // r0; rows past nr get depth 0 and weight 0 (an empty split writes zeros)
    const bool in = tid < nr;
    const int rl = r0 + tid < a.ld ? r0 + tid : r0;
    const long long rr = (long long)u * a.ld + rl;
    const int row = a.uidx[rr];
    const int dep = a.depth[rr];
    const float sc = a.scale[rr];
    const float* f = a.fac + ((long long)u * a.nsplit + split) * G;
    float ev[G], fv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      ev[h] = a.e[((long long)u * G + h) * a.ld + rl];
      fv[h] = f[h];
    }
    rows[tid] = in ? row : 0;
    deps[tid] = in ? dep : 0;
    scl[tid] = in ? sc : 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) pr[tid][h] = in ? ev[h] * fv[h] : 0.f;
  }
  __syncthreads();
  uint32_t dw[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = RPW * wave + 4 * it + rs;
    const int t = deps[r];
    dw[it] = 0u;
    if ((ch >> 2) < t)
      dw[it] = reinterpret_cast<const uint32_t*>(a.vplanes + (gu * a.g.cap + rows[r]) * VREC)[ch];
  }
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int x = 0; x < 8; ++x) o[h][x] = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = RPW * wave + 4 * it + rs;
    // byte c of plane p is byte c % 4 of dword 4 p + c / 4 of the row group;
    // the code of channel 8 c + x is byte x % 4 of word x / 4 of the sum of
    // the planes' spread bytes, plane p weighted 2^(3-p)
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t x = (uint32_t)__shfl((int)dw[it], (lane & ~15) + 4 * p + (ch >> 2));
      const uint2 sp = spread[(x >> (8 * (ch & 3))) & 0xFFu];
      lo |= sp.x << (NP - 1 - p);
      hi |= sp.y << (NP - 1 - p);
    }
    const float s = scl[r];
    const int t = deps[r];
    const float off = s * (t == 0 ? 0.f : ldexpf(1.f, 3 - t) - 8.f);  // s (2^(3-t) - 8), exact
    float vf[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      vf[x] = fmaf(s, (float)((lo >> (8 * x)) & 0xFFu), off);
      vf[4 + x] = fmaf(s, (float)((hi >> (8 * x)) & 0xFFu), off);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float wt = pr[r][h];  // 0 past nr
#pragma unroll
      for (int x = 0; x < 8; ++x) o[h][x] = fmaf(wt, vf[x], o[h][x]);
    }
  }
  // the four row groups of the wavefront
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      float v = o[h][x];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      o[h][x] = v;
    }
  if (rs == 0)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int x = 0; x < 8; ++x) oacc[wave][h][8 * ch + x] = o[h][x];
  __syncthreads();
  for (int e = tid; e < G * D; e += VA_THREADS) {
    const int h = e / D, d = e % D;
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) v += oacc[w2][h][d];
    part[h * D + d] = v;
  }
}

template <int G>
__global__ __launch_bounds__(G * D) void vsum_kernel(const float* part, int nsplit, float* out) {
  const int u = blockIdx.x, e = threadIdx.x;
  float v = 0.f;
  for (int s = 0; s < nsplit; ++s) v += part[((long long)u * nsplit + s) * G * D + e];
  out[(long long)u * G * D + e] = v;
}

struct VWs {
  size_t uidx, umask, ucount, e, stats, fac, scale, vdep, part, total;
  int nsplit;
};

VWs vws_layout(const Geom& g, int k) {
  VWs w;
  const size_t units = (size_t)g.units();
  const size_t sel = (size_t)g.G * k;
  w.nsplit = (int)((sel + ATT_SPLIT_ROWS - 1) / ATT_SPLIT_ROWS);
  size_t off = 0;
  w.uidx = off;   off += align256(units * sel * sizeof(int32_t));
  w.umask = off;  off += align256(units * sel);
  w.ucount = off; off += align256(units * sizeof(int32_t));
  w.e = off;      off += align256(units * g.G * sel * sizeof(float));
  w.stats = off;  off += align256(units * (size_t)w.nsplit * g.G * 2 * sizeof(float));
  w.fac = off;    off += align256(units * (size_t)w.nsplit * g.G * sizeof(float));
  w.scale = off;  off += align256(units * sel * sizeof(float));
  w.vdep = off;   off += align256(units * sel);
  w.part = off;   off += align256(units * (size_t)w.nsplit * g.G * D * sizeof(float));
  w.total = off;
  return w;
}

// rows per thread for a row stride of ld over nt threads
inline int rows_per(long long ld, int nt) {
  return ld <= nt ? 1 : ld <= 2 * nt ? 2 : ld <= 4 * nt ? 4 : ld <= 8 * nt ? 8 : ld <= 16 * nt ? 16 : 32;
}

void launch_vdepth(const VDepthArgs& da, hipStream_t st) {
  const int units = da.g.units();
  switch (rows_per(da.ld, VD_THREADS)) {
    case 1: case 2: vdepth_kernel<2><<<units, VD_THREADS, 0, st>>>(da); break;
    case 4: case 8: vdepth_kernel<8><<<units, VD_THREADS, 0, st>>>(da); break;
    default: vdepth_kernel<VD_PER><<<units, VD_THREADS, 0, st>>>(da); break;
  }
}

template <int G>
void launch_v_g(const VAttDepthArgs& da, const VAccArgs& va, float* out, hipStream_t st) {
  const int units = da.g.units();
  switch (rows_per(da.ld, VF_THREADS)) {
    case 1: vdepth_att_kernel<G, 1><<<units, VF_THREADS, 0, st>>>(da); break;
    case 2: vdepth_att_kernel<G, 2><<<units, VF_THREADS, 0, st>>>(da); break;
    case 4: vdepth_att_kernel<G, 4><<<units, VF_THREADS, 0, st>>>(da); break;
    default: vdepth_att_kernel<G, 8><<<units, VF_THREADS, 0, st>>>(da); break;
  }
  vaccum_kernel<G><<<dim3((unsigned)va.nsplit, (unsigned)units), VA_THREADS, 0, st>>>(va);
  vsum_kernel<G><<<units, G * D, 0, st>>>(va.part, va.nsplit, out);
}

}  // namespace

hipError_t launch_vencode(const Geom& g, int seq, const uint16_t* v_rows, uint8_t* vplanes,
                          uint16_t* vscales, long long n0, long long n_new, hipStream_t st) {
  if (n_new <= 0) return hipSuccess;
  VEncArgs a{g.L, g.H, g.cap, seq, n0, n_new, v_rows, vplanes, vscales};
  dim3 grid((unsigned)((n_new + VENC_ROWS - 1) / VENC_ROWS), (unsigned)(g.L * g.H));
  vencode_kernel<<<grid, 64 * VENC_ROWS / 4, 0, st>>>(a);
  return hipGetLastError();
}

size_t attend_v_ws_bytes(const Geom& g, int k) { return vws_layout(g, k).total; }

hipError_t launch_attend_v(const Geom& g, int k_dtype, const void* k_rows, const uint8_t* vplanes,
                           const uint16_t* vscales, const uint16_t* q, const int32_t* idx, int k,
                           float scale, int v_budget, float* out, int32_t* union_out,
                           uint8_t* vdepth_out, void* ws, bool union_ready, hipStream_t st) {
  if (g.units() == 0) return hipSuccess;
  const VWs w = vws_layout(g, k);
  char* base = static_cast<char*>(ws);
  int32_t* uidx = reinterpret_cast<int32_t*>(base + w.uidx);
  uint8_t* umask = reinterpret_cast<uint8_t*>(base + w.umask);
  int32_t* ucount = reinterpret_cast<int32_t*>(base + w.ucount);
  float* ev = reinterpret_cast<float*>(base + w.e);
  float* stats = reinterpret_cast<float*>(base + w.stats);
  float* fac = reinterpret_cast<float*>(base + w.fac);
  float* vsc = reinterpret_cast<float*>(base + w.scale);
  uint8_t* vdep = reinterpret_cast<uint8_t*>(base + w.vdep);
  float* part = reinterpret_cast<float*>(base + w.part);
  hipError_t e = launch_union_logits(g, k_dtype, k_rows, q, idx, k, scale, uidx, umask, ucount,
                                     ev, stats, vscales, vsc, union_ready, st);
  if (e != hipSuccess) return e;
  const long long sel = (long long)g.G * k;
  const VAttDepthArgs da{g,   sel,      ucount, uidx, ev,   stats,      w.nsplit,
                         vsc, v_budget, fac,    vdep, vdepth_out, union_out};
  const VAccArgs va{g, sel, uidx, ucount, ev, fac, vsc, vdep, vplanes, part, w.nsplit};
  switch (g.G) {
    case 1: launch_v_g<1>(da, va, out, st); break;
    case 2: launch_v_g<2>(da, va, out, st); break;
    case 4: launch_v_g<4>(da, va, out, st); break;
    case 8: launch_v_g<8>(da, va, out, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_value_depth(const Geom& g, const int32_t* rows, const int32_t* n_rows,
                              int row_ld, const float* weights, const uint16_t* vscales,
                              int v_budget, uint8_t* depth, hipStream_t st) {
  if (g.units() == 0) return hipSuccess;
  const VDepthArgs da{g, row_ld, n_rows, rows, weights, vscales, v_budget, depth};
  launch_vdepth(da, st);
  return hipGetLastError();
}

}  // namespace bpk
