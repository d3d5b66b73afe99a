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
//    (attend.hip, launch_union_logits);
// 2. vdepth_kernel, one workgroup per unit: the splits' softmax statistics
//    merged into one factor f_sh = exp(m_sh - M_h) / L_h per (split, head)
//    (the rows' value scales come from the key pass, which fetched them with
//    the key rows),
//    so that p_hr = e_hr f_sh; importances a_r = sum_h p_hr^2, gains
//    w_r = a_r s_r^2, and the depth search: the budget-th largest plane value
//    w_r 4^-t found two bits a pass over the fp32 bit patterns, then the
//    candidates equal to it handed out in (row, plane) order (a prefix count
//    over the threads, only when there are more of them than needed);
// 3. vaccum_kernel, one workgroup per (split of 256 union rows, unit), the
//    row mapping of the exact attention (16 lanes per row, 8 channels a lane):
//    the 16 lanes load the row's planes as 16 dwords (only the dwords of the
//    first t planes), a lane permute hands lane c byte c of every plane, and
//    the 8 channels are rebuilt as s (2^(3-t) - 8 + 8 b0 + 4 b1 + 2 b2 + b3)
//    and accumulated with each head's probability e_hr f_sh;
// 4. vsum_kernel: the splits' partial outputs added in split order.
#include <float.h>

#include "bpk_internal.h"
#include "scan_common.h"

namespace bpk {
namespace {

constexpr int VENC_ROWS = 16;         // value rows per encode workgroup (4 per wavefront)
constexpr int VD_THREADS = 256;       // depth search: one workgroup per unit
constexpr int VD_PER = BPK_MAX_SELECTED / VD_THREADS;  // rows a thread owns at most (32)
constexpr int VD_SPLITS = BPK_MAX_SELECTED / ATT_SPLIT_ROWS;  // attention splits at most (32)
constexpr int VA_ROWS = ATT_SPLIT_ROWS;  // union rows per accumulation workgroup (one split)
constexpr int VA_THREADS = 256;
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

struct VDepthArgs {
  Geom g;
  long long ld;             // rows stride per unit
  const int32_t* count;     // [units] rows of each unit
  const int32_t* rows;      // [units][ld] token of each row
  const float* e;           // attention: [units][G][ld] exp(l - split max)
  const float* stats;       // attention: [units][nsplit][G][2] split max, exp-sum
  float* fac;               // attention: [units][nsplit][G] exp(m_s - M) / L, written
  int nsplit;
  const float* weights;     // given importances: [units][ld]
  const uint16_t* vscales;
  int budget;
  const float* scale_in;    // attention: [units][ld] each row's value scale
  uint8_t* depth;           // [units][ld]
  uint8_t* depth_copy;      // optional second copy of depth
  int32_t* rows_copy;       // optional copy of rows, -1 past the count
};

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// sum over the workgroup (every thread gets it); red holds one int per wavefront
__device__ __forceinline__ int block_sum_i(int v, int* red) {
  v = wave_sum_i(v);
  __syncthreads();  // the previous use of red is over
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < VD_THREADS / 64; ++w) t += red[w];
  return t;
}

// three sums over the workgroup at once (every thread gets them)
__device__ __forceinline__ void block_sum3_i(int& x, int& y, int& z, int (*red)[3]) {
  x = wave_sum_i(x);
  y = wave_sum_i(y);
  z = wave_sum_i(z);
  __syncthreads();  // the previous use of red is over
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6][0] = x;
    red[threadIdx.x >> 6][1] = y;
    red[threadIdx.x >> 6][2] = z;
  }
  __syncthreads();
  x = y = z = 0;
#pragma unroll
  for (int w = 0; w < VD_THREADS / 64; ++w) {
    x += red[w][0];
    y += red[w][1];
    z += red[w][2];
  }
}

// exclusive prefix sum over the threads in thread order
__device__ __forceinline__ int block_prefix_i(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += red[w];
  return before + incl - v;
}

// One workgroup of VD_THREADS per unit; thread t owns rows r = VD_THREADS j + t
// (j < PER), so every load of a row array is coalesced.  GIVEN: importances from a.weights (G unused);
// otherwise p_hr = e_hr f_jh with f_jh = exp(m_jh - M_h) / L_h merged from
// the splits' statistics, and a_r = sum_h p_hr^2.
template <int G, int PER, bool GIVEN>
__global__ __launch_bounds__(VD_THREADS) void vdepth_kernel(VDepthArgs a) {
  __shared__ int redi[VD_THREADS / 64];
  __shared__ int red3[VD_THREADS / 64][3];
  __shared__ float fs[VD_SPLITS][G];
  __shared__ float smax[VD_SPLITS][G], ssum[VD_SPLITS][G];
  const int tid = threadIdx.x, u = blockIdx.x;
  const long long gu = a.g.global_unit(u);
  const long long n = a.g.n[a.g.seq_of(u)];
  const long long ubase = (long long)u * a.ld;
  int count = a.count[u];
  count = count < 0 ? 0 : (count > a.ld ? (int)a.ld : count);

  if constexpr (!GIVEN) {
    const int ns = (count + ATT_SPLIT_ROWS - 1) / ATT_SPLIT_ROWS;  // splits holding rows
    if (tid < ns * G) {
      const float* st = a.stats + ((long long)u * a.nsplit * G + tid) * 2;
      smax[tid / G][tid % G] = st[0];
      ssum[tid / G][tid % G] = st[1];
    }
    __syncthreads();
    float M[G], Ls[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      M[h] = -INFINITY;
      Ls[h] = 0.f;
    }
    for (int sp = 0; sp < ns; ++sp)
#pragma unroll
      for (int h = 0; h < G; ++h) M[h] = fmaxf(M[h], smax[sp][h]);
    for (int sp = 0; sp < ns; ++sp)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float m = smax[sp][h];
        if (m != -INFINITY) Ls[h] = fmaf(ssum[sp][h], expf(m - M[h]), Ls[h]);
      }
    if (tid < ns)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float m = smax[tid][h];
        const float f = (m == -INFINITY || !(Ls[h] > 0.f)) ? 0.f : expf(m - M[h]) / Ls[h];
        fs[tid][h] = f;
        a.fac[((long long)u * a.nsplit + tid) * G + h] = f;
      }
    __syncthreads();
  }

  // gains of the owned rows.  Given importances: the tokens and weights,
  // then the tokens' scales; in the attention, the softmax terms and the
  // scales the key pass fetched.  No branch around the loads: a row index
  // past the count reads row 0 and a token outside [0, n) reads token 0,
  // both masked afterwards.
  float w[PER];
  int tok[GIVEN ? PER : 1];
  float wgt[GIVEN ? PER : 1];
  if constexpr (GIVEN)
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int r = j * VD_THREADS + tid;
      const long long rr = ubase + (r < count ? r : 0);
      tok[j] = a.rows[rr];
      wgt[j] = a.weights[rr];
    }
  constexpr int JB = PER < 8 ? PER : (G > 4 ? 4 : 8);  // rows per batch of the second loads
#pragma unroll
  for (int j0 = 0; j0 < PER; j0 += JB) {
    uint32_t sbits[JB];
    float ev[GIVEN ? 1 : JB][G];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int j = j0 + jj;
      const int r = j * VD_THREADS + tid;
      if constexpr (GIVEN) {
        const int t = tok[j];
        const bool tok_ok = t >= 0 && t < n;
        sbits[jj] = a.vscales[gu * a.g.cap + (tok_ok ? t : 0)];
      } else {
        sbits[jj] = __float_as_uint(a.scale_in[ubase + (r < count ? r : 0)]);
      }
      if constexpr (!GIVEN)
#pragma unroll
        for (int h = 0; h < G; ++h)
          ev[jj][h] = a.e[((long long)u * G + h) * a.ld + (r < count ? r : 0)];
    }
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int j = j0 + jj;
      const int r = j * VD_THREADS + tid;
      const bool in = r < count;
      const float s = GIVEN ? half_bits_to_f32((uint16_t)sbits[jj]) : __uint_as_float(sbits[jj]);
      if constexpr (GIVEN) {
        const int t = tok[j];
        const float wt = wgt[j];
        const bool ok = in && t >= 0 && t < n && wt > 0.f && wt <= FLT_MAX;
        w[j] = ok ? wt * (s * s) : 0.f;
      } else {
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = ev[jj][h] * fs[r / ATT_SPLIT_ROWS][h];
          acc = fmaf(p, p, acc);
        }
        w[j] = in ? acc * (s * s) : 0.f;
      }
    }
  }

  // plane values w 4^-t as fp32 bit patterns (0: no positive gain)
  // (kept in registers for up to 8 rows a thread, recomputed beyond)
  constexpr float quarter[NP] = {1.f, 0.25f, 0.0625f, 0.015625f};
  constexpr bool KEEP = PER <= 8;
  uint32_t kb[KEEP ? PER : 1][NP];
  auto make = [&](int j, int t) {
    const float v = w[j] * quarter[t];
    return v > 0.f ? __float_as_uint(v) : 0u;
  };
  if constexpr (KEEP)
#pragma unroll
    for (int j = 0; j < PER; ++j)
#pragma unroll
      for (int t = 0; t < NP; ++t) kb[j][t] = make(j, t);
  auto key = [&](int j, int t) {
    if constexpr (KEEP) return kb[j][t];
    else return make(j, t);
  };
  int npos = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j)
#pragma unroll
    for (int t = 0; t < NP; ++t) npos += key(j, t) != 0u;
  const int total = block_sum_i(npos, redi);
  // every candidate above T is taken, and the first `need` equal to T in
  // (row, plane) order; T = 0 (every positive candidate) when the budget
  // covers them all, ~0 (nothing) for a zero budget
  uint32_t T = 0;
  int need = 0;
  if (a.budget == 0) {
    T = 0xFFFFFFFFu;
  } else if (total > a.budget) {
    // the largest T with at least `budget` candidates >= T, bit 30 first,
    // then two bits a pass (positive floats: bit 31 clear)
    {
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j)
#pragma unroll
        for (int t = 0; t < NP; ++t) cnt += key(j, t) >= (1u << 30);
      if (block_sum_i(cnt, redi) >= a.budget) T = 1u << 30;
    }
    for (int lo = 28; lo >= 0; lo -= 2) {
      const uint32_t t1 = T | (1u << lo), t2 = T | (2u << lo), t3 = T | (3u << lo);
      int c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j)
#pragma unroll
        for (int t = 0; t < NP; ++t) {
          const uint32_t x = key(j, t);
          c1 += x >= t1;
          c2 += x >= t2;
          c3 += x >= t3;
        }
      block_sum3_i(c1, c2, c3, red3);
      T = c3 >= a.budget ? t3 : c2 >= a.budget ? t2 : c1 >= a.budget ? t1 : T;
    }
    int above = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j)
#pragma unroll
      for (int t = 0; t < NP; ++t) above += key(j, t) > T;
    need = a.budget - block_sum_i(above, redi);
  }
  const bool partial = T != 0u && T != 0xFFFFFFFFu;
  int eq_all = 0;
  if (partial)
#pragma unroll
    for (int j = 0; j < PER; ++j)
#pragma unroll
      for (int t = 0; t < NP; ++t) eq_all += key(j, t) == T;
  // with more candidates equal to T than needed (an exact tie), rank them in
  // (row, plane) order: chunk j, then thread, then plane
  const bool ranked = partial && block_sum_i(eq_all, redi) > need;
  int base = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = j * VD_THREADS + tid;
    int d = 0;
    if (ranked) {
      int eq = 0;
#pragma unroll
      for (int t = 0; t < NP; ++t) eq += key(j, t) == T;
      int rank = base + block_prefix_i(eq, redi);
      base += block_sum_i(eq, redi);
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
    if (r < a.ld) {
      const uint8_t dv = r < count ? (uint8_t)d : (uint8_t)0;
      a.depth[ubase + r] = dv;
      if (a.depth_copy) a.depth_copy[ubase + r] = dv;
      if (a.rows_copy) a.rows_copy[ubase + r] = r < count ? a.rows[ubase + r] : -1;
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
  const uint16_t* vscales;
  float* part;           // [units][nsplit][G][D]
  int nsplit;
};

// bit e of an 8-bit value -> bit 4 e
__device__ __forceinline__ uint32_t spread4(uint32_t b) {
  b = (b | (b << 12)) & 0x000F000Fu;
  b = (b | (b << 6)) & 0x03030303u;
  b = (b | (b << 3)) & 0x11111111u;
  return b;
}

template <int G>
__global__ __launch_bounds__(VA_THREADS) void vaccum_kernel(VAccArgs a) {
  constexpr int RPW = VA_ROWS / (VA_THREADS / 64);  // rows per wavefront (64)
  constexpr int IT = RPW / 4;                        // 4 rows per wavefront step
  __shared__ int32_t rows[VA_ROWS];
  __shared__ int deps[VA_ROWS];
  __shared__ float scl[VA_ROWS];
  __shared__ float pr[VA_ROWS][G];
  __shared__ float oacc[VA_THREADS / 16][G][D];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, rs = lane >> 4, ch = lane & 15;
  const int split = blockIdx.x, u = blockIdx.y;
  const long long gu = a.g.global_unit(u);
  const int count = a.ucount[u];
  const int r0 = split * VA_ROWS;
  const int nr = count - r0 < VA_ROWS ? (count - r0 > 0 ? count - r0 : 0) : VA_ROWS;
  float* part = a.part + (((long long)u * a.nsplit + split) * G) * D;
  if (nr == 0) {
    for (int e = tid; e < G * D; e += VA_THREADS) part[e] = 0.f;
    return;
  }
  {
    // rows past nr: depth 0, weight 0 (their loads read row r0, masked)
    const bool in = tid < nr;
    const long long rr = (long long)u * a.ld + r0 + (in ? tid : 0);
    const int row = a.uidx[rr];
    const int dep = a.depth[rr];
    const float sc = a.scale[rr];
    rows[tid] = in ? row : 0;
    deps[tid] = in ? dep : 0;
    scl[tid] = in ? sc : 0.f;
    const float* f = a.fac + ((long long)u * a.nsplit + split) * G;
    float ev[G], fv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      ev[h] = a.e[((long long)u * G + h) * a.ld + r0 + (in ? tid : 0)];
      fv[h] = f[h];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) pr[tid][h] = in ? ev[h] * fv[h] : 0.f;
  }
  __syncthreads();
  // lane c of a row group loads dword c of the row's planes (plane c / 4)
  // when that plane is read; every load is issued before the arithmetic
  uint32_t dw[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = RPW * wave + 4 * it + rs;
    const int t = deps[r];
    const long long rec = gu * a.g.cap + rows[r];
    dw[it] = 0u;
    if ((ch >> 2) < t) dw[it] = reinterpret_cast<const uint32_t*>(a.vplanes + rec * VREC)[ch];
  }
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = RPW * wave + 4 * it + rs;
    // byte c of plane p is byte c % 4 of dword 4 p + c / 4 of the row group
    uint32_t code = 0;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t x = (uint32_t)__shfl((int)dw[it], (lane & ~15) + 4 * p + (ch >> 2));
      code |= spread4((x >> (8 * (ch & 3))) & 0xFFu) << (NP - 1 - p);
    }
    const float s = scl[r];
    const int t = deps[r];
    const float off = s * (t == 0 ? 0.f : ldexpf(1.f, 3 - t) - 8.f);  // s (2^(3-t) - 8), exact
    float vf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vf[e] = fmaf(s, (float)((code >> (4 * e)) & 15u), off);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float wt = pr[r][h];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = fmaf(wt, vf[e], o[h][e]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[4 * wave + rs][h][8 * ch + e] = o[h][e];
  __syncthreads();
  for (int e = tid; e < G * D; e += VA_THREADS) {
    const int h = e / D, d = e % D;
    float v = 0.f;
    for (int gi = 0; gi < VA_THREADS / 16; ++gi) v += oacc[gi][h][d];
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
  w.nsplit = (int)((sel + VA_ROWS - 1) / VA_ROWS);
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

// rows per depth-search thread for a row stride of ld
inline int vd_per(long long ld) { return ld <= 2 * VD_THREADS ? 2 : ld <= 8 * VD_THREADS ? 8 : VD_PER; }

template <int G, bool GIVEN>
void launch_vdepth(const VDepthArgs& da, hipStream_t st) {
  const int units = da.g.units();
  switch (vd_per(da.ld)) {
    case 2: vdepth_kernel<G, 2, GIVEN><<<units, VD_THREADS, 0, st>>>(da); break;
    case 8: vdepth_kernel<G, 8, GIVEN><<<units, VD_THREADS, 0, st>>>(da); break;
    default: vdepth_kernel<G, VD_PER, GIVEN><<<units, VD_THREADS, 0, st>>>(da); break;
  }
}

template <int G>
void launch_v_g(const VDepthArgs& da, const VAccArgs& va, float* out, hipStream_t st) {
  const int units = da.g.units();
  launch_vdepth<G, false>(da, st);
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
  uint8_t* vdep = reinterpret_cast<uint8_t*>(base + w.vdep);
  float* part = reinterpret_cast<float*>(base + w.part);
  float* vsc = reinterpret_cast<float*>(base + w.scale);
  hipError_t e = launch_union_logits(g, k_dtype, k_rows, q, idx, k, scale, uidx, umask, ucount,
                                     ev, stats, vscales, vsc, union_ready, st);
  if (e != hipSuccess) return e;
  const long long sel = (long long)g.G * k;
  VDepthArgs da{g,       sel,      ucount,  uidx,     ev,   stats,      fac,
                w.nsplit, nullptr, vscales, v_budget, vsc,  vdep,       vdepth_out,
                union_out};
  VAccArgs va{g, sel, uidx, ucount, ev, fac, vsc, vdep, vplanes, vscales, part, w.nsplit};
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
  VDepthArgs da{g,       row_ld,  n_rows,   rows,     nullptr, nullptr, nullptr,
                0,       weights, vscales,  v_budget, nullptr, depth,   nullptr,
                nullptr};
  launch_vdepth<1, true>(da, st);
  return hipGetLastError();
}

}  // namespace bpk
