// Shared by the two key-scan kernels (scan.hip: units reading at most
// SCAN_FAST_ROWS plane rows; scan_wide.hip: the others).  Not part of the ABI.
#pragma once

#include <type_traits>

#include "bpk_internal.h"

namespace bpk {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int SCAN_THREADS = 256;
constexpr int SCAN_GB = 16;              // blocks per step (128-byte reads of a plane row)
constexpr int SCAN_WIDE_SPAN = 1024;     // blocks per workgroup of a wide scan when launched blind
// Fixed-point frame of the row weights: |X_r| < 2^FRAME_BITS (four balanced
// int8 digits; the top one within [-32, 32]).
constexpr int FRAME_BITS = 29;
// 2^52 + 2^51 + 0x80808080: an fp64 sum with it lies in [2^52, 2^53), where
// the ulp is 1 and the low 32 bits of the bit pattern are X + 0x80808080
constexpr double DIGIT_MAGIC64 = 6755401596960896.0;
// bound of |2^8 d1 + d0| for the two low digits of one row
constexpr int LOW_DIGITS_MAX = 128 * 256 + 128;
static_assert(SCAN_MIN_WG_BLOCKS == SCAN_GB, "a workgroup takes whole steps");
static_assert(SAMPLE_GROUP % SCAN_GB == 0 && SAMPLE_STRIDE % SAMPLE_GROUP == 0, "sample plan");

// What a launch does with the scores it computes:
// * SCAN_FULL writes every score ([unit][G][cap]);
// * SCAN_SAMPLE scores only the first SAMPLE_GROUP blocks of every
//   SAMPLE_STRIDE (one workgroup per sampled group) and writes the upper 16
//   bits of each score's order key into [unit][G][sample_ld];
// * SCAN_CAND appends (score, token) of the tokens of [4, n - W) whose score
//   is at or above the head's threshold to the workgroup's candidate region
//   of that head (slots handed out by an LDS counter; the count, which may
//   pass the region's size, is stored at the end).
enum ScanMode { SCAN_FULL = 0, SCAN_SAMPLE = 1, SCAN_CAND = 2 };

struct ScanArgs {
  Geom g;
  const float* __restrict__ q_basis;
  const uint8_t* __restrict__ depth;
  const uint64_t* __restrict__ planes;
  const uint16_t* __restrict__ scales;
  float* __restrict__ out;          // scores (FULL)
  uint16_t* __restrict__ sample;    // SAMPLE: upper halves of the sampled scores' order keys
  long long out_ld;                 // per (unit, head) row length of out or sample
  int wg_blocks;                    // blocks per workgroup (multiple of SCAN_GB)
  int k;                            // top-k (CAND: units with n <= k are skipped)
  const int32_t* __restrict__ unit_flag;  // FULL: if set, only units with flag != 0
  const uint32_t* __restrict__ thresh;    // CAND: [unit][G] order keys
  long long regions;                      // CAND: region stride per (unit, head)
  int32_t* __restrict__ cand_count;       // CAND: [unit][G][regions]
  float* __restrict__ cand_val;           // CAND: [unit][G][regions][CAND_SLOTS]
  int32_t* __restrict__ cand_idx;         // CAND: [unit][G][regions][CAND_SLOTS]
  int part_slots;                         // CAND: candidate slots per (workgroup, head, wavefront)
  int all_rows;                           // wide kernel: take every unit, whatever it reads
  int rows_above;                         // fast kernel: skip units reading at most this many rows
};

// the wide kernel (units reading more than SCAN_FAST_ROWS rows, or every unit
// with all_rows); span = blocks per workgroup (0: the standard scan_wg_blocks /
// SAMPLE_GROUP)
hipError_t launch_scan_wide(const ScanArgs& a, int mode, int span, hipStream_t st);

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off);
    v = o > v ? o : v;
  }
  return v;
}

// the same with DPP moves inside each 16-lane row (quad_perm xor 1, xor 2,
// row_half_mirror, row_mirror) and one read of each row's result; every lane
// of the wavefront must be active
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return mx(mx(r0, r1), mx(r2, r3));
}

// the same maximum within each 16-lane row, in every lane of the row (every
// lane of the row must be active)
__device__ __forceinline__ uint32_t row_max_u32_dpp(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return v;
}

// value of the neighbouring lane (lane ^ 1)
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Largest E with m 2^E < 2^lx (0 for m == 0), clamped so that every later
// scaling by 2^E or 2^-(E+1) stays in the normal range.
__device__ __forceinline__ int frame_exp(float m, int lx) {
  if (!(m > 0.f)) return 0;
  int e;
  frexpf(m, &e);  // m < 2^e
  int E = lx - e;
  return E < -100 ? -100 : (E > 100 ? 100 : E);
}

// The four balanced signed digits of X = round(f s) (to nearest, ties to
// even; |X| < 2^29), packed little-endian: X = d0 + 2^8 d1 + 2^16 d2 + 2^24 d3.
// f s is exact in fp64 (f carries at most 24 significant bits, s 11), so the
// fma rounds once; the low word of the result is X + 0x80808080, whose bytes
// are the digits + 128 each (no carries), and the xor turns each into the
// digit's two's-complement byte.
__device__ __forceinline__ uint32_t x_digits4(double f, double s) {
  const double r = __builtin_fma(f, s, DIGIT_MAGIC64);
  return (uint32_t)__builtin_bit_cast(unsigned long long, r) ^ 0x80808080u;
}

// Column arithmetic of the scan's integer contraction.  A column of the
// products keeps bit bp of each plane byte, so its digit sums carry the
// factor v = 2^bp (bp < 7), or v = -128 for bp = 7 (the int8 byte 0x80);
// d = (D0, D1, D2, D3) are the column's digit sums of sum_r X_r b_r times v,
// dc = (C0 .. C3) the digit sums of C = sum_r X_r (all-one bytes).  The score
// is (2 S - C) 2^-(e+1), formed from the high and low halves
// T_hi = 2 P' - C_hi (units of 2^16) and T_lo = 2 S_lo - C_lo, each exact in
// int32, by one fma (T_lo is exact in fp32 while 3 R 2^15 < 2^24, R < 170;
// beyond, it rounds by at most 3 units).
__device__ __forceinline__ float score4(const i32x4& d, const i32x4& dc, int bp, bool neg, int e) {
  int ph = (d.w >> bp) * 256 + (d.z >> bp);  // P' v / |v|
  int pl = (d.y >> bp) * 256 + (d.x >> bp);  // S_lo v / |v|
  if (neg) {
    ph = -ph;
    pl = -pl;
  }
  const int th = 2 * ph - (dc.w * 256 + dc.z);
  const int tl = 2 * pl - (dc.y * 256 + dc.x);
  return ldexpf(__builtin_fmaf((float)th, 65536.f, (float)tl), -(e + 1));
}

// Candidate test threshold of a (head, block) with frame exponent e, for R
// rows: tau such that every token whose written score is >= theta has
// 2 P' - C_hi >= tau (P' = sum_r (2^8 d3 + d2) b_r, C_hi = 2^8 C3 + C2).
// The written score needs T = 2 S - C >= tp - |tp| 2^-22 - 16 with
// tp = theta 2^(e+1) (the two fp32 roundings of score4 move T by at most
// |tp| 2^-23 + 4), and the dropped low halves move 2^16 (2 P' - C_hi) below T by
// at most 3 R LOW_DIGITS_MAX.  Clamped to +-2^24 (beyond every value of
// 2 P' - C_hi: nobody / everybody passes); the caller keeps tau + 1.
__device__ __forceinline__ int cand_tau(float theta, int e, int R) {
  if (theta == -__builtin_inff()) return -(1 << 24);
  if (!(theta < __builtin_inff())) return 1 << 24;  // +inf or NaN: nothing passes
  const double tp = ldexp((double)theta, e + 1);
  const double need = tp - fabs(tp) * 0x1p-22 - 16.0 - 3.0 * LOW_DIGITS_MAX * (double)R;
  const double t = floor(need * 0x1p-16);
  if (t <= -16777216.0) return -(1 << 24);
  if (t >= 16777216.0) return 1 << 24;
  return (int)t;
}

// Inverse of order_key; 0 and ~0 (everything / nothing is a candidate) map to
// -inf / +inf.
__device__ __forceinline__ float key_to_float(uint32_t k) {
  if (k == 0u) return -__builtin_inff();
  if (k == 0xFFFFFFFFu) return __builtin_inff();
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// the per-part counts of a candidate region filled front to back with total
// candidates (the last part takes any overflow, which the selection flags)
__device__ __forceinline__ void contiguous_part_counts(int32_t* cnt, int total, int part_slots) {
#pragma unroll
  for (int p = 0; p < CAND_PARTS; ++p) {
    int c = total - p * part_slots;
    c = c < 0 ? 0 : c;
    if (p + 1 < CAND_PARTS && c > part_slots) c = part_slots;
    cnt[p] = c;
  }
}

// ds_read_b64_tr_b8: in each 16-lane group, lane i < 8 gets byte i of the 8
// bytes at the addresses of lanes 0, 2, .., 14, and lane i >= 8 gets byte
// i - 8 of those of lanes 1, 3, .., 15 (byte j of the result from the j-th
// of those lanes).
__device__ __forceinline__ i32x2 tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

}  // namespace bpk
