// Shared by the two key-scan kernels (scan.hip: units reading at most
// SCAN_FAST_ROWS plane rows; scan_wide.hip: the others).  Not part of the ABI.
#pragma once

#include <type_traits>

#include "bpk_internal.h"

namespace bpk {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16-byte global words of rows that are only 8-byte aligned (odd capacity / 64)
typedef uint32_t u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int SCAN_THREADS = 256;
constexpr int SCAN_GB = 16;              // blocks per step (128-byte reads of a plane row)
constexpr int SCAN_WIDE_SPAN = 1024;     // blocks per workgroup of a wide scan when launched blind
constexpr float DIGIT_BIAS = 8421504.f;  // 0x808080: X + bias holds three balanced digits + 128 each
static_assert(SCAN_MIN_WG_BLOCKS == SCAN_GB, "a workgroup takes whole steps");
static_assert(SAMPLE_GROUP % SCAN_GB == 0 && SAMPLE_STRIDE % SAMPLE_GROUP == 0, "sample plan");

// What a launch does with the scores it computes:
// * SCAN_FULL writes every score ([unit][G][cap]);
// * SCAN_SAMPLE scores only the first SAMPLE_GROUP blocks of every
//   SAMPLE_STRIDE (one workgroup per sampled group) into [unit][G][sample_ld];
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
  float* __restrict__ out;          // scores (FULL) or sampled scores (SAMPLE)
  long long out_ld;                 // per (unit, head) row length of out
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
