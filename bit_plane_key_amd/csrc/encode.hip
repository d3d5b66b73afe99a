// Bit-plane encoder: per 64-token block, fp16 block scales and channel-major
// planes of the 4-bit symmetric codes (Fathom §3.2).
//
// Keys as stored (encode_tok_kernel): a workgroup codes 16 consecutive
// blocks, each wavefront one block at a time.  Lane (c, t), c = lane % 16,
// t = lane / 16, holds channels 8c .. 8c+7 of tokens 16t .. 16t+15: sixteen
// 16-byte row loads (32-byte for fp32 keys), all in flight together.  A
// channel's block maximum is the lane's own maximum over its 16 tokens
// combined with the three other token groups' (two lane exchanges); the lane
// codes its 16 values of the channel (as nibbles, from which each plane's 16
// bits are gathered) and puts bits 16t .. 16t+15 of the channel's four plane
// words into LDS.  The group's words then leave as one contiguous 128-byte
// run per plane row.
//
// Rotated keys (encode_kernel): one workgroup per (unit, block), one thread
// per channel: the block's rows are staged in LDS, thread j forms z_j of
// every row, keeps the 64 values in registers and assembles the four 64-bit
// plane words of its channel bit by bit (bit i <-> token i).
#include <algorithm>

#include "bpk_internal.h"

namespace bpk {
namespace {

struct EncArgs {
  int L, H;
  long long cap, nbcap;
  int seq;
  long long b0;
  const void* k_rows;
  const float* rot;
  uint64_t* planes;
  uint16_t* scales;
};

template <bool F32, bool ROT>
__global__ __launch_bounds__(128) void encode_kernel(EncArgs a) {
  __shared__ float tile[ROT ? BLK : 1][ROT ? D : 1];
  const int j = threadIdx.x;
  const int lh = blockIdx.y;
  const int l = lh / a.H, h = lh % a.H;
  const long long gu = ((long long)a.seq * a.L + l) * a.H + h;
  const long long blk = a.b0 + blockIdx.x;
  const long long row0 = gu * a.cap + blk * BLK;

  float v[BLK];
  if constexpr (!ROT) {
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
      if constexpr (F32)
        v[i] = static_cast<const float*>(a.k_rows)[(row0 + i) * D + j];
      else
        v[i] = bf16_to_f32(static_cast<const uint16_t*>(a.k_rows)[(row0 + i) * D + j]);
    }
  } else {
    for (int i = 0; i < BLK; ++i) {
      if constexpr (F32)
        tile[i][j] = static_cast<const float*>(a.k_rows)[(row0 + i) * D + j];
      else
        tile[i][j] = bf16_to_f32(static_cast<const uint16_t*>(a.k_rows)[(row0 + i) * D + j]);
    }
    __syncthreads();
    // z_j = sum_d R[d][j] * k_d: each product of two fp32 values is exact in
    // fp64, added in ascending d.
    const float* r = a.rot + (long long)(l * a.H + h) * D * D + j;
    for (int i = 0; i < BLK; ++i) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc = __dadd_rn(acc, (double)r[d * D] * (double)tile[i][d]);
      v[i] = (float)acc;
    }
  }

  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < BLK; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const _Float16 hs = scale_of_max(amax);
  const float s = (float)hs;

  uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll
  for (int i = 0; i < BLK; ++i) {
    const uint64_t c = quant_code(v[i], s);
    w0 |= ((c >> 3) & 1ull) << i;
    w1 |= ((c >> 2) & 1ull) << i;
    w2 |= ((c >> 1) & 1ull) << i;
    w3 |= (c & 1ull) << i;
  }
  const long long pbase = ((gu * D + j) * NP) * a.nbcap + blk;
  a.planes[pbase] = w0;
  a.planes[pbase + a.nbcap] = w1;
  a.planes[pbase + 2 * a.nbcap] = w2;
  a.planes[pbase + 3 * a.nbcap] = w3;
  a.scales[(gu * D + j) * a.nbcap + blk] = __builtin_bit_cast(uint16_t, hs);
}

constexpr int ENC_GROUP = 16;  // blocks per workgroup of encode_tok_kernel (128 bytes of each plane row)
constexpr int ENC_WAVES = 4;   // its wavefronts, one block at a time each

// clip(floor(v / s), -8, 7) + 8 with the exact real floor, given r ~ 1 / s
// (s > 0): floor(v r) is within one of floor(v / s) (|v / s| <= 8 (1 + 2^-11)
// for the values the scale was taken from; beyond, the clip decides), and
// m s, (m + 1) s are exact in fp32, so one corrective step, taken without a
// branch, gives the exact floor
__device__ __forceinline__ uint32_t quant_code_r(float v, float s, float r) {
  const float m0 = floorf(v * r);
  int m = (int)m0;
  m += (fmaf(m0, s, s) <= v) - (m0 * s > v);  // (m0 + 1) s and m0 s are exact
  m = m < -8 ? -8 : (m > 7 ? 7 : m);
  return (uint32_t)(m + 8);
}

// bits k, k + 4, .., k + 28 of x gathered into bits 0 .. 7
__device__ __forceinline__ uint32_t nibble_bits(uint32_t x, int k) {
  x = (x >> k) & 0x11111111u;
  x = (x | (x >> 3)) & 0x03030303u;
  x = (x | (x >> 6)) & 0x000F000Fu;
  return (x | (x >> 12)) & 0xFFu;
}

template <bool F32>
__global__ __launch_bounds__(64 * ENC_WAVES) void encode_tok_kernel(EncArgs a, long long nblocks) {
  // the group's plane words, row (j, p) = 4 j + p, word of block b in slot
  // b ^ (j / 8) (so the 16 channel groups of one store hit 16 banks), and
  // its scales
  __shared__ uint64_t stage[D * NP][ENC_GROUP];
  __shared__ uint16_t sstage[D][ENC_GROUP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = lane & 15, tg = lane >> 4;
  const int lh = blockIdx.y;
  const int l = lh / a.H, h = lh % a.H;
  const long long gu = ((long long)a.seq * a.L + l) * a.H + h;
  const long long g0 = a.b0 + (long long)blockIdx.x * ENC_GROUP;
  const long long left = nblocks - (long long)blockIdx.x * ENC_GROUP;
  const int nv = left < ENC_GROUP ? (int)left : ENC_GROUP;  // blocks of this group
  auto comp = [](const uint4& q, int x) { return x == 0 ? q.x : x == 1 ? q.y : x == 2 ? q.z : q.w; };
  for (int bl = wave; bl < nv; bl += ENC_WAVES) {
    const long long row0 = gu * a.cap + (g0 + bl) * BLK + 16 * tg;
    uint4 raw[F32 ? 32 : 16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (F32) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(a.k_rows) +
                                                          (row0 + i) * D + 8 * cg);
        raw[2 * i] = src[0];
        raw[2 * i + 1] = src[1];
      } else {
        raw[i] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_rows) +
                                                 (row0 + i) * D + 8 * cg);
      }
    }
    auto val = [&](int i, int e) -> float {
      if constexpr (F32) return __uint_as_float(comp(raw[2 * i + e / 4], e % 4));
      const uint32_t w = comp(raw[i], e / 2);
      return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    };
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(val(i, e)));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      const _Float16 hs = scale_of_max(m);
      const float sv = (float)hs;
      const float r = 1.f / sv;
      // the 16 codes as nibbles (token i at bits 4 (i % 8) of word i / 8),
      // then each plane's 16 bits gathered from them
      uint32_t nib[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) nib[i >> 3] |= quant_code_r(val(i, e), sv, r) << (4 * (i & 7));
      uint32_t pc[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int k = NP - 1 - p;
        pc[p] = nibble_bits(nib[0], k) | (nibble_bits(nib[1], k) << 8);
      }
      if (sv == 0.f) {  // a zero scale codes every value as 8 (0b1000)
        pc[0] = 0xFFFFu;
        pc[1] = pc[2] = pc[3] = 0u;
      }
      const int j = 8 * cg + e;
#pragma unroll
      for (int p = 0; p < NP; ++p)
        reinterpret_cast<uint16_t*>(&stage[j * NP + p][bl ^ cg])[tg] = (uint16_t)pc[p];
      if (tg == 0) sstage[j][bl] = __builtin_bit_cast(uint16_t, hs);
    }
  }
  __syncthreads();
  // plane row (j, p) gets the group's nv words in one contiguous run
  uint64_t* pdst = a.planes + gu * D * NP * a.nbcap + g0;
  for (int e = tid; e < D * NP * ENC_GROUP; e += 64 * ENC_WAVES) {
    const int row = e / ENC_GROUP, b = e % ENC_GROUP;
    if (b < nv) pdst[row * a.nbcap + b] = stage[row][b ^ ((row / (8 * NP)) & 15)];
  }
  uint16_t* sdst = a.scales + gu * D * a.nbcap + g0;
  for (int e = tid; e < D * ENC_GROUP; e += 64 * ENC_WAVES) {
    const int j = e / ENC_GROUP, b = e % ENC_GROUP;
    if (b < nv) sdst[j * a.nbcap + b] = sstage[j][b];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void append_rows_kernel(int L, int H, long long cap, int seq,
                                                          long long n0, long long n_new,
                                                          const T* src, T* dst) {
  const int lh = blockIdx.y;
  const int l = lh / H, h = lh % H;
  const long long gu = ((long long)seq * L + l) * H + h;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_new * D) return;
  dst[(gu * cap + n0) * D + e] = src[(long long)lh * n_new * D + e];
}

}  // namespace

hipError_t launch_append_rows(const Geom& g, int seq, int k_dtype, const void* k_new,
                              const uint16_t* v_new, long long n0, long long n_new, void* k_rows,
                              uint16_t* v_rows, hipStream_t st) {
  if (n_new <= 0) return hipSuccess;
  dim3 grid((unsigned)((n_new * D + 255) / 256), (unsigned)(g.L * g.H));
  if (k_dtype == BPK_F32)
    append_rows_kernel<float><<<grid, 256, 0, st>>>(g.L, g.H, g.cap, seq, n0, n_new,
                                                   static_cast<const float*>(k_new),
                                                   static_cast<float*>(k_rows));
  else
    append_rows_kernel<uint16_t><<<grid, 256, 0, st>>>(g.L, g.H, g.cap, seq, n0, n_new,
                                                      static_cast<const uint16_t*>(k_new),
                                                      static_cast<uint16_t*>(k_rows));
  append_rows_kernel<uint16_t><<<grid, 256, 0, st>>>(g.L, g.H, g.cap, seq, n0, n_new, v_new,
                                                    v_rows);
  return hipGetLastError();
}

hipError_t launch_encode(const Geom& g, int seq, int k_dtype, const void* k_rows, const float* rot,
                         uint64_t* planes, uint16_t* scales, long long b0, long long nblocks,
                         hipStream_t st) {
  if (nblocks <= 0) return hipSuccess;
  EncArgs a{g.L, g.H, g.cap, g.nbcap(), seq, b0, k_rows, rot, planes, scales};
  const int lh = g.L * g.H;
  // grid.x is limited to 2^31 - 1 and grid.y to 65535: split long ranges.
  const long long chunk = 1ll << 30;
  for (long long off = 0; off < nblocks; off += chunk) {
    a.b0 = b0 + off;
    dim3 grid((unsigned)std::min(chunk, nblocks - off), (unsigned)lh);
    const bool f32 = (k_dtype == BPK_F32);
    if (rot) {
      if (f32) encode_kernel<true, true><<<grid, 128, 0, st>>>(a);
      else encode_kernel<false, true><<<grid, 128, 0, st>>>(a);
    } else {
      const long long nb = std::min(chunk, nblocks - off);
      dim3 tgrid((unsigned)((nb + ENC_GROUP - 1) / ENC_GROUP), (unsigned)lh);
      if (f32) encode_tok_kernel<true><<<tgrid, 64 * ENC_WAVES, 0, st>>>(a, nb);
      else encode_tok_kernel<false><<<tgrid, 64 * ENC_WAVES, 0, st>>>(a, nb);
    }
  }
  return hipGetLastError();
}

}  // namespace bpk
