// Bit-plane encoder: per 64-token block, fp16 block scales and channel-major
// planes of the 4-bit symmetric codes (Fathom §3.2).  One workgroup per
// (unit, block), one thread per channel: thread j walks the block's 64 rows
// (each row read is a coalesced 256/512-byte line across the workgroup), keeps
// the 64 values in registers, and assembles the four 64-bit plane words of
// its channel bit by bit (bit i <-> token i).
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
      if (f32) encode_kernel<true, false><<<grid, 128, 0, st>>>(a);
      else encode_kernel<false, false><<<grid, 128, 0, st>>>(a);
    }
  }
  return hipGetLastError();
}

}  // namespace bpk
