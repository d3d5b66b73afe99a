// Device-side generator of the synthetic workloads: the same Philox4x32-10
// elements as the host generator in synth/philox.py, bit for bit.
//   element (unit u, row r, column d, stream s):
//     counter = (r & 0xffffffff, r >> 32, d, s), key = keys[u]
//     x = sum of the eight 16-bit halves of the four output words - 262140
//     value = float(x) * mult[u][d]   (one fp32 product, round to nearest even)
//   optionally rotated per row: k_d = sum_j R[d][j] z_j (fp64, j ascending),
//   stored as fp32 or as bf16 (round to nearest even).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int D = 128;

__device__ __forceinline__ void philox_round(uint32_t& x0, uint32_t& x1, uint32_t& x2,
                                             uint32_t& x3, uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  const uint32_t y0 = hi1 ^ x1 ^ k0;
  const uint32_t y2 = hi0 ^ x3 ^ k1;
  x0 = y0;
  x1 = lo1;
  x2 = y2;
  x3 = lo0;
}

__device__ __forceinline__ int32_t irwin_hall8(uint32_t k0, uint32_t k1, uint64_t row, uint32_t col,
                                               uint32_t stream) {
  uint32_t x0 = (uint32_t)row, x1 = (uint32_t)(row >> 32), x2 = col, x3 = stream;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    philox_round(x0, x1, x2, x3, k0, k1);
  }
  const int32_t s = (int32_t)((x0 & 0xFFFFu) + (x0 >> 16) + (x1 & 0xFFFFu) + (x1 >> 16) +
                              (x2 & 0xFFFFu) + (x2 >> 16) + (x3 & 0xFFFFu) + (x3 >> 16));
  return s - 262140;
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  const uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

struct FillArgs {
  const uint32_t* keys;  // [units][2]
  const float* mult;     // [units][D]
  const float* rot;      // NULL or [rot_lh][D][D]
  int rot_lh;
  long long row0, rows, cap;
  uint32_t stream;
  int out_bf16;
  void* out;
};

// one workgroup of 128 threads per (unit, 64 rows); thread d owns column d
template <bool ROT>
__global__ __launch_bounds__(128) void fill_kernel(FillArgs a) {
  __shared__ float z[ROT ? 64 : 1][ROT ? D : 1];
  const int d = threadIdx.x;
  const long long u = blockIdx.y;
  const long long r0 = a.row0 + (long long)blockIdx.x * 64;
  const uint32_t k0 = a.keys[2 * u], k1 = a.keys[2 * u + 1];
  const float m = a.mult[u * D + d];
  const long long rend = a.row0 + a.rows;
  const int nr = (int)((rend - r0) < 64 ? (rend - r0) : 64);
  for (int i = 0; i < nr; ++i) {
    float v = (float)irwin_hall8(k0, k1, (uint64_t)(r0 + i), d, a.stream) * m;
    if constexpr (ROT) {
      z[i][d] = v;
    } else {
      const long long e = (u * a.cap + r0 + i) * D + d;
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[e] = to_bf16(v);
      else
        static_cast<float*>(a.out)[e] = v;
    }
  }
  if constexpr (ROT) {
    __syncthreads();
    const float* r = a.rot + (u % a.rot_lh) * D * D + (long long)d * D;
    for (int i = 0; i < nr; ++i) {
      double acc = 0.0;
      for (int j = 0; j < D; ++j) acc = __dadd_rn(acc, (double)r[j] * (double)z[i][j]);
      const float v = (float)acc;
      const long long e = (u * a.cap + r0 + i) * D + d;
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[e] = to_bf16(v);
      else
        static_cast<float*>(a.out)[e] = v;
    }
  }
}

// Streaming-read probe of the benchmark: every thread reads 16-byte words
// in a grid-stride loop (four loads in flight) and folds them into one word
// per workgroup, so the loads cannot be dropped.  Reads n16 words of buf.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ buf,
                                                          long long n16, uint32_t* out) {
  __shared__ uint32_t part[4];
  const long long stride = (long long)gridDim.x * 256;
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" {

// Read n16 16-byte words of buf (16-byte aligned) with `blocks` workgroups
// of 256 threads, writing one word per workgroup to out[blocks].  Returns 0,
// -1 for bad arguments or -5 for a launch error.
int synth_stream_read(const void* buf, long long n16, int blocks, uint32_t* out, void* stream) {
  if (!buf || !out || n16 < 0 || blocks < 1 || blocks > 65535 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return -1;
  stream_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(buf), n16, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Fill rows [row0, row0 + rows) of `units` units of a [units][cap][128] array.
// keys [units][2] uint32 and mult [units][128] fp32 are device pointers; rot is
// NULL or [rot_lh][128][128] fp32 (unit u uses matrix u % rot_lh).
// Returns 0, or -1 for bad arguments, or -5 for a launch error.
int synth_fill_rows(const uint32_t* keys, const float* mult, const float* rot, int rot_lh, int units,
                    long long row0, long long rows, long long cap, int stream_id, int out_bf16,
                    void* out, void* stream) {
  if (!keys || !mult || !out || units <= 0 || units > 65535 || rows < 0 || row0 < 0 ||
      row0 + rows > cap || (rot && rot_lh <= 0))
    return -1;
  if (rows == 0) return 0;
  FillArgs a{keys, mult, rot, rot_lh, row0, rows, cap, (uint32_t)stream_id, out_bf16, out};
  dim3 grid((unsigned)((rows + 63) / 64), (unsigned)units);
  if (rot)
    fill_kernel<true><<<grid, 128, 0, static_cast<hipStream_t>(stream)>>>(a);
  else
    fill_kernel<false><<<grid, 128, 0, static_cast<hipStream_t>(stream)>>>(a);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
