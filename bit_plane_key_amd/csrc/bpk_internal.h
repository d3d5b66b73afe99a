// Internal declarations shared by the library's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bpk.h"

namespace bpk {

constexpr int D = BPK_HEAD_DIM;
constexpr int BLK = BPK_BLOCK;
constexpr int NP = BPK_PLANES;

// Geometry of the units a launch covers: every sequence, layers [l0, l0 + nl),
// every KV head.  Local unit u -> (s, l, h) with h fastest.
struct Geom {
  int S, L, H, G;
  int l0, nl;
  long long cap;  // tokens per sequence (multiple of 64)
  long long n[BPK_MAX_SEQS];

  __host__ __device__ int units() const { return S * nl * H; }
  __host__ __device__ int seq_of(int u) const { return u / (H * nl); }
  // global unit index (s * L + l) * H + h of local unit u
  __host__ __device__ long long global_unit(int u) const {
    int h = u % H;
    int l = l0 + (u / H) % nl;
    int s = u / (H * nl);
    return ((long long)s * L + l) * H + h;
  }
  __host__ __device__ long long nbcap() const { return cap / BLK; }
};

// ---- launchers (each returns hipGetLastError() of its launches) ----
hipError_t launch_encode(const Geom& g, int seq, int k_dtype, const void* k_rows,
                         const float* rot, uint64_t* planes, uint16_t* scales, long long b0,
                         long long nblocks, hipStream_t st);

hipError_t launch_append_rows(const Geom& g, int seq, int k_dtype, const void* k_new,
                              const uint16_t* v_new, long long n0, long long n_new, void* k_rows,
                              uint16_t* v_rows, hipStream_t st);

hipError_t launch_alloc(const Geom& g, const uint16_t* q, const float* chan_var, const float* rot,
                        int budget, uint8_t* depth, float* q_basis, hipStream_t st);

hipError_t launch_scan(const Geom& g, const float* q_basis, const uint8_t* depth,
                       const uint64_t* planes, const uint16_t* scales, float* scores,
                       hipStream_t st);

hipError_t launch_topk(const Geom& g, const float* scores, int k, int32_t* idx, hipStream_t st);

size_t attend_ws_bytes(const Geom& g, int k);
hipError_t launch_attend(const Geom& g, int k_dtype, const void* k_rows, const uint16_t* v_rows,
                         const uint16_t* q, const int32_t* idx, int k, float scale, float* out,
                         void* ws, hipStream_t st);

// ---- small device helpers ----
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

}  // namespace bpk
