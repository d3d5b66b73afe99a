// Per-query depth allocation by reverse water-filling (Fathom §1 observation 1
// and §3; ReadKV §5.2 and §5.4).  One wavefront per unit: lane l owns channels
// 2l and 2l+1 and their 8 (channel, plane) candidates.  The budget of P planes
// goes to the P candidates of largest value g_j * 4^-t; the P-th largest
// candidate is found by a 41-step bitwise search over the totally ordered keys
// (value bits << 9 | 511 - (4 j + t)), counting with wave ballots, and a
// channel's depth is the number of its candidates at or above that key.
//
// The same kernel also writes the fixed depth vectors of the baselines the
// Fathom page compares against (§2): SparQ's r channels of largest summed
// |q| over the group at full depth (the r-th largest found by the same kind
// of bitwise search), a static channel set at full depth (Double Sparsity),
// or one depth for every channel (t = 2: the 2-bit thumbnail scan).
#include "bpk_internal.h"

namespace bpk {
namespace {

struct AllocArgs {
  Geom g;
  const uint16_t* q;
  const float* chan_var;
  const float* rot;
  int budget;  // WATERFILL: planes; SPARQ: r; CHANNELS: c; UNIFORM: t
  uint8_t* depth;
  float* q_basis;
  int rule;                 // BPK_DEPTH_*
  const uint8_t* channels;  // CHANNELS: [L][H][c] channel indices
  float* gains;             // WATERFILL, if set: g_j of every unit [units][D]
  const int32_t* layer_budget;  // WATERFILL, if set: the budget of each layer of the call [nl]
};

template <int G, bool ROT>
__global__ __launch_bounds__(64) void alloc_kernel(AllocArgs a) {
  __shared__ float sq[ROT ? G : 1][ROT ? D : 1];
  __shared__ uint8_t chosen[D];
  const int u = blockIdx.x;
  const long long gu = a.g.global_unit(u);
  const int lane = threadIdx.x;
  const uint16_t* qu = a.q + (long long)u * G * D;

  float qb[G][2];
  if constexpr (!ROT) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c) qb[h][c] = bf16_to_f32(qu[h * D + 2 * lane + c]);
  } else {
    for (int e = lane; e < G * D; e += 64) sq[e / D][e % D] = bf16_to_f32(qu[e]);
    __syncthreads();
    const int l = a.g.l0 + (u / a.g.H) % a.g.nl;
    const int hh = u % a.g.H;
    const float* r = a.rot + (long long)(l * a.g.H + hh) * D * D;
    // q'_j = sum_d R[d][j] q_d, exact fp64 products added in ascending d;
    // each row of R is read once for every head (lane: columns 2 lane, +1)
    double acc[G][2];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = 0.0;
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
      const float2 rv = *reinterpret_cast<const float2*>(r + d * D + 2 * lane);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const double qd = (double)sq[h][d];
        acc[h][0] = __dadd_rn(acc[h][0], (double)rv.x * qd);
        acc[h][1] = __dadd_rn(acc[h][1], (double)rv.y * qd);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c) qb[h][c] = (float)acc[h][c];
  }
  float* qbo = a.q_basis + (long long)u * G * D;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < 2; ++c) qbo[h * D + 2 * lane + c] = qb[h][c];

  uint8_t* dep = a.depth + (long long)u * D;
  if (a.rule == BPK_DEPTH_UNIFORM) {
    const uint8_t v = (uint8_t)(a.budget < 0 ? 0 : (a.budget > NP ? NP : a.budget));
    dep[2 * lane] = v;
    dep[2 * lane + 1] = v;
    return;
  }
  if (a.rule == BPK_DEPTH_CHANNELS) {
    const int c = a.budget < 0 ? 0 : (a.budget > D ? D : a.budget);
    const int l = a.g.l0 + (u / a.g.H) % a.g.nl;
    const uint8_t* list = a.channels + (long long)(l * a.g.H + u % a.g.H) * c;
    chosen[2 * lane] = chosen[2 * lane + 1] = 0;
    __syncthreads();
    for (int e = lane; e < c; e += 64)
      if (list[e] < D) chosen[list[e]] = 1;  // indices past the head size are ignored
    __syncthreads();
    dep[2 * lane] = chosen[2 * lane] ? NP : 0;
    dep[2 * lane + 1] = chosen[2 * lane + 1] ? NP : 0;
    return;
  }
  if (a.rule == BPK_DEPTH_SPARQ) {
    // s_j = |q_0j| + |q_1j| + ... (fp32, heads ascending); the r largest
    // (s, then the lower channel) are read at full depth
    const int take = a.budget < 0 ? 0 : (a.budget > D ? D : a.budget);
    uint64_t key[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) acc = __fadd_rn(acc, fabsf(qb[h][c]));
      key[c] = ((uint64_t)__float_as_uint(acc) << 7) | (uint64_t)(127u - (2 * lane + c));
    }
    uint64_t prefix = 0;
    if (take > 0) {
      for (int b = 38; b >= 0; --b) {
        const uint64_t cand = prefix | (1ull << b);
        const int cnt = __popcll(__ballot(key[0] >= cand)) + __popcll(__ballot(key[1] >= cand));
        if (cnt >= take) prefix = cand;
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) dep[2 * lane + c] = (take > 0 && key[c] >= prefix) ? NP : 0;
    return;
  }

  // g_j = var_j * (((q_0j^2 + q_1j^2) + ...) + q_(G-1)j^2), one rounding per op
  float gain[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float acc = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) acc = __fadd_rn(acc, __fmul_rn(qb[h][c], qb[h][c]));
    gain[c] = __fmul_rn(a.chan_var[gu * D + 2 * lane + c], acc);
  }
  if (a.gains) {
#pragma unroll
    for (int c = 0; c < 2; ++c) a.gains[(long long)u * D + 2 * lane + c] = gain[c];
  }

  const int budget = a.layer_budget ? a.layer_budget[(u / a.g.H) % a.g.nl] : a.budget;
  const int take = budget < NP * D ? budget : NP * D;
  if (take <= 0 || take >= NP * D) {
    const uint8_t v = take <= 0 ? 0 : NP;
    dep[2 * lane] = v;
    dep[2 * lane + 1] = v;
    return;
  }

  const float quarter_pow[NP] = {1.0f, 0.25f, 0.0625f, 0.015625f};
  uint64_t key[2][NP];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      const float v = __fmul_rn(gain[c], quarter_pow[t]);
      const uint32_t j = 2 * lane + c;
      key[c][t] = ((uint64_t)__float_as_uint(v) << 9) | (uint64_t)(511u - (NP * j + t));
    }

  uint64_t prefix = 0;
  for (int b = 40; b >= 0; --b) {
    const uint64_t cand = prefix | (1ull << b);
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < NP; ++t) cnt += __popcll(__ballot(key[c][t] >= cand));
    if (cnt >= take) prefix = cand;
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    int t_j = 0;
#pragma unroll
    for (int t = 0; t < NP; ++t) t_j += key[c][t] >= prefix ? 1 : 0;
    dep[2 * lane + c] = (uint8_t)t_j;
  }
}

template <int G>
void launch_g(const AllocArgs& a, hipStream_t st) {
  if (a.rot)
    alloc_kernel<G, true><<<a.g.units(), 64, 0, st>>>(a);
  else
    alloc_kernel<G, false><<<a.g.units(), 64, 0, st>>>(a);
}

// Pooled water-filling over every unit of the call (per-layer budget
// calibration): the budget of units * P planes goes to the most valuable
// (unit, channel, plane) candidates g_uj 4^-t, equal values to the lower
// unit, channel, plane.  One workgroup: the threshold key is found bit by
// bit from the top (57-bit keys: value bits, then the candidate index
// complemented), each probe counting every candidate; then each unit's
// count of candidates at or above it.
constexpr int POOL_THREADS = 1024;
__global__ __launch_bounds__(POOL_THREADS) void pooled_kernel(const float* __restrict__ gains,
                                                              int units, long long take,
                                                              int32_t* __restrict__ counts) {
  __shared__ unsigned long long part[POOL_THREADS / 64];
  const int tid = threadIdx.x;
  const long long ncand = (long long)units * D * NP;
  const float qp[NP] = {1.0f, 0.25f, 0.0625f, 0.015625f};
  auto key = [&](long long c) {  // candidate c = (u * D + j) * NP + t
    const float v = __fmul_rn(gains[c / NP], qp[c % NP]);
    return ((unsigned long long)__float_as_uint(v) << 25) |
           ((unsigned long long)(0x1FFFFFFll - c) & 0x1FFFFFFull);
  };
  unsigned long long prefix = 0;
  if (take >= ncand) {
    prefix = 0;  // everything is taken
  } else if (take > 0) {
    for (int b = 56; b >= 0; --b) {
      const unsigned long long cand = prefix | (1ull << b);
      unsigned long long cnt = 0;
      for (long long c = tid; c < ncand; c += POOL_THREADS) cnt += key(c) >= cand;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1)
        cnt += (unsigned long long)__shfl_xor((long long)cnt, off);
      if ((tid & 63) == 0) part[tid >> 6] = cnt;
      __syncthreads();
      unsigned long long tot = 0;
#pragma unroll
      for (int w = 0; w < POOL_THREADS / 64; ++w) tot += part[w];
      __syncthreads();
      if (tot >= (unsigned long long)take) prefix = cand;
    }
  }
  for (int u = tid; u < units; u += POOL_THREADS) {
    int c = 0;
    if (take >= ncand) {
      c = D * NP;
    } else if (take > 0) {
      for (int e = 0; e < D * NP; ++e) c += key((long long)u * D * NP + e) >= prefix;
    }
    counts[u] = c;
  }
}

// Per-layer budgets from pooled counts [queries][units]: a layer's budget is
// the mean count of its units, rounded by largest remainder (ties to the
// lower layer) so that the budgets sum to nl * P.  One wavefront.
__global__ __launch_bounds__(64) void layer_budget_kernel(Geom g, const int32_t* __restrict__ counts,
                                                          int queries, int budget,
                                                          int32_t* __restrict__ out) {
  __shared__ long long per[256];
  __shared__ long long rem[256];
  __shared__ int base[256];
  const int lane = threadIdx.x;
  const int units = g.units();
  const long long denom = (long long)queries * g.S * g.H;
  for (int l = lane; l < g.nl; l += 64) {
    long long sum = 0;
    for (int qi = 0; qi < queries; ++qi)
      for (int s = 0; s < g.S; ++s)
        for (int h = 0; h < g.H; ++h) sum += counts[(long long)qi * units + (s * g.nl + l) * g.H + h];
    per[l] = sum;
    base[l] = (int)(sum / denom);
    rem[l] = sum - (long long)base[l] * denom;
  }
  __syncthreads();
  if (lane == 0) {
    long long used = 0;
    for (int l = 0; l < g.nl; ++l) used += base[l];
    long long shortfall = (long long)g.nl * budget - used;
    // hand out the shortfall one plane at a time: largest remainder first,
    // the lower layer on ties (a layer gets at most one)
    while (shortfall > 0) {
      int best = -1;
      for (int l = 0; l < g.nl; ++l)
        if (rem[l] >= 0 && (best < 0 || rem[l] > rem[best])) best = l;
      if (best < 0) break;
      ++base[best];
      rem[best] = -1;
      --shortfall;
    }
  }
  __syncthreads();
  for (int l = lane; l < g.nl; l += 64) out[l] = base[l];
}

}  // namespace

hipError_t launch_pooled(const Geom& g, const float* gains, int budget, int32_t* counts,
                         hipStream_t st) {
  const int units = g.units();
  if (units == 0) return hipSuccess;
  const long long take = (long long)(budget < NP * D ? budget : NP * D) * units;
  pooled_kernel<<<1, POOL_THREADS, 0, st>>>(gains, units, take, counts);
  return hipGetLastError();
}

hipError_t launch_layer_budgets(const Geom& g, const int32_t* counts, int queries, int budget,
                                int32_t* out, hipStream_t st) {
  layer_budget_kernel<<<1, 64, 0, st>>>(g, counts, queries, budget, out);
  return hipGetLastError();
}

hipError_t launch_alloc(const Geom& g, const uint16_t* q, const float* chan_var, const float* rot,
                        int budget, uint8_t* depth, float* q_basis, hipStream_t st, int rule,
                        const uint8_t* channels, float* gains, const int32_t* layer_budget) {
  AllocArgs a{g, q, chan_var, rot, budget, depth, q_basis, rule, channels, gains, layer_budget};
  switch (g.G) {
    case 1: launch_g<1>(a, st); break;
    case 2: launch_g<2>(a, st); break;
    case 4: launch_g<4>(a, st); break;
    case 8: launch_g<8>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bpk
