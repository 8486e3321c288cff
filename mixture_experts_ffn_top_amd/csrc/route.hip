// Routing: fp32 softmax over all experts, then top-k (ruDNN user guide,
// "4. Routing contract").
//
// One token per group of G lanes of a wavefront (G = E rounded up to a power
// of two when E <= 64, else G = 64 with VPL experts per lane). Softmax
// statistics and the k selection rounds are group reductions over
// cross-lane shuffles; nothing touches LDS.
//
// Selection key: for a finite row every probability p is in [0, 1], so its
// fp32 bit pattern orders like the value. key = (bits(p) << 32) | ~id makes
// "larger key" mean "larger p, then lower id", the contract's order, and a
// 64-bit max-reduction selects the next expert. Taken or padding entries get
// key 0, below every real key (~id > 0 for id < 2^32 - 1).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// Reductions over an aligned group of G lanes (G a power of two <= 64) that
// leave every lane of the group with the result, without LDS. Each step pairs
// a lane with one lane of the other half of its aligned block of twice the
// span: DPP quad permutes for spans 1 and 2 (lane ^ 1, lane ^ 2), then the
// half-row mirror (i <-> 7 - i) and the row mirror (i <-> 15 - i). Rows of 16
// lanes are combined through readlane. Partners always lie in the lane's own
// group, so a group switched off as a whole does not disturb the others.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ uint32_t xlane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ float xlane(float v) {
  return __uint_as_float(xlane<kCtrl>(__float_as_uint(v)));
}
template <int kCtrl>
__device__ __forceinline__ uint64_t xlane(uint64_t v) {
  return ((uint64_t)xlane<kCtrl>((uint32_t)(v >> 32)) << 32) | xlane<kCtrl>((uint32_t)v);
}
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __uint_as_float(lane_value(__float_as_uint(v), l));
}
__device__ __forceinline__ uint64_t lane_value(uint64_t v, int l) {
  return ((uint64_t)lane_value((uint32_t)(v >> 32), l) << 32) | lane_value((uint32_t)v, l);
}

template <int G, typename V, typename Op>
__device__ __forceinline__ V group_reduce(V v, Op op) {
  if constexpr (G >= 2) v = op(v, xlane<kDppXor1>(v));
  if constexpr (G >= 4) v = op(v, xlane<kDppXor2>(v));
  if constexpr (G >= 8) v = op(v, xlane<kDppRowHalfMirror>(v));
  if constexpr (G >= 16) v = op(v, xlane<kDppRowMirror>(v));
  if constexpr (G >= 32) {
    const V lo = op(lane_value(v, 0), lane_value(v, 16));
    const V hi = op(lane_value(v, 32), lane_value(v, 48));
    if constexpr (G == 64) v = op(lo, hi);
    else v = __lane_id() < 32 ? lo : hi;
  }
  return v;
}

template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  return group_reduce<G>(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}
template <int G>
__device__ __forceinline__ float group_max_f32(float v) {
  return group_reduce<G>(v, [](float a, float b) { return fmaxf(a, b); });
}
template <int G>
__device__ __forceinline__ float group_sum_f32(float v) {
  return group_reduce<G>(v, [](float a, float b) { return a + b; });
}
template <int G>
__device__ __forceinline__ int group_or(int v) {
  return (int)group_reduce<G>((uint32_t)v, [](uint32_t a, uint32_t b) { return a | b; });
}

constexpr int kRouteThreads = 256;

template <typename LT, int G, int VPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const LT* __restrict__ logits, int T, int E, int k, int renorm,
    uint32_t* __restrict__ indices, LT* __restrict__ weights) {
  constexpr int kGroupsPerBlock = kRouteThreads / G;
  const int gl = threadIdx.x % G;
  const int t = blockIdx.x * kGroupsPerBlock + threadIdx.x / G;
  const bool active = t < T;  // whole groups share t, so shuffles stay consistent

  float z[VPL];
  int flags = 0;  // bit0: NaN seen, bit1: +inf seen, bit2: a value other than -inf seen
  // Every load is issued (indices clamped into the row), then masked.
  const int64_t row = (int64_t)min(t, T - 1) * E;
#pragma unroll
  for (int v = 0; v < VPL; ++v) z[v] = to_f32(logits[row + min(gl + G * v, E - 1)]);
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    if (!active || gl + G * v >= E) z[v] = -INFINITY;
    if (__builtin_isnan(z[v])) flags |= 1;
    if (z[v] == INFINITY) flags |= 2;
    if (z[v] != -INFINITY) flags |= 4;
  }
  flags = group_or<G>(flags);
  const bool bad = (flags & 3) || !(flags & 4);

  // fp32 softmax statistics over all E experts.
  float m = -INFINITY;
#pragma unroll
  for (int v = 0; v < VPL; ++v) m = fmaxf(m, z[v]);
  m = group_max_f32<G>(m);
  float a[VPL];
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    a[v] = (gl + G * v < E && !bad) ? expf(z[v] - m) : 0.f;
    s += a[v];
  }
  s = group_sum_f32<G>(s);

  uint64_t key[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const uint32_t e = (uint32_t)(gl + G * v);
    const float p = a[v] / s;
    key[v] = (e < (uint32_t)E && !bad) ? (((uint64_t)__float_as_uint(p) << 32) | (uint32_t)~e) : 0ull;
  }

  // k selection rounds; round r's winner is kept by lane r % G in slot r / G.
  float mine_p[VPL];
  uint32_t mine_e[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) { mine_p[v] = 0.f; mine_e[v] = 0u; }
  float sel_sum = 0.f;
  if (!bad) {
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int v = 0; v < VPL; ++v) best = key[v] > best ? key[v] : best;
      best = group_max_u64<G>(best);
      const uint32_t eb = ~(uint32_t)best;
      const float pb = __uint_as_float((uint32_t)(best >> 32));
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if ((uint32_t)(gl + G * v) == eb) key[v] = 0ull;
      if (r % G == gl) {
        const int slot = r / G;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (v == slot) { mine_p[v] = pb; mine_e[v] = eb; }
      }
      sel_sum += pb;  // same order in every lane of the group
    }
  } else {
    // NaN row: all probabilities are NaN and tie, so ids 0..k-1 in order.
#pragma unroll
    for (int v = 0; v < VPL; ++v) { mine_p[v] = NAN; mine_e[v] = (uint32_t)(gl + G * v); }
  }

  if (!active) return;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int r = gl + G * v;
    if (r < k) {
      float wv = mine_p[v];
      if (renorm && !bad) wv = wv / sel_sum;
      indices[(int64_t)t * k + r] = mine_e[v];
      weights[(int64_t)t * k + r] = from_f32<LT>(wv);
    }
  }
}

template <typename LT, int G, int VPL>
hipError_t launch(const void* logits, int T, int E, int k, int renorm, uint32_t* idx, void* w,
                  hipStream_t s) {
  constexpr int kGroupsPerBlock = kRouteThreads / G;
  const int blocks = (T + kGroupsPerBlock - 1) / kGroupsPerBlock;
  hipLaunchKernelGGL((route_kernel<LT, G, VPL>), dim3(blocks), dim3(kRouteThreads), 0, s,
                     static_cast<const LT*>(logits), T, E, k, renorm, idx, static_cast<LT*>(w));
  return hipGetLastError();
}

template <typename LT>
hipError_t dispatch_shape(const void* logits, int T, int E, int k, int renorm, uint32_t* idx,
                          void* w, hipStream_t s) {
  if (E <= 1) return launch<LT, 1, 1>(logits, T, E, k, renorm, idx, w, s);
  if (E <= 2) return launch<LT, 2, 1>(logits, T, E, k, renorm, idx, w, s);
  if (E <= 4) return launch<LT, 4, 1>(logits, T, E, k, renorm, idx, w, s);
  if (E <= 8) return launch<LT, 8, 1>(logits, T, E, k, renorm, idx, w, s);
  if (E <= 16) return launch<LT, 16, 1>(logits, T, E, k, renorm, idx, w, s);
  if (E <= 32) return launch<LT, 32, 1>(logits, T, E, k, renorm, idx, w, s);
  if (E <= 64) return launch<LT, 64, 1>(logits, T, E, k, renorm, idx, w, s);
  if (E <= 128) return launch<LT, 64, 2>(logits, T, E, k, renorm, idx, w, s);
  if (E <= 256) return launch<LT, 64, 4>(logits, T, E, k, renorm, idx, w, s);
  if (E <= 512) return launch<LT, 64, 8>(logits, T, E, k, renorm, idx, w, s);
  return launch<LT, 64, 16>(logits, T, E, k, renorm, idx, w, s);
}

// ---------------------------------------------------------------------------
// Grouped-limited sigmoid routing (ruDNN user guide, "10. Grouped-limited
// sigmoid MoE routing"): s = sigmoid(z) in fp32, corrected score c = s + bias
// (selection only), experts in `groups` equal contiguous groups, each scored
// by the sum of its two largest c (or its largest c); the `selected_groups`
// best groups are kept (ties: lower group), then the k largest c among their
// experts (ties: lower id). Weights: the raw s, divided by their sum when
// renormalising, times scale.
//
// One token per wavefront, kGroupedWaves tokens per block. Corrected and raw
// scores go to LDS; group scores are reduced by 64 / P lanes per group
// (P = groups rounded up to a power of two, at most 64; more than 64 groups
// take two passes), then each group counts the groups ranked above it. The
// k rounds of selection are 64-bit max-reductions over
// (order-preserving bits of c) << 32 | ~id; experts of dropped groups and
// padding get key 0, below every real key. A row whose corrected scores
// contain a NaN selects ids 0..k-1 with NaN weights.
constexpr int kGroupedWaves = 4;
constexpr int kMaxGroups = 128;

// Monotone map of an fp32 (not NaN) to uint32: a < b  <=>  ord(a) < ord(b).
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void top2_push(float x, float& m1, float& m2) {
  if (x > m1) { m2 = m1; m1 = x; }
  else if (x > m2) { m2 = x; }
}

template <typename LT, int VPL>
__global__ __launch_bounds__(64 * kGroupedWaves) void route_grouped_kernel(
    const LT* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k, int groups,
    int sel_groups, int top_two, int renorm, float scale, uint32_t* __restrict__ indices,
    LT* __restrict__ weights) {
  __shared__ float s_c[kGroupedWaves][kMaxExperts];
  __shared__ float s_s[kGroupedWaves][kMaxExperts];
  __shared__ float s_g[kGroupedWaves][kMaxGroups];
  __shared__ int s_kept[kGroupedWaves][kMaxGroups];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * kGroupedWaves + wv;
  const bool active = t < T;  // whole wavefronts share t
  const int gs = E / groups;

  float c_reg[VPL];
  int nan_seen = 0;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane + 64 * v;
    c_reg[v] = 0.f;
    if (active && e < E) {
      const float z = to_f32(logits[(int64_t)t * E + e]);
      const float sg = 1.0f / (1.0f + expf(-z));
      const float c = sg + (bias ? bias[e] : 0.0f) + 0.0f;  // + 0: -0 -> +0
      if (__builtin_isnan(c)) nan_seen = 1;
      s_s[wv][e] = sg;
      s_c[wv][e] = c;
      c_reg[v] = c;
    }
  }
  const bool bad = __any(nan_seen);
  __syncthreads();

  // Group scores: P = groups rounded up to a power of two (<= 64), 64 / P
  // lanes per group, each scanning a strided share of the group.
  int P = 1;
  while (P < groups && P < 64) P <<= 1;
  const int lpg = 64 / P;
  const int sub = lane % lpg;
  for (int pass = 0; pass * P < groups; ++pass) {
    const int g = lane / lpg + pass * P;
    float m1 = -INFINITY, m2 = -INFINITY;
    if (active && g < groups)
      for (int e = g * gs + sub; e < (g + 1) * gs; e += lpg) top2_push(s_c[wv][e], m1, m2);
    for (int d = 1; d < lpg; d <<= 1) {
      const float o1 = __shfl_xor(m1, d, 64);
      const float o2 = __shfl_xor(m2, d, 64);
      const float hi = fmaxf(m1, o1), lo = fminf(m1, o1);
      m2 = fmaxf(lo, fmaxf(m2, o2));
      m1 = hi;
    }
    if (active && g < groups && sub == 0) s_g[wv][g] = top_two ? m1 + m2 : m1;
  }
  __syncthreads();

  // Rank of each group: groups with a larger score, or an equal score and a
  // lower index, come first; the first sel_groups are kept.
  for (int g = lane; g < groups; g += 64) {
    if (!active) break;
    const float sc = s_g[wv][g];
    int rank = 0;
    for (int g2 = 0; g2 < groups; ++g2) {
      const float o = s_g[wv][g2];
      rank += (o > sc) || (o == sc && g2 < g);
    }
    s_kept[wv][g] = rank < sel_groups;
  }
  __syncthreads();
  if (!active) return;

  uint64_t key[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const uint32_t e = (uint32_t)(lane + 64 * v);
    key[v] = (e < (uint32_t)E && !bad && s_kept[wv][e / gs])
                 ? (((uint64_t)ordered_bits(c_reg[v]) << 32) | (uint32_t)~e)
                 : 0ull;
  }
  uint32_t mine_e = (uint32_t)lane;
  float mine_s = NAN;
  float sel_sum = 0.f;
  if (!bad) {
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int v = 0; v < VPL; ++v) best = key[v] > best ? key[v] : best;
      best = group_max_u64<64>(best);
      // best == 0 cannot happen for validated arguments (k <= kept experts);
      // the clamp keeps the LDS read in bounds regardless.
      const uint32_t eb = best ? ~(uint32_t)best : 0u;
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if ((uint32_t)(lane + 64 * v) == eb) key[v] = 0ull;
      const float sb = s_s[wv][eb];
      if (lane == r) { mine_e = eb; mine_s = sb; }
      sel_sum += sb;  // same order in every lane
    }
  }
  if (lane < k) {
    float wv_out = mine_s;
    if (!bad) {
      if (renorm) wv_out = wv_out / sel_sum;
      wv_out = wv_out * scale;
    }
    indices[(int64_t)t * k + lane] = mine_e;
    weights[(int64_t)t * k + lane] = from_f32<LT>(wv_out);
  }
}

template <typename LT, int VPL>
hipError_t launch_grouped(const void* logits, const float* bias, int T, int E, int k, int groups,
                          int sel_groups, int top_two, int renorm, float scale, uint32_t* idx,
                          void* w, hipStream_t s) {
  const int blocks = (T + kGroupedWaves - 1) / kGroupedWaves;
  hipLaunchKernelGGL((route_grouped_kernel<LT, VPL>), dim3(blocks), dim3(64 * kGroupedWaves), 0, s,
                     static_cast<const LT*>(logits), bias, T, E, k, groups, sel_groups, top_two,
                     renorm, scale, idx, static_cast<LT*>(w));
  return hipGetLastError();
}

template <typename LT>
hipError_t grouped_shape(const void* logits, const float* bias, int T, int E, int k, int groups,
                         int sel_groups, int top_two, int renorm, float scale, uint32_t* idx,
                         void* w, hipStream_t s) {
  if (E <= 64) return launch_grouped<LT, 1>(logits, bias, T, E, k, groups, sel_groups, top_two, renorm, scale, idx, w, s);
  if (E <= 128) return launch_grouped<LT, 2>(logits, bias, T, E, k, groups, sel_groups, top_two, renorm, scale, idx, w, s);
  if (E <= 256) return launch_grouped<LT, 4>(logits, bias, T, E, k, groups, sel_groups, top_two, renorm, scale, idx, w, s);
  if (E <= 512) return launch_grouped<LT, 8>(logits, bias, T, E, k, groups, sel_groups, top_two, renorm, scale, idx, w, s);
  return launch_grouped<LT, 16>(logits, bias, T, E, k, groups, sel_groups, top_two, renorm, scale, idx, w, s);
}

}  // namespace

hipError_t launch_route(const void* logits, int logits_dt, int T, int E, int k, int renorm,
                        uint32_t* indices, void* weights, hipStream_t s) {
  switch (logits_dt) {
    case kF32: return dispatch_shape<float>(logits, T, E, k, renorm, indices, weights, s);
    case kF16: return dispatch_shape<f16>(logits, T, E, k, renorm, indices, weights, s);
    default: return dispatch_shape<bf16>(logits, T, E, k, renorm, indices, weights, s);
  }
}

hipError_t launch_route_grouped(const void* logits, int logits_dt, const float* bias, int T, int E,
                                int k, int groups, int sel_groups, int top_two, int renorm,
                                float scale, uint32_t* indices, void* weights, hipStream_t s) {
  if (T == 0) return hipSuccess;
  switch (logits_dt) {
    case kF32: return grouped_shape<float>(logits, bias, T, E, k, groups, sel_groups, top_two, renorm, scale, indices, weights, s);
    case kF16: return grouped_shape<f16>(logits, bias, T, E, k, groups, sel_groups, top_two, renorm, scale, indices, weights, s);
    default: return grouped_shape<bf16>(logits, bias, T, E, k, groups, sel_groups, top_two, renorm, scale, indices, weights, s);
  }
}

}  // namespace moe
