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

template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
#pragma unroll
  for (int d = 1; d < G; d <<= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, d, G);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, G);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

template <int G>
__device__ __forceinline__ float group_max_f32(float v) {
#pragma unroll
  for (int d = 1; d < G; d <<= 1) v = fmaxf(v, __shfl_xor(v, d, G));
  return v;
}

template <int G>
__device__ __forceinline__ float group_sum_f32(float v) {
#pragma unroll
  for (int d = 1; d < G; d <<= 1) v += __shfl_xor(v, d, G);
  return v;
}

template <int G>
__device__ __forceinline__ int group_or(int v) {
#pragma unroll
  for (int d = 1; d < G; d <<= 1) v |= __shfl_xor(v, d, G);
  return v;
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
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = gl + G * v;
    z[v] = -INFINITY;
    if (active && e < E) {
      z[v] = to_f32(logits[(int64_t)t * E + e]);
      if (__builtin_isnan(z[v])) flags |= 1;
      if (z[v] == INFINITY) flags |= 2;
      if (z[v] != -INFINITY) flags |= 4;
    }
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

}  // namespace

hipError_t launch_route(const void* logits, int logits_dt, int T, int E, int k, int renorm,
                        uint32_t* indices, void* weights, hipStream_t s) {
  switch (logits_dt) {
    case kF32: return dispatch_shape<float>(logits, T, E, k, renorm, indices, weights, s);
    case kF16: return dispatch_shape<f16>(logits, T, E, k, renorm, indices, weights, s);
    default: return dispatch_shape<bf16>(logits, T, E, k, renorm, indices, weights, s);
  }
}

}  // namespace moe
