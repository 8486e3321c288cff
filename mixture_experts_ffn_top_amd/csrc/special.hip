// Combine with special experts (zero / copy / constant) and an activity mask
// (aclnnMoeDistributeCombineAddRmsNormV2, "function description": the
// special-expert formulas, and the parameters zeroExpertNum, copyExpertNum,
// constExpertNum, oriXOptional, constExpert*Optional and
// xActiveMaskOptional), with the optional residual Add + RMSNorm.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Combine with special experts and an activity mask
// (aclnnMoeDistributeCombineAddRmsNormV2: zeroExpertNum, copyExpertNum,
// constExpertNum with oriXOptional / constExpertAlpha1Optional /
// constExpertAlpha2Optional / constExpertVOptional, and xActiveMaskOptional).
// Slot (t, j) with expert id e contributes w[t,j] * (m + shared[t]) where m is
//   e < E                       the dispatched expert row,
//   E <= e < E+nz               0 (zero expert),
//   next nc ids                 ori_x[t] (copy expert),
//   next nq ids (const q)       alpha1[q] * ori_x[t] + alpha2[q] * V[q];
// a larger id, or a real-expert slot that was not dispatched, makes the row
// NaN. Slots switched off by the mask contribute nothing (a token with every
// slot off combines to 0). All arithmetic fp32; with kNorm the residual Add
// and RMSNorm follow as in combine_norm_kernel.
struct SpecialArgs {
  const void* y;
  const int32_t* row_of_slot;
  const uint32_t* indices;
  const void* w;
  int k, H, E, n_zero, n_copy, n_const;
  const void* ori_x;
  const void* alpha1;
  const void* alpha2;
  const void* v;
  const uint8_t* active;
  int mask_dims;
  const void* shared;
  const void* residual;
  const float* gamma;
  float eps;
  void* out;  // combined rows, or y of the RMSNorm
  void* x_out;
  float* rstd;
};

constexpr int kSpecialThreads = 256;

template <typename T, typename WT, int VPT, bool kNorm>
__global__ __launch_bounds__(kSpecialThreads) void combine_special_kernel(SpecialArgs a) {
  __shared__ float red[kSpecialThreads / kWave];
  const int t = blockIdx.x;
  const int H = a.H, k = a.k, nvec = H / 8;
  const T* y = static_cast<const T*>(a.y);
  const T* ori = static_cast<const T*>(a.ori_x);
  const T* vv = static_cast<const T*>(a.v);
  float x[VPT][8];
#pragma unroll
  for (int q = 0; q < VPT; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[q][i] = 0.f;
  float wsum = 0.f;
  bool lost = false;
  for (int j = 0; j < k; ++j) {  // same (t, j) for the whole block: uniform branches
    const int64_t sl = (int64_t)t * k + j;
    if (a.mask_dims == 1 && !a.active[t]) continue;
    if (a.mask_dims == 2 && !a.active[sl]) continue;
    const uint32_t e = a.indices[sl];
    const float wj = to_f32(static_cast<const WT*>(a.w)[sl]);
    int kind = -1, row = -1, q = 0;
    float a1 = 0.f, a2 = 0.f;
    const int64_t d = (int64_t)e - a.E;  // position among the special experts
    if (d < 0) {
      row = a.row_of_slot[sl];
      kind = row >= 0 ? 0 : -1;
    } else if (d < a.n_zero) {
      kind = 1;
    } else if (d < (int64_t)a.n_zero + a.n_copy) {
      kind = 2;
    } else if (d < (int64_t)a.n_zero + a.n_copy + a.n_const) {
      kind = 3;
      q = (int)(d - a.n_zero - a.n_copy);
      a1 = to_f32(static_cast<const T*>(a.alpha1)[q]);
      a2 = to_f32(static_cast<const T*>(a.alpha2)[q]);
    }
    if (kind < 0) {
      lost = true;
      continue;
    }
    wsum += wj;
    if (kind == 1) continue;
#pragma unroll
    for (int qv = 0; qv < VPT; ++qv) {
      const int v = threadIdx.x + qv * kSpecialThreads;
      if (v < nvec) {
        float m[8];
        if (kind == 0) {
          Vec8<T> r;
          r.load(y + (int64_t)row * H + v * 8);
#pragma unroll
          for (int i = 0; i < 8; ++i) m[i] = r.get(i);
        } else {
          Vec8<T> o;
          o.load(ori + (int64_t)t * H + v * 8);
#pragma unroll
          for (int i = 0; i < 8; ++i) m[i] = o.get(i);
          if (kind == 3) {
            Vec8<T> c;
            c.load(vv + (int64_t)q * H + v * 8);
#pragma unroll
            for (int i = 0; i < 8; ++i) m[i] = fmaf(a1, m[i], a2 * c.get(i));
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) x[qv][i] = fmaf(wj, m[i], x[qv][i]);
      }
    }
  }
  const T* sh = static_cast<const T*>(a.shared);
  const T* res = static_cast<const T*>(a.residual);
  float ss = 0.f;
#pragma unroll
  for (int qv = 0; qv < VPT; ++qv) {
    const int v = threadIdx.x + qv * kSpecialThreads;
    if (v < nvec) {
      Vec8<T> shv, rsv, o;
      if (sh) shv.load(sh + (int64_t)t * H + v * 8);
      if (kNorm) rsv.load(res + (int64_t)t * H + v * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // sum over active slots of w (m + s) = sum w m + (sum w) s
        float xv = x[qv][i];
        if (sh) xv = fmaf(wsum, shv.get(i), xv);
        if (kNorm) xv = xv + rsv.get(i);
        if (lost) xv = NAN;
        x[qv][i] = xv;
        ss = fmaf(xv, xv, ss);
        o.set(i, xv);
      }
      o.store(static_cast<T*>(kNorm ? a.x_out : a.out) + (int64_t)t * H + v * 8);
    }
  }
  if constexpr (kNorm) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, kWave);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < kSpecialThreads / kWave; ++i) tot += red[i];
    const float rstd = 1.0f / sqrtf(tot / (float)H + a.eps);
    if (threadIdx.x == 0) a.rstd[t] = rstd;
#pragma unroll
    for (int qv = 0; qv < VPT; ++qv) {
      const int v = threadIdx.x + qv * kSpecialThreads;
      if (v < nvec) {
        const float4 g0 = *reinterpret_cast<const float4*>(a.gamma + v * 8);
        const float4 g1 = *reinterpret_cast<const float4*>(a.gamma + v * 8 + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        Vec8<T> yo;
#pragma unroll
        for (int i = 0; i < 8; ++i) yo.set(i, x[qv][i] * rstd * g[i]);
        yo.store(static_cast<T*>(a.out) + (int64_t)t * H + v * 8);
      }
    }
  }
}

template <typename T, typename WT, bool kNorm>
hipError_t special_vpt(const SpecialArgs& a, int T_, hipStream_t s) {
  const int per = (a.H / 8 + kSpecialThreads - 1) / kSpecialThreads;
  const dim3 grid(T_), block(kSpecialThreads);
  if (per <= 1) hipLaunchKernelGGL((combine_special_kernel<T, WT, 1, kNorm>), grid, block, 0, s, a);
  else if (per <= 2) hipLaunchKernelGGL((combine_special_kernel<T, WT, 2, kNorm>), grid, block, 0, s, a);
  else if (per <= 4) hipLaunchKernelGGL((combine_special_kernel<T, WT, 4, kNorm>), grid, block, 0, s, a);
  else if (per <= 8) hipLaunchKernelGGL((combine_special_kernel<T, WT, 8, kNorm>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((combine_special_kernel<T, WT, 16, kNorm>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename T, bool kNorm>
hipError_t special_w(const SpecialArgs& a, int w_dt, int T_, hipStream_t s) {
  switch (w_dt) {
    case kF32: return special_vpt<T, float, kNorm>(a, T_, s);
    case kF16: return special_vpt<T, f16, kNorm>(a, T_, s);
    default: return special_vpt<T, bf16, kNorm>(a, T_, s);
  }
}

template <bool kNorm>
hipError_t special_dt(const SpecialArgs& a, int w_dt, int dt, int T_, hipStream_t s) {
  switch (dt) {
    case kF32: return special_w<float, kNorm>(a, w_dt, T_, s);
    case kF16: return special_w<f16, kNorm>(a, w_dt, T_, s);
    default: return special_w<bf16, kNorm>(a, w_dt, T_, s);
  }
}

}  // namespace

hipError_t launch_combine_special(const SpecialCombine& c, int T, hipStream_t s) {
  if (T == 0) return hipSuccess;
  SpecialArgs a;
  a.y = c.expert_out; a.row_of_slot = c.row_of_slot; a.indices = c.indices; a.w = c.weights;
  a.k = c.k; a.H = c.H; a.E = c.E; a.n_zero = c.n_zero; a.n_copy = c.n_copy; a.n_const = c.n_const;
  a.ori_x = c.ori_x; a.alpha1 = c.alpha1; a.alpha2 = c.alpha2; a.v = c.const_v;
  a.active = c.active; a.mask_dims = c.active ? c.mask_dims : 0;
  a.shared = c.shared; a.residual = c.residual; a.gamma = c.gamma; a.eps = c.eps;
  a.out = c.out; a.x_out = c.x_out; a.rstd = c.rstd;
  return c.residual ? special_dt<true>(a, c.w_dt, c.dt, T, s) : special_dt<false>(a, c.w_dt, c.dt, T, s);
}

}  // namespace moe
