// Combine: restore token order and merge expert outputs with the routing
// weights (ruDNN user guide, "6. Calling MoE"), and the fused variant with
// the shared-expert term, residual Add and RMSNorm
// (aclnnMoeDistributeCombineAddRmsNormV2, "function description", formula;
// ruDNN user guide, "7. LayerNorm, RMSNorm and Softmax" for fp32 statistics
// and F32 gamma).
//
// Both kernels read expert rows through row_of_slot with 16-byte loads; all
// arithmetic is fp32, summed over the k slots in slot order; there are no
// atomics, so results are bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kChunkK = 8;  // expert rows whose loads are issued together

// The fused epilogue touches every byte once: streaming (non-temporal)
// loads and stores.
#define LOAD(v, p) (v).load_nt(p)
#define STORE(v, p) (v).store_nt(p)

// Grid T * ceil(H/8/256) (token-major); each thread produces 8 consecutive
// outputs. The k expert rows are fetched kChunkK at a time, all loads of a
// chunk issued before any is used, then summed in slot order.
template <typename T, typename WT>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y,
                                                       const int32_t* __restrict__ row_of_slot,
                                                       const WT* __restrict__ w, int k, int H,
                                                       int blocks_per_token,
                                                       T* __restrict__ out) {
  const int t = blockIdx.x / blocks_per_token;
  const int v = (blockIdx.x % blocks_per_token) * blockDim.x + threadIdx.x;
  if (v * 8 >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  bool lost = false;
  for (int j0 = 0; j0 < k; j0 += kChunkK) {
    Vec8<T> d[kChunkK];
    float wj[kChunkK];
#pragma unroll
    for (int j = 0; j < kChunkK; ++j) {
      wj[j] = 0.f;
      if (j0 + j < k) {
        const int r = row_of_slot[(int64_t)t * k + j0 + j];
        wj[j] = to_f32(w[(int64_t)t * k + j0 + j]);
        if (r < 0) lost = true;
        else d[j].load(y + (int64_t)r * H + v * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < kChunkK; ++j) {
      if (j0 + j < k && !lost) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[j], d[j].get(i), acc[i]);
      }
    }
  }
  Vec8<T> o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o.set(i, lost ? NAN : acc[i]);
  o.store(out + (int64_t)t * H + v * 8);
}

// As combine_kernel, but expert rows are split-K partial sums: each row is
// summed over the splits in order and rounded to T before it is weighted.
template <typename T, typename WT>
__global__ __launch_bounds__(256) void combine_partials_kernel(
    const float* __restrict__ partial, int splits, int64_t split_stride,
    const int32_t* __restrict__ row_of_slot, const WT* __restrict__ w, int k, int H,
    int blocks_per_token, T* __restrict__ out) {
  const int t = blockIdx.x / blocks_per_token;
  const int v = (blockIdx.x % blocks_per_token) * blockDim.x + threadIdx.x;
  if (v * 8 >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  bool lost = false;
  constexpr int kC = 4;
  for (int j0 = 0; j0 < k; j0 += kC) {
    float4 a0[kC], a1[kC];
    float wj[kC];
    const float* src[kC];
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      wj[j] = 0.f;
      src[j] = nullptr;
      if (j0 + j < k) {
        const int r = row_of_slot[(int64_t)t * k + j0 + j];
        wj[j] = to_f32(w[(int64_t)t * k + j0 + j]);
        if (r < 0) {
          lost = true;
        } else {
          src[j] = partial + (int64_t)r * H + v * 8;
          a0[j] = *reinterpret_cast<const float4*>(src[j]);
          a1[j] = *reinterpret_cast<const float4*>(src[j] + 4);
        }
      }
    }
    for (int sp = 1; sp < splits; ++sp) {
#pragma unroll
      for (int j = 0; j < kC; ++j) {
        if (src[j]) {
          const float4 b0 = *reinterpret_cast<const float4*>(src[j] + sp * split_stride);
          const float4 b1 = *reinterpret_cast<const float4*>(src[j] + sp * split_stride + 4);
          a0[j].x += b0.x; a0[j].y += b0.y; a0[j].z += b0.z; a0[j].w += b0.w;
          a1[j].x += b1.x; a1[j].y += b1.y; a1[j].z += b1.z; a1[j].w += b1.w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      if (src[j]) {
        const float y[8] = {a0[j].x, a0[j].y, a0[j].z, a0[j].w, a1[j].x, a1[j].y, a1[j].z, a1[j].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[j], to_f32(from_f32<T>(y[i])), acc[i]);
      }
    }
  }
  Vec8<T> o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o.set(i, lost ? NAN : acc[i]);
  o.store(out + (int64_t)t * H + v * 8);
}

// One workgroup per token, up to 1024 threads; thread owns VPT groups of 8
// columns strided by the workgroup and keeps x in registers between the sum
// of squares and the scaling. The k expert rows of a group are fetched
// kChunkK at a time with all loads issued before any is used.
template <typename T, typename WT, int VPT>
__global__ __launch_bounds__(1024) void combine_norm_kernel(
    const T* __restrict__ y, const int32_t* __restrict__ row_of_slot, const WT* __restrict__ w,
    const T* __restrict__ shared, const T* __restrict__ residual, const float* __restrict__ gamma,
    float eps, int k, int H, T* __restrict__ y_out, T* __restrict__ x_out,
    float* __restrict__ rstd_out) {
  __shared__ float red[1024 / kWave];
  const int t = blockIdx.x;
  const int nvec = H / 8;
  const int nthreads = blockDim.x;
  float x[VPT][8];
#pragma unroll
  for (int q = 0; q < VPT; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[q][i] = 0.f;

  float wsum = 0.f;
  bool lost = false;
  for (int j0 = 0; j0 < k; j0 += kChunkK) {
    int rows[kChunkK];
    float wj[kChunkK];
#pragma unroll
    for (int j = 0; j < kChunkK; ++j) {
      rows[j] = -1;
      wj[j] = 0.f;
      if (j0 + j < k) {
        rows[j] = row_of_slot[(int64_t)t * k + j0 + j];
        wj[j] = to_f32(w[(int64_t)t * k + j0 + j]);
        wsum += wj[j];
        if (rows[j] < 0) lost = true;
      }
    }
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int v = threadIdx.x + q * nthreads;
      if (v < nvec) {
        Vec8<T> d[kChunkK];
#pragma unroll
        for (int j = 0; j < kChunkK; ++j)
          if (rows[j] >= 0) LOAD(d[j], y + (int64_t)rows[j] * H + v * 8);
#pragma unroll
        for (int j = 0; j < kChunkK; ++j)
          if (rows[j] >= 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[q][i] = fmaf(wj[j], d[j].get(i), x[q][i]);
          }
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < VPT; ++q) {
    const int v = threadIdx.x + q * nthreads;
    if (v < nvec) {
      Vec8<T> rs;
      LOAD(rs, residual + (int64_t)t * H + v * 8);
      Vec8<T> sh;
      if (shared) LOAD(sh, shared + (int64_t)t * H + v * 8);
      Vec8<T> xo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // sum_j w_j * (y_j + s) = sum_j w_j y_j + (sum_j w_j) s
        float xv = x[q][i];
        if (shared) xv = fmaf(wsum, sh.get(i), xv);
        xv = lost ? NAN : xv + rs.get(i);
        x[q][i] = xv;
        ss = fmaf(xv, xv, ss);
        xo.set(i, xv);
      }
      STORE(xo, x_out + (int64_t)t * H + v * 8);
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < nthreads / kWave; ++i) tot += red[i];
  const float rstd = 1.0f / sqrtf(tot / (float)H + eps);
  if (threadIdx.x == 0) rstd_out[t] = rstd;
#pragma unroll
  for (int q = 0; q < VPT; ++q) {
    const int v = threadIdx.x + q * nthreads;
    if (v < nvec) {
      const float4 g0 = *reinterpret_cast<const float4*>(gamma + v * 8);
      const float4 g1 = *reinterpret_cast<const float4*>(gamma + v * 8 + 4);
      const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      Vec8<T> yo;
#pragma unroll
      for (int i = 0; i < 8; ++i) yo.set(i, x[q][i] * rstd * g[i]);
      STORE(yo, y_out + (int64_t)t * H + v * 8);
    }
  }
}

template <typename T, typename WT>
hipError_t combine_t(const void* y, const int32_t* ros, const void* w, int T_, int k, int H,
                     void* out, hipStream_t s) {
  const int bpt = (H / 8 + 255) / 256;
  hipLaunchKernelGGL((combine_kernel<T, WT>), dim3((int64_t)T_ * bpt), dim3(256), 0, s,
                     static_cast<const T*>(y), ros, static_cast<const WT*>(w), k, H, bpt,
                     static_cast<T*>(out));
  return hipGetLastError();
}

template <typename T>
hipError_t combine_w(const void* y, const int32_t* ros, const void* w, int w_dt, int T_, int k,
                     int H, void* out, hipStream_t s) {
  switch (w_dt) {
    case kF32: return combine_t<T, float>(y, ros, w, T_, k, H, out, s);
    case kF16: return combine_t<T, f16>(y, ros, w, T_, k, H, out, s);
    default: return combine_t<T, bf16>(y, ros, w, T_, k, H, out, s);
  }
}

template <typename T, typename WT, int VPT>
hipError_t norm_launch(const void* y, const int32_t* ros, const void* w, const void* sh,
                       const void* res, const float* gamma, float eps, int T_, int k, int H,
                       void* yo, void* xo, float* rstd, hipStream_t s) {
  const int nvec = H / 8;
  int threads = (nvec + VPT - 1) / VPT;
  threads = (threads + kWave - 1) / kWave * kWave;
  hipLaunchKernelGGL((combine_norm_kernel<T, WT, VPT>), dim3(T_), dim3(threads), 0, s,
                     static_cast<const T*>(y), ros, static_cast<const WT*>(w),
                     static_cast<const T*>(sh), static_cast<const T*>(res), gamma, eps, k, H,
                     static_cast<T*>(yo), static_cast<T*>(xo), rstd);
  return hipGetLastError();
}

// Groups of 8 columns per thread: at least two (measured best on the
// DeepSeek-V3-shaped epilogue), more once H/8 exceeds 1024 threads.
#ifndef MOE_NORM_MIN_VPT
#define MOE_NORM_MIN_VPT 2
#endif
template <typename T, typename WT>
hipError_t norm_vpt(const void* y, const int32_t* ros, const void* w, const void* sh,
                    const void* res, const float* gamma, float eps, int T_, int k, int H,
                    void* yo, void* xo, float* rstd, hipStream_t s) {
  int per = (H / 8 + 1023) / 1024;
  if (per < MOE_NORM_MIN_VPT) per = MOE_NORM_MIN_VPT;
  if (per <= 1) return norm_launch<T, WT, 1>(y, ros, w, sh, res, gamma, eps, T_, k, H, yo, xo, rstd, s);
  if (per <= 2) return norm_launch<T, WT, 2>(y, ros, w, sh, res, gamma, eps, T_, k, H, yo, xo, rstd, s);
  if (per <= 4) return norm_launch<T, WT, 4>(y, ros, w, sh, res, gamma, eps, T_, k, H, yo, xo, rstd, s);
  return norm_launch<T, WT, 8>(y, ros, w, sh, res, gamma, eps, T_, k, H, yo, xo, rstd, s);
}

template <typename T>
hipError_t norm_w(const void* y, const int32_t* ros, const void* w, int w_dt, const void* sh,
                  const void* res, const float* gamma, float eps, int T_, int k, int H, void* yo,
                  void* xo, float* rstd, hipStream_t s) {
  switch (w_dt) {
    case kF32: return norm_vpt<T, float>(y, ros, w, sh, res, gamma, eps, T_, k, H, yo, xo, rstd, s);
    case kF16: return norm_vpt<T, f16>(y, ros, w, sh, res, gamma, eps, T_, k, H, yo, xo, rstd, s);
    default: return norm_vpt<T, bf16>(y, ros, w, sh, res, gamma, eps, T_, k, H, yo, xo, rstd, s);
  }
}

template <typename T, typename WT>
hipError_t combine_partials_t(const DownPartials& part, const int32_t* ros, const void* w, int T_,
                              int k, int H, void* out, hipStream_t s) {
  const int bpt = (H / 8 + 255) / 256;
  hipLaunchKernelGGL((combine_partials_kernel<T, WT>), dim3((int64_t)T_ * bpt), dim3(256), 0, s,
                     part.partial, part.splits, part.split_stride, ros, static_cast<const WT*>(w),
                     k, H, bpt, static_cast<T*>(out));
  return hipGetLastError();
}

template <typename T>
hipError_t combine_partials_w(const DownPartials& part, const int32_t* ros, const void* w,
                              int w_dt, int T_, int k, int H, void* out, hipStream_t s) {
  switch (w_dt) {
    case kF32: return combine_partials_t<T, float>(part, ros, w, T_, k, H, out, s);
    case kF16: return combine_partials_t<T, f16>(part, ros, w, T_, k, H, out, s);
    default: return combine_partials_t<T, bf16>(part, ros, w, T_, k, H, out, s);
  }
}

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

hipError_t launch_combine_partials(const DownPartials& part, const int32_t* row_of_slot,
                                   const void* weights, int w_dt, int T, int k, int H, int dt,
                                   void* out, hipStream_t s) {
  if (dt == kF16) return combine_partials_w<f16>(part, row_of_slot, weights, w_dt, T, k, H, out, s);
  return combine_partials_w<bf16>(part, row_of_slot, weights, w_dt, T, k, H, out, s);
}

hipError_t launch_combine(const void* expert_out, const int32_t* row_of_slot, const void* weights,
                          int w_dt, int T, int k, int H, int dt, void* out, hipStream_t s) {
  switch (dt) {
    case kF32: return combine_w<float>(expert_out, row_of_slot, weights, w_dt, T, k, H, out, s);
    case kF16: return combine_w<f16>(expert_out, row_of_slot, weights, w_dt, T, k, H, out, s);
    default: return combine_w<bf16>(expert_out, row_of_slot, weights, w_dt, T, k, H, out, s);
  }
}

hipError_t launch_combine_add_rmsnorm(const void* expert_out, const int32_t* row_of_slot,
                                      const void* weights, int w_dt, const void* shared,
                                      const void* residual, const float* gamma, float eps, int T,
                                      int k, int H, int dt, void* y, void* x_out, float* rstd,
                                      hipStream_t s) {
  switch (dt) {
    case kF32:
      return norm_w<float>(expert_out, row_of_slot, weights, w_dt, shared, residual, gamma, eps, T,
                           k, H, y, x_out, rstd, s);
    case kF16:
      return norm_w<f16>(expert_out, row_of_slot, weights, w_dt, shared, residual, gamma, eps, T,
                         k, H, y, x_out, rstd, s);
    default:
      return norm_w<bf16>(expert_out, row_of_slot, weights, w_dt, shared, residual, gamma, eps, T,
                          k, H, y, x_out, rstd, s);
  }
}

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
