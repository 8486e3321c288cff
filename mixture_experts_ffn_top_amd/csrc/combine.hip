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

// One expert output row as a buffer resource. A dropped slot (row < 0) gets
// an empty range, so its loads read zeros without touching memory and no
// load has to sit behind a branch.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const T* y, int row, int H) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(y + (int64_t)max(row, 0) * H), (short)0,
                                           row >= 0 ? H * (int)sizeof(T) : 0, kBufferFlags);
}

// Adds w_j * y[row_of_slot[s0 + j]] for the C slots s0 .. s0 + C - 1, in slot
// order, to this thread's VPT groups of 8 columns (group q starts at column
// 8 * (v0 + q * vstride); groups past the row read zeros). The C indices and
// weights are read first, then the row loads are issued for QB column groups
// at a time (at most kPieces 16-byte pieces held at once) before any is used.
// wsum gets the weights' sum; lost is set if a slot has no row.
template <int C, int VPT, int kPieces, typename T, typename WT>
__device__ __forceinline__ void add_slots(const T* __restrict__ y,
                                          const int32_t* __restrict__ row_of_slot,
                                          const WT* __restrict__ w, int64_t s0, int H, int v0,
                                          int vstride, float (&x)[VPT][8], float& wsum,
                                          bool& lost) {
  __amdgpu_buffer_rsrc_t r[C];
  float wj[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int row = row_of_slot[s0 + j];
    wj[j] = to_f32(w[s0 + j]);
    wsum += wj[j];
    lost = lost || row < 0;
    r[j] = row_rsrc(y, row, H);
  }
  constexpr int kPer = C * Vec8<T>::kChunks;  // pieces per column group
  constexpr int QB = VPT * kPer <= kPieces ? VPT : (kPieces / kPer > 0 ? kPieces / kPer : 1);
#pragma unroll
  for (int q0 = 0; q0 < VPT; q0 += QB) {
    Vec8<T> d[QB][C];
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int j = 0; j < C; ++j)
        d[q][j].load_nt(r[j], (uint32_t)(v0 + (q0 + q) * vstride) * (uint32_t)sizeof(Vec8<T>));
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[q0 + q][i] = fmaf(wj[j], d[q][j].get(i), x[q0 + q][i]);
  }
}

// All k slots of token t: chunks of kChunkK, then a tail of 4, 2 and 1.
template <int VPT, int kPieces, typename T, typename WT>
__device__ __forceinline__ void add_token_slots(const T* __restrict__ y,
                                                const int32_t* __restrict__ row_of_slot,
                                                const WT* __restrict__ w, int t, int k, int H,
                                                int v0, int vstride, float (&x)[VPT][8],
                                                float& wsum, bool& lost) {
  const int64_t s = (int64_t)t * k;
  int j = 0;
  for (; j + kChunkK <= k; j += kChunkK)
    add_slots<kChunkK, VPT, kPieces>(y, row_of_slot, w, s + j, H, v0, vstride, x, wsum, lost);
  if (k - j >= 4) {
    add_slots<4, VPT, kPieces>(y, row_of_slot, w, s + j, H, v0, vstride, x, wsum, lost);
    j += 4;
  }
  if (k - j >= 2) {
    add_slots<2, VPT, kPieces>(y, row_of_slot, w, s + j, H, v0, vstride, x, wsum, lost);
    j += 2;
  }
  if (k - j >= 1) add_slots<1, VPT, kPieces>(y, row_of_slot, w, s + j, H, v0, vstride, x, wsum, lost);
}

// Grid T * ceil(H/8/256) (token-major); each thread produces 8 consecutive
// outputs, the k expert rows summed in slot order.
template <typename T, typename WT>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y,
                                                       const int32_t* __restrict__ row_of_slot,
                                                       const WT* __restrict__ w, int k, int H,
                                                       int blocks_per_token,
                                                       T* __restrict__ out) {
  const int t = blockIdx.x / blocks_per_token;
  const int v = (blockIdx.x % blocks_per_token) * blockDim.x + threadIdx.x;
  float x[1][8] = {{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
  float wsum = 0.f;
  bool lost = false;
  add_token_slots<1, 16>(y, row_of_slot, w, t, k, H, v, 0, x, wsum, lost);
  if (v * 8 >= H) return;
  Vec8<T> o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o.set(i, lost ? NAN : x[0][i]);
  o.store(out + (int64_t)t * H + v * 8);
}

// One workgroup per token, one thread per VPT groups of 8 columns (strided
// by the workgroup); x stays in registers between the sum of squares and the
// scaling. The expert rows' loads are issued first, at most 16 16-byte
// pieces a thread at a time; the residual and shared rows follow.
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
  add_token_slots<VPT, 16>(y, row_of_slot, w, t, k, H, threadIdx.x, nthreads, x, wsum, lost);
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < VPT; ++q) {
    const int v = threadIdx.x + q * nthreads;
    if (v < nvec) {
      Vec8<T> rs, sh;
      LOAD(rs, residual + (int64_t)t * H + v * 8);
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

// Four groups of 8 columns per thread (H <= 32768: at most 1024 threads).
// On the DeepSeek-V3-shaped epilogue (H 7168) four measured faster than one
// or two per thread, with every token's workgroup resident at once.
constexpr int kNormVpt = 4;
template <typename T, typename WT>
hipError_t norm_vpt(const void* y, const int32_t* ros, const void* w, const void* sh,
                    const void* res, const float* gamma, float eps, int T_, int k, int H,
                    void* yo, void* xo, float* rstd, hipStream_t s) {
  return norm_launch<T, WT, kNormVpt>(y, ros, w, sh, res, gamma, eps, T_, k, H, yo, xo, rstd, s);
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

}  // namespace

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

}  // namespace moe
