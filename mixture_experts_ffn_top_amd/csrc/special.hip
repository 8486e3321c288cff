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

constexpr int kSpecialMaxThreads = 1024;  // one workgroup per token, up to this many threads
#ifndef MOE_SPECIAL_MIN_VPT
#define MOE_SPECIAL_MIN_VPT 2
#endif
constexpr int kSpecialMinVpt = MOE_SPECIAL_MIN_VPT;  // groups of 8 columns per thread, at least

// Per-token sums of the special experts' terms, formed while the slots are
// walked: the token row enters with c_ori = sum of w (copy) and w * alpha1[q]
// (constant q); constant rows V[q] with w * alpha2[q] (has_const marks a
// token with such a slot; they are added in a second, rare pass).
struct SpecialSums {
  float wsum = 0.f;
  float c_ori = 0.f;
  bool lost = false;
  bool has_ori = false;
  bool has_const = false;
  bool ori_in_regs = false;  // the token row was fetched with the first chunk
};

// C consecutive slots j0 .. j0+C-1 of token t, in slot order. A real-expert
// slot adds w * its expert row; each row is a buffer resource, empty for a
// slot that has no row to add, so every load of the chunk is issued
// (unconditionally, QB column groups at a time) before any is used. The
// slot descriptors are the same for the whole workgroup (one token); their
// loads go out in batches with indices clamped into range.
template <int C, int VPT, int kPieces, typename T, typename WT>
__device__ __forceinline__ void special_slots(const SpecialArgs& a, int t, int j0, bool tok_on,
                                              float (&x)[VPT][8], SpecialSums& S,
                                              Vec8<T> (&ov)[VPT]) {
  const int H = a.H;
  const int64_t s0 = (int64_t)t * a.k + j0;
  const T* y = static_cast<const T*>(a.y);
  uint32_t e[C];
  int row[C];
  float wj[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    e[j] = a.indices[s0 + j];
    row[j] = a.row_of_slot[s0 + j];
    wj[j] = to_f32(static_cast<const WT*>(a.w)[s0 + j]);
  }
  bool on[C];
#pragma unroll
  for (int j = 0; j < C; ++j) on[j] = tok_on;
  if (a.mask_dims == 2) {
    uint8_t m[C];
#pragma unroll
    for (int j = 0; j < C; ++j) m[j] = a.active[s0 + j];
#pragma unroll
    for (int j = 0; j < C; ++j) on[j] = m[j] != 0;
  }
  const int64_t dz = a.n_zero, dc = dz + a.n_copy, dq = dc + a.n_const;
  float ca1[C];
#pragma unroll
  for (int j = 0; j < C; ++j) ca1[j] = 0.f;
  if (a.n_const > 0) {
    T v1[C];
#pragma unroll
    for (int j = 0; j < C; ++j)
      v1[j] = static_cast<const T*>(a.alpha1)[min(max((int64_t)e[j] - a.E - dc, (int64_t)0),
                                                   (int64_t)a.n_const - 1)];
#pragma unroll
    for (int j = 0; j < C; ++j) ca1[j] = to_f32(v1[j]);
  }
  __amdgpu_buffer_rsrc_t r[C];
  float W[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int64_t d = (int64_t)e[j] - a.E;  // position among the special experts
    bool expert = false, bad = false;
    if (d < 0) {
      expert = row[j] >= 0;
      bad = !expert;
    } else if (d >= dq) {
      bad = true;
    }
    if (on[j] && bad) S.lost = true;
    const bool use = on[j] && !bad;
    if (use) S.wsum += wj[j];
    if (use && d >= dz && d < dc) {  // copy expert
      S.c_ori += wj[j];
      S.has_ori = true;
    }
    if (use && d >= dc && d < dq) {  // constant expert
      S.c_ori += wj[j] * ca1[j];
      S.has_ori = true;
      S.has_const = true;
    }
    r[j] = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(y + (int64_t)max(row[j], 0) * H), (short)0,
                                             use && expert ? H * (int)sizeof(T) : 0, kBufferFlags);
    W[j] = use && expert ? wj[j] : 0.f;
  }
  // The first chunk also fetches the token row for the copy and constant
  // experts, next to the expert rows (an empty range when no slot so far
  // needs it; a later chunk that does adds it after the walk).
  if (j0 == 0) {
    const bool need = S.has_ori;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(need ? static_cast<const T*>(a.ori_x) + (int64_t)t * H : y), (short)0,
        need ? H * (int)sizeof(T) : 0, kBufferFlags);
#pragma unroll
    for (int q = 0; q < VPT; ++q)
      ov[q].load_nt(ro, (uint32_t)(threadIdx.x + q * blockDim.x) * (uint32_t)sizeof(Vec8<T>));
    S.ori_in_regs = need;
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
        d[q][j].load_nt(r[j], (uint32_t)(threadIdx.x + (q0 + q) * blockDim.x) * (uint32_t)sizeof(Vec8<T>));
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[q0 + q][i] = fmaf(W[j], d[q][j].get(i), x[q0 + q][i]);
  }
}

template <typename T, typename WT, int VPT, bool kNorm>
__global__ __launch_bounds__(kSpecialMaxThreads) void combine_special_kernel(SpecialArgs a) {
  __shared__ float red[kSpecialMaxThreads / kWave];
  const int t = blockIdx.x;
  const int H = a.H, k = a.k, nvec = H / 8;
  const T* sh = static_cast<const T*>(a.shared);
  const T* res = static_cast<const T*>(a.residual);
  float x[VPT][8];
#pragma unroll
  for (int q = 0; q < VPT; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[q][i] = 0.f;
  // The shared and residual rows do not depend on the routing: when the
  // registers allow, their loads go out first.
  constexpr bool kEarly = VPT * Vec8<T>::kChunks <= 2;
  Vec8<T> shv[VPT], rsv[VPT];
  auto load_sr = [&](int q) {
    const int v = threadIdx.x + q * (int)blockDim.x;
    if (v < nvec) {
      if (sh) shv[q].load_nt(sh + (int64_t)t * H + v * 8);
      if (kNorm) rsv[q].load_nt(res + (int64_t)t * H + v * 8);
    }
  };
  if (kEarly) {
#pragma unroll
    for (int q = 0; q < VPT; ++q) load_sr(q);
  }
  SpecialSums S;
  Vec8<T> ov[VPT];
  const bool tok_on = a.mask_dims != 1 || a.active[t] != 0;
  constexpr int kPieces = VPT * Vec8<T>::kChunks <= 2 ? 16 : 8;
  // real-expert rows, slots in order: chunks of 8, then a tail of 4, 2 and 1
  int j = 0;
  for (; j + 8 <= k; j += 8) special_slots<8, VPT, kPieces, T, WT>(a, t, j, tok_on, x, S, ov);
  if (k - j >= 4) {
    special_slots<4, VPT, kPieces, T, WT>(a, t, j, tok_on, x, S, ov);
    j += 4;
  }
  if (k - j >= 2) {
    special_slots<2, VPT, kPieces, T, WT>(a, t, j, tok_on, x, S, ov);
    j += 2;
  }
  if (k - j >= 1) special_slots<1, VPT, kPieces, T, WT>(a, t, j, tok_on, x, S, ov);
  // the token row of the copy and constant experts, once
  if (S.has_ori) {
    if (!S.ori_in_regs) {
      const T* ori = static_cast<const T*>(a.ori_x) + (int64_t)t * H;
#pragma unroll
      for (int q = 0; q < VPT; ++q) {
        const int v = threadIdx.x + q * (int)blockDim.x;
        if (v < nvec) ov[q].load(ori + v * 8);
      }
    }
#pragma unroll
    for (int q = 0; q < VPT; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[q][i] = fmaf(S.c_ori, ov[q].get(i), x[q][i]);
  }
  // the constant experts' rows V[q], slot by slot (tokens routed to them are few)
  if (S.has_const) {
    const int64_t dc = (int64_t)a.n_zero + a.n_copy;
    for (int js = 0; js < k; ++js) {
      const int64_t sl = (int64_t)t * k + js;
      const int64_t q = (int64_t)a.indices[sl] - a.E - dc;
      const bool on = a.mask_dims == 2 ? a.active[sl] != 0 : tok_on;
      if (!on || q < 0 || q >= a.n_const) continue;
      const float c = to_f32(static_cast<const WT*>(a.w)[sl]) *
                      to_f32(static_cast<const T*>(a.alpha2)[q]);
      const T* vrow = static_cast<const T*>(a.v) + q * H;
#pragma unroll
      for (int qq = 0; qq < VPT; ++qq) {
        const int v = threadIdx.x + qq * (int)blockDim.x;
        if (v < nvec) {
          Vec8<T> cv;
          cv.load(vrow + v * 8);
#pragma unroll
          for (int i = 0; i < 8; ++i) x[qq][i] = fmaf(c, cv.get(i), x[qq][i]);
        }
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int qv = 0; qv < VPT; ++qv) {
    const int v = threadIdx.x + qv * (int)blockDim.x;
    if (v < nvec) {
      if (!kEarly) load_sr(qv);
      Vec8<T> o;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // sum over active slots of w (m + s) = sum w m + (sum w) s
        float xv = x[qv][i];
        if (sh) xv = fmaf(S.wsum, shv[qv].get(i), xv);
        if (kNorm) xv = xv + rsv[qv].get(i);
        if (S.lost) xv = NAN;
        x[qv][i] = xv;
        ss = fmaf(xv, xv, ss);
        o.set(i, xv);
      }
      o.store_nt(static_cast<T*>(kNorm ? a.x_out : a.out) + (int64_t)t * H + v * 8);
    }
  }
  if constexpr (kNorm) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ss += __shfl_xor(ss, d, kWave);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < (int)blockDim.x / kWave; ++i) tot += red[i];
    const float rstd = 1.0f / sqrtf(tot / (float)H + a.eps);
    if (threadIdx.x == 0) a.rstd[t] = rstd;
#pragma unroll
    for (int qv = 0; qv < VPT; ++qv) {
      const int v = threadIdx.x + qv * (int)blockDim.x;
      if (v < nvec) {
        const float4 g0 = *reinterpret_cast<const float4*>(a.gamma + v * 8);
        const float4 g1 = *reinterpret_cast<const float4*>(a.gamma + v * 8 + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        Vec8<T> yo;
#pragma unroll
        for (int i = 0; i < 8; ++i) yo.set(i, x[qv][i] * rstd * g[i]);
        yo.store_nt(static_cast<T*>(a.out) + (int64_t)t * H + v * 8);
      }
    }
  }
}

template <typename T, typename WT, bool kNorm>
hipError_t special_vpt(const SpecialArgs& a, int T_, hipStream_t s) {
  // Groups of 8 columns per thread: as few as the 1024-thread limit allows,
  // so a chunk's row loads go out in one batch. H <= 32768 (checked by the
  // entry points) gives at most 4.
  const int nvec = a.H / 8;
  int per = (nvec + kSpecialMaxThreads - 1) / kSpecialMaxThreads;
  if (per > 4) return hipErrorInvalidValue;
  if (per < kSpecialMinVpt) per = kSpecialMinVpt;
  const int vpt = per <= 1 ? 1 : per <= 2 ? 2 : 4;
  const int threads = ((nvec + vpt - 1) / vpt + kWave - 1) / kWave * kWave;
  const dim3 grid(T_), block(threads);
  if (vpt == 1) hipLaunchKernelGGL((combine_special_kernel<T, WT, 1, kNorm>), grid, block, 0, s, a);
  else if (vpt == 2) hipLaunchKernelGGL((combine_special_kernel<T, WT, 2, kNorm>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((combine_special_kernel<T, WT, 4, kNorm>), grid, block, 0, s, a);
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
