// Weight-only quantised experts on the decode path (aclnnFFN, formula of the
// pseudo-quantization scenario: each weight matrix W, stored as INT8 or
// INT4, enters the product as (W + antiquantOffset) * antiquantScale, with
// one scale/offset per output channel, or, for INT4, per group of
// consecutive input channels).
//
// Layouts (K = input channels, contiguous like the bf16 weights):
//   INT8  [E, N, K] int8;  INT4 [E, N, K/2] bytes, element k in byte k/2,
//   low nibble first, two's complement (-8..7);
//   scale, offset [E, N, G] in the model dtype, G groups of K/G consecutive
//   input channels (G = 1: per channel; K/G a multiple of 128, so a
//   K-iteration (128 channels) never straddles two groups); offset may be
//   absent (0).
//
// The formula is computed as written, without rounding the dequantised
// weights: for output channel n and group g,
//   sum_k x_k (q_k + o) s = s (sum_k x_k c_k) + s (o - C) (sum_k x_k)
// where c_k = q_k + C is the code shifted by a constant C so that it is an
// exact small integer in the model dtype that a few bit operations build
// (INT4: 128 + the unsigned nibble; INT8: the unsigned byte, converted).
// The MFMA contracts the activations with the codes (exact products, fp32
// accumulation), a second MFMA against ones gives sum_k x_k, and the scale
// and offset are applied to those fp32 sums once per group.
//
// One workgroup of 4 wavefronts per (expert, block of 64 weight rows), K
// split four ways and reduced in LDS, MFMA 16x16x32 with A = 16 token rows
// and B = 16 weight rows, D[token][weight row]: a lane's outputs share one
// weight row, so it needs one scale and offset per tile. Every weight load
// is 16 bytes per lane, four lanes side by side on a row (64 contiguous
// bytes per row and instruction): 16 INT8 or 32 INT4 codes, i.e. 2 or 4 MFMA
// k-slices of 8. The k order inside a lane's span differs from the MFMA's
// native one, and the activations are loaded in the same order, so the
// contraction is unchanged. The next K-iteration's weight and activation
// loads are issued before the current iteration's MFMAs; the scales are
// loaded once when a wavefront's K range lies in one scale group
// (per-channel scales, or groups at least that long), else with each
// iteration's loads.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRsrcFlagsQ = 0x00020000;
constexpr uint32_t kOutOfRangeQ = 0x80000000u;
constexpr int kQTiles = 4;              // MFMA tiles of 16 weight rows per workgroup
constexpr int kQRows = 16 * kQTiles;    // weight rows per workgroup
constexpr int kQTokens = 16;
constexpr int kQWaves = 4;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct MfmaQ;
template <> struct MfmaQ<bf16> {
  typedef bf16x8 Frag;
  static __device__ __forceinline__ f32x4 run(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct MfmaQ<f16> {
  typedef f16x8 Frag;
  static __device__ __forceinline__ f32x4 run(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float silu_q(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// K-iteration geometry: one 16-byte load per lane and tile covers kSpan / 4
// codes of a row (kSpan across the 4 lanes of the row), i.e. kMf MFMA
// k-slices of 8; one K-iteration is kLoads such loads per tile, side by side
// (kIter = kLoads * kSpan input channels). INT8 takes two (128 channels, 128
// contiguous bytes of each row, up to 16 KB of weights in flight per
// wavefront at two wavefronts per SIMD, i.e. two workgroups per CU); INT4 one
// (its dequantisation needs more registers and more wavefronts to hide it:
// three per SIMD). Scale groups are multiples of 128 channels and INT4-only,
// so an iteration never straddles two groups.
template <int kBits> struct QGeo {
  static constexpr int kSpan = kBits == 8 ? 64 : 128;
  static constexpr int kLoads = kBits == 8 ? 2 : 1;
  static constexpr int kIter = kSpan * kLoads;
  static constexpr int kMf = kSpan / 32;
  static constexpr int kWavesPerSimd = kBits == 8 ? 2 : 3;  // occupancy target (launch bounds)
};

typedef float f32x2q __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2q __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2q __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even into one dword of T (a first).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (std::is_same<T, bf16>::value)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2q{a, b}, bf16x2q));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2q{a, b}, f16x2q));
}

__device__ __forceinline__ uint32_t word_of(const uint4& q, int i) {
  return i < 2 ? (i == 0 ? q.x : q.y) : (i == 2 ? q.z : q.w);
}

// The shift C of the codes: c = q + C is what enters the MFMA.
//  INT8: c = q + 128, the unsigned byte (0..255, exact in bf16 and fp16).
//  INT4: c = 128 + u with u = q + 8 the unsigned nibble (bf16: exponent of
//        128, u in the low mantissa bits); fp16: c = 1024 + u.
template <typename T, int kBits>
__device__ __forceinline__ constexpr float code_shift() {
  return kBits == 8 ? 128.0f : (std::is_same<T, bf16>::value ? 136.0f : 1032.0f);
}

// The 8 codes of MFMA slice m of a lane's 16 bytes, as an MFMA operand of T.
//  INT8: codes 8m .. 8m+7 are the bytes of words 2m, 2m+1; with the sign bit
//        flipped each byte is q + 128, converted exactly.
//  INT4: codes 8m .. 8m+7 are the nibbles of word m, low nibble first; with
//        each nibble's top bit flipped it is u = q + 8, and the pair of codes
//        2d, 2d+1 (byte d of the word) becomes one dword of two T values by
//        placing u in the mantissa field of 128 (bf16) or 1024 (fp16).
template <typename T, int kBits>
__device__ __forceinline__ uint4 codes8(const uint4& q, int m, uint32_t nib_mask) {
  if constexpr (kBits == 8) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)((word_of(q, 2 * m + (i >> 2)) ^ 0x80808080u) >> (8 * (i & 3)) & 0xFFu);
    uint4 r;
    r.x = pack2<T>(f[0], f[1]);
    r.y = pack2<T>(f[2], f[3]);
    r.z = pack2<T>(f[4], f[5]);
    r.w = pack2<T>(f[6], f[7]);
    return r;
  } else {
    const uint32_t x = word_of(q, m) ^ 0x88888888u;
    // nib_mask (0x0F0F0F0F) comes from the kernel arguments (a compile-time
    // mask would let the compiler split the byte moves into bit-field ops)
    const uint32_t lo = x & nib_mask, hi = (x >> 4) & nib_mask;
    constexpr uint32_t kBase = std::is_same<T, bf16>::value ? 0x43004300u : 0x64006400u;
    // byte permute: selectors 0-3 take the bytes of the second source (lo),
    // 4-7 those of the first (hi), 12 gives a zero byte; dword b holds byte
    // b of lo in its low half and byte b of hi in its high half
    uint32_t d[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      d[b] = __builtin_amdgcn_perm(hi, lo, 0x0C000C00u | ((uint32_t)(4 + b) << 16) | (uint32_t)b) | kBase;
    return uint4{d[0], d[1], d[2], d[3]};
  }
}

struct QuantArgs {
  const void* a;          // activations [a_rows, K]
  const int32_t* a_map;   // optional: A row r is a[a_map[r] / a_div]
  int a_div, a_rows;
  const uint8_t* b0;      // quantised gate (GEMM 1) or down (GEMM 2)
  const uint8_t* b1;      // quantised up (GEMM 1)
  const void* s0;         // scales  [E, N, G]
  const void* s1;
  const void* o0;         // offsets [E, N, G] or null
  const void* o1;
  void* c;                // [rows, N]
  const int32_t* offsets; // [E+1]
  int rows, N, K, G, E, n_blocks, k_quarter;
  uint32_t nib_mask;      // 0x0F0F0F0F
};

// The 4 wavefronts of a workgroup form 4 / kSplitK groups; each group owns a
// block of kQRows weight rows (or kQRows / 2 gate and as many up rows) and
// its kSplitK wavefronts split K, their partial sums meeting in LDS.
template <typename T, bool kSwiGlu, int kBits, int kSplitK>
__global__ __launch_bounds__(64 * kQWaves, QGeo<kBits>::kWavesPerSimd) void skinny_quant_kernel(QuantArgs p) {
  typedef typename MfmaQ<T>::Frag Frag;
  static_assert(kQWaves % kSplitK == 0, "whole groups of wavefronts");
  constexpr int kGroups = kQWaves / kSplitK;
  __shared__ f32x4 red[kGroups][kSplitK > 1 ? kSplitK - 1 : 1][kQTiles][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wk = wave % kSplitK, wn = wave / kSplitK;  // K slice, row block of the workgroup
  const int e = blockIdx.x / p.n_blocks;
  const int nb = (blockIdx.x - e * p.n_blocks) * kGroups + wn;
  if (e >= p.E) return;
  const int r_begin = max(__builtin_amdgcn_readfirstlane(p.offsets[e]), 0);
  const int r_end = min(__builtin_amdgcn_readfirstlane(p.offsets[e + 1]), p.rows);
  if (r_end <= r_begin) return;
  if (kSplitK == 1 && nb * (kSwiGlu ? kQRows / 2 : kQRows) >= p.N) return;  // no barriers without a K split

  const int K = p.K, N = p.N, G = p.G;
  const int gsz = K / G;  // input channels per group (multiple of 8)
  const int k_lo = wk * p.k_quarter;
  const int k_hi = min(K, k_lo + p.k_quarter);
  const uint32_t qrow = (uint32_t)K * kBits / 8;  // bytes per quantised row
  const int64_t expert_rows = (int64_t)e * N;
  const int q_bytes = (int)((uint32_t)N * qrow);
  const __amdgpu_buffer_rsrc_t rw0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.b0 + expert_rows * qrow), (short)0, q_bytes, kRsrcFlagsQ);
  const __amdgpu_buffer_rsrc_t rw1 = kSwiGlu
      ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b1 + expert_rows * qrow), (short)0,
                                          q_bytes, kRsrcFlagsQ)
      : rw0;
  const uint32_t xrow = (uint32_t)K * sizeof(T);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.a), (short)0, (int)((uint32_t)p.a_rows * xrow), kRsrcFlagsQ);

  // Weight rows of the 4 tiles; rows past N read as zero and get scale 0.
  typedef QGeo<kBits> Geo;
  const int g = lane >> 4;
  constexpr int kHalf = kQTiles / 2;
  uint32_t vo_w[kQTiles];
  int wrow[kQTiles];
#pragma unroll
  for (int t = 0; t < kQTiles; ++t) {
    const int n = kSwiGlu ? nb * (16 * kHalf) + (t % kHalf) * 16 + (lane & 15) : nb * kQRows + t * 16 + (lane & 15);
    wrow[t] = n;
    vo_w[t] = (uint32_t)n * qrow + (uint32_t)g * 16u;  // this lane's 16 bytes of each span
  }
  const T* sp0 = static_cast<const T*>(p.s0) + expert_rows * G;
  const T* sp1 = kSwiGlu ? static_cast<const T*>(p.s1) + expert_rows * G : sp0;
  const T* op0 = p.o0 ? static_cast<const T*>(p.o0) + expert_rows * G : nullptr;
  const T* op1 = kSwiGlu ? (p.o1 ? static_cast<const T*>(p.o1) + expert_rows * G : nullptr) : op0;
  const bool has_o0 = op0 != nullptr, has_o1 = op1 != nullptr;
  const T* ob0 = has_o0 ? op0 : sp0;
  const T* ob1 = has_o1 ? op1 : sp1;

  T* C = static_cast<T*>(p.c);
  for (int rg = r_begin; rg < r_end; rg += kQTokens) {
    const int xr = rg + (lane & 15);
    uint32_t vo_x = kOutOfRangeQ;
    if (xr < r_end) {
      const int src = p.a_map ? min(max(p.a_map[xr] / p.a_div, 0), p.a_rows - 1) : xr;
      vo_x = (uint32_t)src * xrow + (uint32_t)(g * (Geo::kSpan / 4)) * (uint32_t)sizeof(T);
    }
    f32x4 acc[kQTiles];
#pragma unroll
    for (int t = 0; t < kQTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Scale and offset*scale of tile t for the group holding the 128
    // input channels of the K-iteration at kb (groups are multiples of 128 long).
    // Every load is issued (row and group clamped into range), then masked,
    // so none waits behind a branch.
    typedef float Sc[kQTiles][Geo::kLoads];
    auto load_sc = [&](int kb, Sc& sc, Sc& os, int n_loads) {
#pragma unroll
      for (int l = 0; l < Geo::kLoads; ++l) {
        if (l >= n_loads) {
#pragma unroll
          for (int t = 0; t < kQTiles; ++t) { sc[t][l] = sc[t][0]; os[t][l] = os[t][0]; }
          continue;
        }
        const int kl = kb + l * Geo::kSpan;
        const int grp = min(kl, K - 1) / gsz;
        T sv[kQTiles], ov[kQTiles];
#pragma unroll
        for (int t = 0; t < kQTiles; ++t) {
          const bool up = kSwiGlu && t >= kHalf;
          const int64_t at = (int64_t)min(wrow[t], N - 1) * G + grp;
          sv[t] = (up ? sp1 : sp0)[at];
          ov[t] = (up ? ob1 : ob0)[at];  // the scales stand in for absent offsets
        }
        // Masked by clearing the bits (+0), not by a select the compiler would
        // turn back into a branch around the load.
#pragma unroll
        for (int t = 0; t < kQTiles; ++t) {
          const bool up = kSwiGlu && t >= kHalf;
          const bool on = wrow[t] < N && kl < k_hi;
          const uint16_t ms = on ? 0xFFFFu : 0u;
          const uint16_t mo = on && (up ? has_o1 : has_o0) ? 0xFFFFu : 0u;
          const float s = to_f32(__builtin_bit_cast(T, (uint16_t)(__builtin_bit_cast(uint16_t, sv[t]) & ms)));
          const float o = to_f32(__builtin_bit_cast(T, (uint16_t)(__builtin_bit_cast(uint16_t, ov[t]) & mo)));
          sc[t][l] = s;
          os[t][l] = (o - code_shift<T, kBits>()) * s;  // the codes enter as q + C
        }
      }
    };
    // Per iteration at input channel kb: load w of tile t holds channels
    // kb + w*kSpan + g*kSpan/4 .. +kSpan/4-1 of the tile's row; MFMA m of that
    // load takes its codes 8m .. 8m+7, and activation chunk [w][m] holds the
    // same 8 channels. Codes past K or past this wavefront's K range meet
    // activations masked to zero (8-channel granularity).
    uint4 wa[kQTiles][Geo::kLoads], wb[kQTiles][Geo::kLoads];
    uint4 xa[Geo::kLoads][Geo::kMf], xb[Geo::kLoads][Geo::kMf];
    Sc sa_, oa, sb_, ob;
    auto load = [&](int kb, uint4 (&w)[kQTiles][Geo::kLoads], uint4 (&x)[Geo::kLoads][Geo::kMf]) {
      const uint32_t soff_q = (uint32_t)kb * kBits / 8;
      const uint32_t soff_x = (uint32_t)kb * sizeof(T);
#pragma unroll
      for (int l = 0; l < Geo::kLoads; ++l) {
        const int k0 = kb + l * Geo::kSpan + g * (Geo::kSpan / 4);
        const bool okw = k0 < k_hi;
#pragma unroll
        for (int t = 0; t < kQTiles; ++t)
          w[t][l] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
              (kSwiGlu && t >= kHalf) ? rw1 : rw0,
              okw ? vo_w[t] + (uint32_t)(l * Geo::kSpan * kBits / 8) : kOutOfRangeQ, soff_q, 0));
#pragma unroll
        for (int m = 0; m < Geo::kMf; ++m) {
          const bool okx = k0 + m * 8 < k_hi;
          x[l][m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
              rx, okx ? vo_x + (uint32_t)((l * Geo::kSpan + m * 8) * (int)sizeof(T)) : kOutOfRangeQ, soff_x, 0));
        }
      }
    };
    // Codes against activations (cacc, per tile) and ones against
    // activations (xsum: every column the sum of the token's activations),
    // both in fp32; finish() applies the group's scale and offset.
    f32x4 cacc[kQTiles], xsum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kQTiles; ++t) cacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const Frag ones = __builtin_bit_cast(
        Frag, std::is_same<T, bf16>::value ? uint4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                                           : uint4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});
    auto compute = [&](const uint4 (&w)[kQTiles][Geo::kLoads], const uint4 (&x)[Geo::kLoads][Geo::kMf]) {
#pragma unroll
      for (int l = 0; l < Geo::kLoads; ++l)
#pragma unroll
        for (int m = 0; m < Geo::kMf; ++m) {
          const Frag xf = __builtin_bit_cast(Frag, x[l][m]);
#pragma unroll
          for (int t = 0; t < kQTiles; ++t)
            cacc[t] = MfmaQ<T>::run(xf, __builtin_bit_cast(Frag, codes8<T, kBits>(w[t][l], m, p.nib_mask)), cacc[t]);
          xsum = MfmaQ<T>::run(xf, ones, xsum);
        }
    };
    // acc += s * cacc + s (o - C) * xsum for the group just finished (all of
    // an iteration's loads lie in one group: index 0 of sc, os).
    auto finish = [&](const Sc& sc, const Sc& os) {
#pragma unroll
      for (int t = 0; t < kQTiles; ++t) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] += sc[t][0] * cacc[t][v] + os[t][0] * xsum[v];
        cacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      xsum = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    const int n_iter = (k_hi - k_lo + Geo::kIter - 1) / Geo::kIter;
    // One scale group over this wavefront's whole K range (per-channel
    // scales, or groups no shorter than the range): the scales are loaded once.
    const bool one_group = n_iter > 0 && k_lo / gsz == (k_hi - 1) / gsz;
    if (one_group) {
      load_sc(k_lo, sa_, oa, 1);
      load(k_lo, wa, xa);
      int it = 0;
      for (; it + 2 <= n_iter; it += 2) {
        load(k_lo + (it + 1) * Geo::kIter, wb, xb);
        compute(wa, xa);
        load(k_lo + (it + 2) * Geo::kIter, wa, xa);
        compute(wb, xb);
      }
      if (it < n_iter) compute(wa, xa);  // odd count: wa holds the last iteration
      finish(sa_, oa);
    } else if (n_iter > 0) {
      // the group ends after iteration it when the next one starts a new group
      auto group_ends = [&](int it) {
        const int kn = k_lo + (it + 1) * Geo::kIter;
        return it + 1 == n_iter || kn % gsz == 0;
      };
      load(k_lo, wa, xa);
      load_sc(k_lo, sa_, oa, Geo::kLoads);
      int it = 0;
      for (; it + 2 <= n_iter; it += 2) {
        load(k_lo + (it + 1) * Geo::kIter, wb, xb);
        load_sc(k_lo + (it + 1) * Geo::kIter, sb_, ob, Geo::kLoads);
        compute(wa, xa);
        if (group_ends(it)) finish(sa_, oa);
        load(k_lo + (it + 2) * Geo::kIter, wa, xa);
        load_sc(k_lo + (it + 2) * Geo::kIter, sa_, oa, Geo::kLoads);
        compute(wb, xb);
        if (group_ends(it + 1)) finish(sb_, ob);
      }
      if (it < n_iter) {
        compute(wa, xa);
        finish(sa_, oa);
      }
    }

    // Partial sums of a group's wavefronts 1.. meet its wavefront 0's in LDS
    // (fixed order).
    if (kSplitK > 1) {
      if (wk > 0) {
#pragma unroll
        for (int t = 0; t < kQTiles; ++t) red[wn][wk - 1][t][lane] = acc[t];
      }
      __syncthreads();
    }
    if (wk == 0) {
#pragma unroll
      for (int w = 0; w < kSplitK - 1; ++w)
#pragma unroll
        for (int t = 0; t < kQTiles; ++t) acc[t] += red[wn][w][t][lane];
      // D element v of lane l: token (l/16)*4 + v, weight row l%16 of the tile.
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = rg + g * 4 + v;
        if (tok >= r_end) continue;
        T* crow = C + (int64_t)tok * N;
        if (kSwiGlu) {
#pragma unroll
          for (int t = 0; t < kHalf; ++t) {
            const int col = nb * (16 * kHalf) + t * 16 + (lane & 15);
            if (col < N) crow[col] = from_f32<T>(silu_q(acc[t][v]) * acc[t + kHalf][v]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < kQTiles; ++t) {
            const int col = nb * kQRows + t * 16 + (lane & 15);
            if (col < N) crow[col] = from_f32<T>(acc[t][v]);
          }
        }
      }
    }
    if (kSplitK > 1) __syncthreads();  // red[] is reused by the next row group
  }
}

// Wavefronts per K range (kSplitK) of each GEMM and bit width, measured on
// the decode shape: 4 everywhere except the INT8 down GEMM (K = I, short
// rows), where two row blocks of two K halves each ran faster than one row
// block of four K quarters; the INT4 GEMMs were slower with 2 or 1.
#ifndef MOE_Q_SPLIT_GU8
#define MOE_Q_SPLIT_GU8 4
#endif
#ifndef MOE_Q_SPLIT_DN8
#define MOE_Q_SPLIT_DN8 2
#endif
#ifndef MOE_Q_SPLIT_GU4
#define MOE_Q_SPLIT_GU4 4
#endif
#ifndef MOE_Q_SPLIT_DN4
#define MOE_Q_SPLIT_DN4 4
#endif
template <typename T, int kBits, bool kSwiGlu, int kSplitK>
void launch_q_split(QuantArgs p, hipStream_t s) {
  const int rows_per_wave = kSwiGlu ? kQRows / 2 : kQRows;  // output columns of one row block
  const int rows_per_group = rows_per_wave * (kQWaves / kSplitK);
  p.n_blocks = (p.N + rows_per_group - 1) / rows_per_group;
  constexpr int kIter = QGeo<kBits>::kIter;
  const int iters = (p.K + kIter - 1) / kIter;
  p.k_quarter = (iters + kSplitK - 1) / kSplitK * kIter;
  const dim3 grid((unsigned)((int64_t)p.E * p.n_blocks));
  hipLaunchKernelGGL((skinny_quant_kernel<T, kSwiGlu, kBits, kSplitK>), grid, dim3(64 * kQWaves), 0, s, p);
}

template <typename T, int kBits>
void launch_q(QuantArgs p, bool swiglu, hipStream_t s) {
  if (swiglu) launch_q_split<T, kBits, true, kBits == 8 ? MOE_Q_SPLIT_GU8 : MOE_Q_SPLIT_GU4>(p, s);
  else launch_q_split<T, kBits, false, kBits == 8 ? MOE_Q_SPLIT_DN8 : MOE_Q_SPLIT_DN4>(p, s);
}

template <typename T>
void launch_q_bits(const QuantArgs& p, int bits, bool swiglu, hipStream_t s) {
  if (bits == 8) launch_q<T, 8>(p, swiglu, s);
  else launch_q<T, 4>(p, swiglu, s);
}

}  // namespace

hipError_t launch_experts_quant(const QuantExperts& q, hipStream_t s) {
  if (q.rows == 0) return hipSuccess;
  QuantArgs p = {};
  p.nib_mask = 0x0F0F0F0Fu;
  p.offsets = q.offsets;
  p.rows = q.rows;
  p.E = q.E;
  // GEMM 1: h = SiLU(x Wg^T) * (x Wu^T), K = H, N = I
  p.a = q.x; p.a_map = q.row_map; p.a_div = q.map_div > 0 ? q.map_div : 1;
  p.a_rows = q.row_map ? (q.rows + p.a_div - 1) / p.a_div : q.rows;
  p.b0 = static_cast<const uint8_t*>(q.w_gate); p.b1 = static_cast<const uint8_t*>(q.w_up);
  p.s0 = q.s_gate; p.s1 = q.s_up; p.o0 = q.o_gate; p.o1 = q.o_up;
  p.c = q.h; p.N = q.I; p.K = q.H; p.G = q.groups;
  if (q.dt == kF16) launch_q_bits<f16>(p, q.bits, true, s);
  else launch_q_bits<bf16>(p, q.bits, true, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // GEMM 2: expert_out = h Wd^T, K = I, N = H
  p.a = q.h; p.a_map = nullptr; p.a_div = 1; p.a_rows = q.rows;
  p.b0 = static_cast<const uint8_t*>(q.w_down); p.b1 = nullptr;
  p.s0 = q.s_down; p.s1 = nullptr; p.o0 = q.o_down; p.o1 = nullptr;
  p.c = q.expert_out; p.N = q.H; p.K = q.I;
  if (q.dt == kF16) launch_q_bits<f16>(p, q.bits, false, s);
  else launch_q_bits<bf16>(p, q.bits, false, s);
  return hipGetLastError();
}

}  // namespace moe
