// First-order training of the MoE FFN (ruDNN user guide, "12. MoE
// first-order training"): router weights for a fixed selection and their
// gradient, combine_backward, the experts' training forward (with its
// cache) and backward, and dispatch_backward.
//
// Expert GEMMs of the backward pass (per expert e, rows n_e):
//   dh     = dY W_down[e]            [n_e, I]  K = H   W_down read along N
//   dinput = [dg | du] [W_gate; W_up] [n_e, H]  K = 2I  weights read along N
//   ddown  = dY^T h                  [H, I]    K = n_e rows
//   dgate | dup = [dg | du]^T X      [2I, H]   K = n_e rows
// and of the training forward the plain projection [g | u] = X [W_gate;
// W_up]^T (K = H, both operands along K; used for decode-sized batches, the
// larger ones take the inference gate/up GEMM with a cache epilogue). One
// MFMA kernel serves them all: each operand is either K-contiguous (element
// (mn, k) at mn * ld + k) or MN-contiguous (at k * ld + mn), and K may run
// over two segments held by different tensors (dg with W_gate, du with
// W_up). Both kinds of tile go to LDS as they lie in memory; MN-contiguous
// ones are read back with gfx950's transposing LDS read, so the MFMA gets
// its 8-element K-runs either way.
//
// Grouping. "M-grouped" GEMMs take their rows from the expert offsets (one
// M-tile never spans two experts; tiles are found through a device-built
// prefix of M-tiles per expert). "K-grouped" GEMMs (the weight gradients)
// run one output tile per (expert, M-tile, N-tile) and loop over the
// expert's rows as K; an expert without rows writes zeros.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTM = 256;           // output tile rows
constexpr int kTN = 256;           // output tile columns
constexpr int kTK = 64;            // K per LDS stage
constexpr int kTWaves = 8;         // 4 (M) x 2 (N); 64 x 128 outputs per wavefront
constexpr int kTThreads = 64 * kTWaves;
constexpr int kNGroup = 32;        // N-tiles per group in the M-grouped tile order
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, no format, no swizzle (gfx9 family)
constexpr uint32_t kOOR = 0x80000000u;  // voffset past every buffer built here: reads zeros
constexpr int kRecords = 0x7FFFFFF0;    // buffer size in bytes: every real offset is smaller

enum Epilogue { kEpiStore = 0, kEpiStoreF32 = 1, kEpiSwiGluBwd = 2 };

// One GEMM operand. Element (mn, k) of K-segment s for expert e lies at
//   K-contiguous:  p[s] + e * estride + mn * ld + kofs[s] + k
//   MN-contiguous: p[s] + e * estride + (kofs[s] + k) * ld + mn
struct TOp {
  const void* p[2];
  int64_t ld;
  int64_t estride;
  int64_t kofs[2];
};

struct TrainGemm {
  TOp a, b;
  int nseg;                    // M-grouped: K segments (1 or 2), each a multiple of 8 long
  int64_t seg_len[2];
  const int32_t* offsets;      // [E+1]
  const int32_t* tile_prefix;  // M-grouped: [E+1] prefix of M-tiles per expert
  int E;
  int M, N;                    // M-grouped: M unused
  int m_tiles, n_tiles;        // M-grouped: m_tiles is the bound the grid is sized for
  void* out0;
  void* out1;
  int64_t out_split;           // output rows >= out_split go to out1
  int64_t ldc;
  int64_t out_estride;         // K-grouped outputs: elements between experts
  const void* gu;              // SwiGLU backward: cache [rows, 2N] = (g | u)
};

template <typename T> struct TMfma;
template <> struct TMfma<bf16> {
  static __device__ __forceinline__ f32x16 run(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct TMfma<f16> {
  static __device__ __forceinline__ f32x16 run(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <typename T> using Frag = typename std::conditional<std::is_same<T, bf16>::value, bf16x8, f16x8>::type;

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// One LDS object per (operand, stage), 32 KB each: 256 rows x 64 k (K-
// contiguous operand) or 64 k-rows x 256 (MN-contiguous operand).
template <typename T, int kOperand, int kStage>
__device__ __forceinline__ T* tbuf() {
  __shared__ __attribute__((aligned(1024))) T buf[kTM * kTK];
  return buf;
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t vo) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, vo, 0, 0, 0);
}

// Copies one operand's k-tile into LDS with buffer loads straight to LDS:
// instruction j of wavefront w fills the 1 KB block q = 8j + w, lane l its
// 16 bytes at 16 l; the lane fetches the global chunk the swizzle puts there.
//  K-contiguous: block q = rows 8q .. 8q+7 (128-byte rows, 8 chunks); chunk c
//    of row r sits in slot c ^ ((r >> 1) & 7), so the 16 lanes of a 128-bit
//    fragment read (16 consecutive rows, one chunk) hit 16 bank groups.
//  MN-contiguous: block q = k-rows 2q, 2q+1 (512-byte rows, 32 chunks); chunk
//    c of k-row k sits in slot c ^ 4 (k & 3), so a transposed read (4 k-rows x
//    64 bytes per 32 lanes) hits 16 distinct bank groups.
// Rows at or past mn_end, and k at or past k_valid, read as zeros.
template <typename T, bool kKC>
__device__ __forceinline__ void load_tile(const TOp& op, int seg, int e, int64_t mn0, int64_t mn_end,
                                          int64_t kbase, int k_valid, T* dst, int wave, int lane) {
  if (kKC) {
    const T* base = static_cast<const T*>(op.p[seg]) + (int64_t)e * op.estride + mn0 * op.ld + kbase;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, kRecords, kRsrcFlags);
    const int c = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    const bool kok = c * 8 < k_valid;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = j * kTWaves + wave;
      const int r = q * 8 + (lane >> 3);
      const bool ok = kok && mn0 + r < mn_end;
      dma16(rs, dst + q * 512, ok ? (uint32_t)(((int64_t)r * op.ld + c * 8) * (int64_t)sizeof(T)) : kOOR);
    }
  } else {
    const T* base = static_cast<const T*>(op.p[seg]) + (int64_t)e * op.estride + kbase * op.ld + mn0;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, kRecords, kRsrcFlags);
    const int c = (lane & 31) ^ (4 * ((2 * (wave & 1) + (lane >> 5)) & 3));
    const bool mok = mn0 + c * 8 < mn_end;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = j * kTWaves + wave;
      const int kr = q * 2 + (lane >> 5);
      const bool ok = mok && kr < k_valid;
      dma16(rs, dst + q * 512, ok ? (uint32_t)(((int64_t)kr * op.ld + c * 8) * (int64_t)sizeof(T)) : kOOR);
    }
  }
}

// MFMA 32x32x16 operand fragment: lane l holds row (or column) R0 + l % 32 at
// k = 16 s + 8 (l / 32) .. +7.
template <typename T>
__device__ __forceinline__ Frag<T> frag_kc(const T* buf, int R0, int s, int lane) {
  const int r = R0 + (lane & 31);
  const int c = (2 * s + (lane >> 5)) ^ ((r >> 1) & 7);
  return *reinterpret_cast<const Frag<T>*>(buf + r * kTK + c * 8);
}

// The same fragment from an MN-contiguous tile with two transposed 8-byte
// LDS reads: in each group of 16 lanes, lane i receives element i % 4 of the
// 8-byte pieces addressed by lanes 4m + i / 4 (m = 0..3). Lane j of group g
// addresses k-row k0 + j / 4 at column C0 + 16 (g & 1) + 4 (j % 4), so lane i
// ends up with column C0 + 16 (g & 1) + i at k0 .. k0 + 3, k0 = 16 s + 8 (g / 2)
// (+ 4 for the second read).
template <typename T>
__device__ __forceinline__ Frag<T> frag_mn(const T* buf, int C0, int s, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int mn = C0 + (g & 1) * 16 + 4 * (i & 3);
  s16x4 v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = s * 16 + (g >> 1) * 8 + h * 4 + (i >> 2);
    const int off = k * kTM + (((mn >> 3) ^ (4 * (k & 3))) << 3) + (mn & 7);
    v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + off));
  }
  const s16x8 w = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
  return __builtin_bit_cast(Frag<T>, w);
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// One butterfly round of a 4 x 4 transpose across the lanes of a quad: the
// lane swaps with lane ^ kBit the two values whose index bit kBit differs
// from its own lane bit (quad-permute DPP moves).
template <int kBit>
__device__ __forceinline__ void quad_round(float (&x)[4], int lane) {
  constexpr int kCtrl = kBit == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] or [2,3,0,1]
  const bool hi = (lane & kBit) != 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i & kBit) continue;
    const float send = hi ? x[i] : x[i | kBit];
    const float recv = __builtin_bit_cast(float,
        __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), kCtrl, 0xF, 0xF, false));
    if (hi) x[i] = recv;
    else x[i | kBit] = recv;
  }
}

// On return x[c] of lane q of a quad holds what x[q] of lane c held.
__device__ __forceinline__ void quad_transpose(float (&x)[4], int lane) {
  quad_round<1>(x, lane);
  quad_round<2>(x, lane);
}

// Scheduling order for one k16 sub-step: each of its 8 MFMAs followed by
// its share of the next sub-step's kReads LDS reads.
template <int kReads, int X>
__device__ __forceinline__ void interleave() {
  if constexpr (X < 8) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int n = (kReads + 7 - X) / 8;
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);
    interleave<kReads, X + 1>();
  }
}

// Grouped GEMM C[m, n] = sum_k A(m, k) B(n, k) over 256 x 256 tiles, 8
// wavefronts, K staged 64 at a time through two LDS stages: the loads of
// k-step t+1 are issued before the MFMAs of k-step t and waited for at its end.
template <typename T, bool kAK, bool kBK, int kEpi, bool kGroupK>
__global__ __launch_bounds__(kTThreads) void train_gemm_kernel(TrainGemm p) {
  int e, m_idx, n_idx;
  int64_t m0, m_end, kstart;
  int64_t seg_len[2];
  int nseg;
  if (kGroupK) {
    const int per_e = p.m_tiles * p.n_tiles;
    e = blockIdx.x / per_e;
    const int t = blockIdx.x % per_e;
    m_idx = t / p.n_tiles;
    n_idx = t % p.n_tiles;
    m0 = (int64_t)m_idx * kTM;
    m_end = p.M;
    kstart = p.offsets[e];
    nseg = 1;
    seg_len[0] = p.offsets[e + 1] - kstart;
    seg_len[1] = 0;
  } else {
    const int per_group = kNGroup * p.m_tiles;
    const int g = blockIdx.x / per_group;
    const int within = blockIdx.x % per_group;
    const int n_in = min(kNGroup, p.n_tiles - g * kNGroup);
    m_idx = within / n_in;
    n_idx = g * kNGroup + within % n_in;
    if (m_idx >= p.tile_prefix[p.E]) return;
    int lo = 0, hi = p.E - 1;  // the expert e with prefix[e] <= m_idx < prefix[e+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.tile_prefix[mid] <= m_idx) lo = mid; else hi = mid - 1;
    }
    e = lo;
    m0 = p.offsets[e] + (int64_t)(m_idx - p.tile_prefix[e]) * kTM;
    m_end = p.offsets[e + 1];
    kstart = 0;
    nseg = p.nseg;
    seg_len[0] = p.seg_len[0];
    seg_len[1] = p.seg_len[1];
  }
  const int64_t n0 = (int64_t)n_idx * kTN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t nk0 = (seg_len[0] + kTK - 1) / kTK;
  const int64_t nk = nk0 + (nseg > 1 ? (seg_len[1] + kTK - 1) / kTK : 0);
  const int64_t nk_pad = (nk + 1) & ~(int64_t)1;

  auto issue = [&](int64_t t, T* la, T* lb) {
    const int seg = t >= nk0 ? 1 : 0;
    const int64_t k0 = (t - (seg ? nk0 : 0)) * kTK;
    const int kval = t < nk ? (int)min((int64_t)kTK, seg_len[seg] - k0) : 0;
    load_tile<T, kAK>(p.a, seg, e, m0, m_end, kstart + p.a.kofs[seg] + k0, kval, la, wave, lane);
    load_tile<T, kBK>(p.b, seg, e, n0, p.N, kstart + p.b.kofs[seg] + k0, kval, lb, wave, lane);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Fragments are double-buffered across the four k16 sub-steps: the reads
  // of sub-step s+1 are interleaved with the MFMAs of sub-step s. The last
  // sub-step's MFMAs are split around the stage barrier: half before it, and
  // half after, overlapping the first fragment reads of the next stage, so a
  // wavefront that reaches the barrier early still has MFMAs queued.
  Frag<T> fa[2][2], fb[2][4];
  auto read = [&](const T* la, const T* lb, int s, int slot) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      fa[slot][i] = kAK ? frag_kc<T>(la, wm * 64 + i * 32, s, lane) : frag_mn<T>(la, wm * 64 + i * 32, s, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[slot][j] = kBK ? frag_kc<T>(lb, wn * 128 + j * 32, s, lane) : frag_mn<T>(lb, wn * 128 + j * 32, s, lane);
  };
  auto mfmas = [&](int slot, int from, int to) {
#pragma unroll
    for (int x = from; x < to; ++x) acc[x >> 2][x & 3] = TMfma<T>::run(fa[slot][x >> 2], fb[slot][x & 3], acc[x >> 2][x & 3]);
  };
  constexpr int kReads = (kAK ? 2 : 4) + (kBK ? 4 : 8);  // LDS read instructions per sub-step
  // One k-step from stage (la, lb); (na, nb) is the stage the next k-step reads.
  auto step = [&](const T* la, const T* lb, const T* na, const T* nb, bool more) {
#pragma unroll
    for (int s = 0; s + 1 < kTK / 16; ++s) {
      read(la, lb, s + 1, (s + 1) & 1);
      mfmas(s & 1, 0, 8);
      interleave<kReads, 0>();
    }
    mfmas(1, 0, 4);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (more) read(na, nb, 0, 0);
    mfmas(1, 4, 8);
  };

  if (nk_pad > 0) {
    issue(0, tbuf<T, 0, 0>(), tbuf<T, 1, 0>());
    wait_vmem<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    read(tbuf<T, 0, 0>(), tbuf<T, 1, 0>(), 0, 0);
  }
  for (int64_t t = 0; t < nk_pad; t += 2) {
    issue(t + 1, tbuf<T, 0, 1>(), tbuf<T, 1, 1>());
    step(tbuf<T, 0, 0>(), tbuf<T, 1, 0>(), tbuf<T, 0, 1>(), tbuf<T, 1, 1>(), true);
    if (t + 2 < nk_pad) issue(t + 2, tbuf<T, 0, 0>(), tbuf<T, 1, 0>());
    step(tbuf<T, 0, 1>(), tbuf<T, 1, 1>(), tbuf<T, 0, 0>(), tbuf<T, 1, 0>(), t + 2 < nk_pad);
  }

  // ---- epilogue ----
  // Accumulator element v of lane l sits at row (v/4)*8 + (l/32)*4 + v%4 and
  // column l%32 of its 32 x 32 block. Each run of 4 rows is transposed within
  // the quad of lanes holding 4 adjacent columns, after which lane l holds
  // columns 4*((l%32)/4) .. +3 of one row: one 16-byte (fp32) or 8-byte
  // store instead of four. N is a multiple of 8, so the 4 columns are all
  // inside or all outside.
  const int col4 = (lane & 31) & ~3;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float x[4] = {acc[i][j][4 * g4], acc[i][j][4 * g4 + 1], acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]};
        quad_transpose(x, lane);
        const int64_t m = m0 + wm * 64 + i * 32 + g4 * 8 + (lane >> 5) * 4 + (lane & 3);
        const int64_t n = n0 + wn * 128 + j * 32 + col4;
        if (m >= m_end || n >= p.N) continue;
        if (kEpi == kEpiSwiGluBwd) {
          // dh = x; g, u from the cache; dg, du into out0 (same [rows, 2N] layout)
          const int64_t at = m * 2 * (int64_t)p.N + n;
          const uint2 gw = *reinterpret_cast<const uint2*>(static_cast<const T*>(p.gu) + at);
          const uint2 uw = *reinterpret_cast<const uint2*>(static_cast<const T*>(p.gu) + at + p.N);
          const T* gv = reinterpret_cast<const T*>(&gw);
          const T* uv = reinterpret_cast<const T*>(&uw);
          T dg[4], du[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float g = to_f32(gv[c]), u = to_f32(uv[c]);
            const float sg = sigmoidf_(g);
            dg[c] = from_f32<T>(x[c] * u * sg * (1.0f + g * (1.0f - sg)));
            du[c] = from_f32<T>(x[c] * g * sg);
          }
          T* o = static_cast<T*>(p.out0);
          *reinterpret_cast<uint2*>(o + at) = *reinterpret_cast<const uint2*>(dg);
          *reinterpret_cast<uint2*>(o + at + p.N) = *reinterpret_cast<const uint2*>(du);
        } else {
          const bool hi = m >= p.out_split;
          const int64_t row = hi ? m - p.out_split : m;
          const int64_t at = (kGroupK ? (int64_t)e * p.out_estride : 0) + row * p.ldc + n;
          void* base = hi ? p.out1 : p.out0;
          if (kEpi == kEpiStoreF32) {
            // fp32 weight gradients: written once and not read again in
            // the step, so streamed past the caches (measured 7 % faster)
            typedef float f4v __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(f4v{x[0], x[1], x[2], x[3]},
                                        reinterpret_cast<f4v*>(static_cast<float*>(base) + at));
          } else {
            T h[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) h[c] = from_f32<T>(x[c]);
            *reinterpret_cast<uint2*>(static_cast<T*>(base) + at) = *reinterpret_cast<const uint2*>(h);
          }
        }
      }
}


// prefix[e] = number of M-tiles of experts before e; prefix[E] = total.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int bm, int32_t* __restrict__ prefix) {
  const int e = threadIdx.x;
  int n = 0;
  if (e < E) n = (offsets[e + 1] - offsets[e] + bm - 1) / bm;
  int total = 0;
  const int before = block_exclusive_scan(n, &total);
  if (e < E) prefix[e] = before;
  if (e == 0) prefix[E] = total;
}

// h = SiLU(g) * u from the cached projections, 8 columns per thread.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_cache_kernel(const T* __restrict__ gu, T* __restrict__ h,
                                                          int64_t rows, int I) {
  const int64_t chunks = (int64_t)I / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * chunks) return;
  const int64_t r = idx / chunks, c = (idx % chunks) * 8;
  Vec8<T> g, u, o;
  g.load(gu + r * 2 * I + c);
  u.load(gu + r * 2 * I + I + c);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float gv = g.get(i);
    o.set(i, gv * sigmoidf_(gv) * u.get(i));
  }
  o.store(h + r * I + c);
}

// ---- combine / dispatch backward -------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// One block per token: dexpert[row(t,j)] = w[t,j] * grad_out[t]; dweights[t,j]
// = <grad_out[t], expert_out[row(t,j)]> (fp32); NaN for a slot without a row.
template <typename T, typename WT>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const T* __restrict__ y, const int32_t* __restrict__ row_of_slot, const WT* __restrict__ w,
    const T* __restrict__ go, int k, int H, T* __restrict__ dexp, float* __restrict__ dw) {
  __shared__ float part[4][64];
  const int t = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunks = H / 8;
  for (int j = 0; j < k; ++j) {
    const int r = row_of_slot[(int64_t)t * k + j];
    float dot = 0.f;
    if (r >= 0) {
      const float wj = to_f32(w[(int64_t)t * k + j]);
      for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        Vec8<T> g, yv, d;
        g.load(go + (int64_t)t * H + c * 8);
        yv.load(y + (int64_t)r * H + c * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dot = fmaf(g.get(i), yv.get(i), dot);
          d.set(i, wj * g.get(i));
        }
        d.store(dexp + (int64_t)r * H + c * 8);
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) part[wave][j & 63] = r >= 0 ? dot : __builtin_nanf("");
    if ((j & 63) == 63 || j == k - 1) {
      __syncthreads();
      const int jj = threadIdx.x;
      const int base = j & ~63;
      if (jj <= (j & 63)) dw[(int64_t)t * k + base + jj] = part[0][jj] + part[1][jj] + part[2][jj] + part[3][jj];
      __syncthreads();
    }
  }
}

// One block per token: dx[t] = sum over dispatched slots of dinput[row(t,j)].
template <typename T>
__global__ __launch_bounds__(256) void dispatch_backward_kernel(const T* __restrict__ dinput,
                                                               const int32_t* __restrict__ row_of_slot,
                                                               int k, int H, T* __restrict__ dx) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < H / 8; c += blockDim.x) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int r = row_of_slot[(int64_t)t * k + j];
      if (r < 0) continue;
      Vec8<T> v;
      v.load(dinput + (int64_t)r * H + c * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] += v.get(i);
    }
    Vec8<T> o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o.set(i, s[i]);
    o.store(dx + (int64_t)t * H + c * 8);
  }
}

// ---- router weights and their gradient for a fixed selection ---------------------

template <typename IT>
__device__ __forceinline__ int64_t read_index(const IT* idx, int64_t at) { return (int64_t)idx[at]; }

// Per token (one wavefront): the max and the sum of exp over the row for the
// softmax (fp32, as the routing contract computes it).
template <typename LT>
__device__ __forceinline__ void softmax_stats(const LT* z, int E, float* zmax, float* zsum) {
  const int lane = __lane_id();
  float m = -INFINITY;
  bool nan = false;
  for (int e = lane; e < E; e += kWave) {
    const float v = to_f32(z[e]);
    nan |= v != v;
    m = fmaxf(m, v);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
  float s = 0.f;
  for (int e = lane; e < E; e += kWave) s += expf(to_f32(z[e]) - m);
  s = wave_sum(s);
  const bool any_nan = __any(nan);
  *zmax = m;
  *zsum = any_nan ? __builtin_nanf("") : s;
}

template <typename LT, typename IT>
__global__ __launch_bounds__(256) void router_weights_kernel(const LT* __restrict__ logits,
                                                             const IT* __restrict__ indices, int T,
                                                             int E, int k, int scoring, int normalize,
                                                             float scale, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const LT* z = logits + (int64_t)t * E;
  float zmax = 0.f, zsum = 1.f;
  if (scoring == 0) softmax_stats(z, E, &zmax, &zsum);
  int64_t i = 0;
  bool bad = false;
  float a = 0.f;
  if (lane < k) {
    i = read_index(indices, (int64_t)t * k + lane);
    bad = i < 0 || i >= E;
    if (!bad) {
      const float v = to_f32(z[i]);
      a = scoring == 0 ? expf(v - zmax) / zsum : sigmoidf_(v);
    }
  }
  const bool row_bad = __any(bad);
  const float S = normalize ? wave_sum(lane < k ? a : 0.f) : 1.f;
  if (lane < k) w[(int64_t)t * k + lane] = row_bad ? __builtin_nanf("") : (normalize ? a / S : a) * scale;
}

// Gradient for the fixed selection (c = scale, a_j the gathered score, S the
// sum of gathered scores when normalising, G_e = sum of grad_weights over the
// slots selecting e, n_e their number):
//   softmax:  dz_e = c p_e (G_e - sum_j g_j p_{i_j})               no normalize
//             dz_e = c p_e / S (G_e - n_e sum_j g_j p_{i_j} / S)   normalize
//   sigmoid:  dz_e = c s_e (1 - s_e) G_e                           no normalize
//             dz_e = c s_e (1 - s_e) / S (G_e - n_e sum_j g_j s_{i_j} / S)
// An unselected expert of a sigmoid row has no dependence: 0.
template <typename LT, typename IT>
__global__ __launch_bounds__(256) void router_backward_kernel(
    const LT* __restrict__ logits, const IT* __restrict__ indices, const float* __restrict__ gw,
    int T, int E, int k, int scoring, int normalize, float scale, LT* __restrict__ dz) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const LT* z = logits + (int64_t)t * E;
  LT* out = dz + (int64_t)t * E;
  float zmax = 0.f, zsum = 1.f;
  if (scoring == 0) softmax_stats(z, E, &zmax, &zsum);
  int my_i = -1;
  bool bad = false;
  float a = 0.f, g = 0.f;
  if (lane < k) {
    const int64_t i = read_index(indices, (int64_t)t * k + lane);
    bad = i < 0 || i >= E;
    my_i = bad ? -1 : (int)i;
    g = gw[(int64_t)t * k + lane];
    if (!bad) {
      const float v = to_f32(z[i]);
      a = scoring == 0 ? expf(v - zmax) / zsum : sigmoidf_(v);
    }
  }
  const float S = normalize ? wave_sum(lane < k ? a : 0.f) : 1.f;
  // An invalid index, or normalising by a sum that is zero or NaN (0/0 in
  // every term of the derivative), makes the whole row NaN.
  if (__any(bad) || !(S > 0.f)) {
    for (int e = lane; e < E; e += kWave) out[e] = from_f32<LT>(__builtin_nanf(""));
    return;
  }
  const float A = wave_sum(lane < k ? g * a : 0.f);
  for (int e = lane; e < E; e += kWave) {
    float G = 0.f;
    int n = 0;
    for (int j = 0; j < k; ++j) {
      const int ij = __shfl(my_i, j, kWave);
      const float gj = __shfl(g, j, kWave);
      if (ij == e) { G += gj; ++n; }
    }
    const float v = to_f32(z[e]);
    float d;
    if (scoring == 0) {
      const float pe = expf(v - zmax) / zsum;
      d = normalize ? scale * pe / S * (G - n * A / S) : scale * pe * (G - A);
    } else if (n == 0) {
      d = 0.f;  // a sigmoid score depends on its own logit only
    } else {
      const float s = sigmoidf_(v);
      const float ds = s * (1.0f - s);
      d = normalize ? scale * ds / S * (G - n * A / S) : scale * ds * G;
    }
    out[e] = from_f32<LT>(d);
  }
}

// ---- launch helpers ------------------------------------------------------------

int64_t mtile_bound(int64_t rows, int64_t E) {
  return (rows + kTM - 1) / kTM + std::min<int64_t>(E, rows);
}

template <typename T, bool kAK, bool kBK, int kEpi, bool kGroupK>
void launch_tg(const TrainGemm& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.m_tiles * p.n_tiles * (kGroupK ? p.E : 1);
  if (blocks == 0) return;
  hipLaunchKernelGGL((train_gemm_kernel<T, kAK, kBK, kEpi, kGroupK>), dim3((unsigned)blocks),
                     dim3(kTThreads), 0, s, p);
}

// Operand with one K-segment, or two (p1 and its K offset for segment 1).
TOp opnd(const void* p0, int64_t ld, int64_t estride, const void* p1 = nullptr, int64_t kofs0 = 0,
         int64_t kofs1 = 0) {
  return TOp{{p0, p1 ? p1 : p0}, ld, estride, {kofs0, kofs1}};
}

template <typename T>
hipError_t experts_forward_training_t(const TrainExperts& q, hipStream_t s) {
  const int64_t R = q.rows, H = q.H, I = q.I;
  int32_t* prefix = static_cast<int32_t*>(q.ws);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, q.offsets, q.E, kTM, prefix);
  T* gu = static_cast<T*>(q.cache);
  T* h = gu + R * 2 * I;
  TrainGemm p = {};
  p.offsets = q.offsets; p.tile_prefix = prefix; p.E = q.E;
  p.m_tiles = (int)mtile_bound(R, q.E);
  p.nseg = 1; p.seg_len[0] = H;
  p.N = (int)I; p.n_tiles = (int)((I + kTN - 1) / kTN);
  p.out_split = INT64_MAX; p.ldc = 2 * I;
  p.a = opnd(q.x, H, 0);
  // g = X W_gate^T into columns [0, I) of the cache, u = X W_up^T into [I, 2I)
  p.b = opnd(q.w_gate, H, I * H);
  p.out0 = p.out1 = gu;
  launch_tg<T, true, true, kEpiStore, false>(p, s);
  p.b = opnd(q.w_up, H, I * H);
  p.out0 = p.out1 = gu + I;
  launch_tg<T, true, true, kEpiStore, false>(p, s);
  const int64_t n8 = R * (I / 8);
  hipLaunchKernelGGL(swiglu_cache_kernel<T>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, gu, h, R, (int)I);
  return hipGetLastError();
}

template <typename T>
hipError_t experts_backward_t(const TrainExperts& q, hipStream_t s) {
  const int64_t R = q.rows, H = q.H, I = q.I;
  int32_t* prefix = static_cast<int32_t*>(q.ws);
  T* dgu = reinterpret_cast<T*>(static_cast<char*>(q.ws) + train_prefix_bytes(q.E));
  const T* gu = static_cast<const T*>(q.cache);
  const T* h = gu + R * 2 * I;
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, q.offsets, q.E, kTM, prefix);
  TrainGemm p = {};
  p.offsets = q.offsets; p.tile_prefix = prefix; p.E = q.E;
  p.m_tiles = (int)mtile_bound(R, q.E);
  // dh = dY W_down (W_down [H, I] read along I), fused SwiGLU backward -> dg | du
  p.a = opnd(q.dy, H, 0);
  p.b = opnd(q.w_down, I, H * I);
  p.nseg = 1; p.seg_len[0] = H;
  p.N = (int)I; p.n_tiles = (int)((I + kTN - 1) / kTN);
  p.out0 = dgu; p.gu = gu;
  launch_tg<T, true, false, kEpiSwiGluBwd, false>(p, s);
  // dinput = dg W_gate + du W_up: two K-segments of I (weights [I, H] read along H)
  p.a = opnd(dgu, 2 * I, 0, dgu, 0, I);
  p.b = opnd(q.w_gate, H, I * H, q.w_up, 0, 0);
  p.nseg = 2; p.seg_len[0] = I; p.seg_len[1] = I;
  p.N = (int)H; p.n_tiles = (int)((H + kTN - 1) / kTN);
  p.out0 = p.out1 = q.dx; p.out_split = INT64_MAX; p.ldc = H; p.gu = nullptr;
  launch_tg<T, true, false, kEpiStore, false>(p, s);
  // ddown[e] = dY_e^T h_e  [H, I], K = rows of e
  TrainGemm w = {};
  w.offsets = q.offsets; w.E = q.E; w.nseg = 1;
  w.a = opnd(q.dy, H, 0);
  w.b = opnd(h, I, 0);
  w.M = (int)H; w.N = (int)I;
  w.m_tiles = (int)((H + kTM - 1) / kTM); w.n_tiles = (int)((I + kTN - 1) / kTN);
  w.out0 = w.out1 = q.d_down; w.out_split = INT64_MAX; w.ldc = I; w.out_estride = H * I;
  launch_tg<T, false, false, kEpiStoreF32, true>(w, s);
  // dgate[e] | dup[e] = [dg | du]_e^T X_e  [2I, H], K = rows of e
  w.a = opnd(dgu, 2 * I, 0);
  w.b = opnd(q.x, H, 0);
  w.M = (int)(2 * I); w.N = (int)H;
  w.m_tiles = (int)((2 * I + kTM - 1) / kTM); w.n_tiles = (int)((H + kTN - 1) / kTN);
  w.out0 = q.d_gate; w.out1 = q.d_up; w.out_split = I; w.ldc = H; w.out_estride = I * H;
  launch_tg<T, false, false, kEpiStoreF32, true>(w, s);
  return hipGetLastError();
}

template <typename LT, typename IT>
void launch_router_t(const RouterGrad& r, hipStream_t s) {
  const dim3 grid((unsigned)((r.T + 3) / 4)), block(256);
  if (r.grad_weights)
    hipLaunchKernelGGL((router_backward_kernel<LT, IT>), grid, block, 0, s,
                       static_cast<const LT*>(r.logits), static_cast<const IT*>(r.indices),
                       r.grad_weights, r.T, r.E, r.k, r.scoring, r.normalize, r.scale,
                       static_cast<LT*>(r.grad_logits));
  else
    hipLaunchKernelGGL((router_weights_kernel<LT, IT>), grid, block, 0, s,
                       static_cast<const LT*>(r.logits), static_cast<const IT*>(r.indices), r.T,
                       r.E, r.k, r.scoring, r.normalize, r.scale, r.weights);
}

template <typename LT>
void launch_router_lt(const RouterGrad& r, hipStream_t s) {
  if (r.idx_dt == 0) launch_router_t<LT, uint32_t>(r, s);
  else if (r.idx_dt == 1) launch_router_t<LT, int32_t>(r, s);
  else launch_router_t<LT, int64_t>(r, s);
}

template <typename T, typename WT>
void launch_cb(const void* y, const int32_t* ros, const void* w, const void* go, int T_, int k, int H,
               void* dexp, float* dw, hipStream_t s) {
  hipLaunchKernelGGL((combine_backward_kernel<T, WT>), dim3(T_), dim3(256), 0, s,
                     static_cast<const T*>(y), ros, static_cast<const WT*>(w),
                     static_cast<const T*>(go), k, H, static_cast<T*>(dexp), dw);
}

template <typename T>
void launch_cb_w(const void* y, const int32_t* ros, const void* w, int w_dt, const void* go, int T_,
                 int k, int H, void* dexp, float* dw, hipStream_t s) {
  if (w_dt == kF32) launch_cb<T, float>(y, ros, w, go, T_, k, H, dexp, dw, s);
  else if (w_dt == kF16) launch_cb<T, f16>(y, ros, w, go, T_, k, H, dexp, dw, s);
  else launch_cb<T, bf16>(y, ros, w, go, T_, k, H, dexp, dw, s);
}

}  // namespace

size_t train_prefix_bytes(int64_t E) { return ((size_t)(E + 1) * 4 + 255) / 256 * 256; }

hipError_t launch_experts_forward_training(const TrainExperts& q, hipStream_t s) {
  if (q.rows == 0) return hipSuccess;
  void* h = static_cast<char*>(q.cache) + (size_t)q.rows * 2 * q.I * 2;
  void* scratch = static_cast<char*>(q.ws) + train_prefix_bytes(q.E);
  hipError_t e;
  if (gate_up_can_cache(q.rows, q.E, q.dt))
    // the inference gate/up GEMM, also writing the rounded g and u
    e = launch_gate_up(q.x, nullptr, 1, q.offsets, q.rows, q.E, q.H, q.I, q.w_gate, q.w_up, q.dt, h,
                       scratch, s, q.cache);
  else
    e = q.dt == kF16 ? experts_forward_training_t<f16>(q, s) : experts_forward_training_t<bf16>(q, s);
  if (e != hipSuccess) return e;
  return launch_down(h, q.offsets, q.rows, q.E, q.H, q.I, q.w_down, q.dt, q.y, scratch, s);
}

hipError_t launch_experts_backward(const TrainExperts& q, hipStream_t s) {
  return q.dt == kF16 ? experts_backward_t<f16>(q, s) : experts_backward_t<bf16>(q, s);
}

hipError_t launch_router_grad(const RouterGrad& r, hipStream_t s) {
  if (r.T == 0) return hipSuccess;
  if (r.logits_dt == kF32) launch_router_lt<float>(r, s);
  else if (r.logits_dt == kF16) launch_router_lt<f16>(r, s);
  else launch_router_lt<bf16>(r, s);
  return hipGetLastError();
}

hipError_t launch_combine_backward(const void* y, const int32_t* row_of_slot, const void* w, int w_dt,
                                   const void* grad_out, int T, int k, int H, int dt, void* dexpert,
                                   float* dweights, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dt == kF32) launch_cb_w<float>(y, row_of_slot, w, w_dt, grad_out, T, k, H, dexpert, dweights, s);
  else if (dt == kF16) launch_cb_w<f16>(y, row_of_slot, w, w_dt, grad_out, T, k, H, dexpert, dweights, s);
  else launch_cb_w<bf16>(y, row_of_slot, w, w_dt, grad_out, T, k, H, dexpert, dweights, s);
  return hipGetLastError();
}

hipError_t launch_dispatch_backward(const void* dinput, const int32_t* row_of_slot, int T, int k,
                                    int H, int dt, void* dx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dt == kF32)
    hipLaunchKernelGGL(dispatch_backward_kernel<float>, dim3(T), dim3(256), 0, s,
                       static_cast<const float*>(dinput), row_of_slot, k, H, static_cast<float*>(dx));
  else if (dt == kF16)
    hipLaunchKernelGGL(dispatch_backward_kernel<f16>, dim3(T), dim3(256), 0, s,
                       static_cast<const f16*>(dinput), row_of_slot, k, H, static_cast<f16*>(dx));
  else
    hipLaunchKernelGGL(dispatch_backward_kernel<bf16>, dim3(T), dim3(256), 0, s,
                       static_cast<const bf16*>(dinput), row_of_slot, k, H, static_cast<bf16*>(dx));
  return hipGetLastError();
}

}  // namespace moe
