// Bias-free SwiGLU experts as two grouped GEMMs (ruDNN user guide, "3. MoE
// workflow" and "5. Expert weights and dispatch"):
//   GEMM 1:  h = SiLU(X_e W_gate[e]^T) * (X_e W_up[e]^T)   [n_e, I], K = H
//   GEMM 2:  Y = h W_down[e]^T                              [n_e, H], K = I
// Weights are [E, N, K] with K contiguous, like the rows of X, so both MFMA
// operands are read along K.
//
// Tile list. The rows of expert e are offsets[e]..offsets[e+1]-1 (device
// data). A one-block plan kernel cuts every expert into M-tiles of BM rows and
// writes (expert, first row) per tile plus the tile count; the GEMM grid is
// sized on the host from the bound ceil(rows/BM) + min(E, rows) and
// workgroups past the device tile count exit at once. Expert counts never
// travel to the host.
//
// bf16/f16 kernel (gfx950 MFMA 32x32x16): workgroup tile 256 x 256 x 64, 512
// threads = 8 wavefronts as 4 (M) x 2 (N), 64 x 128 per wavefront. A and B
// tiles are staged through LDS, double-buffered, with a register prefetch of
// the next K-step issued before the current step's MFMAs. LDS rows are 64
// elements (eight 16-byte chunks); chunk c of row r is stored at c ^ (r & 7),
// so the 16-byte fragment reads of eight consecutive rows hit eight distinct
// chunk positions. In GEMM 1 the B tile holds 128 gate rows and the same 128
// up rows, and every wavefront owns matching gate and up accumulators, so
// SiLU(g) * u is formed in registers and only h reaches memory.
//
// Workgroup order: the hardware deals workgroups round-robin to the 8 XCDs;
// the kernel remaps its id so that each XCD receives a contiguous range of
// logical tiles, M-tile fastest, so the workgroups sharing one weight tile run
// on the same XCD and share its L2.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBM = 256;      // rows per M-tile (MFMA path)
constexpr int kBK = 64;       // K per pipeline step
constexpr int kBNB = 256;     // B-tile rows per workgroup
constexpr int kThreads = 512;
constexpr int kBMSimt = 64;   // rows per M-tile (fp32 path)

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E,
                                                     int rows, int bm, int max_tiles,
                                                     int32_t* __restrict__ tiles,
                                                     int32_t* __restrict__ tile_count) {
  const int e = threadIdx.x;
  int lo = 0, n = 0;
  if (e < E) {
    lo = max(offsets[e], 0);
    const int hi = min(offsets[e + 1], rows);
    n = hi > lo ? (hi - lo + bm - 1) / bm : 0;
  }
  int total = 0;
  const int first = block_exclusive_scan(n, &total);
  for (int i = 0; i < n; ++i) {
    const int t = first + i;
    if (t < max_tiles) {
      tiles[2 * t] = e;
      tiles[2 * t + 1] = lo + i * bm;
    }
  }
  if (threadIdx.x == 0) *tile_count = min(total, max_tiles);
}

struct GemmArgs {
  const void* a;           // [*, K] rows of X (or h)
  const int32_t* a_map;    // optional: A row r is a[a_map[r] / a_div]
  int a_div;
  int a_rows;              // rows of `a` when a_map is given (gather bound)
  const void* b0;          // [E, N, K] gate (GEMM 1) or down (GEMM 2)
  const void* b1;          // [E, N, K] up (GEMM 1 only)
  void* c;                 // [rows, N]
  const int32_t* offsets;  // [E+1]
  const int32_t* tiles;    // [max_tiles][2]
  const int32_t* tile_count;
  int rows, N, K, max_tiles, n_tiles_n;
};

template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  typedef bf16x8 Frag;
  static __device__ __forceinline__ f32x16 run(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<f16> {
  typedef f16x8 Frag;
  static __device__ __forceinline__ f32x16 run(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Maps the workgroup id to (M-tile, N-tile); false if this workgroup has no tile.
__device__ __forceinline__ bool tile_of_block(const GemmArgs& p, int& m_t, int& n_t) {
  const int G = gridDim.x;  // multiple of 8
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (G >> 3) + (bid >> 3);
  m_t = logical % p.max_tiles;
  n_t = logical / p.max_tiles;
  if (n_t >= p.n_tiles_n) return false;
  return m_t < *p.tile_count;
}

template <typename T, bool kSwiGlu>
__global__ __launch_bounds__(kThreads) void mfma_gemm_kernel(GemmArgs p) {
  typedef typename Mfma<T>::Frag Frag;
  __shared__ __attribute__((aligned(16))) T lds_a[2][kBM * kBK];
  __shared__ __attribute__((aligned(16))) T lds_b[2][kBNB * kBK];

  int m_t, n_t;
  if (!tile_of_block(p, m_t, n_t)) return;
  const int e = p.tiles[2 * m_t];
  const int row0 = p.tiles[2 * m_t + 1];
  const int row_end = min(p.offsets[e + 1], p.rows);
  const int mrows = min(kBM, row_end - row0);
  if (mrows <= 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // 0..3
  const int wn = wave & 1;   // 0..1
  const int K = p.K;
  const int N = p.N;

  // Global -> LDS copy assignment: thread owns chunk lc of rows lr + 64*i.
  const int lr = tid >> 3;
  const int lc = tid & 7;
  const T* a_ptr[4];
  const T* b_ptr[4];
  const T* A = static_cast<const T*>(p.a);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grow = row0 + min(lr + 64 * i, mrows - 1);
    const int64_t src = p.a_map ? (int64_t)min(max(p.a_map[grow] / p.a_div, 0), p.a_rows - 1)
                                : (int64_t)grow;
    a_ptr[i] = A + src * K + lc * 8;
    const int brow = lr + 64 * i;
    int n;
    const T* base;
    if (kSwiGlu) {
      n = n_t * (kBNB / 2) + (brow & (kBNB / 2 - 1));
      base = static_cast<const T*>(brow < kBNB / 2 ? p.b0 : p.b1);
    } else {
      n = n_t * kBNB + brow;
      base = static_cast<const T*>(p.b0);
    }
    n = min(n, N - 1);
    b_ptr[i] = base + ((int64_t)e * N + n) * K + lc * 8;
  }
  int st_off[4];  // swizzled LDS element offset of this thread's chunks
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lr + 64 * i;
    st_off[i] = r * kBK + ((lc ^ (r & 7)) * 8);
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  uint4 ra[4], rb[4];
  auto load_step = [&](int kt) {
    const int k0 = kt * kBK;
    const bool ok = k0 + lc * 8 < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ok ? *reinterpret_cast<const uint4*>(a_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = ok ? *reinterpret_cast<const uint4*>(b_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(&lds_a[buf][st_off[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&lds_b[buf][st_off[i]]) = rb[i];
    }
  };

  // Fragment rows of this wavefront (MFMA A: lane holds row lane%32; B: lane
  // holds column lane%32, i.e. weight row).
  int a_row[2], b_row[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) a_row[mb] = wm * 64 + mb * 32 + (lane & 31);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    if (kSwiGlu)
      b_row[nb] = (nb >> 1) * (kBNB / 2) + wn * 64 + (nb & 1) * 32 + (lane & 31);
    else
      b_row[nb] = wn * 128 + nb * 32 + (lane & 31);
  }
  const int sw = lane & 7;  // == row & 7 for every fragment row above

  const int nk = (K + kBK - 1) / kBK;
  load_step(0);
  store_step(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_step(kt + 1);
    const T* la = lds_a[cur];
    const T* lb = lds_b[cur];
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int c = ((2 * s + (lane >> 5)) ^ sw) * 8;
      Frag fa[2], fb[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) fa[mb] = *reinterpret_cast<const Frag*>(la + a_row[mb] * kBK + c);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) fb[nb] = *reinterpret_cast<const Frag*>(lb + b_row[nb] * kBK + c);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = Mfma<T>::run(fa[mb], fb[nb], acc[mb][nb]);
    }
    if (kt + 1 < nk) store_step(cur ^ 1);
    __syncthreads();
  }

  // Epilogue. Accumulator element v of lane l sits at row
  // (v/4)*8 + (l/32)*4 + v%4 and column l%32 of its 32x32 block.
  T* C = static_cast<T*>(p.c);
  const int col_lane = lane & 31;
  const int row_lane = (lane >> 5) * 4;
  if (kSwiGlu) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n_t * (kBNB / 2) + wn * 64 + nb * 32 + col_lane;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lrow = wm * 64 + mb * 32 + (v >> 2) * 8 + row_lane + (v & 3);
          if (lrow < mrows && col < N)
            C[(int64_t)(row0 + lrow) * N + col] =
                from_f32<T>(silu(acc[mb][nb][v]) * acc[mb][nb + 2][v]);
        }
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = n_t * kBNB + wn * 128 + nb * 32 + col_lane;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lrow = wm * 64 + mb * 32 + (v >> 2) * 8 + row_lane + (v & 3);
          if (lrow < mrows && col < N)
            C[(int64_t)(row0 + lrow) * N + col] = from_f32<T>(acc[mb][nb][v]);
        }
      }
  }
}

// fp32 path on the vector ALUs: tile 64 x 64 outputs, K step 16, 256 threads
// with 4 x 4 outputs each (gate and up accumulators in GEMM 1).
template <bool kSwiGlu>
__global__ __launch_bounds__(256) void simt_gemm_kernel(GemmArgs p) {
  constexpr int BN = 64, BK = 16, BNB = kSwiGlu ? 2 * BN : BN;
  __shared__ float sa[BK][kBMSimt + 4];
  __shared__ float sb[BK][BNB + 4];

  int m_t, n_t;
  if (!tile_of_block(p, m_t, n_t)) return;
  const int e = p.tiles[2 * m_t];
  const int row0 = p.tiles[2 * m_t + 1];
  const int mrows = min(kBMSimt, min(p.offsets[e + 1], p.rows) - row0);
  if (mrows <= 0) return;
  const int K = p.K, N = p.N, tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  const float* A = static_cast<const float*>(p.a);

  // A loader: row tid/4, four k values (tid%4)*4.
  const int arow = tid / 4, akq = (tid % 4) * 4;
  const int grow = row0 + min(arow, mrows - 1);
  const int64_t asrc = p.a_map ? (int64_t)min(max(p.a_map[grow] / p.a_div, 0), p.a_rows - 1)
                                : (int64_t)grow;
  const float* a_ptr = A + asrc * K + akq;
  // B loader: rows tid/4 and 64 + tid/4 (GEMM 1: gate then up).
  const float* b_ptr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int brow = arow + 64 * i;
    int n;
    const float* base;
    if (kSwiGlu) {
      n = n_t * BN + (brow & (BN - 1));
      base = static_cast<const float*>(brow < BN ? p.b0 : p.b1);
    } else {
      n = n_t * BN + brow;
      base = static_cast<const float*>(p.b0);
    }
    n = min(n, N - 1);
    b_ptr[i] = base + ((int64_t)e * N + n) * K + akq;
  }

  float accg[4][4] = {}, accu[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool ok = k0 + akq < K;
    const float4 av = ok ? *reinterpret_cast<const float4*>(a_ptr + k0) : make_float4(0, 0, 0, 0);
    sa[akq + 0][arow] = av.x; sa[akq + 1][arow] = av.y; sa[akq + 2][arow] = av.z; sa[akq + 3][arow] = av.w;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i == 1 && BNB == BN) break;
      const float4 bv = ok ? *reinterpret_cast<const float4*>(b_ptr[i] + k0) : make_float4(0, 0, 0, 0);
      const int br = arow + 64 * i;
      sb[akq + 0][br] = bv.x; sb[akq + 1][br] = bv.y; sb[akq + 2][br] = bv.z; sb[akq + 3][br] = bv.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], bg[4], bu[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sa[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bg[j] = sb[kk][tx * 4 + j];
        bu[j] = kSwiGlu ? sb[kk][BN + tx * 4 + j] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          accg[i][j] = fmaf(a[i], bg[j], accg[i][j]);
          if (kSwiGlu) accu[i][j] = fmaf(a[i], bu[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
  float* C = static_cast<float*>(p.c);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lrow = ty * 4 + i;
    if (lrow >= mrows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n_t * BN + tx * 4 + j;
      if (col < N)
        C[(int64_t)(row0 + lrow) * N + col] = kSwiGlu ? silu(accg[i][j]) * accu[i][j] : accg[i][j];
    }
  }
}

inline int round_up8(int64_t g) { return (int)((g + 7) / 8 * 8); }

}  // namespace

ExpertsPlan experts_plan(int64_t rows, int64_t E, int dt) {
  ExpertsPlan p;
  p.bm = dt == kF32 ? kBMSimt : kBM;
  p.max_tiles = (int)((rows + p.bm - 1) / p.bm + (E < rows ? E : rows));
  return p;
}

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

size_t tile_scratch_bytes(int64_t rows, int64_t E, int dt) {
  const ExpertsPlan p = experts_plan(rows, E, dt);
  return align256((size_t)p.max_tiles * 2 * sizeof(int32_t)) + 256;
}

size_t experts_scratch_bytes(int64_t rows, int64_t E, int64_t I, int dt) {
  return tile_scratch_bytes(rows, E, dt) + align256((size_t)rows * (size_t)I * dtype_size(dt));
}

namespace {

// Carves the tile list out of `scratch` and enqueues the plan kernel.
GemmArgs plan_tiles(const int32_t* offsets, int rows, int E, int dt, void* scratch,
                    hipStream_t s) {
  const ExpertsPlan plan = experts_plan(rows, E, dt);
  char* ws = static_cast<char*>(scratch);
  GemmArgs g = {};
  int32_t* tiles = reinterpret_cast<int32_t*>(ws);
  int32_t* tile_count = reinterpret_cast<int32_t*>(ws + align256((size_t)plan.max_tiles * 2 * sizeof(int32_t)));
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, E, rows, plan.bm,
                     plan.max_tiles, tiles, tile_count);
  g.offsets = offsets;
  g.tiles = tiles;
  g.tile_count = tile_count;
  g.rows = rows;
  g.max_tiles = plan.max_tiles;
  return g;
}

template <bool kSwiGlu>
void launch_gemm(const GemmArgs& g, int dt, hipStream_t s) {
  const dim3 grid(round_up8((int64_t)g.max_tiles * g.n_tiles_n));
  if (dt == kF32)
    hipLaunchKernelGGL(simt_gemm_kernel<kSwiGlu>, grid, dim3(256), 0, s, g);
  else if (dt == kF16)
    hipLaunchKernelGGL((mfma_gemm_kernel<f16, kSwiGlu>), grid, dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL((mfma_gemm_kernel<bf16, kSwiGlu>), grid, dim3(kThreads), 0, s, g);
}

int n_tiles(int N, int dt, bool swiglu) {
  const int bn = dt == kF32 ? 64 : (swiglu ? kBNB / 2 : kBNB);
  return (N + bn - 1) / bn;
}

void setup_gate_up(GemmArgs& g, const void* a, const int32_t* a_map, int a_div, int H, int I,
                   const void* w_gate, const void* w_up, int dt, void* h) {
  g.a = a; g.a_map = a_map; g.a_div = a_div > 0 ? a_div : 1;
  g.a_rows = (g.rows + g.a_div - 1) / g.a_div;
  g.b0 = w_gate; g.b1 = w_up; g.c = h;
  g.N = I; g.K = H; g.n_tiles_n = n_tiles(I, dt, true);
}

void setup_down(GemmArgs& g, const void* h, int H, int I, const void* w_down, int dt,
                void* expert_out) {
  g.a = h; g.a_map = nullptr; g.a_div = 1;
  g.b0 = w_down; g.b1 = nullptr; g.c = expert_out;
  g.N = H; g.K = I; g.n_tiles_n = n_tiles(H, dt, false);
}

}  // namespace

hipError_t launch_gate_up(const void* a, const int32_t* a_map, int a_div, const int32_t* offsets,
                          int rows, int E, int H, int I, const void* w_gate, const void* w_up,
                          int dt, void* h, void* scratch, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  GemmArgs g = plan_tiles(offsets, rows, E, dt, scratch, s);
  setup_gate_up(g, a, a_map, a_div, H, I, w_gate, w_up, dt, h);
  launch_gemm<true>(g, dt, s);
  return hipGetLastError();
}

hipError_t launch_down(const void* h, const int32_t* offsets, int rows, int E, int H, int I,
                       const void* w_down, int dt, void* expert_out, void* scratch,
                       hipStream_t s) {
  if (rows == 0) return hipSuccess;
  GemmArgs g = plan_tiles(offsets, rows, E, dt, scratch, s);
  setup_down(g, h, H, I, w_down, dt, expert_out);
  launch_gemm<false>(g, dt, s);
  return hipGetLastError();
}

hipError_t launch_experts(const void* a, const int32_t* a_map, int a_div,
                          const int32_t* offsets, int rows, int E, int H, int I,
                          const void* w_gate, const void* w_up, const void* w_down, int dt,
                          void* expert_out, void* scratch, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  void* h = static_cast<char*>(scratch) + tile_scratch_bytes(rows, E, dt);
  GemmArgs g1 = plan_tiles(offsets, rows, E, dt, scratch, s);
  GemmArgs g2 = g1;
  setup_gate_up(g1, a, a_map, a_div, H, I, w_gate, w_up, dt, h);
  setup_down(g2, h, H, I, w_down, dt, expert_out);
  launch_gemm<true>(g1, dt, s);
  launch_gemm<false>(g2, dt, s);
  return hipGetLastError();
}

}  // namespace moe
