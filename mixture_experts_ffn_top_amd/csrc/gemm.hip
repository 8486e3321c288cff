// Bias-free SwiGLU experts as two grouped GEMMs (ruDNN user guide, "3. MoE
// workflow" and "5. Expert weights and dispatch"):
//   GEMM 1:  h = SiLU(X_e W_gate[e]^T) * (X_e W_up[e]^T)   [n_e, I], K = H
//   GEMM 2:  Y = h W_down[e]^T                              [n_e, H], K = I
// Weights are [E, N, K] with K contiguous, like the rows of X, so both MFMA
// operands are read along K.
//
// Schedule. The rows of expert e are offsets[e]..offsets[e+1]-1 (device
// data). A plan kernel cuts every expert into M-tiles of BM rows
// and writes, for every workgroup of the GEMM grid, one 16-byte entry
// (expert and K-split, first row, end row, N-tile) or "no tile". The grid is
// sized on the host from the bound ceil(rows/BM) + min(E, rows) on the
// M-tile count; workgroups without a tile exit at once. Expert counts never
// travel to the host.
//
// Order of the schedule (schedule.h). The hardware deals workgroups
// round-robin to the 8 XCDs (each with its own L2), so workgroup b runs on
// XCD b % 8, and each XCD starts its workgroups in the order b / 8. The plan
// gives XCD x a contiguous slice of the tile list, so the ~32 workgroups
// resident on one XCD at a time are neighbours in the list. Inside an expert
// the list takes groups of up to 8 M-tiles, and inside such a group runs of
// N-tiles wide enough that one run covers about 8 tiles (4 M-tiles x 2
// N-tiles, 8 x 1, 1 x 8 ...), N first inside a run: the ~32 tiles resident
// together (four consecutive runs) share their weight tiles and activation
// tiles through that XCD's L2, and a run never mixes two experts' weights.
// (Runs of 8 measured about 1 % faster than one run of 32 covering the same
// tiles.)
//
// bf16/f16 kernel (gfx950 MFMA 32x32x16), two tile shapes:
//  - 256 x kBNB tiles, 512 threads = 8 wavefronts as 4 (M) x 2 (N), 64 x
//    kBNB/2 outputs per wavefront, K = 64 a stage, two 32 KB stages of the
//    activation tile and three of the weight tile (160 KB): k-step kt
//    requests the activations of kt+1 and the weights of kt+2;
//  - weight streaming (at most 128 rows an expert on average, where the
//    weights are read about once per 128 rows and the stream of weight tiles
//    sets the time): 128 x kBNB tiles, 8 wavefronts of 32 x kBNB/2 outputs,
//    three 48 KB stages, the loads of k-step kt+2 issued at the top of kt, so
//    two k-steps of weights are in flight per CU instead of one.
// Global tiles go straight into LDS with buffer loads (buffer_load_dwordx4 ...
// lds): each lane's 16 bytes land at LDS base + 16 * lane, so the swizzle is
// applied by choosing which global chunk each lane fetches. A load past the
// buffer's byte count returns zeros, which covers the N tail of the weights,
// A rows past the expert's last row and (with a deliberately out-of-range
// offset) the K tail. A stage is waited for (vmcnt) only just before the
// barrier that precedes its first read. Fragment registers are
// double-buffered across the k16 sub-steps of a stage so LDS reads overlap
// MFMAs.
//
// LDS rows are 64 elements (eight 16-byte chunks, 128 bytes). gfx950 serves
// a 128-bit LDS read 16 lanes per cycle across 64 banks (two 128-byte rows),
// so the 16 rows read together must cover all 16 (row mod 2, chunk) slots:
// chunk c of row r is stored at c ^ ((r >> 1) & 7).
//
// Split-K of the last round (GEMM 2): the tiles left over after the full
// rounds of workgroups are split along K, each K range written as fp32
// partial sums to a block of its own; a separate pass adds them in K-range
// order, so results do not depend on scheduling. Every other tile covers all
// of K and stores its output directly.
//
// In GEMM 1 the B tile holds 128 gate rows and the same 128 up rows, and
// every wavefront owns matching gate and up accumulators, so SiLU(g) * u is
// formed in registers and only h reaches memory.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "schedule.h"


namespace moe {
namespace {

constexpr int kBM = 256;      // rows per M-tile (MFMA path)
constexpr int kBK = 64;       // K per LDS stage
constexpr int kBMSimt = 64;   // rows per M-tile (fp32 path)
constexpr int kXcds = sched::kXcds;
// Third dword of a raw buffer resource on gfx9-family parts (no format, no swizzle).
constexpr int kRsrcFlags = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;  // voffset past any buffer we build (< 2^31 bytes)

// One schedule entry per slot: x = expert | (K-range << 16) | (K-ranges of
// the tile << 20), y = first row, z = end row (exclusive), w = N-tile | (index
// of a split tile among the last round's << 16); x < 0: no tile. The list,
// its XCD slices and the split of the last round are those of schedule.h.
// With a split last round, split[0] = (r, s) and split[1 + u] = (expert,
// first row, end row, N-tile) of split tile u, for the reduction of its
// partial sums; split[0].y = 1 otherwise.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E,
                                                     int rows, int bm, int max_tiles,
                                                     int n_tiles_n, int cap, int costed, int wgs, int grid,
                                                     int4* __restrict__ sched, int4* __restrict__ split) {
  __shared__ int s_first[kMaxExperts + 1], s_cfirst[kMaxExperts + 1], s_lo[kMaxExperts], s_hi[kMaxExperts];
  const int e = threadIdx.x;
  int lo = 0, hi = 0, n = 0;
  if (e < E) {
    lo = max(offsets[e], 0);
    hi = min(offsets[e + 1], rows);
    n = hi > lo ? (hi - lo + bm - 1) / bm : 0;
  }
  int total = 0, ctotal = 0;
  const int first = block_exclusive_scan(n, &total);
  const int cfirst = block_exclusive_scan(costed ? sched::expert_cost(hi - lo, bm, n_tiles_n) : 0, &ctotal);
  if (e < E) {
    s_first[e] = first;
    s_cfirst[e] = cfirst;
    s_lo[e] = lo;
    s_hi[e] = hi;
  }
  if (e == 0) {
    s_first[E] = total;
    s_cfirst[E] = ctotal;
  }
  __syncthreads();
  sched::Table t;
  t.first = s_first;
  t.lo = s_lo;
  t.hi = s_hi;
  t.cfirst = nullptr;
  t.E = E;
  t.bm = bm;
  t.n_tiles_n = n_tiles_n;
  t.tiles = min(total, max_tiles) * n_tiles_n;
  const sched::Rounds d = sched::rounds_of(t, wgs, cap);
  if (costed && d.s == 1) t.cfirst = s_cfirst;  // slices of equal cost
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < grid; b += gridDim.x * blockDim.x) {
    sched::Entry en;
    int4 v = make_int4(-1, 0, 0, 0);
    if (sched::slot_entry(t, d, b, &en))
      v = make_int4(en.ex | (en.ks << 16) | (en.s << 20), en.row0, en.row_end, en.n_t | (en.u << 16));
    sched[b] = v;
  }
  if (split != nullptr && blockIdx.x == 0) {
    if (threadIdx.x == 0) split[0] = make_int4(d.r, d.s, 0, 0);
    if (d.s > 1)
      for (int u = threadIdx.x; u < d.r; u += blockDim.x) {
        const sched::Entry en = sched::entry_at(t, d.q * d.W + u);
        split[1 + u] = make_int4(en.ex, en.row0, en.row_end, en.n_t);
      }
  }
}

struct GemmArgs {
  const void* a;           // [a_rows, K] rows of X (or h)
  const int32_t* a_map;    // optional: A row r is a[a_map[r] / a_div]
  int a_div;
  int a_rows;              // rows of `a`
  const void* b0;          // [E, N, K] gate (GEMM 1) or down (GEMM 2)
  const void* b1;          // [E, N, K] up (GEMM 1 only)
  void* c;                 // [rows, N]
  const int32_t* offsets;  // [E+1]
  const int4* sched;       // [grid] entries written by plan_kernel
  int rows, N, K, max_tiles, n_tiles_n, grid;
  int wgs;  // workgroups of the persistent MFMA kernel (a multiple of 8)
  int bm;   // rows per M-tile of the schedule (selects the kernel's tile shape)
  // GEMM 2 only: a tile of the last round whose K is split s ways writes the
  // fp32 partial sums of K-range ks to partial + (u * s + ks) * bm * 256, a
  // bm x 256 block (u: its index among the split tiles); they are added in
  // K-range order afterwards.
  float* partial;
  // GEMM 1 of the experts' training forward: also store g and u, rounded to
  // T, into cache[rows, 2N] = (g | u), and form h from those rounded values.
  void* cache;
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

// SiLU with the hardware reciprocal (1 ulp) in place of a full division.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

inline int64_t grid_tiles(int64_t max_tiles, int64_t n_tiles_n) {
  return (max_tiles * n_tiles_n + kXcds - 1) / kXcds * kXcds;
}

struct Tile {
  int e, ks, s, u, row0, row_end, n_t;
};

// Schedule entry v (wave-uniform); false past the grid or if it holds no tile.
__device__ __forceinline__ bool tile_of_block(const GemmArgs& p, int v, Tile& t) {
  if (v >= p.grid) return false;
  const int4 e = p.sched[v];
  const int x = __builtin_amdgcn_readfirstlane(e.x);
  if (x < 0) return false;
  t.e = x & 0xFFFF;
  t.ks = (x >> 16) & 0xF;
  t.s = x >> 20;
  t.row0 = __builtin_amdgcn_readfirstlane(e.y);
  t.row_end = __builtin_amdgcn_readfirstlane(e.z);
  const int w = __builtin_amdgcn_readfirstlane(e.w);
  t.n_t = w & 0xFFFF;
  t.u = w >> 16;
  return t.row0 < t.row_end;
}

// One butterfly round of a 4 x 4 transpose across the lanes of a quad: the
// lane swaps with lane ^ kBit the two values whose index bit kBit differs
// from its own lane bit, through a quad-permute DPP move.
template <int kBit>
__device__ __forceinline__ void transpose4_round(float (&x)[4], int lane) {
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

// 4 x 4 transpose across the 4 lanes of each quad: on return x[c] of lane j
// holds what x[j] of lane c held.
__device__ __forceinline__ void transpose4(float (&x)[4], int lane) {
  transpose4_round<1>(x, lane);
  transpose4_round<2>(x, lane);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds, uint32_t voffset,
                                           uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds, 16, voffset, soffset, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One LDS object per (operand, stage): with distinct objects the compiler's
// wait-count pass can tell that an LDS-DMA load into one stage does not
// alias fragment reads from another, and does not stall the reads on vmcnt.
template <typename T, int kElems, int kOperand, int kStage>
__device__ __forceinline__ T* stage_buf() {
  __shared__ __attribute__((aligned(1024))) T buf[kElems];
  return buf;
}

// LDS slot of 16-byte chunk c in row r is c ^ swizzle(r). A 128-bit LDS
// read is served 16 lanes at a time, and the MFMA fragment reads of those 16
// lanes touch 16 consecutive rows at one logical chunk, so the slots must
// fall in 16 distinct 16-byte bank groups of the 256-byte bank window:
//  - 64-byte rows (4 chunks): a window holds 4 rows; rows r..r+3 differ in
//    r & 3, and (r >> 2) & 3 spreads the four 4-row groups over the chunks.
//  - 128-byte rows (8 chunks): a window holds 2 rows; (r >> 1) & 7 gives the
//    8 even and the 8 odd rows of a 16-row group 8 distinct chunks each.
template <int kChunksT>
__device__ __forceinline__ int swizzle(int r) {
  static_assert(kChunksT == 4 || kChunksT == 8, "64- or 128-byte LDS rows");
  return kChunksT == 4 ? (r >> 2) & 3 : (r >> 1) & 7;
}

// kWaveM: rows per wavefront, 64 (8 wavefronts, 4 x 2) or 128 (4 wavefronts,
// 2 x 2; 256 accumulators per lane, one wavefront per SIMD).
template <int kWaveM, int kBMt = kBM>
constexpr int gemm_threads() { return 64 * (kBMt / kWaveM) * 2; }

// Persistent grouped GEMM. The grid holds one workgroup per CU; workgroup b
// takes schedule entries b, b + G, b + 2G, ... (G = grid size, a multiple of
// 8, so every entry it takes belongs to its own XCD's slice of the list).
//
// K is staged kBKT (64) elements at a time through LDS stages. A stage row
// is 128 bytes, and each buffer load instruction fills 8 rows with 128-byte
// row segments, which move through the load path about twice as fast as
// 64-byte ones. 256-row tiles: two A stages and three B stages; k-step kt
// requests A(kt+1) and B(kt+2) at its top, and the barrier that ends it
// waits for A(kt+1) and B(kt+1) only. 128-row tiles: three stages of both;
// the loads of k-step kt+2 are issued at the top of k-step kt.
//
// Between tiles: once every wavefront has finished reading LDS, the first
// stage of the next tile is requested, and only then are the finished
// tile's results written out, so the store traffic overlaps the next tile's
// first loads instead of leaving the CU idle.
template <typename T, bool kSwiGlu, int kBNB, int kBKT, int kWaveM, bool kCache = false, int kBMt = kBM,
          int kStg = 2>
__global__ __launch_bounds__((gemm_threads<kWaveM, kBMt>())) void mfma_gemm_kernel(GemmArgs p) {
  typedef typename Mfma<T>::Frag Frag;
  static_assert((kStg == 2 && kBMt == 256) || (kStg == 3 && kBMt == 128),
                "256-row tiles (2 activation + 3 weight stages) or 128-row tiles (3 + 3)");
  constexpr int kWaves = (kBMt / kWaveM) * 2;
  constexpr int kThreadsK = 64 * kWaves;
  constexpr int kCh = kBKT / 8;                       // 16-byte chunks per LDS row
  constexpr int kRowsPerInst = 64 / kCh;              // rows filled by one load instruction
  constexpr int kSub = kBKT / 16;                     // MFMA k16 sub-steps per stage
  constexpr int kMB = kWaveM / 32;                    // 32-row blocks per wavefront
  constexpr int kNB = kBNB / 64;                      // 32-column blocks per wavefront
  constexpr int kLoadsA = kBMt * kCh / kThreadsK;     // 16-byte chunks per thread per stage
  constexpr int kLoadsB = kBNB * kCh / kThreadsK;
  constexpr int kLoads = kLoadsA + kLoadsB;
  static_assert(!kSwiGlu || kBNB == 256, "fused gate/up uses 128 + 128 B rows");
  static_assert(kSub >= 2, "at least two k16 sub-steps per stage");
  static_assert((kBNB / 2) % (kWaves * kRowsPerInst) == 0, "gate/up split between instructions");
  // 256 x 256 tiles with two stages and no training cache: the MFMAs take
  // the weight fragment as their row operand, so that each lane's 16
  // accumulators of a 32 x 32 block hold one output row (token) and four
  // runs of four consecutive output columns; the epilogue stages the block
  // through the LDS stage that holds no k-step between two tiles and stores
  // 16-byte row chunks (split-K partials go out directly, four fp32 at a
  // time). The other shapes keep the token fragment as row operand and
  // transpose in registers.
  constexpr bool kLdsEpi = kStg == 2 && !kCache && kBMt == 256 && kWaveM == 64 && kBNB == 256;
  // 256-row tiles: two A stages and three B stages (160 KB of LDS), so that
  // weight tiles, which mostly come from HBM, are requested two k-steps
  // ahead and activation tiles, which mostly hit the caches, one. 128-row
  // tiles: three stages of both (step / main_loop below).
  constexpr bool kB3 = kStg == 2;

  int v = blockIdx.x;
  Tile tile;
  if (!tile_of_block(p, v, tile)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;  // 0 .. kWaves/2 - 1
  const int wn = wave & 1;   // 0..1
  const int K = p.K;
  const int N = p.N;
  const uint32_t row_bytes = (uint32_t)K * sizeof(T);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.a), (short)0, (int)((uint32_t)p.a_rows * row_bytes), kRsrcFlags);
  const int b_bytes = (int)((uint32_t)N * row_bytes);

  // Copy assignment: instruction j of wavefront w fills LDS chunks
  // (j*kWaves + w)*64 + lane, i.e. row (j*kWaves + w)*kRowsPerInst +
  // lane/kCh, slot lane%kCh; the lane fetches the global chunk that the
  // swizzle puts in that slot. The slot's chunk is the same for every j.
  const int c_lane = (lane % kCh) ^ swizzle<kCh>(wave * kRowsPerInst + lane / kCh);
  const int kc = c_lane * 8;  // element offset of this lane's chunk within a stage

  // Per-tile load state.
  // the expert's weight bases (the buffer resources are rebuilt at each
  // use from these scalars)
  const T* wb0;
  const T* wb1;
  uint32_t vo_a[kLoadsA], vo_b[kLoadsB];
  int e, ks, ts, tu, row0, n_t, mrows, k_begin, k_end;
  // Source rows of this lane's A chunks (through the row map when there is
  // one). Fetched for the next tile at the start of the current one, so the
  // map's latency is hidden behind its k-steps.
  auto a_src = [&](const Tile& t, int (&src)[kLoadsA]) {
    const int mr = min(kBMt, t.row_end - t.row0);
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
      const int r = (j * kWaves + wave) * kRowsPerInst + lane / kCh;
      const int grow = t.row0 + min(r, mr - 1);
      src[j] = p.a_map ? min(max(p.a_map[grow] / p.a_div, 0), p.a_rows - 1) : grow;
    }
  };
  auto setup = [&](const Tile& t, const int (&src)[kLoadsA]) {
    e = t.e; ks = t.ks; ts = t.s; tu = t.u; row0 = t.row0; n_t = t.n_t;
    mrows = min(kBMt, t.row_end - row0);
    sched::k_range(K, kBKT, ks, ts, &k_begin, &k_end);
    const int64_t expert_elems = (int64_t)e * N * K;
    wb0 = static_cast<const T*>(p.b0) + expert_elems;
    wb1 = kSwiGlu ? static_cast<const T*>(p.b1) + expert_elems : wb0;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
      const int r = (j * kWaves + wave) * kRowsPerInst + lane / kCh;
      // rows past the expert's last row are not fetched (they read as zero)
      vo_a[j] = r < mrows ? (uint32_t)src[j] * row_bytes + (uint32_t)c_lane * 16u : kOutOfRange;
    }
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j) {
      const int r = (j * kWaves + wave) * kRowsPerInst + lane / kCh;
      // rows past N fall beyond the buffer and read as zero
      const int n = kSwiGlu ? n_t * (kBNB / 2) + (r & (kBNB / 2 - 1)) : n_t * kBNB + r;
      vo_b[j] = (uint32_t)n * row_bytes + (uint32_t)c_lane * 16u;
    }
  };

  auto issue_a = [&](int kt, T* la) __attribute__((always_inline)) {
    const int k0 = k_begin + kt * kBKT;
    const uint32_t soff = (uint32_t)k0 * sizeof(T);
    const bool in_k = k0 + kc < k_end;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j)
      load_lds16(rsrc_a, la + (j * kWaves + wave) * 64 * 8, in_k ? vo_a[j] : kOutOfRange, soff);
  };
  auto issue_b = [&](int kt, T* lb) __attribute__((always_inline)) {
    const int k0 = k_begin + kt * kBKT;
    const uint32_t soff = (uint32_t)k0 * sizeof(T);
    const bool in_k = k0 + kc < k_end;
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j)
      load_lds16(__builtin_amdgcn_make_buffer_rsrc(
                     const_cast<T*>(kSwiGlu && j * kWaves * kRowsPerInst >= kBNB / 2 ? wb1 : wb0), (short)0,
                     b_bytes, kRsrcFlags),
                 lb + (j * kWaves + wave) * 64 * 8, in_k ? vo_b[j] : kOutOfRange, soff);
  };
  auto issue_loads = [&](int kt, T* la, T* lb) {
    const int k0 = k_begin + kt * kBKT;
    const uint32_t soff = (uint32_t)k0 * sizeof(T);
    const bool in_k = k0 + kc < k_end;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j)
      load_lds16(rsrc_a, la + (j * kWaves + wave) * 64 * 8, in_k ? vo_a[j] : kOutOfRange, soff);
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j)
      // fused gate/up: B rows 0..127 come from gate, 128..255 from up; the
      // split falls between instructions
      load_lds16(__builtin_amdgcn_make_buffer_rsrc(
                     const_cast<T*>(kSwiGlu && j * kWaves * kRowsPerInst >= kBNB / 2 ? wb1 : wb0), (short)0,
                     b_bytes, kRsrcFlags),
                 lb + (j * kWaves + wave) * 64 * 8, in_k ? vo_b[j] : kOutOfRange, soff);
  };

  // Fragment rows of this wavefront (MFMA A: lane holds row lane%32; B: lane
  // holds column lane%32, i.e. weight row). All block bases are multiples of
  // 32, so every fragment row has the same swizzle as row lane%32.
  int a_row[kMB], b_row[kNB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) a_row[mb] = (wm * kWaveM + mb * 32 + (lane & 31)) * kBKT;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int r = kSwiGlu ? (nb >> 1) * (kBNB / 2) + wn * 64 + (nb & 1) * 32 + (lane & 31)
                          : wn * (kBNB / 2) + nb * 32 + (lane & 31);
    b_row[nb] = r * kBKT;
  }
  const int sw = swizzle<kCh>(lane & 31);

  f32x16 acc[kMB][kNB];
  Frag fa[2][kMB], fb[2][kNB];
  auto read_frags = [&](const T* la, const T* lb, int s, int slot) __attribute__((always_inline)) {
    const int c = ((2 * s + (lane >> 5)) ^ sw) * 8;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) fa[slot][mb] = *reinterpret_cast<const Frag*>(la + a_row[mb] + c);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) fb[slot][nb] = *reinterpret_cast<const Frag*>(lb + b_row[nb] + c);
  };
  auto mfmas = [&](int slot, int from, int to) __attribute__((always_inline)) {
#pragma unroll
    for (int i = from; i < to; ++i) {
      if constexpr (kLdsEpi)
        acc[i / kNB][i % kNB] = Mfma<T>::run(fb[slot][i % kNB], fa[slot][i / kNB], acc[i / kNB][i % kNB]);
      else
        acc[i / kNB][i % kNB] = Mfma<T>::run(fa[slot][i / kNB], fb[slot][i % kNB], acc[i / kNB][i % kNB]);
    }
  };
  constexpr int kMfma = kMB * kNB;   // MFMAs per k16 sub-step
  constexpr int kReads = kMB + kNB;  // fragment reads per sub-step

  // 128-row tiles, one K-stage: compute from stage S while stage L is
  // refilled for k-step kt+2 (none in the tile's last two padded steps). The
  // barrier is a plain s_barrier (a scheduling boundary): a fenced
  // __syncthreads would make the compiler drain every LDS-DMA load in flight.
  // Order: [loads, sub-step s MFMAs interleaved with sub-step s+1 fragment
  // reads ..., half of the last sub-step] wait + barrier [next stage's
  // sub-step 0 fragment reads overlapping the other half of the last
  // sub-step]. A wavefront whose rows all lie past the expert's last row
  // (short M-tiles) runs the same loads and barriers without reads or MFMAs.
  auto step = [&](auto stage, auto compute, int kt, int nk_pad) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    constexpr bool kCompute = decltype(compute)::value;
    constexpr int X = (S + 1) % kStg;        // stage read next
    constexpr int L = (S + kStg - 1) % kStg; // stage refilled now, for k-step kt + kStg - 1
    T* ca = stage_buf<T, kBMt * kBKT, 0, S>();
    T* cb = stage_buf<T, kBNB * kBKT, 1, S>();
    const bool refill = kt + kStg - 1 < nk_pad;
    if (refill) issue_loads(kt + kStg - 1, stage_buf<T, kBMt * kBKT, 0, L>(), stage_buf<T, kBNB * kBKT, 1, L>());
    // Stage X (k-step kt+1) must have landed by the barrier; the loads just
    // issued for kt+2 may stay in flight.
    auto wait_next = [&]() {
      if (refill)
        wait_vmem<kLoads>();
      else
        wait_vmem<0>();
    };
    if constexpr (!kCompute) {
      wait_next();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      return;
    }
#pragma unroll
    for (int sub = 0; sub + 1 < kSub; ++sub) {
      read_frags(ca, cb, sub + 1, (sub + 1) & 1);
      mfmas(sub & 1, 0, kMfma);
#pragma unroll
      for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (sub == 0 && i < kLoads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if (i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    constexpr int kLast = (kSub - 1) & 1;
    mfmas(kLast, 0, kMfma / 2);
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma / 2, 0);
    // MFMAs are not memory operations and would otherwise drift across the
    // barrier, leaving too few of them to cover the next stage's reads.
    __builtin_amdgcn_sched_barrier(0);
    wait_next();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    read_frags(stage_buf<T, kBMt * kBKT, 0, X>(), stage_buf<T, kBNB * kBKT, 1, X>(), 0, 0);
    mfmas(kLast, kMfma / 2, kMfma);
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i < kMfma / 2) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  // Three B stages: k-step kt reads A slot kt % 2 and B slot kt % 3,
  // requests A(kt+1) and B(kt+2) at its top (their slots were last read in
  // k-step kt-1), and before its barrier waits for A(kt+1) and B(kt+1)
  // (issued a k-step earlier), leaving B(kt+2) in flight.
  auto step3 = [&](auto jc, auto compute, int kt, int nk) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    constexpr bool kCompute = decltype(compute)::value;
    T* ca = stage_buf<T, kBMt * kBKT, 0, J % 2>();
    T* cb = stage_buf<T, kBNB * kBKT, 1, J % 3>();
    const bool more_a = kt + 1 < nk, more_b = kt + 2 < nk;
    if (more_a) issue_a(kt + 1, stage_buf<T, kBMt * kBKT, 0, (J + 1) % 2>());
    if (more_b) issue_b(kt + 2, stage_buf<T, kBNB * kBKT, 1, (J + 2) % 3>());
    auto wait_next = [&]() __attribute__((always_inline)) {
      if (more_b)
        wait_vmem<kLoadsB>();
      else
        wait_vmem<0>();
    };
    if constexpr (!kCompute) {
      wait_next();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      return;
    }
#pragma unroll
    for (int sub = 0; sub + 1 < kSub; ++sub) {
      read_frags(ca, cb, sub + 1, (sub + 1) & 1);
      mfmas(sub & 1, 0, kMfma);
#pragma unroll
      for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (sub == 0 && i < kLoads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if (i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    constexpr int kLast = (kSub - 1) & 1;
    // MFMAs of the last sub-step left for after the barrier, where they
    // cover the next stage's first fragment reads: 6 of 8 in gate/up, half
    // in the down GEMM (measured: 6 or 8 helped gate/up by 1-3 %, 8 slowed
    // the down GEMM by 2 %)
    constexpr int kDefer = kSwiGlu ? 6 : kMfma / 2;
    mfmas(kLast, 0, kMfma - kDefer);
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kDefer, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_next();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    read_frags(stage_buf<T, kBMt * kBKT, 0, (J + 1) % 2>(), stage_buf<T, kBNB * kBKT, 1, (J + 1) % 3>(), 0, 0);
    mfmas(kLast, kMfma - kDefer, kMfma);
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i < kDefer) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    static_assert(kDefer <= kReads, "deferred MFMAs pair with the next stage's reads");
  };
  // Unrolled by 6 (the slot periods 2 and 3), leaving after the tile's last
  // k-step wherever it falls.
  auto main_loop3 = [&](auto compute, int nk) __attribute__((always_inline)) {
    if constexpr (decltype(compute)::value)
      read_frags(stage_buf<T, kBMt * kBKT, 0, 0>(), stage_buf<T, kBNB * kBKT, 1, 0>(), 0, 0);
    const int nk6 = nk / 6 * 6;
    for (int kt = 0; kt < nk6; kt += 6) {
      step3(std::integral_constant<int, 0>{}, compute, kt, nk);
      step3(std::integral_constant<int, 1>{}, compute, kt + 1, nk);
      step3(std::integral_constant<int, 2>{}, compute, kt + 2, nk);
      step3(std::integral_constant<int, 3>{}, compute, kt + 3, nk);
      step3(std::integral_constant<int, 4>{}, compute, kt + 4, nk);
      step3(std::integral_constant<int, 5>{}, compute, kt + 5, nk);
    }
    // the last nk % 6 k-steps (slots continue from 0)
    const int r = nk - nk6;
    if (r > 0) step3(std::integral_constant<int, 0>{}, compute, nk6, nk);
    if (r > 1) step3(std::integral_constant<int, 1>{}, compute, nk6 + 1, nk);
    if (r > 2) step3(std::integral_constant<int, 2>{}, compute, nk6 + 2, nk);
    if (r > 3) step3(std::integral_constant<int, 3>{}, compute, nk6 + 3, nk);
    if (r > 4) step3(std::integral_constant<int, 4>{}, compute, nk6 + 4, nk);
  };
  // Main loop over one tile, unrolled by the stages so every LDS pointer is
  // a fixed object. The trip count is padded to a multiple of the stage
  // count: loads past K are masked to zeros, so a padding step adds nothing.
  auto main_loop = [&](auto compute, int nk_pad) __attribute__((always_inline)) {
    if constexpr (decltype(compute)::value)
      read_frags(stage_buf<T, kBMt * kBKT, 0, 0>(), stage_buf<T, kBNB * kBKT, 1, 0>(), 0, 0);
    for (int kt = 0; kt < nk_pad; kt += kStg) {
      step(std::integral_constant<int, 0>{}, compute, kt, nk_pad);
      step(std::integral_constant<int, 1>{}, compute, kt + 1, nk_pad);
      step(std::integral_constant<int, 2>{}, compute, kt + 2, nk_pad);
    }
  };
  // The first loads of a tile, requested ahead of its loop.
  auto issue_first = [&]() {
    if constexpr (kB3) {
      // A(0), B(0), then B(1) (which may stay in flight when the tile starts)
      issue_a(0, stage_buf<T, kBMt * kBKT, 0, 0>());
      issue_b(0, stage_buf<T, kBNB * kBKT, 1, 0>());
      issue_b(1, stage_buf<T, kBNB * kBKT, 1, 1>());
      return;
    }
    issue_loads(0, stage_buf<T, kBMt * kBKT, 0, 0>(), stage_buf<T, kBNB * kBKT, 1, 0>());
    issue_loads(1, stage_buf<T, kBMt * kBKT, 0, 1>(), stage_buf<T, kBNB * kBKT, 1, 1>());
  };

  {
    int src[kLoadsA];
    a_src(tile, src);
    setup(tile, src);
  }
  issue_first();
  T* C = static_cast<T*>(p.c);
  const int row_lane = (lane >> 5) * 4;
  // Epilogue stores per computing wavefront: 4 per 32x32 output block (3
  // blocks, h, g and u, per h block when the training cache is written).
  constexpr int kStores = (kSwiGlu ? kMB * 2 : kMB * kNB) * 4 * (kCache ? 3 : 1);
  static_assert(kStores + kLoads < 64, "vmcnt holds 6 bits");
  // Stores of the LDS epilogue: 64 rows x 64 columns (one pass) per gate/up
  // wavefront, 64 x 128 (two passes) per down wavefront, 8 per pass.
  constexpr int kStoresLds = kSwiGlu ? 8 : 16;
  // The next tile waits for its first stage with vmcnt(this): never more
  // than the stores any wavefront issued after those loads.
  constexpr int kStoresWait = kLdsEpi ? kStoresLds : kStores;
  int stores_prev = 0;
  for (;;) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
    const int nk = (k_end - k_begin + kBKT - 1) / kBKT;
    const int nk_pad = (nk + kStg - 1) / kStg * kStg;
    // This tile's first loads have been requested; wait for k-step 0's (not
    // for the weights of k-step 1, or the loads of k-step 1 with 128-row
    // tiles, or the previous tile's stores, all issued after them).
    constexpr int kAhead = kB3 ? kLoadsB : kLoads;
    if (stores_prev)
      wait_vmem<kStoresWait + kAhead>();
    else
      wait_vmem<kAhead>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const bool has_rows = wm * kWaveM < mrows;
    // The next tile's schedule entry and A-row sources, requested now and
    // used after the main loop.
    Tile next;
    const bool more = tile_of_block(p, v + gridDim.x, next);
    int nsrc[kLoadsA];
    if (more) a_src(next, nsrc);
    if constexpr (kB3) {
      if (has_rows)
        main_loop3(std::true_type{}, nk);
      else
        main_loop3(std::false_type{}, nk);
    } else {
      if (has_rows)
        main_loop(std::true_type{}, nk_pad);
      else
        main_loop(std::false_type{}, nk_pad);
    }
    // Every wavefront is done with LDS before the next tile's loads land.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int t_row0 = row0, t_mrows = mrows, t_nt = n_t, t_slot = tu * ts + ks;
    const bool part = !kSwiGlu && ts > 1;  // a split tile of the down GEMM
    v += gridDim.x;
    if (more) {
      setup(next, nsrc);
      issue_first();
    }

    // Epilogue. Accumulator element i of lane l sits at row
    // (i/4)*8 + (l/32)*4 + i%4 and column l%32 of its 32x32 block. Each run
    // of 4 rows is transposed within the quad of lanes holding 4 adjacent
    // columns, after which lane l holds columns 4*((l%32)/4) .. +3 of one
    // row: one 8-byte store (16 for fp32 partials) in place of four 2-byte
    // ones. Stores go through a buffer resource covering this tile's rows,
    // with out-of-range offsets for rows past the expert or columns past N
    // (N is a multiple of 8, so 4 columns are all in or all out); every
    // wavefront that computed thus issues exactly kStores stores, issued
    // after the next tile's first loads, and the next tile waits for its
    // loads with vmcnt(kStores) without draining the stores.
    int stores_out = 0;
    if (kLdsEpi && has_rows) {
      // Lane l holds, for accumulator i of block (mb, nb), output row
      // mb*32 + l%32 of the wavefront and column nb*32 + (i/4)*8 + 4*(l/32)
      // + i%4: four consecutive columns per group of four accumulators.
      const int m32 = lane & 31, h4 = (lane >> 5) * 4;
      if (part) {
        // fp32 split-K partials: 16 bytes per lane and group, straight out
        // to the tile's own kBMt x kBNB block; its rows past the expert fall
        // beyond the byte count, its columns past N are stored and never
        // read, so every offset is this lane's base plus a constant
        const __amdgpu_buffer_rsrc_t rsrc_p = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<char*>(p.partial + (int64_t)t_slot * kBMt * kBNB), (short)0,
            t_mrows * kBNB * 4, kRsrcFlags);
        const uint32_t vb = (uint32_t)((wm * kWaveM + m32) * kBNB + wn * (kBNB / 2) + h4) * 4u;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              // copied out first: a bit cast of a vector element reads the
              // vector's first element
              const float x0 = acc[mb][nb][4 * g], x1 = acc[mb][nb][4 * g + 1];
              const float x2 = acc[mb][nb][4 * g + 2], x3 = acc[mb][nb][4 * g + 3];
              const i32x4 d = {__builtin_bit_cast(int, x0), __builtin_bit_cast(int, x1),
                               __builtin_bit_cast(int, x2), __builtin_bit_cast(int, x3)};
              __builtin_amdgcn_raw_buffer_store_b128(
                  d, rsrc_p, vb + (uint32_t)((mb * 32 * kBNB + nb * 32 + g * 8) * 4), 0, 0);
            }
      } else {
        // Wavefront w's block goes to its own 8 KB of stage 1 (waves 0-3 in
        // the A half, 4-7 in the B half): 64 rows of 64 elements, 16-byte
        // chunk c of row r at slot c ^ ((r >> 1) & 7), so that the 32 rows
        // of an 8-byte write instruction and the 8 rows of a 16-byte read
        // spread over all banks.
        T* const blk = wave < 4 ? stage_buf<T, kBMt * kBKT, 0, 1>() + wave * 4096
                                : stage_buf<T, kBNB * kBKT, 1, 2>() + (wave - 4) * 4096;
        const __amdgpu_buffer_rsrc_t rsrc_c = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<char*>(C + (int64_t)t_row0 * N), (short)0, t_mrows * N * (int)sizeof(T), kRsrcFlags);
        // four values at row mb*32 + m32, columns nbx*32 + g*8 + h4 .. +3
        const int wrow = m32 * 64 + h4;
        const int wsw = (m32 >> 1) & 7;
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        typedef T tx4 __attribute__((ext_vector_type(4)));
        auto put4 = [&](float x0, float x1, float x2, float x3, int mb, int nbx, int g) {
          const f32x4v xv = {x0, x1, x2, x3};
          *reinterpret_cast<tx4*>(blk + mb * 2048 + wrow + (((nbx * 4 + g) ^ wsw) << 3)) =
              __builtin_convertvector(xv, tx4);
        };
        // 64 rows x 64 columns from output column col_base: lane l reads
        // chunk l%8 of rows l/8 + 8j; rows past the tile fall beyond the
        // buffer's byte count, a chunk past N gets an out-of-range offset
        // (N is a multiple of 8)
        const int rr = lane >> 3, ch = lane & 7;
        const T* const rd0 = blk + rr * 64 + ((ch ^ (rr >> 1)) << 3);
        const T* const rd1 = blk + rr * 64 + ((ch ^ (rr >> 1) ^ 4) << 3);
        auto drain = [&](int col_base) {
          const int col = col_base + ch * 8;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const i32x4 d = *reinterpret_cast<const i32x4*>((j & 1 ? rd1 : rd0) + j * 512);
            const int row = wm * kWaveM + rr + 8 * j;
            const uint32_t vo = col < N ? (uint32_t)(row * N + col) * (uint32_t)sizeof(T) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(d, rsrc_c, vo, 0, 0);
          }
        };
        if constexpr (kSwiGlu) {
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                float hv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  // the product is rounded to fp32 before the conversion, as
                  // on the register path: the empty asm keeps the compiler
                  // from fusing multiply and conversion into one rounding
                  hv[q] = silu(acc[mb][nb][4 * g + q]) * acc[mb][nb + 2][4 * g + q];
                  asm("" : "+v"(hv[q]));
                }
                put4(hv[0], hv[1], hv[2], hv[3], mb, nb, g);
              }
          drain(t_nt * (kBNB / 2) + wn * 64);
        } else {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
              for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  const f32x16& a = acc[mb][2 * hf + nb];
                  put4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3], mb, nb, g);
                }
            drain(t_nt * kBNB + wn * (kBNB / 2) + hf * 64);
          }
        }
      }
      stores_out = 1;
    } else if (has_rows) {
      // split-K partials go to the tile's own kBMt x kBNB block (row
      // stride kBNB, columns from the tile's first), outputs to C
      const int esz = part ? 4 : (int)sizeof(T);
      const int ld = part ? kBNB : N;
      const int col_off = part ? t_nt * kBNB : 0;
      char* base = part ? reinterpret_cast<char*>(p.partial + (int64_t)t_slot * kBMt * kBNB)
                        : reinterpret_cast<char*>(C + (int64_t)t_row0 * N);
      const __amdgpu_buffer_rsrc_t rsrc_c =
          __builtin_amdgcn_make_buffer_rsrc(base, (short)0, t_mrows * ld * esz, kRsrcFlags);
      const int col4 = (lane & 31) & ~3;
      auto store_block = [&](float (&val)[16], int row_base, int col_base) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float x[4] = {val[4 * g], val[4 * g + 1], val[4 * g + 2], val[4 * g + 3]};
          transpose4(x, lane);
          const int lrow = row_base + g * 8 + row_lane + (lane & 3);
          const int col = col_base + col4;
          // (a partial block's columns past N are stored and never read)
          const uint32_t vo = (lrow < t_mrows && (part || col < N))
                                  ? (uint32_t)(lrow * ld + col - col_off) * (uint32_t)esz
                                  : kOutOfRange;
          if (part) {
            const i32x4 d = {__builtin_bit_cast(int, x[0]), __builtin_bit_cast(int, x[1]),
                             __builtin_bit_cast(int, x[2]), __builtin_bit_cast(int, x[3])};
            __builtin_amdgcn_raw_buffer_store_b128(d, rsrc_c, vo, 0, 0);
          } else {
            const T h0 = from_f32<T>(x[0]), h1 = from_f32<T>(x[1]);
            const T h2 = from_f32<T>(x[2]), h3 = from_f32<T>(x[3]);
            const i32x2 d = {(int)((uint32_t)__builtin_bit_cast(uint16_t, h0) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16)),
                             (int)((uint32_t)__builtin_bit_cast(uint16_t, h2) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16))};
            __builtin_amdgcn_raw_buffer_store_b64(d, rsrc_c, vo, 0, 0);
          }
        }
      };
      if (kSwiGlu && kCache) {
        // g and u rounded to T go to the cache ([rows, 2N], g then u); h is
        // formed from the rounded values
        const __amdgpu_buffer_rsrc_t rsrc_gu = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<T*>(p.cache) + (int64_t)t_row0 * 2 * N, (short)0, t_mrows * 2 * N * (int)sizeof(T),
            kRsrcFlags);
        // col_base: the block's column of h; half 0 stores into the g half of
        // the cache row, half 1 into the u half (N further on)
        auto store_gu = [&](float (&val)[16], int row_base, int col_base, int half) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float x[4] = {val[4 * g], val[4 * g + 1], val[4 * g + 2], val[4 * g + 3]};
            transpose4(x, lane);
            const int lrow = row_base + g * 8 + row_lane + (lane & 3);
            const int col = col_base + col4;
            const uint32_t vo = (lrow < t_mrows && col < N)
                                    ? (uint32_t)(lrow * 2 * N + half * N + col) * (uint32_t)sizeof(T)
                                    : kOutOfRange;
            const i32x2 d = {(int)((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(x[0])) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(x[1])) << 16)),
                             (int)((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(x[2])) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(x[3])) << 16))};
            __builtin_amdgcn_raw_buffer_store_b64(d, rsrc_gu, vo, 0, 0);
          }
        };
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int col_base = t_nt * (kBNB / 2) + wn * 64 + nb * 32;
            float g[16], u[16], val[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              g[i] = to_f32(from_f32<T>(acc[mb][nb][i]));
              u[i] = to_f32(from_f32<T>(acc[mb][nb + 2][i]));
              val[i] = silu(g[i]) * u[i];
            }
            store_gu(g, wm * kWaveM + mb * 32, col_base, 0);
            store_gu(u, wm * kWaveM + mb * 32, col_base, 1);
            store_block(val, wm * kWaveM + mb * 32, col_base);
          }
      } else if (kSwiGlu) {
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            float val[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) val[i] = silu(acc[mb][nb][i]) * acc[mb][nb + 2][i];
            store_block(val, wm * kWaveM + mb * 32, t_nt * (kBNB / 2) + wn * 64 + nb * 32);
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            float val[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) val[i] = acc[mb][nb][i];
            store_block(val, wm * kWaveM + mb * 32, t_nt * kBNB + wn * (kBNB / 2) + nb * 32);
          }
      }
      stores_out = 1;
    }
    if (!more) break;
    stores_prev = stores_out;
  }
}

// Decode gate/up GEMM for a few rows per expert: weight-bandwidth bound, so
// weights stream from HBM straight into registers (no reuse to stage through
// LDS) and the MFMA work is sized to the rows that exist. One workgroup of 4
// wavefronts per (expert, block of 32 gate rows and the same 32 up rows); the
// wavefronts split K four ways and their partial sums meet in LDS, so the
// grid has enough independent streams to keep every CU busy. Rows of A
// (tokens) are taken 16 at a time. MFMA 16x16x32 with A = 16 weight rows and
// B = 16 rows of X, D[weight row][token]. In a K-iteration of 128, load c
// (= MFMA step c) gives lane group g = lane/16 the 8 elements at
// k = kb + 32c + 8g, the MFMA's own operand layout, so the four lanes of a
// row read 64 contiguous bytes per load. All loads of the next iteration are
// issued before the current one's MFMAs.
constexpr int kSkinnyTokens = 16;
constexpr int kSkinnyKIter = 128;
constexpr int kSkinnyWaves = 4;

template <typename T> struct Mfma16;
template <> struct Mfma16<bf16> {
  typedef bf16x8 Frag;
  static __device__ __forceinline__ f32x4 run(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma16<f16> {
  typedef f16x8 Frag;
  static __device__ __forceinline__ f32x4 run(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

struct SkinnyArgs {
  GemmArgs g;
  int E;
  int n_blocks;   // weight-row blocks per expert (one workgroup each)
  int k_quarter;  // K elements per wavefront (multiple of kSkinnyKIter)
};

template <typename T>
__global__ __launch_bounds__(64 * kSkinnyWaves) void skinny_gate_up_kernel(SkinnyArgs sa) {
  typedef typename Mfma16<T>::Frag Frag;
  __shared__ f32x4 red[kSkinnyWaves - 1][4][64];
  const GemmArgs& p = sa.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = blockIdx.x / sa.n_blocks;
  const int nb = blockIdx.x - e * sa.n_blocks;
  if (e >= sa.E) return;
  const int r_begin = max(__builtin_amdgcn_readfirstlane(p.offsets[e]), 0);
  const int r_end = min(__builtin_amdgcn_readfirstlane(p.offsets[e + 1]), p.rows);
  if (r_end <= r_begin) return;

  const int K = p.K, N = p.N;
  const int k_lo = wave * sa.k_quarter;
  const int k_hi = min(K, k_lo + sa.k_quarter);
  const uint32_t row_bytes = (uint32_t)K * sizeof(T);
  const int64_t expert_elems = (int64_t)e * N * K;
  const int b_bytes = (int)((uint32_t)N * row_bytes);
  const __amdgpu_buffer_rsrc_t rw0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(static_cast<const T*>(p.b0) + expert_elems), (short)0, b_bytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rw1 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(static_cast<const T*>(p.b1) + expert_elems), (short)0, b_bytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.a), (short)0, (int)((uint32_t)p.a_rows * row_bytes), kRsrcFlags);

  // Weight rows of the 4 tiles: gate rows nb*32 .. +31 (tiles 0, 1), the
  // same up rows (tiles 2, 3); rows past N read as zero.
  const int g = lane >> 4;
  uint32_t vo_w[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = nb * 32 + (t & 1) * 16 + (lane & 15);
    vo_w[t] = (uint32_t)n * row_bytes + (uint32_t)g * 16u;
  }
  const int n_it = max((k_hi - k_lo + kSkinnyKIter - 1) / kSkinnyKIter, 0);  // this wavefront's K-iterations

  T* C = static_cast<T*>(p.c);
  for (int rg = r_begin; rg < r_end; rg += kSkinnyTokens) {
    const int xr = rg + (lane & 15);
    uint32_t vo_x = kOutOfRange;
    if (xr < r_end) {
      const int src = p.a_map ? min(max(p.a_map[xr] / p.a_div, 0), p.a_rows - 1) : xr;
      vo_x = (uint32_t)src * row_bytes + (uint32_t)g * 16u;
    }
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Two register buffers, named (not indexed) so they stay in registers;
    // loads past this wavefront's K range or its last iteration read as zero.
    uint4 wa[4][4], xa[4], wb[4][4], xb[4];
    auto load = [&](int it, uint4 (&w)[4][4], uint4 (&x)[4]) {
      const int kb = k_lo + it * kSkinnyKIter;
      const uint32_t soff = (uint32_t)kb * sizeof(T);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool ok = it < n_it && kb + c * 32 + g * 8 < k_hi;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          w[t][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
              t >= 2 ? rw1 : rw0, ok ? vo_w[t] + c * 64u : kOutOfRange, soff, 0));
        x[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            rx, ok ? vo_x + c * 64u : kOutOfRange, soff, 0));
      }
    };
    auto compute = [&](const uint4 (&w)[4][4], const uint4 (&x)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[t] = Mfma16<T>::run(__builtin_bit_cast(Frag, w[t][c]), __builtin_bit_cast(Frag, x[c]),
                                  acc[t]);
    };
    // Partial sums of wavefronts 1..3 meet wavefront 0's in LDS (fixed
    // order), wavefront 0 stores. Every wavefront calls this once per token
    // group (the same barriers, whatever its K range).
    auto finish = [&]() {
      if (wave > 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) red[wave - 1][t][lane] = acc[t];
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int w = 0; w < kSkinnyWaves - 1; ++w)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t] += red[w][t][lane];
        // D element v of lane l: weight row (l/16)*4 + v of the tile, token l%16.
        const int tok = rg + (lane & 15);
        if (tok < r_end) {
          T* crow = C + (int64_t)tok * N;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int col = nb * 32 + t * 16 + g * 4;
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (col + v < N) crow[col + v] = from_f32<T>(silu(acc[t][v]) * acc[t + 2][v]);
          }
        }
      }
      __syncthreads();  // red[] is reused by the next token group
    };

    if (n_it > 0) {
      // keep every load of the next iteration ahead of this one's MFMAs
      constexpr int kLoadsPerIter = 4 * 4 + 4;
      load(0, wa, xa);
      int it = 0;
      for (; it + 2 <= n_it; it += 2) {
        load(it + 1, wb, xb);
        compute(wa, xa);
        __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerIter, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        load(it + 2, wa, xa);
        compute(wb, xb);
        __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerIter, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      }
      if (it < n_it) compute(wa, xa);  // odd count: wa holds the last iteration
    }
    finish();
  }
}

// Decode down GEMM, one wavefront per 16 output columns over the whole of K:
// the wavefront streams its 16 weight rows from HBM straight into MFMA
// operands, kDepth K-iterations of loads in flight, no K split and no LDS
// (each wavefront reads whole rows: a K split made the short K = I rows of
// the down projection into pieces of a few hundred bytes per wavefront). MFMA 16x16x32, A = 16 weight rows, B = 16
// token rows, D[weight row][token]; load c of a K-iteration of 128 gives lane
// group g = lane/16 the 8 elements at k = kb + 32c + 8g, so the four lanes of
// a row read 64 contiguous bytes per load.
constexpr int kRowsWaves = 4;  // wavefronts per workgroup
constexpr int kRowsDepth = 2;  // K-iterations of loads in flight per wavefront

template <typename T, int kDepth>
__global__ __launch_bounds__(64 * kRowsWaves) void skinny_down_kernel(SkinnyArgs sa) {
  typedef typename Mfma16<T>::Frag Frag;
  constexpr int kT = 1;  // weight tiles per wavefront
  const GemmArgs& p = sa.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = blockIdx.x / sa.n_blocks;
  const int nb = blockIdx.x - e * sa.n_blocks;
  if (e >= sa.E) return;
  const int r_begin = max(__builtin_amdgcn_readfirstlane(p.offsets[e]), 0);
  const int r_end = min(__builtin_amdgcn_readfirstlane(p.offsets[e + 1]), p.rows);
  const int K = p.K, N = p.N;
  const int col0 = (nb * kRowsWaves + wave) * 16;  // this wavefront's output columns
  if (r_end <= r_begin || col0 >= N) return;        // no barriers in this kernel

  const uint32_t row_bytes = (uint32_t)K * sizeof(T);
  const int64_t expert_elems = (int64_t)e * N * K;
  const int b_bytes = (int)((uint32_t)N * row_bytes);
  const __amdgpu_buffer_rsrc_t rw0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(static_cast<const T*>(p.b0) + expert_elems), (short)0, b_bytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.a), (short)0, (int)((uint32_t)p.a_rows * row_bytes), kRsrcFlags);
  const int g = lane >> 4;
  // weight row col0 + lane % 16 (rows past N read as zero)
  const uint32_t vo_w = (uint32_t)(col0 + (lane & 15)) * row_bytes + (uint32_t)g * 16u;
  const int n_it = (K + kSkinnyKIter - 1) / kSkinnyKIter;

  T* C = static_cast<T*>(p.c);
  for (int rg = r_begin; rg < r_end; rg += kSkinnyTokens) {
    const int xr = rg + (lane & 15);
    uint32_t vo_x = kOutOfRange;
    if (xr < r_end) {
      const int src = p.a_map ? min(max(p.a_map[xr] / p.a_div, 0), p.a_rows - 1) : xr;
      vo_x = (uint32_t)src * row_bytes + (uint32_t)g * 16u;
    }
    f32x4 acc[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // kDepth register buffers, indexed only by unrolled constants so they
    // stay in registers; K-iterations past the end read as zero.
    uint4 w[kDepth][kT][4], x[kDepth][4];
    auto load = [&](int it, uint4 (&wd)[kT][4], uint4 (&xd)[4]) {
      const int kb = it * kSkinnyKIter;
      const uint32_t soff = (uint32_t)kb * sizeof(T);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool ok = it < n_it && kb + c * 32 + g * 8 < K;
#pragma unroll
        for (int t = 0; t < kT; ++t)
          wd[t][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
              rw0, ok ? vo_w + c * 64u : kOutOfRange, soff, 0));
        xd[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            rx, ok ? vo_x + c * 64u : kOutOfRange, soff, 0));
      }
    };
    constexpr int kLoadsPerIter = kT * 4 + 4;
    auto mfma = [&](const uint4 (&wd)[kT][4], const uint4 (&xd)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < kT; ++t)
          acc[t] = Mfma16<T>::run(__builtin_bit_cast(Frag, wd[t][c]), __builtin_bit_cast(Frag, xd[c]), acc[t]);
    };
#pragma unroll
    for (int d = 0; d + 1 < kDepth; ++d) load(d, w[d], x[d]);
    // Loads run kDepth - 1 iterations ahead of the MFMAs. Full blocks of
    // kDepth iterations whose loads all lie before the last iteration run
    // without branches; the rest (fewer than 2 kDepth - 1 iterations) issues
    // no load past the last iteration (such loads, all out of range, had
    // cost 3 % of the launch's time on the decode shape).
    int it0 = 0;
    for (; it0 + 2 * kDepth - 2 < n_it; it0 += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        load(it0 + d + kDepth - 1, w[(d + kDepth - 1) % kDepth], x[(d + kDepth - 1) % kDepth]);
        mfma(w[d], x[d]);
        __builtin_amdgcn_sched_group_barrier(0x020, kLoadsPerIter, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * kT, 0);
      }
    }
#pragma unroll
    for (int d = 0; d < 2 * kDepth - 2; ++d) {
      if (it0 + d >= n_it) break;
      if (it0 + d + kDepth - 1 < n_it)
        load(it0 + d + kDepth - 1, w[(d + kDepth - 1) % kDepth], x[(d + kDepth - 1) % kDepth]);
      mfma(w[d % kDepth], x[d % kDepth]);
    }
    // D element v of lane l: weight row (l/16)*4 + v of the tile, token l%16.
    const int tok = rg + (lane & 15);
    if (tok < r_end) {
      T* crow = C + (int64_t)tok * N;
      const int col = col0 + g * 4;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (col + v < N)
          crow[col + v] = from_f32<T>(acc[0][v]);
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

  Tile tile;
  if (!tile_of_block(p, blockIdx.x, tile)) return;
  const int e = tile.e, row0 = tile.row0, n_t = tile.n_t;
  const int mrows = min(kBMSimt, tile.row_end - row0);
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

}  // namespace

constexpr int kCUs = 256;

#ifndef MOE_GEMM_WAVE_M
#define MOE_GEMM_WAVE_M 64
#endif
constexpr int kWaveMGemm = MOE_GEMM_WAVE_M;
// Weight-streaming shape (at most kBMStream rows an expert on average): 128-row
// M-tiles of 8 wavefronts (32 rows each) and three 48 KB LDS stages, so two
// k-steps of weights are in flight per CU instead of one.
constexpr int kBMStream = 128;
constexpr int kWaveMStream = 32;

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// N-tile width of each GEMM kernel: 128 h columns (256 gate + up weight rows)
// or 256 output columns on the MFMA path, 64 on the fp32 path.
static int64_t tile_n(int64_t N, int dt, bool swiglu) {
  const int64_t w = dt == kF32 ? 64 : (swiglu ? 128 : 256);
  return (N + w - 1) / w;
}

// Split-K of the down GEMM's last round: at most kSplitCap K-ranges a tile,
// each at least kSplitMinSteps K-steps long (64 elements a step), on at most
// kCUs workgroups (so at most kCUs split entries). (The gate/up GEMM's last
// round split the same way, its reduction forming SiLU(g) * u, measured no
// faster on the many-expert shape, the one whose last round is short.)
constexpr int kSplitCap = 8;
constexpr int kSplitMinSteps = 32;

ExpertsPlan experts_plan(int64_t rows, int64_t E, int64_t H, int64_t I, int dt) {
  ExpertsPlan p;
  p.bm = dt == kF32 ? kBMSimt : (rows <= kBMStream * E ? kBMStream : kBM);
  p.max_tiles = (int)((rows + p.bm - 1) / p.bm + (E < rows ? E : rows));
  p.split_cap = dt == kF32 ? 1
                            : (int)std::max<int64_t>(
                                  1, std::min<int64_t>(kSplitCap, (I + kBK - 1) / kBK / kSplitMinSteps));
  const int64_t n_gate_up = tile_n(I, dt, true), n_down = tile_n(H, dt, false);
  const int64_t tiles_gu = grid_tiles(p.max_tiles, n_gate_up), tiles_dn = grid_tiles(p.max_tiles, n_down);
  p.split_slots = p.split_cap > 1 ? (int)std::min<int64_t>(kCUs, tiles_dn * p.split_cap) : 0;
  // slots of the schedule (cost slices or a split last round) on at most
  // kCUs workgroups
  p.sched_entries = std::max(sched::slots_bound((int)tiles_gu, kCUs), sched::slots_bound((int)tiles_dn, kCUs));
  return p;
}

// Scratch of one GEMM call: the schedule, the split tiles' table (a header
// and up to kCUs entries) and their fp32 partial-sum blocks.
static size_t tile_list_bytes(const ExpertsPlan& p) {
  return align256((size_t)p.sched_entries * sizeof(int4));
}
static size_t split_table_bytes() { return align256((size_t)(1 + kCUs) * sizeof(int4)); }
static size_t partial_bytes(const ExpertsPlan& p) {
  return align256((size_t)p.split_slots * (size_t)p.bm * 256 * sizeof(float));
}

size_t gemm_scratch_bytes(int64_t rows, int64_t E, int64_t H, int64_t I, int dt) {
  const ExpertsPlan p = experts_plan(rows, E, H, I, dt);
  return tile_list_bytes(p) + split_table_bytes() + partial_bytes(p);
}

size_t experts_scratch_bytes(int64_t rows, int64_t E, int64_t H, int64_t I, int dt) {
  return gemm_scratch_bytes(rows, E, H, I, dt) + align256((size_t)rows * (size_t)I * dtype_size(dt));
}

namespace {

// The split tiles of the down GEMM's last round: for each split tile u
// (split[1 + u]), its s fp32 partial blocks are added in K-range order and
// the tile's rows of out stored; nothing when the last round was not split
// (split[0] = (r, s)). Eight columns a thread, 32 threads a row; workgroups
// take 8-row pieces of the split tiles in turn.
template <typename T>
__global__ __launch_bounds__(256) void reduce_split_tiles_kernel(const float* __restrict__ partial,
                                                                 const int4* __restrict__ split, int bm,
                                                                 int N, T* __restrict__ out) {
  const int4 hd = split[0];
  const int r = hd.x, s = hd.y;
  if (s <= 1) return;
  const int pieces = bm / 8;  // pieces of a tile
  const int c = (threadIdx.x & 31) * 8;
  const int64_t stride = (int64_t)bm * 256;
  for (int pc = blockIdx.x; pc < r * pieces; pc += gridDim.x) {
    const int u = pc / pieces;
    const int lr = (pc - u * pieces) * 8 + (threadIdx.x >> 5);
    const int4 d = split[1 + u];
    const int col = d.w * 256 + c;
    if (lr >= min(bm, d.z - d.y) || col >= N) continue;  // N is a multiple of 8
    const float* src = partial + (int64_t)u * s * stride + lr * 256 + c;
    float acc[8];
    {
      const float4 a0 = *reinterpret_cast<const float4*>(src);
      const float4 a1 = *reinterpret_cast<const float4*>(src + 4);
      acc[0] = a0.x; acc[1] = a0.y; acc[2] = a0.z; acc[3] = a0.w;
      acc[4] = a1.x; acc[5] = a1.y; acc[6] = a1.z; acc[7] = a1.w;
    }
    for (int k = 1; k < s; ++k) {
      const float4 a0 = *reinterpret_cast<const float4*>(src + k * stride);
      const float4 a1 = *reinterpret_cast<const float4*>(src + k * stride + 4);
      acc[0] += a0.x; acc[1] += a0.y; acc[2] += a0.z; acc[3] += a0.w;
      acc[4] += a1.x; acc[5] += a1.y; acc[6] += a1.z; acc[7] += a1.w;
    }
    Vec8<T> o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o.set(j, acc[j]);
    o.store(out + (int64_t)(d.y + lr) * N + col);
  }
}

// Workgroups of the persistent MFMA GEMM: one per CU (its 144-160 KB of LDS
// stages leave room for no second one), at most one per schedule entry; a
// multiple of 8 so each workgroup stays on the XCD its entries belong to.
static int persistent_grid(int64_t entries) {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = kCUs;
    cus[dev] = n / 8 * 8;
  }
  return (int)std::min<int64_t>(entries, cus[dev]);
}

int4* split_table(const ExpertsPlan& plan, void* scratch) {
  return reinterpret_cast<int4*>(static_cast<char*>(scratch) + tile_list_bytes(plan));
}

float* partial_buffer(const ExpertsPlan& plan, void* scratch) {
  return plan.split_slots > 0
             ? reinterpret_cast<float*>(static_cast<char*>(scratch) + tile_list_bytes(plan) + split_table_bytes())
             : nullptr;
}

// Carves the schedule out of `scratch` and enqueues the plan kernel for the
// GEMM described by g (N set; the down GEMM with split = true may split its
// last round's K).
void plan_tiles(GemmArgs& g, const ExpertsPlan& plan, int E, int dt, bool swiglu, bool split, void* scratch,
                hipStream_t s) {
  g.max_tiles = plan.max_tiles;
  g.bm = plan.bm;
  g.n_tiles_n = (int)tile_n(g.N, dt, swiglu);
  const int64_t tiles = grid_tiles(plan.max_tiles, g.n_tiles_n);
  const int cap = split && plan.split_slots > 0 ? plan.split_cap : 1;
  // workgroups, at most kCUs (the schedule and the split entries' partial
  // blocks are sized for kCUs): with a possible split, enough for every split
  // entry
  if (cap > 1)
    g.wgs = std::min(persistent_grid(tiles * cap), plan.split_slots);
  else
    g.wgs = std::min(persistent_grid(tiles), kCUs);
  // slices of equal estimated cost for the gate/up GEMM on the 256-row tile
  // (many-expert shape: 0.46 -> 0.43 ms); equal count for the down GEMM
  // (its 12-k-step tiles measured 1-3 % slower with cost slices) and on the
  // fp32 path, which launches one workgroup per slot
  const bool costed = dt != kF32 && plan.bm == kBM && swiglu;
  g.grid = dt != kF32 ? sched::slots_bound((int)tiles, g.wgs) : (int)tiles;
  g.partial = cap > 1 ? partial_buffer(plan, scratch) : nullptr;
  int4* sched = static_cast<int4*>(scratch);
  // Each workgroup repeats the expert scan and fills 1024 entries: the entry
  // arithmetic (a binary search and several divisions) dominates, and one
  // workgroup on one CU would take it in series.
  const int blocks = std::max(1, std::min((g.grid + 1023) / 1024, 64));
  hipLaunchKernelGGL(plan_kernel, dim3(blocks), dim3(1024), 0, s, g.offsets, E, g.rows, plan.bm,
                     plan.max_tiles, g.n_tiles_n, cap, costed ? 1 : 0, g.wgs, g.grid, sched,
                     cap > 1 ? split_table(plan, scratch) : nullptr);
  g.sched = sched;
}

template <typename T>
void launch_mfma(const GemmArgs& g, bool swiglu, hipStream_t s) {
  const dim3 grid(g.wgs);
  if (g.bm == kBMStream) {
    constexpr int kThreads = gemm_threads<kWaveMStream, kBMStream>();
    if (swiglu && g.cache)
      hipLaunchKernelGGL((mfma_gemm_kernel<T, true, 256, kBK, kWaveMStream, true, kBMStream, 3>), grid,
                         dim3(kThreads), 0, s, g);
    else if (swiglu)
      hipLaunchKernelGGL((mfma_gemm_kernel<T, true, 256, kBK, kWaveMStream, false, kBMStream, 3>), grid,
                         dim3(kThreads), 0, s, g);
    else
      hipLaunchKernelGGL((mfma_gemm_kernel<T, false, 256, kBK, kWaveMStream, false, kBMStream, 3>), grid,
                         dim3(kThreads), 0, s, g);
    return;
  }
  if (swiglu && g.cache)
    hipLaunchKernelGGL((mfma_gemm_kernel<T, true, 256, kBK, kWaveMGemm, true>), grid,
                       dim3(gemm_threads<kWaveMGemm>()), 0, s, g);
  else if (swiglu)
    hipLaunchKernelGGL((mfma_gemm_kernel<T, true, 256, kBK, kWaveMGemm>), grid,
                       dim3(gemm_threads<kWaveMGemm>()), 0, s, g);
  else
    hipLaunchKernelGGL((mfma_gemm_kernel<T, false, 256, kBK, kWaveMGemm>), grid,
                       dim3(gemm_threads<kWaveMGemm>()), 0, s, g);
}

template <bool kSwiGlu>
void launch_gemm(const GemmArgs& g, int dt, hipStream_t s) {
  if (dt == kF32) {
    hipLaunchKernelGGL(simt_gemm_kernel<kSwiGlu>, dim3(g.grid), dim3(256), 0, s, g);
  } else if (dt == kF16) {
    launch_mfma<f16>(g, kSwiGlu, s);
  } else {
    launch_mfma<bf16>(g, kSwiGlu, s);
  }
}

void setup_gate_up(GemmArgs& g, const void* a, const int32_t* a_map, int a_div, int H, int I,
                   const void* w_gate, const void* w_up, void* h) {
  g.a = a; g.a_map = a_map; g.a_div = a_div > 0 ? a_div : 1;
  g.a_rows = a_map ? (g.rows + g.a_div - 1) / g.a_div : g.rows;
  g.b0 = w_gate; g.b1 = w_up; g.c = h;
  g.N = I; g.K = H;
  g.partial = nullptr;
}

void setup_down(GemmArgs& g, const void* h, int H, int I, const void* w_down, void* expert_out) {
  g.a = h; g.a_map = nullptr; g.a_div = 1; g.a_rows = g.rows;
  g.b0 = w_down; g.b1 = nullptr; g.c = expert_out;
  g.N = H; g.K = I;
  g.partial = nullptr;
}

// Few rows per expert (decode-shaped batches): weight streaming dominates.
bool use_skinny(int rows, int E, int dt) { return dt != kF32 && rows <= 4 * E; }

// Decode-sized batches: the gate/up GEMM (K = H) on skinny_gate_up_kernel
// (4 wavefronts split K), the down GEMM (K = I, usually short) on
// skinny_down_kernel (each wavefront streams whole weight rows); on the
// decode workload each measured faster than the other kernel's scheme.
template <typename T>
void launch_rows(const SkinnyArgs& sa, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)sa.E * sa.n_blocks));
  hipLaunchKernelGGL((skinny_down_kernel<T, kRowsDepth>), grid, dim3(64 * kRowsWaves), 0, s, sa);
}

void launch_skinny(const GemmArgs& g, int E, int dt, bool swiglu, hipStream_t s) {
  SkinnyArgs sa;
  sa.g = g;
  sa.E = E;
  if (!swiglu) {
    sa.n_blocks = (g.N + 16 * kRowsWaves - 1) / (16 * kRowsWaves);
    sa.k_quarter = 0;
    if (dt == kF16) launch_rows<f16>(sa, s);
    else launch_rows<bf16>(sa, s);
    return;
  }
  sa.n_blocks = (g.N + 31) / 32;
  const int iters = (g.K + kSkinnyKIter - 1) / kSkinnyKIter;
  sa.k_quarter = (iters + kSkinnyWaves - 1) / kSkinnyWaves * kSkinnyKIter;
  const dim3 grid((unsigned)((int64_t)E * sa.n_blocks));
  if (dt == kF16) hipLaunchKernelGGL((skinny_gate_up_kernel<f16>), grid, dim3(64 * kSkinnyWaves), 0, s, sa);
  else hipLaunchKernelGGL((skinny_gate_up_kernel<bf16>), grid, dim3(64 * kSkinnyWaves), 0, s, sa);
}

// Adds the down GEMM's split last-round tiles into expert_out: 8-row pieces
// of up to g.wgs split tiles.
hipError_t reduce_split_tiles(const GemmArgs& g, const ExpertsPlan& plan, void* scratch, int dt, void* out,
                              hipStream_t s) {
  const int4* table = split_table(plan, scratch);
  const dim3 grid(std::min(2048, g.wgs * (plan.bm / 8))), block(256);
  if (dt == kF16)
    hipLaunchKernelGGL(reduce_split_tiles_kernel<f16>, grid, block, 0, s, g.partial, table, plan.bm, g.N,
                       static_cast<f16*>(out));
  else
    hipLaunchKernelGGL(reduce_split_tiles_kernel<bf16>, grid, block, 0, s, g.partial, table, plan.bm, g.N,
                       static_cast<bf16*>(out));
  return hipGetLastError();
}

}  // namespace

bool gate_up_can_cache(int64_t rows, int64_t E, int dt) {
  return dt != kF32 && !use_skinny(rows, E, dt);
}

hipError_t launch_gate_up(const void* a, const int32_t* a_map, int a_div, const int32_t* offsets,
                          int rows, int E, int H, int I, const void* w_gate, const void* w_up,
                          int dt, void* h, void* scratch, hipStream_t s, void* cache) {
  if (rows == 0) return hipSuccess;
  if (cache && !gate_up_can_cache(rows, E, dt)) return hipErrorInvalidValue;
  if (use_skinny(rows, E, dt)) {
    GemmArgs g = {};
    g.offsets = offsets; g.rows = rows;
    setup_gate_up(g, a, a_map, a_div, H, I, w_gate, w_up, h);
    launch_skinny(g, E, dt, true, s);
    return hipGetLastError();
  }
  const ExpertsPlan plan = experts_plan(rows, E, H, I, dt);
  GemmArgs g = {};
  g.offsets = offsets; g.rows = rows;
  setup_gate_up(g, a, a_map, a_div, H, I, w_gate, w_up, h);
  g.cache = cache;
  plan_tiles(g, plan, E, dt, true, false, scratch, s);
  launch_gemm<true>(g, dt, s);
  return hipGetLastError();
}

hipError_t launch_down(const void* h, const int32_t* offsets, int rows, int E, int H, int I,
                       const void* w_down, int dt, void* expert_out, void* scratch, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (use_skinny(rows, E, dt)) {
    GemmArgs g = {};
    g.offsets = offsets; g.rows = rows;
    setup_down(g, h, H, I, w_down, expert_out);
    launch_skinny(g, E, dt, false, s);
    return hipGetLastError();
  }
  const ExpertsPlan plan = experts_plan(rows, E, H, I, dt);
  GemmArgs g = {};
  g.offsets = offsets; g.rows = rows;
  setup_down(g, h, H, I, w_down, expert_out);
  plan_tiles(g, plan, E, dt, false, true, scratch, s);
  launch_gemm<false>(g, dt, s);
  if (g.partial != nullptr) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return reduce_split_tiles(g, plan, scratch, dt, expert_out, s);
  }
  return hipGetLastError();
}

hipError_t launch_experts(const void* a, const int32_t* a_map, int a_div,
                          const int32_t* offsets, int rows, int E, int H, int I,
                          const void* w_gate, const void* w_up, const void* w_down, int dt,
                          void* expert_out, void* scratch, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  void* h = static_cast<char*>(scratch) + gemm_scratch_bytes(rows, E, H, I, dt);
  hipError_t e = launch_gate_up(a, a_map, a_div, offsets, rows, E, H, I, w_gate, w_up, dt, h,
                                scratch, s);
  if (e != hipSuccess) return e;
  return launch_down(h, offsets, rows, E, H, I, w_down, dt, expert_out, scratch, s);
}

}  // namespace moe
