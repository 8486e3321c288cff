// Dispatch: compact grouping of the T*k (token, slot) pairs by expert with no
// capacity drop, plus the saved maps that restore token order (ruDNN user
// guide, "5. Expert weights and dispatch").
//
// Deterministic counting sort in three launches:
//   1. hist    - each block of slots counts its slots per expert (LDS);
//   2. scan    - one block turns the per-block counts into expert offsets and
//                per-(block, expert) starting rows;
//   3. scatter - each block walks its slots in order, one wavefront-wide
//                chunk at a time; a slot's row is its expert's running row
//                plus its rank among equal ids in the chunk (a match mask
//                built from one ballot per id bit).
// Rows inside an expert therefore follow increasing flat slot t*k+j, the same
// for every run. Up to kOneBlockSlots slots the same three steps run in one
// workgroup, with its 16 wavefronts in the role of the blocks and the counts
// in LDS (one launch instead of three). A further launch gathers the token
// rows into x_disp.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kMaxBlocks = 256;

// The ids of kIdBatch chunks of 64 slots starting at c, read at once
// (indices clamped into range, so no load waits behind a branch); slots at or
// past s_end, ids > E and inactive slots give E.
constexpr int kIdBatch = 4;

__device__ __forceinline__ void load_ids(const uint32_t* __restrict__ idx, int64_t c, int s_end,
                                         int n_slots, int E, const uint8_t* __restrict__ active,
                                         int mask_dims, int k, uint32_t (&e)[kIdBatch]) {
  const int lane = threadIdx.x & (kWave - 1);
  int sc[kIdBatch];  // clamped below n_slots: fits in int
#pragma unroll
  for (int b = 0; b < kIdBatch; ++b) {
    const int64_t s = c + b * kWave + lane;
    sc[b] = s < n_slots ? (int)s : n_slots - 1;
    e[b] = idx[sc[b]];
  }
  uint8_t on[kIdBatch];
#pragma unroll
  for (int b = 0; b < kIdBatch; ++b) on[b] = mask_dims ? active[mask_dims == 1 ? sc[b] / k : sc[b]] : 1;
#pragma unroll
  for (int b = 0; b < kIdBatch; ++b) {
    const int64_t s = c + b * kWave + lane;
    if (e[b] > (uint32_t)E || !on[b] || s >= s_end) e[b] = (uint32_t)E;
  }
}

// Rows of a batch of ids, in slot order: an expert's running row (run[e])
// plus the rank among equal ids of the same 64-slot chunk, found with one
// ballot per id bit; the lane holding the last equal id advances run[e]. All
// lanes read run[] before that write (one wavefront, LDS operations in order).
__device__ __forceinline__ void place_batch(const uint32_t (&ev)[kIdBatch], int64_t c, int s_end,
                                            int E, int nbits, int* run,
                                            int32_t* __restrict__ slot_of_row,
                                            int32_t* __restrict__ row_of_slot) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int b = 0; b < kIdBatch; ++b) {
    const int64_t s = c + b * kWave + lane;
    const bool in = s < s_end;
    const uint32_t e = ev[b];
    uint64_t same = __ballot(in);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool v = (e >> bit) & 1u;
      const uint64_t m = __ballot(v);
      same &= v ? m : ~m;
    }
    const int rank = __popcll(same & lanemask_lt());
    const bool last = (same >> lane) == 1ull;  // no equal id in a higher lane
    int row = -1;
    if (in && e < (uint32_t)E) {
      row = run[e] + rank;
      slot_of_row[row] = (int32_t)s;
    }
    if (in) row_of_slot[s] = row;
    if (in && e < (uint32_t)E && last) run[e] = row + 1;
  }
}

__global__ __launch_bounds__(kWave) void hist_kernel(const uint32_t* __restrict__ idx, int n_slots,
                                                      int E, int per_block,
                                                      int32_t* __restrict__ hist,
                                                      const uint8_t* __restrict__ active,
                                                      int mask_dims, int k) {
  __shared__ int cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kWave) cnt[e] = 0;
  __syncthreads();
  const int s0 = (int)std::min<int64_t>((int64_t)blockIdx.x * per_block, n_slots);
  const int s_end = (int)std::min<int64_t>((int64_t)s0 + per_block, n_slots);
  for (int64_t c = s0; c < s_end; c += kIdBatch * kWave) {
    uint32_t e[kIdBatch];
    load_ids(idx, c, s_end, n_slots, E, active, mask_dims, k, e);
#pragma unroll
    for (int b = 0; b < kIdBatch; ++b)
      if (e[b] < (uint32_t)E) atomicAdd(&cnt[e[b]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kWave) hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// One block of 1024 threads, thread e owns expert e. The per-block counts are
// read kScanBatch blocks at a time (block index clamped into range, so the
// loads of a batch are all in flight together): once for the totals, once
// more to write each block's first row.
constexpr int kScanBatch = 16;

// When the whole table fits in LDS (kScanLds counts) it is instead staged
// there with coalesced loads, all issued at once, and written back the same way.
constexpr int kScanLds = 16384;

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ hist, int n_blocks,
                                                     int E, int32_t* __restrict__ offsets) {
  __shared__ int tab[kScanLds];
  const int e = threadIdx.x;
  const bool mine = e < E;
  const int n = n_blocks * E;
  if (n <= kScanLds) {
    constexpr int kPer = kScanLds / 1024;
    int c[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = hist[min(i * 1024 + e, n - 1)];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (i * 1024 + e < n) tab[i * 1024 + e] = c[i];
    __syncthreads();
    int total = 0;
    if (mine)
      for (int b = 0; b < n_blocks; ++b) total += tab[b * E + e];
    int all = 0;
    const int off = block_exclusive_scan(total, &all);
    if (mine) {
      int run = off;
      for (int b = 0; b < n_blocks; ++b) {
        const int cnt = tab[b * E + e];
        tab[b * E + e] = run;
        run += cnt;
      }
      offsets[e] = off;
    }
    if (e == 0) offsets[E] = all;
    __syncthreads();
    for (int i = e; i < n; i += 1024) hist[i] = tab[i];
    return;
  }
  const int ec = min(e, E - 1);
  int total = 0;
  for (int b0 = 0; b0 < n_blocks; b0 += kScanBatch) {
    int c[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) c[i] = hist[(int64_t)min(b0 + i, n_blocks - 1) * E + ec];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      if (mine && b0 + i < n_blocks) total += c[i];
  }
  int all = 0;
  const int off = block_exclusive_scan(total, &all);
  int run = off;
  for (int b0 = 0; b0 < n_blocks; b0 += kScanBatch) {
    int c[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) c[i] = hist[(int64_t)min(b0 + i, n_blocks - 1) * E + ec];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) {
      if (mine && b0 + i < n_blocks) {
        hist[(int64_t)(b0 + i) * E + e] = run;
        run += c[i];
      }
    }
  }
  if (mine) offsets[e] = off;
  if (e == 0) offsets[E] = all;
}

__global__ __launch_bounds__(kWave) void scatter_kernel(const uint32_t* __restrict__ idx,
                                                         int n_slots, int E, int per_block,
                                                         const int32_t* __restrict__ base,
                                                         int32_t* __restrict__ slot_of_row,
                                                         int32_t* __restrict__ row_of_slot,
                                                         const uint8_t* __restrict__ active,
                                                         int mask_dims, int k) {
  __shared__ int run[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kWave) run[e] = base[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  const int nbits = 32 - __clz(E);  // ids 0..E (E = "not dispatched") fit in nbits
  const int s0 = (int)std::min<int64_t>((int64_t)blockIdx.x * per_block, n_slots);
  const int s_end = (int)std::min<int64_t>((int64_t)s0 + per_block, n_slots);
  for (int64_t c = s0; c < s_end; c += kIdBatch * kWave) {
    uint32_t ev[kIdBatch];
    load_ids(idx, c, s_end, n_slots, E, active, mask_dims, k, ev);
    place_batch(ev, c, s_end, E, nbits, run, slot_of_row, row_of_slot);
  }
}

// One workgroup of kOneBlockWaves wavefronts; wavefront w owns the slots
// [w * per, (w + 1) * per) and its counts per expert live in LDS. Up to
// kOneBlockSlots slots (measured: faster than the three launches up to 16K
// slots, slower at 64K, where one CU walks all of them).
constexpr int kOneBlockWaves = 16;
constexpr int kOneBlockSlots = 16384;

__global__ __launch_bounds__(kOneBlockWaves * kWave) void dispatch_one_block_kernel(
    const uint32_t* __restrict__ idx, int n_slots, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of_row, int32_t* __restrict__ row_of_slot,
    const uint8_t* __restrict__ active, int mask_dims, int k) {
  __shared__ int cnt[kOneBlockWaves * kMaxExperts];  // [wave][E]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kOneBlockWaves * E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int per = ((n_slots + kOneBlockWaves - 1) / kOneBlockWaves + kWave - 1) / kWave * kWave;
  const int s_begin = min(wave * per, n_slots);
  const int s_end = min(s_begin + per, n_slots);
  int* my = cnt + wave * E;

  // 1. counts of this wavefront's slots per expert
  for (int64_t c = s_begin; c < s_end; c += kIdBatch * kWave) {
    uint32_t e[kIdBatch];
    load_ids(idx, c, s_end, n_slots, E, active, mask_dims, k, e);
#pragma unroll
    for (int b = 0; b < kIdBatch; ++b)
      if (e[b] < (uint32_t)E) atomicAdd(&my[e[b]], 1);
  }
  __syncthreads();

  // 2. thread e: expert e's offset and each wavefront's first row in it
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    for (int w = 0; w < kOneBlockWaves; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = total;
      total += c;
    }
  }
  int all = 0;
  const int off = block_exclusive_scan(total, &all);
  if (e < E) {
    offsets[e] = off;
    for (int w = 0; w < kOneBlockWaves; ++w) cnt[w * E + e] += off;
  }
  if (e == 0) offsets[E] = all;
  __syncthreads();

  // 3. rows in slot order: running row per expert plus the rank among equal
  // ids of the chunk (as scatter_kernel)
  const int nbits = 32 - __clz(E);
  for (int64_t c = s_begin; c < s_end; c += kIdBatch * kWave) {
    uint32_t ev[kIdBatch];
    load_ids(idx, c, s_end, n_slots, E, active, mask_dims, k, ev);
    place_batch(ev, c, s_end, E, nbits, my, slot_of_row, row_of_slot);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ x, int H, int k,
                                                      const int32_t* __restrict__ slot_of_row,
                                                      const int32_t* __restrict__ offsets_end,
                                                      T* __restrict__ x_disp) {
  const int vec_per_row = H / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = i / vec_per_row;
  const int v = (int)(i % vec_per_row);
  if (row >= *offsets_end) return;
  const int64_t src = slot_of_row[row] / k;
  Vec8<T> d;
  d.load(x + src * H + v * 8);
  d.store(x_disp + row * H + v * 8);
}

}  // namespace

DispatchPlan dispatch_plan(int64_t n_slots, int64_t E) {
  (void)E;
  DispatchPlan p;
  p.n_slots = (int)n_slots;
  int64_t per = (n_slots + kMaxBlocks - 1) / kMaxBlocks;
  if (per < 1024) per = 1024;
  per = (per + kWave - 1) / kWave * kWave;
  p.slots_per_block = (int)per;
  p.n_blocks = (int)((n_slots + per - 1) / per);
  if (p.n_blocks < 1) p.n_blocks = 1;
  return p;
}

size_t dispatch_scratch_bytes(int64_t n_slots, int64_t E) {
  const DispatchPlan p = dispatch_plan(n_slots, E);
  return (size_t)p.n_blocks * (size_t)E * sizeof(int32_t);
}

hipError_t launch_dispatch_maps(const uint32_t* indices, int n_slots, int E, int32_t* offsets,
                                int32_t* slot_of_row, int32_t* row_of_slot, int32_t* scratch,
                                hipStream_t s, const uint8_t* active, int mask_dims, int k) {
  if (!active) mask_dims = 0;
  if (k < 1) k = 1;
  if (n_slots <= kOneBlockSlots) {
    hipLaunchKernelGGL(dispatch_one_block_kernel, dim3(1), dim3(kOneBlockWaves * kWave), 0, s,
                       indices, n_slots, E, offsets, slot_of_row, row_of_slot, active, mask_dims, k);
    return hipGetLastError();
  }
  const DispatchPlan p = dispatch_plan(n_slots, E);
  hipLaunchKernelGGL(hist_kernel, dim3(p.n_blocks), dim3(kWave), 0, s, indices, n_slots, E,
                     p.slots_per_block, scratch, active, mask_dims, k);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, scratch, p.n_blocks, E, offsets);
  hipLaunchKernelGGL(scatter_kernel, dim3(p.n_blocks), dim3(kWave), 0, s, indices, n_slots, E,
                     p.slots_per_block, scratch, slot_of_row, row_of_slot, active, mask_dims, k);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, int dt, int H, int k, const int32_t* slot_of_row,
                              const int32_t* offsets_end, int max_rows, void* x_disp,
                              hipStream_t s) {
  const int64_t n = (int64_t)max_rows * (H / 8);
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256);
  switch (dt) {
    case kF32:
      hipLaunchKernelGGL(gather_kernel<float>, dim3(blocks), dim3(256), 0, s,
                         static_cast<const float*>(x), H, k, slot_of_row, offsets_end,
                         static_cast<float*>(x_disp));
      break;
    case kF16:
      hipLaunchKernelGGL(gather_kernel<f16>, dim3(blocks), dim3(256), 0, s,
                         static_cast<const f16*>(x), H, k, slot_of_row, offsets_end,
                         static_cast<f16*>(x_disp));
      break;
    default:
      hipLaunchKernelGGL(gather_kernel<bf16>, dim3(blocks), dim3(256), 0, s,
                         static_cast<const bf16*>(x), H, k, slot_of_row, offsets_end,
                         static_cast<bf16*>(x_disp));
  }
  return hipGetLastError();
}

}  // namespace moe
