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
// for every run. A fourth launch gathers the token rows into x_disp.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kMaxBlocks = 256;

// Expert id slot s is dispatched to, or E for "not dispatched": ids >= E and
// slots switched off by the activity mask (mask_dims 1: one flag per token,
// 2: one per slot; 0: no mask) are not dispatched.
__device__ __forceinline__ uint32_t slot_expert(const uint32_t* idx, int64_t s, int E,
                                                const uint8_t* active, int mask_dims, int k) {
  uint32_t e = idx[s];
  if (e > (uint32_t)E) e = (uint32_t)E;
  if (mask_dims == 1 && !active[s / k]) e = (uint32_t)E;
  if (mask_dims == 2 && !active[s]) e = (uint32_t)E;
  return e;
}

__global__ __launch_bounds__(kWave) void hist_kernel(const uint32_t* __restrict__ idx, int n_slots,
                                                      int E, int per_block,
                                                      int32_t* __restrict__ hist,
                                                      const uint8_t* __restrict__ active,
                                                      int mask_dims, int k) {
  __shared__ int cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kWave) cnt[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * per_block;
  for (int i = threadIdx.x; i < per_block; i += kWave) {
    const int64_t s = s0 + i;
    if (s < n_slots) {
      const uint32_t e = slot_expert(idx, s, E, active, mask_dims, k);
      if (e < (uint32_t)E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kWave) hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// One block of 1024 threads, thread e owns expert e.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ hist, int n_blocks,
                                                     int E, int32_t* __restrict__ offsets) {
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    for (int b = 0; b < n_blocks; ++b) {
      const int c = hist[(int64_t)b * E + e];
      hist[(int64_t)b * E + e] = total;
      total += c;
    }
  }
  int all = 0;
  const int off = block_exclusive_scan(total, &all);
  if (e < E) {
    offsets[e] = off;
    for (int b = 0; b < n_blocks; ++b) hist[(int64_t)b * E + e] += off;
  }
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
  const int lane = threadIdx.x;
  const int nbits = 32 - __clz(E);  // ids 0..E (E = "not dispatched") fit in nbits
  const int64_t s0 = (int64_t)blockIdx.x * per_block;
  for (int c = 0; c < per_block; c += kWave) {
    const int64_t s = s0 + c + lane;
    const bool in = s < n_slots;
    const uint32_t e = in ? slot_expert(idx, s, E, active, mask_dims, k) : (uint32_t)E;
    uint64_t same = __ballot(in);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1u;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & lanemask_lt());
    const bool last = (same >> lane) == 1ull;  // no equal id in a higher lane
    int row = -1;
    if (in && e < (uint32_t)E) {
      row = run[e] + rank;
      slot_of_row[row] = (int32_t)s;
    }
    if (in) row_of_slot[s] = row;
    // All lanes have read run[] above (same instruction stream, LDS ops in
    // order); the last lane of each id advances that expert's counter.
    if (in && e < (uint32_t)E && last) run[e] = row + 1;
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
  const DispatchPlan p = dispatch_plan(n_slots, E);
  if (!active) mask_dims = 0;
  if (k < 1) k = 1;
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
