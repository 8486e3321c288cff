// Internal helpers shared by the HIP kernels of libmoe_ffn (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef _Float16 f16;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
// Buffer resources: word-3 flags of a raw (unswizzled, stride 0) buffer and
// the non-temporal cache policy of buffer loads.
constexpr int kBufferFlags = 0x00020000;
constexpr int kCachePolicyNT = 2;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v) { return (T)v; }

// Eight consecutive elements of T, moved with 16-byte memory operations.
template <typename T>
struct Vec8 {
  static constexpr int kBytes = 8 * (int)sizeof(T);
  static constexpr int kChunks = kBytes / 16;  // 1 for 2-byte types, 2 for fp32
  uint4 raw[kChunks];

  __device__ __forceinline__ void load(const T* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) raw[i] = q[i];
  }
  __device__ __forceinline__ void store(T* p) const {
    uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) q[i] = raw[i];
  }
  // Streaming variants: data touched once, marked non-temporal.
  __device__ __forceinline__ void load_nt(const T* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) raw[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(q + i));
  }
  __device__ __forceinline__ void store_nt(T* p) const {
    u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, raw[i]), q + i);
  }
  // Streaming load at byte offset `off` of a buffer resource; an offset past
  // the resource's range reads zeros and touches no memory.
  __device__ __forceinline__ void load_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      raw[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * (uint32_t)i, 0, kCachePolicyNT));
  }
  __device__ __forceinline__ float get(int i) const {
    return to_f32(reinterpret_cast<const T*>(raw)[i]);
  }
  __device__ __forceinline__ void set(int i, float v) {
    reinterpret_cast<T*>(raw)[i] = from_f32<T>(v);
  }
};

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << __lane_id()) - 1ull;
}

// Exclusive prefix sum over the threads of a block (blockDim.x <= 1024,
// multiple of 64). Returns this thread's exclusive prefix; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wave_sums[16];
  const int lane = __lane_id();
  const int wave = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  const int nwaves = blockDim.x / kWave;
  if (wave == 0) {
    int s = lane < nwaves ? wave_sums[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      int o = __shfl_up(s, d, kWave);
      if (lane >= d) s += o;
    }
    if (lane < nwaves) wave_sums[lane] = s;  // inclusive
  }
  __syncthreads();
  int before = wave ? wave_sums[wave - 1] : 0;
  *total = wave_sums[nwaves - 1];
  __syncthreads();
  return before + incl - v;
}

}  // namespace moe
