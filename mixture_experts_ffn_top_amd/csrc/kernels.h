// Internal launchers of libmoe_ffn (host side; not part of the ABI). Each
// enqueues its kernels on `s` and returns hipGetLastError(). Arguments are
// already validated by the C-ABI layer in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum DType { kF32 = 0, kF16 = 1, kBF16 = 2 };

inline size_t dtype_size(int dt) { return dt == kF32 ? 4 : 2; }

// ---- routing ----------------------------------------------------------------
hipError_t launch_route(const void* logits, int logits_dt, int T, int E, int k, int renorm,
                        uint32_t* indices, void* weights, hipStream_t s);

// ---- dispatch ---------------------------------------------------------------
// Scratch: one int32 histogram row of E entries per block of slots.
struct DispatchPlan {
  int n_slots;          // T * k
  int slots_per_block;  // multiple of 64
  int n_blocks;
};
DispatchPlan dispatch_plan(int64_t n_slots, int64_t E);
size_t dispatch_scratch_bytes(int64_t n_slots, int64_t E);
hipError_t launch_dispatch_maps(const uint32_t* indices, int n_slots, int E, int32_t* offsets,
                                int32_t* slot_of_row, int32_t* row_of_slot, int32_t* scratch,
                                hipStream_t s);
// x_disp[r] = x[slot_of_row[r] / k] for r < offsets[E] (read on the device).
hipError_t launch_gather_rows(const void* x, int dt, int H, int k, const int32_t* slot_of_row,
                              const int32_t* offsets_end, int max_rows, void* x_disp,
                              hipStream_t s);

// ---- experts (grouped GEMMs) ---------------------------------------------------
// The M-tile list: for each tile, (expert, first row). Built on the device
// from the expert offsets; its length is stored at tile_count.
struct ExpertsPlan {
  int bm;         // rows per M-tile
  int max_tiles;  // host upper bound of the tile count
};
ExpertsPlan experts_plan(int64_t rows, int64_t E, int dt);
size_t experts_scratch_bytes(int64_t rows, int64_t E, int64_t I, int dt);
// Scratch of one GEMM call on its own (the tile list only).
size_t tile_scratch_bytes(int64_t rows, int64_t E, int dt);
hipError_t launch_gate_up(const void* a, const int32_t* a_map, int a_div, const int32_t* offsets,
                          int rows, int E, int H, int I, const void* w_gate, const void* w_up,
                          int dt, void* h, void* scratch, hipStream_t s);
hipError_t launch_down(const void* h, const int32_t* offsets, int rows, int E, int H, int I,
                       const void* w_down, int dt, void* expert_out, void* scratch,
                       hipStream_t s);
// a_map: optional; when given, A row r is row a_map[r] / a_div of `a`
// (gathering tokens straight from x instead of a materialised x_disp).
hipError_t launch_experts(const void* a, const int32_t* a_map, int a_div,
                          const int32_t* offsets, int rows, int E, int H, int I,
                          const void* w_gate, const void* w_up, const void* w_down, int dt,
                          void* expert_out, void* scratch, hipStream_t s);

// ---- combine ------------------------------------------------------------------
hipError_t launch_combine(const void* expert_out, const int32_t* row_of_slot, const void* weights,
                          int w_dt, int T, int k, int H, int dt, void* out, hipStream_t s);
hipError_t launch_combine_add_rmsnorm(const void* expert_out, const int32_t* row_of_slot,
                                      const void* weights, int w_dt, const void* shared,
                                      const void* residual, const float* gamma, float eps, int T,
                                      int k, int H, int dt, void* y, void* x_out, float* rstd,
                                      hipStream_t s);

}  // namespace moe
