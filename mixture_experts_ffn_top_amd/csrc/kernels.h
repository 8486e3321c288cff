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
// Grouped-limited sigmoid routing; bias may be null. Arguments validated by the caller.
hipError_t launch_route_grouped(const void* logits, int logits_dt, const float* bias, int T, int E,
                                int k, int groups, int sel_groups, int top_two, int renorm,
                                float scale, uint32_t* indices, void* weights, hipStream_t s);

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
                                hipStream_t s,
                                const uint8_t* active = nullptr, int mask_dims = 0, int k = 1);
// x_disp[r] = x[slot_of_row[r] / k] for r < offsets[E] (read on the device).
hipError_t launch_gather_rows(const void* x, int dt, int H, int k, const int32_t* slot_of_row,
                              const int32_t* offsets_end, int max_rows, void* x_disp,
                              hipStream_t s);

// ---- experts (grouped GEMMs) ---------------------------------------------------
// The schedule of the MFMA path is built on the device from the expert
// offsets (plan kernel). The down GEMM may split the K of its last round's
// tiles (fp32 partial sums, added in K-range order into expert_out).
struct ExpertsPlan {
  int bm;           // rows per M-tile
  int max_tiles;    // host upper bound of the M-tile count
  int split_cap;    // most K-ranges a tile of the down GEMM's last round may take (1: none)
  int split_slots;  // partial-sum blocks reserved for split tiles (0: none)
  int64_t sched_entries;  // schedule slots, the larger of the two GEMMs'
};
ExpertsPlan experts_plan(int64_t rows, int64_t E, int64_t H, int64_t I, int dt);
// Scratch of one GEMM call (schedule, split-tile table and partial sums).
size_t gemm_scratch_bytes(int64_t rows, int64_t E, int64_t H, int64_t I, int dt);
// Scratch of both GEMMs (the above + h).
size_t experts_scratch_bytes(int64_t rows, int64_t E, int64_t H, int64_t I, int dt);

// a_map: optional; when given, A row r is row a_map[r] / a_div of `a`
// (gathering tokens straight from x instead of a materialised x_disp).
// cache (optional): also write g and u rounded to dt into cache[rows, 2I] and
// form h from those rounded values (the experts' training forward); only
// where gate_up_can_cache() holds (the MFMA path, not the decode path).
hipError_t launch_gate_up(const void* a, const int32_t* a_map, int a_div, const int32_t* offsets,
                          int rows, int E, int H, int I, const void* w_gate, const void* w_up,
                          int dt, void* h, void* scratch, hipStream_t s, void* cache = nullptr);
bool gate_up_can_cache(int64_t rows, int64_t E, int dt);
hipError_t launch_down(const void* h, const int32_t* offsets, int rows, int E, int H, int I,
                       const void* w_down, int dt, void* expert_out, void* scratch, hipStream_t s);
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

// Combine with special experts (zero / copy / constant) and an activity mask;
// with residual != nullptr the residual Add + RMSNorm follow (out = y).
struct SpecialCombine {
  const void* expert_out;
  const int32_t* row_of_slot;
  const uint32_t* indices;
  const void* weights;
  int w_dt, dt, k, H, E, n_zero, n_copy, n_const;
  const void* ori_x;
  const void* alpha1;
  const void* alpha2;
  const void* const_v;
  const uint8_t* active;
  int mask_dims;
  const void* shared;
  const void* residual;
  const float* gamma;
  float eps;
  void* out;
  void* x_out;
  float* rstd;
};
hipError_t launch_combine_special(const SpecialCombine& c, int T, hipStream_t s);

// Weight-only quantised experts (INT8 / INT4 with per-channel or per-group
// scale and offset) on the decode path: both GEMMs, h in the caller's buffer.
struct QuantExperts {
  const void* x;            // tokens [*, H] read through row_map / map_div, or dispatched rows
  const int32_t* row_map;
  int map_div;
  const int32_t* offsets;   // [E+1]
  int rows, E, H, I, dt, bits, groups;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* s_gate;
  const void* s_up;
  const void* s_down;
  const void* o_gate;
  const void* o_up;
  const void* o_down;
  void* h;                  // [rows, I]
  void* expert_out;         // [rows, H]
};
hipError_t launch_experts_quant(const QuantExperts& q, hipStream_t s);

// ---- first-order training ------------------------------------------------------
// Experts' training forward (fills the cache, then the down GEMM) and backward.
// cache: [rows, 2I] = (g | u) followed by [rows, I] = h, all in dt (bf16/f16).
// ws: train_prefix_bytes(E), then for the forward gemm_scratch_bytes(...),
// for the backward [rows, 2I] dt (dg | du).
struct TrainExperts {
  const void* x;            // dispatched rows [rows, H]
  const int32_t* offsets;   // [E+1]
  int rows, E, H, I, dt;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  void* cache;
  void* y;                  // forward: expert_out [rows, H]
  const void* dy;           // backward: dexpert [rows, H]
  void* dx;                 // backward: dinput [rows, H]
  float* d_gate;            // backward: [E, I, H]
  float* d_up;              // backward: [E, I, H]
  float* d_down;            // backward: [E, H, I]
  void* ws;
};
size_t train_prefix_bytes(int64_t E);
hipError_t launch_experts_forward_training(const TrainExperts& q, hipStream_t s);
hipError_t launch_experts_backward(const TrainExperts& q, hipStream_t s);

// Router weights of a fixed selection (grad_weights == nullptr) or their
// gradient with respect to the logits.
struct RouterGrad {
  const void* logits;
  int logits_dt;
  const void* indices;
  int idx_dt;               // 0 uint32, 1 int32, 2 int64
  int T, E, k, scoring, normalize;
  float scale;
  float* weights;
  const float* grad_weights;
  void* grad_logits;
};
hipError_t launch_router_grad(const RouterGrad& r, hipStream_t s);
hipError_t launch_combine_backward(const void* y, const int32_t* row_of_slot, const void* w, int w_dt,
                                   const void* grad_out, int T, int k, int H, int dt, void* dexpert,
                                   float* dweights, hipStream_t s);
hipError_t launch_dispatch_backward(const void* dinput, const int32_t* row_of_slot, int T, int k,
                                    int H, int dt, void* dx, hipStream_t s);

}  // namespace moe
