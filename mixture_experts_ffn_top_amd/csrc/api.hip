// C ABI of libmoe_ffn: host-side validation, workspace carving and launches.
// Every check runs before anything is enqueued; on error nothing is enqueued.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <stdint.h>

#include "kernels.h"
#include <cmath>
#include "moe_ffn.h"

using namespace moe;

namespace {

constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxNormH = 32768;

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

struct Span {
  const void* p;
  size_t n;
};

bool overlaps(Span a, Span b) {
  if (!a.p || !b.p || !a.n || !b.n) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Each output must be disjoint from every input and every other output.
bool any_overlap(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(outs[i], outs[j])) return true;
  }
  return false;
}

bool valid_dt(int dt) { return dt == MOE_F32 || dt == MOE_F16 || dt == MOE_BF16; }

moe_status stream_device(hipStream_t s, int* dev) {
  if (s == nullptr) return hipGetDevice(dev) == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP;
  if (hipStreamGetDevice(s, dev) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERROR_HIP;
  }
  return MOE_SUCCESS;
}

// Pointers must be device (or managed) memory of the stream's device.
moe_status check_device(const void* const* ptrs, int n, hipStream_t s) {
  int dev = 0;
  moe_status st = stream_device(s, &dev);
  if (st != MOE_SUCCESS) return st;
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) continue;
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, ptrs[i]) != hipSuccess) {
      (void)hipGetLastError();
      return MOE_ERROR_DEVICE;
    }
    if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged) return MOE_ERROR_DEVICE;
    if (at.device != dev) return MOE_ERROR_DEVICE;
  }
  return MOE_SUCCESS;
}

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_HIP; }

moe_status check_route_args(int64_t T, int64_t E, int64_t top_k, moe_dtype logits_dt) {
  if (T < 0 || E < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(logits_dt)) return MOE_ERROR_DTYPE;
  if (top_k < 1 || top_k > E) return MOE_ERROR_ARGUMENT;
  if (E > kMaxE || T * top_k > INT32_MAX) return MOE_ERROR_UNSUPPORTED;
  return MOE_SUCCESS;
}

bool row_len_ok(int64_t n) { return n > 0 && n % 8 == 0; }
// The combine kernels address one expert row through a buffer resource whose
// 32-bit range is the row's byte length.
bool row_bytes_ok(int64_t H, moe_dtype dt) { return H * (int64_t)dtype_size(dt) <= INT32_MAX; }

// n * m * ds < 2^31 without overflowing (n, m >= 0, m * ds <= 2^33).
bool below_2g(int64_t n, int64_t m, int64_t ds) {
  return n == 0 || m == 0 || (m <= INT32_MAX && n <= INT32_MAX / (m * ds));
}

// The bf16 / f16 expert GEMMs (the tiled matrix-core kernel and the decode
// kernel) address every operand through a buffer resource with a 32-bit byte
// range, and mask a load or store by giving it the offset 2^31, which must
// lie outside every range. So the token rows they read (a_rows x H), h
// (rows x I), one expert's weight matrix (I x H), and one 256-row output tile
// of up to 2I fp32 columns (the training cache stores g and u side by side)
// must each stay below 2^31 bytes. The fp32 path uses 64-bit pointers and is
// not limited.
bool gemm_bytes_ok(int64_t a_rows, int64_t rows, int64_t H, int64_t I, moe_dtype dt) {
  if (dt == MOE_F32) return true;
  const int64_t ds = (int64_t)dtype_size(dt);
  return below_2g(a_rows, H, ds) && below_2g(rows, I, ds) && below_2g(I, H, ds) &&
         below_2g(256, std::max(H, 2 * I), 4);
}

// Options of the grouped-limited sigmoid router (ruDNN user guide, "10.
// Grouped-limited sigmoid MoE routing"), validated after check_route_args.
moe_status check_grouped_args(int64_t E, int64_t top_k, int64_t groups, int64_t selected_groups,
                              int group_top_two, float scale) {
  if (groups < 1 || groups > 128 || E % groups != 0) return MOE_ERROR_ARGUMENT;
  if (selected_groups < 1 || selected_groups > groups) return MOE_ERROR_ARGUMENT;
  const int64_t gs = E / groups;
  if (top_k > 64 || top_k > selected_groups * gs) return MOE_ERROR_ARGUMENT;
  if (group_top_two && gs < 2) return MOE_ERROR_ARGUMENT;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return MOE_ERROR_ARGUMENT;
  return MOE_SUCCESS;
}

// Weight-only quantised experts (aclnnFFN, pseudo-quantization scenario).
struct QuantWeights {
  int bits = 0;  // 8 or 4; 0: not quantised
  int64_t groups = 1;
  const void *s_gate = nullptr, *s_up = nullptr, *s_down = nullptr;
  const void *o_gate = nullptr, *o_up = nullptr, *o_down = nullptr;
};

moe_status check_quant_args(int64_t rows, int64_t E, int64_t H, int64_t I, int bits, int64_t groups,
                            moe_dtype dt) {
  if (bits != 8 && bits != 4) return MOE_ERROR_ARGUMENT;
  if (groups < 1 || H % groups != 0 || I % groups != 0) return MOE_ERROR_ARGUMENT;
  if (groups > 1 && bits != 4) return MOE_ERROR_ARGUMENT;  // per-group mode is INT4 only
  if (dt != MOE_BF16 && dt != MOE_F16) return MOE_ERROR_UNSUPPORTED;
  if (groups > 1 && ((H / groups) % 128 != 0 || (I / groups) % 128 != 0)) return MOE_ERROR_UNSUPPORTED;
  if (!row_len_ok(H) || !row_len_ok(I) || E > kMaxE) return MOE_ERROR_UNSUPPORTED;
  if (rows > 4 * E) return MOE_ERROR_UNSUPPORTED;  // decode-sized batches only
  // one expert's codes and the activation rows are addressed with 32-bit offsets
  if (H * I * bits / 8 > INT32_MAX || 4 * E * std::max(H, I) * 2 > INT32_MAX) return MOE_ERROR_UNSUPPORTED;
  return MOE_SUCCESS;
}

// Bytes of one quantised weight tensor [E, N, K].
size_t quant_bytes(int64_t E, int64_t N, int64_t K, int bits) {
  return (size_t)E * (size_t)N * (size_t)K * (size_t)bits / 8;
}

// Routing step of a forward pass: writes indices [T,k] and weights [T,k].
struct Router {
  bool grouped = false;
  int renormalize = 0;
  const float* bias = nullptr;
  int groups = 1, selected_groups = 1, group_top_two = 0;
  float scale = 1.0f;
  hipError_t run(const void* logits, int logits_dt, int T, int E, int k, uint32_t* idx, void* w,
                 hipStream_t s) const {
    return grouped ? launch_route_grouped(logits, logits_dt, bias, T, E, k, groups, selected_groups,
                                          group_top_two, renormalize, scale, idx, w, s)
                   : launch_route(logits, logits_dt, T, E, k, renormalize, idx, w, s);
  }
};

// Layout of the moe_forward workspace; every piece 256-byte aligned.
struct ForwardLayout {
  size_t indices, weights, offsets, slot_of_row, row_of_slot, dispatch, expert_out, experts, total;
};

ForwardLayout forward_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int dt,
                             int logits_dt) {
  ForwardLayout L;
  const size_t slots = (size_t)(T * k);
  size_t o = 0;
  L.indices = o;     o += align256(slots * 4);
  L.weights = o;     o += align256(slots * dtype_size(logits_dt));
  L.offsets = o;     o += align256((size_t)(E + 1) * 4);
  L.slot_of_row = o; o += align256(slots * 4);
  L.row_of_slot = o; o += align256(slots * 4);
  L.dispatch = o;    o += align256(dispatch_scratch_bytes((int64_t)slots, E));
  L.expert_out = o;  o += align256(slots * (size_t)H * dtype_size(dt));
  L.experts = o;     o += align256(experts_scratch_bytes((int64_t)slots, E, H, I, dt));
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_SUCCESS: return "MOE_SUCCESS";
    case MOE_ERROR_NULL_POINTER: return "MOE_ERROR_NULL_POINTER";
    case MOE_ERROR_SHAPE: return "MOE_ERROR_SHAPE";
    case MOE_ERROR_DTYPE: return "MOE_ERROR_DTYPE";
    case MOE_ERROR_ARGUMENT: return "MOE_ERROR_ARGUMENT";
    case MOE_ERROR_DEVICE: return "MOE_ERROR_DEVICE";
    case MOE_ERROR_WORKSPACE: return "MOE_ERROR_WORKSPACE";
    case MOE_ERROR_UNSUPPORTED: return "MOE_ERROR_UNSUPPORTED";
    case MOE_ERROR_HIP: return "MOE_ERROR_HIP";
  }
  return "MOE_ERROR_UNKNOWN";
}

moe_status moe_route(const void* logits, moe_dtype logits_dt, int64_t T, int64_t E, int64_t top_k,
                     int renormalize, uint32_t* indices, void* weights, hipStream_t stream) {
  moe_status st = check_route_args(T, E, top_k, logits_dt);
  if (st != MOE_SUCCESS) return st;
  if (T == 0) return MOE_SUCCESS;
  if (!logits || !indices || !weights) return MOE_ERROR_NULL_POINTER;
  const size_t ls = dtype_size(logits_dt);
  const Span outs[] = {{indices, (size_t)(T * top_k) * 4}, {weights, (size_t)(T * top_k) * ls}};
  const Span ins[] = {{logits, (size_t)(T * E) * ls}};
  if (any_overlap(outs, 2, ins, 1)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {logits, indices, weights};
  if ((st = check_device(ptrs, 3, stream)) != MOE_SUCCESS) return st;
  return from_hip(launch_route(logits, logits_dt, (int)T, (int)E, (int)top_k, renormalize ? 1 : 0,
                               indices, weights, stream));
}

size_t moe_dispatch_workspace_size(int64_t T, int64_t top_k, int64_t E) {
  if (T < 0 || top_k < 1 || E < 1 || E > kMaxE || T * top_k > INT32_MAX) return 0;
  return align256(dispatch_scratch_bytes(T * top_k, E));
}

}  // extern "C"

namespace {

moe_status dispatch_impl(const uint32_t* indices, const uint8_t* active, int mask_dims, int64_t T,
                         int64_t top_k, int64_t E, const void* x, moe_dtype dt, int64_t H,
                         void* x_disp, int32_t* expert_offsets, int32_t* slot_of_row,
                         int32_t* row_of_slot, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || E < 1 || H < 0) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt)) return MOE_ERROR_DTYPE;
  if (top_k < 1) return MOE_ERROR_ARGUMENT;
  if (mask_dims < 0 || mask_dims > 2 || (mask_dims > 0) != (active != nullptr)) return MOE_ERROR_ARGUMENT;
  if (E > kMaxE || T * top_k > INT32_MAX) return MOE_ERROR_UNSUPPORTED;
  if (x_disp && !row_len_ok(H)) return MOE_ERROR_UNSUPPORTED;
  if (!expert_offsets) return MOE_ERROR_NULL_POINTER;
  if (T > 0 && (!indices || !slot_of_row || !row_of_slot)) return MOE_ERROR_NULL_POINTER;
  if (x_disp && !x) return MOE_ERROR_NULL_POINTER;
  const size_t need = moe_dispatch_workspace_size(T, top_k, E);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < need) return MOE_ERROR_WORKSPACE;
  const size_t slots = (size_t)(T * top_k), ds = dtype_size(dt);
  const Span outs[] = {{x_disp, x_disp ? slots * (size_t)H * ds : 0},
                       {expert_offsets, (size_t)(E + 1) * 4},
                       {slot_of_row, slots * 4},
                       {row_of_slot, slots * 4},
                       {ws, need}};
  const Span ins[] = {{indices, slots * 4}, {x, x ? (size_t)T * (size_t)H * ds : 0},
                      {active, mask_dims == 1 ? (size_t)T : mask_dims == 2 ? slots : 0}};
  if (any_overlap(outs, 5, ins, 3)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {indices, x, x_disp, expert_offsets, slot_of_row, row_of_slot, ws, active};
  moe_status st = check_device(ptrs, 8, stream);
  if (st != MOE_SUCCESS) return st;
  hipError_t e = launch_dispatch_maps(indices, (int)slots, (int)E, expert_offsets, slot_of_row,
                                      row_of_slot, static_cast<int32_t*>(ws), stream, active,
                                      mask_dims, (int)top_k);
  if (e == hipSuccess && x_disp && slots)
    e = launch_gather_rows(x, dt, (int)H, (int)top_k, slot_of_row, expert_offsets + E, (int)slots,
                           x_disp, stream);
  return from_hip(e);
}

}  // namespace

extern "C" {

moe_status moe_dispatch(const uint32_t* indices, int64_t T, int64_t top_k, int64_t E,
                        const void* x, moe_dtype dt, int64_t H, void* x_disp,
                        int32_t* expert_offsets, int32_t* slot_of_row, int32_t* row_of_slot,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  if (top_k > E && E >= 1) return MOE_ERROR_ARGUMENT;
  return dispatch_impl(indices, nullptr, 0, T, top_k, E, x, dt, H, x_disp, expert_offsets,
                       slot_of_row, row_of_slot, ws, ws_bytes, stream);
}

moe_status moe_dispatch_masked(const uint32_t* indices, const uint8_t* active, int mask_dims,
                               int64_t T, int64_t top_k, int64_t E, const void* x, moe_dtype dt,
                               int64_t H, void* x_disp, int32_t* expert_offsets,
                               int32_t* slot_of_row, int32_t* row_of_slot, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  return dispatch_impl(indices, active, mask_dims, T, top_k, E, x, dt, H, x_disp, expert_offsets,
                       slot_of_row, row_of_slot, ws, ws_bytes, stream);
}

size_t moe_experts_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I, moe_dtype dt) {
  if (rows < 0 || E < 1 || E > kMaxE || rows > INT32_MAX || H < 1 || I < 1 || !valid_dt(dt))
    return 0;
  return align256(experts_scratch_bytes(rows, E, H, I, dt));
}

moe_status moe_experts_forward_dispatched(const void* x_disp, const int32_t* expert_offsets,
                                          int64_t rows, int64_t E, int64_t H, int64_t I,
                                          const void* w_gate, const void* w_up,
                                          const void* w_down, moe_dtype dt, void* expert_out,
                                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (rows < 0 || E < 1 || H < 1 || I < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt)) return MOE_ERROR_DTYPE;
  if (E > kMaxE || rows > INT32_MAX || !row_len_ok(H) || !row_len_ok(I) ||
      !gemm_bytes_ok(rows, rows, H, I, dt))
    return MOE_ERROR_UNSUPPORTED;
  if (rows == 0) return MOE_SUCCESS;
  if (!x_disp || !expert_offsets || !w_gate || !w_up || !w_down || !expert_out)
    return MOE_ERROR_NULL_POINTER;
  const size_t need = moe_experts_workspace_size(rows, E, H, I, dt);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < need) return MOE_ERROR_WORKSPACE;
  const size_t ds = dtype_size(dt), wbytes = (size_t)E * (size_t)I * (size_t)H * ds;
  const Span outs[] = {{expert_out, (size_t)rows * (size_t)H * ds}, {ws, need}};
  const Span ins[] = {{x_disp, (size_t)rows * (size_t)H * ds},
                      {expert_offsets, (size_t)(E + 1) * 4},
                      {w_gate, wbytes}, {w_up, wbytes}, {w_down, wbytes}};
  if (any_overlap(outs, 2, ins, 5)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {x_disp, expert_offsets, w_gate, w_up, w_down, expert_out, ws};
  moe_status st = check_device(ptrs, 7, stream);
  if (st != MOE_SUCCESS) return st;
  return from_hip(launch_experts(x_disp, nullptr, 1, expert_offsets, (int)rows, (int)E, (int)H,
                                 (int)I, w_gate, w_up, w_down, dt, expert_out, ws, stream));
}

size_t moe_experts_gemm_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I,
                                       moe_dtype dt) {
  if (rows < 0 || E < 1 || E > kMaxE || rows > INT32_MAX || H < 1 || I < 1 || !valid_dt(dt))
    return 0;
  return align256(gemm_scratch_bytes(rows, E, H, I, dt));
}

moe_status moe_experts_gate_up(const void* x, const int32_t* row_map, int64_t map_div,
                               const int32_t* expert_offsets, int64_t rows, int64_t E, int64_t H,
                               int64_t I, const void* w_gate, const void* w_up, moe_dtype dt,
                               void* h, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (rows < 0 || E < 1 || H < 1 || I < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt)) return MOE_ERROR_DTYPE;
  if (row_map && (map_div < 1 || map_div > rows)) return MOE_ERROR_ARGUMENT;
  if (E > kMaxE || rows > INT32_MAX || !row_len_ok(H) || !row_len_ok(I) ||
      !gemm_bytes_ok(row_map ? (rows + map_div - 1) / map_div : rows, rows, H, I, dt))
    return MOE_ERROR_UNSUPPORTED;
  if (rows == 0) return MOE_SUCCESS;
  if (!x || !expert_offsets || !w_gate || !w_up || !h) return MOE_ERROR_NULL_POINTER;
  const size_t need = moe_experts_gemm_workspace_size(rows, E, H, I, dt);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < need) return MOE_ERROR_WORKSPACE;
  const size_t ds = dtype_size(dt), wbytes = (size_t)E * (size_t)I * (size_t)H * ds;
  const size_t x_rows = row_map ? (size_t)((rows + map_div - 1) / map_div) : (size_t)rows;
  const Span outs[] = {{h, (size_t)rows * (size_t)I * ds}, {ws, need}};
  const Span ins[] = {{x, x_rows * (size_t)H * ds}, {row_map, row_map ? (size_t)rows * 4 : 0},
                      {expert_offsets, (size_t)(E + 1) * 4}, {w_gate, wbytes}, {w_up, wbytes}};
  if (any_overlap(outs, 2, ins, 5)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {x, row_map, expert_offsets, w_gate, w_up, h, ws};
  moe_status st = check_device(ptrs, 7, stream);
  if (st != MOE_SUCCESS) return st;
  return from_hip(launch_gate_up(x, row_map, row_map ? (int)map_div : 1, expert_offsets, (int)rows,
                                 (int)E, (int)H, (int)I, w_gate, w_up, dt, h, ws, stream));
}

moe_status moe_experts_down(const void* h, const int32_t* expert_offsets, int64_t rows, int64_t E,
                            int64_t H, int64_t I, const void* w_down, moe_dtype dt,
                            void* expert_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (rows < 0 || E < 1 || H < 1 || I < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt)) return MOE_ERROR_DTYPE;
  if (E > kMaxE || rows > INT32_MAX || !row_len_ok(H) || !row_len_ok(I) ||
      !gemm_bytes_ok(rows, rows, H, I, dt))
    return MOE_ERROR_UNSUPPORTED;
  if (rows == 0) return MOE_SUCCESS;
  if (!h || !expert_offsets || !w_down || !expert_out) return MOE_ERROR_NULL_POINTER;
  const size_t need = moe_experts_gemm_workspace_size(rows, E, H, I, dt);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < need) return MOE_ERROR_WORKSPACE;
  const size_t ds = dtype_size(dt), wbytes = (size_t)E * (size_t)I * (size_t)H * ds;
  const Span outs[] = {{expert_out, (size_t)rows * (size_t)H * ds}, {ws, need}};
  const Span ins[] = {{h, (size_t)rows * (size_t)I * ds}, {expert_offsets, (size_t)(E + 1) * 4},
                      {w_down, wbytes}};
  if (any_overlap(outs, 2, ins, 3)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {h, expert_offsets, w_down, expert_out, ws};
  moe_status st = check_device(ptrs, 5, stream);
  if (st != MOE_SUCCESS) return st;
  return from_hip(launch_down(h, expert_offsets, (int)rows, (int)E, (int)H, (int)I, w_down, dt,
                              expert_out, ws, stream));
}

moe_status moe_combine(const void* expert_out, const int32_t* row_of_slot, const void* weights,
                       moe_dtype w_dt, int64_t T, int64_t top_k, int64_t H, moe_dtype dt,
                       void* out, hipStream_t stream) {
  if (T < 0 || top_k < 1 || H < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt) || !valid_dt(w_dt)) return MOE_ERROR_DTYPE;
  if (T * top_k > INT32_MAX || !row_len_ok(H) || !row_bytes_ok(H, dt)) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!expert_out || !row_of_slot || !weights || !out) return MOE_ERROR_NULL_POINTER;
  const size_t ds = dtype_size(dt), slots = (size_t)(T * top_k);
  // expert_out holds at most T*top_k rows (one per dispatched slot).
  const Span outs[] = {{out, (size_t)T * (size_t)H * ds}};
  const Span ins[] = {{expert_out, slots * (size_t)H * ds}, {row_of_slot, slots * 4},
                      {weights, slots * dtype_size(w_dt)}};
  if (any_overlap(outs, 1, ins, 3)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {expert_out, row_of_slot, weights, out};
  moe_status st = check_device(ptrs, 4, stream);
  if (st != MOE_SUCCESS) return st;
  return from_hip(launch_combine(expert_out, row_of_slot, weights, w_dt, (int)T, (int)top_k,
                                 (int)H, dt, out, stream));
}

moe_status moe_combine_add_rmsnorm(const void* expert_out, const int32_t* row_of_slot,
                                   const void* weights, moe_dtype w_dt, const void* shared,
                                   const void* residual, const float* gamma, float eps,
                                   int64_t T, int64_t top_k, int64_t H, moe_dtype dt, void* y,
                                   void* x_out, float* rstd, hipStream_t stream) {
  if (T < 0 || top_k < 1 || H < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt) || !valid_dt(w_dt)) return MOE_ERROR_DTYPE;
  if (!isfinite(eps) || eps <= 0.f) return MOE_ERROR_ARGUMENT;
  if (T * top_k > INT32_MAX || !row_len_ok(H) || H > kMaxNormH) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!expert_out || !row_of_slot || !weights || !residual || !gamma || !y || !x_out || !rstd)
    return MOE_ERROR_NULL_POINTER;
  const size_t ds = dtype_size(dt), slots = (size_t)(T * top_k), th = (size_t)T * (size_t)H * ds;
  const Span outs[] = {{y, th}, {x_out, th}, {rstd, (size_t)T * 4}};
  const Span ins[] = {{expert_out, slots * (size_t)H * ds}, {row_of_slot, slots * 4},
                      {weights, slots * dtype_size(w_dt)}, {shared, shared ? th : 0},
                      {residual, th}, {gamma, (size_t)H * 4}};
  if (any_overlap(outs, 3, ins, 6)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {expert_out, row_of_slot, weights, shared, residual, gamma, y, x_out, rstd};
  moe_status st = check_device(ptrs, 9, stream);
  if (st != MOE_SUCCESS) return st;
  return from_hip(launch_combine_add_rmsnorm(expert_out, row_of_slot, weights, w_dt, shared,
                                             residual, gamma, eps, (int)T, (int)top_k, (int)H, dt,
                                             y, x_out, rstd, stream));
}

size_t moe_forward_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                                  moe_dtype dt, moe_dtype logits_dt) {
  if (check_route_args(T, E, top_k, logits_dt) != MOE_SUCCESS) return 0;
  if (H < 1 || I < 1 || !valid_dt(dt)) return 0;
  return forward_layout(T, H, I, E, top_k, dt, logits_dt).total;
}

}  // extern "C"

namespace {

moe_status forward_impl(const void* x, const void* logits, moe_dtype logits_dt, int64_t T,
                        int64_t H, int64_t I, int64_t E, int64_t top_k, const Router& router,
                        const void* w_gate, const void* w_up, const void* w_down, moe_dtype dt,
                        void* out, uint32_t* indices_out, void* weights_out,
                        int32_t* offsets_out, void* ws, size_t ws_bytes,
                        hipEvent_t* stage_events, hipStream_t stream,
                        const QuantWeights* quant = nullptr, bool ws_is_library_scratch = false) {
  if (H < 1 || I < 1) return MOE_ERROR_SHAPE;
  moe_status st = MOE_SUCCESS;
  if (!valid_dt(dt)) return MOE_ERROR_DTYPE;
  if (!row_len_ok(H) || !row_len_ok(I) || !row_bytes_ok(H, dt)) return MOE_ERROR_UNSUPPORTED;
  if (!quant && !gemm_bytes_ok(T, T * top_k, H, I, dt)) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !logits || !w_gate || !w_up || !w_down || !out) return MOE_ERROR_NULL_POINTER;
  const ForwardLayout L = forward_layout(T, H, I, E, top_k, dt, logits_dt);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < L.total) return MOE_ERROR_WORKSPACE;
  const size_t ds = dtype_size(dt), ls = dtype_size(logits_dt), slots = (size_t)(T * top_k);
  const size_t wbytes = quant ? quant_bytes(E, I, H, quant->bits) : (size_t)E * (size_t)I * (size_t)H * ds;
  const Span outs[] = {{out, (size_t)T * (size_t)H * ds}, {indices_out, indices_out ? slots * 4 : 0},
                       {weights_out, weights_out ? slots * ls : 0},
                       {offsets_out, offsets_out ? (size_t)(E + 1) * 4 : 0}, {ws, L.total}};
  const Span ins[] = {{x, (size_t)T * (size_t)H * ds}, {logits, (size_t)(T * E) * ls},
                      {w_gate, wbytes}, {w_up, wbytes}, {w_down, wbytes}};
  const Span bias_in[] = {{router.bias, router.bias ? (size_t)E * 4 : 0}};
  if (any_overlap(outs, 5, ins, 5) || any_overlap(outs, 5, bias_in, 1)) return MOE_ERROR_ARGUMENT;
  // the library's own scratch array is device memory of the stream's device by construction
  const void* ptrs[] = {x,           logits,      w_gate,      w_up,
                        w_down,      out,         indices_out, weights_out,
                        offsets_out, ws_is_library_scratch ? nullptr : ws, router.bias};
  if ((st = check_device(ptrs, 11, stream)) != MOE_SUCCESS) return st;

  char* base = static_cast<char*>(ws);
  uint32_t* idx = indices_out ? indices_out : reinterpret_cast<uint32_t*>(base + L.indices);
  void* w = weights_out ? weights_out : static_cast<void*>(base + L.weights);
  int32_t* offsets = offsets_out ? offsets_out : reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* sor = reinterpret_cast<int32_t*>(base + L.slot_of_row);
  int32_t* ros = reinterpret_cast<int32_t*>(base + L.row_of_slot);
  void* y = base + L.expert_out;

  auto mark = [&](int i) -> hipError_t {
    return stage_events ? hipEventRecord(stage_events[i], stream) : hipSuccess;
  };
  hipError_t e = mark(0);
  if (e == hipSuccess) e = router.run(logits, logits_dt, (int)T, (int)E, (int)top_k, idx, w, stream);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess)
    e = launch_dispatch_maps(idx, (int)slots, (int)E, offsets, sor, ros,
                             reinterpret_cast<int32_t*>(base + L.dispatch), stream);
  if (e == hipSuccess) e = mark(2);
  // The gate/up GEMM gathers token rows through slot_of_row; x_disp is never
  // materialised on this path.
  void* h = base + L.experts + gemm_scratch_bytes((int64_t)slots, E, H, I, dt);
  if (quant) {
    QuantExperts q = {};
    q.x = x; q.row_map = sor; q.map_div = (int)top_k; q.offsets = offsets;
    q.rows = (int)slots; q.E = (int)E; q.H = (int)H; q.I = (int)I; q.dt = dt;
    q.bits = quant->bits; q.groups = (int)quant->groups;
    q.w_gate = w_gate; q.w_up = w_up; q.w_down = w_down;
    q.s_gate = quant->s_gate; q.s_up = quant->s_up; q.s_down = quant->s_down;
    q.o_gate = quant->o_gate; q.o_up = quant->o_up; q.o_down = quant->o_down;
    q.h = h; q.expert_out = y;
    if (e == hipSuccess) e = launch_experts_quant(q, stream);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = mark(4);
    if (e == hipSuccess)
      e = launch_combine(y, ros, w, logits_dt, (int)T, (int)top_k, (int)H, dt, out, stream);
    if (e == hipSuccess) e = mark(5);
    return from_hip(e);
  }
  if (e == hipSuccess)
    e = launch_gate_up(x, sor, (int)top_k, offsets, (int)slots, (int)E, (int)H, (int)I, w_gate,
                       w_up, dt, h, base + L.experts, stream);
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess)
    e = launch_down(h, offsets, (int)slots, (int)E, (int)H, (int)I, w_down, dt, y,
                    base + L.experts, stream);
  if (e == hipSuccess) e = mark(4);
  if (e == hipSuccess)
    e = launch_combine(y, ros, w, logits_dt, (int)T, (int)top_k, (int)H, dt, out, stream);
  if (e == hipSuccess) e = mark(5);
  return from_hip(e);
}

}  // namespace

extern "C" {

moe_status moe_forward(const void* x, const void* logits, moe_dtype logits_dt, int64_t T,
                       int64_t H, int64_t I, int64_t E, int64_t top_k, int renormalize,
                       const void* w_gate, const void* w_up, const void* w_down, moe_dtype dt,
                       void* out, uint32_t* indices_out, void* weights_out,
                       int32_t* offsets_out, void* ws, size_t ws_bytes,
                       hipEvent_t* stage_events, hipStream_t stream) {
  if (H < 1 || I < 1) return MOE_ERROR_SHAPE;
  const moe_status st = check_route_args(T, E, top_k, logits_dt);
  if (st != MOE_SUCCESS) return st;
  Router r;
  r.renormalize = renormalize ? 1 : 0;
  return forward_impl(x, logits, logits_dt, T, H, I, E, top_k, r, w_gate, w_up, w_down, dt, out,
                      indices_out, weights_out, offsets_out, ws, ws_bytes, stage_events, stream);
}

}  // extern "C"

// ---- moe_forward_noalloc: moe_forward on the library's own scratch array ----
// For callers that cannot allocate. One array per device, shared by every
// call on that device and kept until the process ends; calls that overlap on
// one device race on it. Host code never names the array itself (that name is
// a host-side stand-in): it uses the device address looked up once per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on `dev`, looked up (with `dev` current) the
// first time a call runs there.
moe_status scratch_on_device(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERROR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) {
      (void)hipGetLastError();
      return MOE_ERROR_HIP;
    }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      return MOE_ERROR_HIP;
    }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != dev) (void)hipSetDevice(prev);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_ERROR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_SUCCESS;
}

}  // namespace

extern "C" {

moe_status moe_forward_noalloc(const void* x, const void* logits, moe_dtype logits_dt, int64_t T,
                               int64_t H, int64_t I, int64_t E, int64_t top_k, int renormalize,
                               const void* w_gate, const void* w_up, const void* w_down,
                               moe_dtype dt, void* out, uint32_t* indices_out, void* weights_out,
                               int32_t* offsets_out, hipEvent_t* stage_events,
                               hipStream_t stream) {
  if (H < 1 || I < 1) return MOE_ERROR_SHAPE;
  moe_status st = check_route_args(T, E, top_k, logits_dt);
  if (st != MOE_SUCCESS) return st;
  if (T == 0) return MOE_SUCCESS;
  int dev = 0;
  if ((st = stream_device(stream, &dev)) != MOE_SUCCESS) return st;
  void* ws = nullptr;
  if ((st = scratch_on_device(dev, &ws)) != MOE_SUCCESS) return st;
  Router r;
  r.renormalize = renormalize ? 1 : 0;
  // too large a batch: the scratch is smaller than the workspace it needs (WORKSPACE)
  return forward_impl(x, logits, logits_dt, T, H, I, E, top_k, r, w_gate, w_up, w_down, dt, out,
                      indices_out, weights_out, offsets_out, ws, MOE_NOALLOC_SCRATCH_BYTES,
                      stage_events, stream, nullptr, true);
}

moe_status moe_route_sigmoid_grouped(const void* logits, moe_dtype logits_dt, int64_t T, int64_t E,
                                     const float* bias, int64_t top_k, int64_t groups,
                                     int64_t selected_groups, int group_top_two, int renormalize,
                                     float scale, uint32_t* indices, void* weights,
                                     hipStream_t stream) {
  moe_status st = check_route_args(T, E, top_k, logits_dt);
  if (st != MOE_SUCCESS) return st;
  if ((st = check_grouped_args(E, top_k, groups, selected_groups, group_top_two, scale)) != MOE_SUCCESS)
    return st;
  if (T == 0) return MOE_SUCCESS;
  if (!logits || !indices || !weights) return MOE_ERROR_NULL_POINTER;
  const size_t ls = dtype_size(logits_dt);
  const Span outs[] = {{indices, (size_t)(T * top_k) * 4}, {weights, (size_t)(T * top_k) * ls}};
  const Span ins[] = {{logits, (size_t)(T * E) * ls}, {bias, bias ? (size_t)E * 4 : 0}};
  if (any_overlap(outs, 2, ins, 2)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {logits, indices, weights, bias};
  if ((st = check_device(ptrs, 4, stream)) != MOE_SUCCESS) return st;
  return from_hip(launch_route_grouped(logits, logits_dt, bias, (int)T, (int)E, (int)top_k,
                                       (int)groups, (int)selected_groups, group_top_two ? 1 : 0,
                                       renormalize ? 1 : 0, scale, indices, weights, stream));
}

moe_status moe_forward_sigmoid_grouped(const void* x, const void* logits, moe_dtype logits_dt,
                                       int64_t T, int64_t H, int64_t I, int64_t E,
                                       const float* bias, int64_t top_k, int64_t groups,
                                       int64_t selected_groups, int group_top_two,
                                       int renormalize, float scale, const void* w_gate,
                                       const void* w_up, const void* w_down, moe_dtype dt,
                                       void* out, uint32_t* indices_out, void* weights_out,
                                       int32_t* offsets_out, void* ws, size_t ws_bytes,
                                       hipEvent_t* stage_events, hipStream_t stream) {
  if (H < 1 || I < 1) return MOE_ERROR_SHAPE;
  moe_status st = check_route_args(T, E, top_k, logits_dt);
  if (st != MOE_SUCCESS) return st;
  if ((st = check_grouped_args(E, top_k, groups, selected_groups, group_top_two, scale)) != MOE_SUCCESS)
    return st;
  Router r;
  r.grouped = true;
  r.renormalize = renormalize ? 1 : 0;
  r.bias = bias;
  r.groups = (int)groups;
  r.selected_groups = (int)selected_groups;
  r.group_top_two = group_top_two ? 1 : 0;
  r.scale = scale;
  return forward_impl(x, logits, logits_dt, T, H, I, E, top_k, r, w_gate, w_up, w_down, dt, out,
                      indices_out, weights_out, offsets_out, ws, ws_bytes, stage_events, stream);
}

}  // extern "C"

namespace {

moe_status combine_special_impl(const void* expert_out, const int32_t* row_of_slot,
                                const uint32_t* indices, const void* weights, moe_dtype w_dt,
                                int64_t T, int64_t top_k, int64_t H, moe_dtype dt, int64_t E,
                                int64_t zero_num, int64_t copy_num, int64_t const_num,
                                const void* ori_x, const void* const_alpha1,
                                const void* const_alpha2, const void* const_v,
                                const uint8_t* active, int mask_dims, const void* shared,
                                const void* residual, const float* gamma, float eps, void* out,
                                void* x_out, float* rstd, hipStream_t stream) {
  const bool norm = residual != nullptr || gamma != nullptr || x_out != nullptr || rstd != nullptr;
  if (T < 0 || top_k < 1 || H < 1 || E < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt) || !valid_dt(w_dt)) return MOE_ERROR_DTYPE;
  if (zero_num < 0 || copy_num < 0 || const_num < 0 ||
      E + zero_num + copy_num + const_num > INT32_MAX)
    return MOE_ERROR_ARGUMENT;
  if (mask_dims < 0 || mask_dims > 2 || (mask_dims > 0) != (active != nullptr)) return MOE_ERROR_ARGUMENT;
  if (norm && (!isfinite(eps) || eps <= 0.f)) return MOE_ERROR_ARGUMENT;
  if (T * top_k > INT32_MAX || !row_len_ok(H) || H > kMaxNormH) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!expert_out || !row_of_slot || !indices || !weights || !out) return MOE_ERROR_NULL_POINTER;
  if ((copy_num > 0 || const_num > 0) && !ori_x) return MOE_ERROR_NULL_POINTER;
  if (const_num > 0 && (!const_alpha1 || !const_alpha2 || !const_v)) return MOE_ERROR_NULL_POINTER;
  if (norm && (!residual || !gamma || !x_out || !rstd)) return MOE_ERROR_NULL_POINTER;
  const size_t ds = dtype_size(dt), slots = (size_t)(T * top_k), th = (size_t)T * (size_t)H * ds;
  const size_t nq = (size_t)const_num;
  const Span outs[] = {{out, th}, {x_out, x_out ? th : 0}, {rstd, rstd ? (size_t)T * 4 : 0}};
  const Span ins[] = {{expert_out, slots * (size_t)H * ds}, {row_of_slot, slots * 4},
                      {indices, slots * 4}, {weights, slots * dtype_size(w_dt)},
                      {ori_x, ori_x ? th : 0}, {const_alpha1, const_alpha1 ? nq * ds : 0},
                      {const_alpha2, const_alpha2 ? nq * ds : 0},
                      {const_v, const_v ? nq * (size_t)H * ds : 0},
                      {active, mask_dims == 1 ? (size_t)T : mask_dims == 2 ? slots : 0},
                      {shared, shared ? th : 0}, {residual, residual ? th : 0},
                      {gamma, gamma ? (size_t)H * 4 : 0}};
  if (any_overlap(outs, 3, ins, 12)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {expert_out, row_of_slot, indices, weights, ori_x, const_alpha1, const_alpha2,
                        const_v, active, shared, residual, gamma, out, x_out, rstd};
  moe_status st = check_device(ptrs, 15, stream);
  if (st != MOE_SUCCESS) return st;
  SpecialCombine c;
  c.expert_out = expert_out; c.row_of_slot = row_of_slot; c.indices = indices; c.weights = weights;
  c.w_dt = w_dt; c.dt = dt; c.k = (int)top_k; c.H = (int)H; c.E = (int)E;
  c.n_zero = (int)zero_num; c.n_copy = (int)copy_num; c.n_const = (int)const_num;
  c.ori_x = ori_x; c.alpha1 = const_alpha1; c.alpha2 = const_alpha2; c.const_v = const_v;
  c.active = active; c.mask_dims = mask_dims; c.shared = shared;
  c.residual = norm ? residual : nullptr; c.gamma = gamma; c.eps = eps;
  c.out = out; c.x_out = x_out; c.rstd = rstd;
  return from_hip(launch_combine_special(c, (int)T, stream));
}

}  // namespace

extern "C" {

moe_status moe_combine_special(const void* expert_out, const int32_t* row_of_slot,
                               const uint32_t* indices, const void* weights, moe_dtype w_dt,
                               int64_t T, int64_t top_k, int64_t H, moe_dtype dt, int64_t E,
                               int64_t zero_num, int64_t copy_num, int64_t const_num,
                               const void* ori_x, const void* const_alpha1,
                               const void* const_alpha2, const void* const_v,
                               const uint8_t* active, int mask_dims, const void* shared,
                               void* out, hipStream_t stream) {
  return combine_special_impl(expert_out, row_of_slot, indices, weights, w_dt, T, top_k, H, dt, E,
                              zero_num, copy_num, const_num, ori_x, const_alpha1, const_alpha2,
                              const_v, active, mask_dims, shared, nullptr, nullptr, 0.f, out,
                              nullptr, nullptr, stream);
}

moe_status moe_combine_add_rmsnorm_special(
    const void* expert_out, const int32_t* row_of_slot, const uint32_t* indices,
    const void* weights, moe_dtype w_dt, int64_t T, int64_t top_k, int64_t H, moe_dtype dt,
    int64_t E, int64_t zero_num, int64_t copy_num, int64_t const_num, const void* ori_x,
    const void* const_alpha1, const void* const_alpha2, const void* const_v,
    const uint8_t* active, int mask_dims, const void* shared, const void* residual,
    const float* gamma, float eps, void* y, void* x_out, float* rstd, hipStream_t stream) {
  if (!residual || !gamma || !x_out || !rstd) {
    if (T < 0 || top_k < 1 || H < 1 || E < 1) return MOE_ERROR_SHAPE;
    if (T > 0) return MOE_ERROR_NULL_POINTER;
  }
  return combine_special_impl(expert_out, row_of_slot, indices, weights, w_dt, T, top_k, H, dt, E,
                              zero_num, copy_num, const_num, ori_x, const_alpha1, const_alpha2,
                              const_v, active, mask_dims, shared, residual, gamma, eps, y, x_out,
                              rstd, stream);
}

size_t moe_experts_quant_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I,
                                        moe_dtype dt) {
  if (rows < 0 || E < 1 || H < 1 || I < 1 || !valid_dt(dt)) return 0;
  return align256((size_t)rows * (size_t)I * dtype_size(dt)) + 256;
}

moe_status moe_experts_forward_dispatched_quant(
    const void* x_disp, const int32_t* expert_offsets, int64_t rows, int64_t E, int64_t H, int64_t I,
    const void* w_gate, const void* w_up, const void* w_down, int bits, int64_t groups,
    const void* scale_gate, const void* scale_up, const void* scale_down, const void* offset_gate,
    const void* offset_up, const void* offset_down, moe_dtype dt, void* expert_out, void* ws,
    size_t ws_bytes, hipStream_t stream) {
  if (rows < 0 || E < 1 || H < 1 || I < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt)) return MOE_ERROR_DTYPE;
  moe_status st = check_quant_args(rows, E, H, I, bits, groups, dt);
  if (st != MOE_SUCCESS) return st;
  if (rows == 0) return MOE_SUCCESS;
  if (!x_disp || !expert_offsets || !w_gate || !w_up || !w_down || !expert_out || !scale_gate ||
      !scale_up || !scale_down)
    return MOE_ERROR_NULL_POINTER;
  const size_t need = moe_experts_quant_workspace_size(rows, E, H, I, dt);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < need) return MOE_ERROR_WORKSPACE;
  const size_t ds = dtype_size(dt), qb = quant_bytes(E, I, H, bits);
  const size_t sb = (size_t)E * (size_t)groups * ds;
  const Span outs[] = {{expert_out, (size_t)rows * (size_t)H * ds}, {ws, need}};
  const Span ins[] = {{x_disp, (size_t)rows * (size_t)H * ds}, {expert_offsets, (size_t)(E + 1) * 4},
                      {w_gate, qb}, {w_up, qb}, {w_down, qb},
                      {scale_gate, sb * (size_t)I}, {scale_up, sb * (size_t)I}, {scale_down, sb * (size_t)H},
                      {offset_gate, offset_gate ? sb * (size_t)I : 0}, {offset_up, offset_up ? sb * (size_t)I : 0},
                      {offset_down, offset_down ? sb * (size_t)H : 0}};
  if (any_overlap(outs, 2, ins, 11)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {x_disp, expert_offsets, w_gate, w_up, w_down, scale_gate, scale_up,
                        scale_down, offset_gate, offset_up, offset_down, expert_out, ws};
  if ((st = check_device(ptrs, 13, stream)) != MOE_SUCCESS) return st;
  QuantExperts q = {};
  q.x = x_disp; q.row_map = nullptr; q.map_div = 1; q.offsets = expert_offsets;
  q.rows = (int)rows; q.E = (int)E; q.H = (int)H; q.I = (int)I; q.dt = dt;
  q.bits = bits; q.groups = (int)groups;
  q.w_gate = w_gate; q.w_up = w_up; q.w_down = w_down;
  q.s_gate = scale_gate; q.s_up = scale_up; q.s_down = scale_down;
  q.o_gate = offset_gate; q.o_up = offset_up; q.o_down = offset_down;
  q.h = ws; q.expert_out = expert_out;
  return from_hip(launch_experts_quant(q, stream));
}

moe_status moe_forward_quant(const void* x, const void* logits, moe_dtype logits_dt, int64_t T,
                             int64_t H, int64_t I, int64_t E, int64_t top_k, int renormalize,
                             const void* w_gate, const void* w_up, const void* w_down, int bits,
                             int64_t groups, const void* scale_gate, const void* scale_up,
                             const void* scale_down, const void* offset_gate,
                             const void* offset_up, const void* offset_down, moe_dtype dt,
                             void* out, uint32_t* indices_out, void* weights_out,
                             int32_t* offsets_out, void* ws, size_t ws_bytes,
                             hipEvent_t* stage_events, hipStream_t stream) {
  if (H < 1 || I < 1) return MOE_ERROR_SHAPE;
  moe_status st = check_route_args(T, E, top_k, logits_dt);
  if (st != MOE_SUCCESS) return st;
  if (!valid_dt(dt)) return MOE_ERROR_DTYPE;
  if ((st = check_quant_args(T * top_k, E, H, I, bits, groups, dt)) != MOE_SUCCESS) return st;
  if (T > 0 && (!scale_gate || !scale_up || !scale_down)) return MOE_ERROR_NULL_POINTER;
  const size_t ds = dtype_size(dt), sb = (size_t)E * (size_t)groups * ds;
  const Span scales[] = {{scale_gate, sb * (size_t)I}, {scale_up, sb * (size_t)I},
                         {scale_down, sb * (size_t)H}, {offset_gate, offset_gate ? sb * (size_t)I : 0},
                         {offset_up, offset_up ? sb * (size_t)I : 0},
                         {offset_down, offset_down ? sb * (size_t)H : 0}};
  const Span outs[] = {{out, (size_t)T * (size_t)H * ds}, {ws, ws_bytes}};
  if (any_overlap(outs, 2, scales, 6)) return MOE_ERROR_ARGUMENT;
  const void* sptrs[] = {scale_gate, scale_up, scale_down, offset_gate, offset_up, offset_down};
  if (T > 0 && (st = check_device(sptrs, 6, stream)) != MOE_SUCCESS) return st;
  Router r;
  r.renormalize = renormalize ? 1 : 0;
  QuantWeights qw;
  qw.bits = bits; qw.groups = groups;
  qw.s_gate = scale_gate; qw.s_up = scale_up; qw.s_down = scale_down;
  qw.o_gate = offset_gate; qw.o_up = offset_up; qw.o_down = offset_down;
  return forward_impl(x, logits, logits_dt, T, H, I, E, top_k, r, w_gate, w_up, w_down, dt, out,
                      indices_out, weights_out, offsets_out, ws, ws_bytes, stage_events, stream, &qw);
}

// ---- first-order training (ruDNN user guide, "12. MoE first-order training") ----

static size_t index_size(int idx_dt) { return idx_dt == MOE_IDX_I64 ? 8 : 4; }

static moe_status router_grad_impl(const void* logits, moe_dtype logits_dt, const void* indices,
                                   moe_index_dtype idx_dt, const float* grad_weights, int64_t T,
                                   int64_t E, int64_t top_k, moe_scoring scoring, int normalize,
                                   float scale, float* weights, void* grad_logits,
                                   hipStream_t stream) {
  if (T < 0 || E < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(logits_dt)) return MOE_ERROR_DTYPE;
  if (idx_dt != MOE_IDX_U32 && idx_dt != MOE_IDX_I32 && idx_dt != MOE_IDX_I64) return MOE_ERROR_DTYPE;
  if (top_k < 1 || top_k > E || top_k > 64) return MOE_ERROR_ARGUMENT;
  if (scoring != MOE_SCORE_SOFTMAX && scoring != MOE_SCORE_SIGMOID) return MOE_ERROR_ARGUMENT;
  if (!(scale > 0.0f) || !std::isfinite(scale)) return MOE_ERROR_ARGUMENT;
  if (E > kMaxE || T * top_k > INT32_MAX) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  const bool bwd = grad_logits != nullptr;
  if (!logits || !indices || (bwd ? !grad_weights : !weights)) return MOE_ERROR_NULL_POINTER;
  const size_t slots = (size_t)(T * top_k);
  const Span ins[] = {{logits, (size_t)T * (size_t)E * dtype_size(logits_dt)},
                      {indices, slots * index_size(idx_dt)}, {grad_weights, bwd ? slots * 4 : 0}};
  const Span outs[] = {bwd ? Span{grad_logits, (size_t)T * (size_t)E * dtype_size(logits_dt)}
                           : Span{weights, slots * 4}};
  if (any_overlap(outs, 1, ins, 3)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {logits, indices, bwd ? (const void*)grad_weights : nullptr,
                        bwd ? grad_logits : (void*)weights};
  moe_status st = check_device(ptrs, 4, stream);
  if (st != MOE_SUCCESS) return st;
  RouterGrad r = {};
  r.logits = logits; r.logits_dt = logits_dt; r.indices = indices; r.idx_dt = idx_dt;
  r.T = (int)T; r.E = (int)E; r.k = (int)top_k; r.scoring = scoring; r.normalize = normalize ? 1 : 0;
  r.scale = scale; r.weights = weights; r.grad_weights = bwd ? grad_weights : nullptr;
  r.grad_logits = grad_logits;
  return from_hip(launch_router_grad(r, stream));
}

moe_status moe_router_weights(const void* logits, moe_dtype logits_dt, const void* indices,
                              moe_index_dtype idx_dt, int64_t T, int64_t E, int64_t top_k,
                              moe_scoring scoring, int normalize, float scale, float* weights,
                              hipStream_t stream) {
  if (T > 0 && !weights) return MOE_ERROR_NULL_POINTER;
  return router_grad_impl(logits, logits_dt, indices, idx_dt, nullptr, T, E, top_k, scoring,
                          normalize, scale, weights, nullptr, stream);
}

moe_status moe_router_backward(const void* logits, moe_dtype logits_dt, const void* indices,
                               moe_index_dtype idx_dt, const float* grad_weights, int64_t T,
                               int64_t E, int64_t top_k, moe_scoring scoring, int normalize,
                               float scale, void* grad_logits, hipStream_t stream) {
  if (T > 0 && !grad_logits) return MOE_ERROR_NULL_POINTER;
  return router_grad_impl(logits, logits_dt, indices, idx_dt, grad_weights, T, E, top_k, scoring,
                          normalize, scale, nullptr, grad_logits, stream);
}

moe_status moe_combine_backward(const void* expert_out, const int32_t* row_of_slot,
                                const void* weights, moe_dtype w_dt, const void* grad_out,
                                int64_t T, int64_t top_k, int64_t H, int64_t rows, moe_dtype dt,
                                void* dexpert, float* dweights, hipStream_t stream) {
  if (T < 0 || top_k < 1 || H < 1 || rows < 0 || rows > T * top_k) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt) || !valid_dt(w_dt)) return MOE_ERROR_DTYPE;
  if (T * top_k > INT32_MAX || !row_len_ok(H)) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!expert_out || !row_of_slot || !weights || !grad_out || !dexpert || !dweights)
    return MOE_ERROR_NULL_POINTER;
  const size_t ds = dtype_size(dt), slots = (size_t)(T * top_k);
  const Span outs[] = {{dexpert, (size_t)rows * (size_t)H * ds}, {dweights, slots * 4}};
  const Span ins[] = {{expert_out, (size_t)rows * (size_t)H * ds}, {row_of_slot, slots * 4},
                      {weights, slots * dtype_size(w_dt)}, {grad_out, (size_t)T * (size_t)H * ds}};
  if (any_overlap(outs, 2, ins, 4)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {expert_out, row_of_slot, weights, grad_out, dexpert, dweights};
  moe_status st = check_device(ptrs, 6, stream);
  if (st != MOE_SUCCESS) return st;
  return from_hip(launch_combine_backward(expert_out, row_of_slot, weights, w_dt, grad_out, (int)T,
                                          (int)top_k, (int)H, dt, dexpert, dweights, stream));
}

moe_status moe_dispatch_backward(const void* dinput, const int32_t* row_of_slot, int64_t T,
                                 int64_t top_k, int64_t H, int64_t rows, moe_dtype dt, void* dx,
                                 hipStream_t stream) {
  if (T < 0 || top_k < 1 || H < 1 || rows < 0 || rows > T * top_k) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt)) return MOE_ERROR_DTYPE;
  if (T * top_k > INT32_MAX || !row_len_ok(H)) return MOE_ERROR_UNSUPPORTED;
  if (T == 0) return MOE_SUCCESS;
  if (!dinput || !row_of_slot || !dx) return MOE_ERROR_NULL_POINTER;
  const size_t ds = dtype_size(dt), slots = (size_t)(T * top_k);
  const Span outs[] = {{dx, (size_t)T * (size_t)H * ds}};
  const Span ins[] = {{dinput, (size_t)rows * (size_t)H * ds}, {row_of_slot, slots * 4}};
  if (any_overlap(outs, 1, ins, 2)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {dinput, row_of_slot, dx};
  moe_status st = check_device(ptrs, 3, stream);
  if (st != MOE_SUCCESS) return st;
  return from_hip(launch_dispatch_backward(dinput, row_of_slot, (int)T, (int)top_k, (int)H, dt, dx,
                                           stream));
}

static moe_status check_train_args(int64_t rows, int64_t E, int64_t H, int64_t I, moe_dtype dt) {
  if (rows < 0 || E < 1 || H < 1 || I < 1) return MOE_ERROR_SHAPE;
  if (!valid_dt(dt)) return MOE_ERROR_DTYPE;
  if (dt == MOE_F32) return MOE_ERROR_UNSUPPORTED;  // the matrix-core path is bf16 / f16
  if (E > kMaxE || rows > INT32_MAX || !row_len_ok(H) || !row_len_ok(I)) return MOE_ERROR_UNSUPPORTED;
  if ((int64_t)E * I * H > INT64_MAX / 8 || 2 * I > INT32_MAX) return MOE_ERROR_UNSUPPORTED;
  // the training forward runs the inference gate/up and down GEMMs
  if (!gemm_bytes_ok(rows, rows, H, I, dt)) return MOE_ERROR_UNSUPPORTED;
  // the training GEMM keeps a lane's offset inside a 256-row tile in 32 bits
  // (leading dimensions up to 2^22 elements) and numbers its tiles in int
  if (H > (1 << 22) || 2 * I > (1 << 22)) return MOE_ERROR_UNSUPPORTED;
  const int64_t n_tiles = (std::max<int64_t>(H, 2 * I) + 255) / 256;
  if (((rows + 255) / 256 + E) * n_tiles > INT32_MAX || E * n_tiles * n_tiles > INT32_MAX)
    return MOE_ERROR_UNSUPPORTED;
  return MOE_SUCCESS;
}

size_t moe_experts_training_cache_size(int64_t rows, int64_t I, moe_dtype dt) {
  if (rows < 0 || I < 1 || !valid_dt(dt)) return 0;
  return (size_t)rows * (size_t)I * 3 * dtype_size(dt);
}

size_t moe_experts_forward_training_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I,
                                                   moe_dtype dt) {
  if (check_train_args(rows, E, H, I, dt) != MOE_SUCCESS) return 0;
  return train_prefix_bytes(E) + align256(gemm_scratch_bytes(rows, E, H, I, dt));
}

size_t moe_experts_backward_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I,
                                           moe_dtype dt) {
  if (check_train_args(rows, E, H, I, dt) != MOE_SUCCESS) return 0;
  return train_prefix_bytes(E) + align256((size_t)rows * (size_t)I * 2 * dtype_size(dt));
}

moe_status moe_experts_forward_training(const void* x_disp, const int32_t* expert_offsets,
                                        int64_t rows, int64_t E, int64_t H, int64_t I,
                                        const void* w_gate, const void* w_up, const void* w_down,
                                        moe_dtype dt, void* expert_out, void* cache, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_train_args(rows, E, H, I, dt);
  if (st != MOE_SUCCESS) return st;
  if (rows == 0) return MOE_SUCCESS;
  if (!x_disp || !expert_offsets || !w_gate || !w_up || !w_down || !expert_out || !cache)
    return MOE_ERROR_NULL_POINTER;
  const size_t need = moe_experts_forward_training_workspace_size(rows, E, H, I, dt);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < need) return MOE_ERROR_WORKSPACE;
  const size_t ds = dtype_size(dt), wbytes = (size_t)E * (size_t)I * (size_t)H * ds;
  const Span outs[] = {{expert_out, (size_t)rows * (size_t)H * ds},
                       {cache, moe_experts_training_cache_size(rows, I, dt)}, {ws, need}};
  const Span ins[] = {{x_disp, (size_t)rows * (size_t)H * ds}, {expert_offsets, (size_t)(E + 1) * 4},
                      {w_gate, wbytes}, {w_up, wbytes}, {w_down, wbytes}};
  if (any_overlap(outs, 3, ins, 5)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {x_disp, expert_offsets, w_gate, w_up, w_down, expert_out, cache, ws};
  if ((st = check_device(ptrs, 8, stream)) != MOE_SUCCESS) return st;
  TrainExperts q = {};
  q.x = x_disp; q.offsets = expert_offsets; q.rows = (int)rows; q.E = (int)E; q.H = (int)H;
  q.I = (int)I; q.dt = dt; q.w_gate = w_gate; q.w_up = w_up; q.w_down = w_down;
  q.cache = cache; q.y = expert_out; q.ws = ws;
  return from_hip(launch_experts_forward_training(q, stream));
}

moe_status moe_experts_backward(const void* x_disp, const int32_t* expert_offsets, int64_t rows,
                                int64_t E, int64_t H, int64_t I, const void* w_gate,
                                const void* w_up, const void* w_down, moe_dtype dt,
                                const void* cache, const void* dexpert, void* dinput,
                                float* dgate, float* dup, float* ddown, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  moe_status st = check_train_args(rows, E, H, I, dt);
  if (st != MOE_SUCCESS) return st;
  if (!expert_offsets || !w_gate || !w_up || !w_down || !dgate || !dup || !ddown)
    return MOE_ERROR_NULL_POINTER;
  if (rows > 0 && (!x_disp || !cache || !dexpert || !dinput)) return MOE_ERROR_NULL_POINTER;
  const size_t need = moe_experts_backward_workspace_size(rows, E, H, I, dt);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < need) return MOE_ERROR_WORKSPACE;
  const size_t ds = dtype_size(dt), wbytes = (size_t)E * (size_t)I * (size_t)H * ds;
  const size_t gbytes = (size_t)E * (size_t)I * (size_t)H * 4, rh = (size_t)rows * (size_t)H * ds;
  const Span outs[] = {{dinput, rh}, {dgate, gbytes}, {dup, gbytes}, {ddown, gbytes}, {ws, need}};
  const Span ins[] = {{x_disp, rh}, {expert_offsets, (size_t)(E + 1) * 4}, {w_gate, wbytes},
                      {w_up, wbytes}, {w_down, wbytes},
                      {cache, moe_experts_training_cache_size(rows, I, dt)}, {dexpert, rh}};
  if (any_overlap(outs, 5, ins, 7)) return MOE_ERROR_ARGUMENT;
  const void* ptrs[] = {x_disp, expert_offsets, w_gate, w_up, w_down, cache, dexpert, dinput,
                        dgate, dup, ddown, ws};
  if ((st = check_device(ptrs, 12, stream)) != MOE_SUCCESS) return st;
  TrainExperts q = {};
  q.x = x_disp; q.offsets = expert_offsets; q.rows = (int)rows; q.E = (int)E; q.H = (int)H;
  q.I = (int)I; q.dt = dt; q.w_gate = w_gate; q.w_up = w_up; q.w_down = w_down;
  q.cache = const_cast<void*>(cache); q.dy = dexpert; q.dx = dinput;
  q.d_gate = dgate; q.d_up = dup; q.d_down = ddown; q.ws = ws;
  return from_hip(launch_experts_backward(q, stream));
}

}  // extern "C"
