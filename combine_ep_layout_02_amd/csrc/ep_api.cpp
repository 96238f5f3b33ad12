// C ABI of the gfx950 MoE dispatch / combine library (declared in
// include/ep.h): host-side argument checks, sizing, and kernel launches.
// Every check runs before anything is enqueued.
#include "ep.h"

#include <hip/hip_runtime.h>

#include "ep_internal.hpp"

#define EP_EXPORT extern "C" __attribute__((visibility("default")))

static_assert(ep::kMaxTopk == EP_MAX_TOPK, "device top-k limit must match the ABI's");

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxRows = (int64_t)1 << 31;  // slots and pair ids are int32
constexpr int kMaxHidden = 1 << 24;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

ep_status_t check_shape(const ep_shape_t* s) {
  if (!s) return EP_ERR_INVALID_ARG;
  if (s->num_tokens < 0 || s->hidden <= 0 || s->num_topk <= 0 || s->num_experts <= 0 || s->num_ranks <= 0)
    return EP_ERR_INVALID_ARG;
  if (s->num_experts % s->num_ranks != 0 || s->num_topk > s->num_experts) return EP_ERR_INVALID_ARG;
  if (s->expert_alignment < 1 || s->capacity < 0) return EP_ERR_INVALID_ARG;
  if (s->expert_alignment > 1 && s->capacity > 0) return EP_ERR_INVALID_ARG;
  if (s->num_cus < 0) return EP_ERR_INVALID_ARG;
  if (s->num_cus > EP_MAX_NUM_CUS) return EP_ERR_UNSUPPORTED;
  if (s->num_experts > EP_MAX_EXPERTS || s->num_topk > EP_MAX_TOPK) return EP_ERR_UNSUPPORTED;
  if (s->hidden % 8 != 0 || s->hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
  const int64_t T = s->num_tokens, k = s->num_topk, E = s->num_experts;
  if (T * k >= kMaxRows) return EP_ERR_UNSUPPORTED;
  // work items (token, 512-column chunk) are counted in int32 on the device
  if (T * ((s->hidden + 511) / 512) >= kMaxRows) return EP_ERR_UNSUPPORTED;
  const int64_t rows = s->capacity > 0 ? E * s->capacity : T * k + E * (s->expert_alignment - 1);
  if (rows >= kMaxRows) return EP_ERR_UNSUPPORTED;
  return EP_OK;
}

int64_t recv_rows_of(const ep_shape_t* s) {
  const int64_t T = s->num_tokens, k = s->num_topk, E = s->num_experts;
  return s->capacity > 0 ? E * s->capacity : T * k + E * (s->expert_alignment - 1);
}

ep_status_t hip_status(hipError_t err) {
  if (err == hipSuccess) return EP_OK;
  g_last_hip_error = (int)err;
  return EP_ERR_HIP;
}

}  // namespace

EP_EXPORT int ep_abi_version(void) { return EP_ABI_VERSION; }

EP_EXPORT int ep_last_hip_error(void) { return g_last_hip_error; }

EP_EXPORT const char* ep_status_string(ep_status_t status) {
  switch (status) {
    case EP_OK: return "EP_OK";
    case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG: null pointer or inconsistent shape";
    case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED: shape outside the supported limits";
    case EP_ERR_MISALIGNED: return "EP_ERR_MISALIGNED: a row pointer is not 16-byte aligned";
    case EP_ERR_WORKSPACE: return "EP_ERR_WORKSPACE: layout workspace missing or too small";
    case EP_ERR_HIP: return "EP_ERR_HIP: a HIP launch failed (see ep_last_hip_error)";
  }
  return "unknown ep_status_t";
}

EP_EXPORT ep_status_t ep_recv_rows(const ep_shape_t* shape, int64_t* rows) {
  const ep_status_t st = check_shape(shape);
  if (st != EP_OK) return st;
  if (!rows) return EP_ERR_INVALID_ARG;
  *rows = recv_rows_of(shape);
  return EP_OK;
}

EP_EXPORT ep_status_t ep_layout_workspace_bytes(const ep_shape_t* shape, size_t* bytes) {
  const ep_status_t st = check_shape(shape);
  if (st != EP_OK) return st;
  if (!bytes) return EP_ERR_INVALID_ARG;
  *bytes = ep::plan_layout(shape->num_tokens, shape->num_topk, shape->num_experts, shape->num_ranks).ws_bytes;
  return EP_OK;
}

namespace {

// Checks of ep_layout's arguments (shape already checked) and its parameters.
ep_status_t layout_args(const ep_shape_t* shape, const int32_t* topk_idx, int32_t* expert_count,
                        int32_t* expert_offset, int32_t* rank_count, int32_t* rank_offset, int32_t* slot,
                        int32_t* src_pair, int32_t* diag, void* workspace, size_t workspace_bytes,
                        ep::LayoutPlan& pl, ep::LayoutParams& p) {
  const int T = shape->num_tokens;
  if (!expert_count || !expert_offset || !rank_count || !rank_offset) return EP_ERR_INVALID_ARG;
  if (T > 0 && (!topk_idx || !slot)) return EP_ERR_INVALID_ARG;
  const int32_t* ptrs[] = {topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot, src_pair, diag};
  for (const int32_t* q : ptrs)
    if (!aligned(q, 4)) return EP_ERR_MISALIGNED;
  pl = ep::plan_layout(T, shape->num_topk, shape->num_experts, shape->num_ranks);
  if (!workspace || workspace_bytes < pl.ws_bytes) return EP_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return EP_ERR_MISALIGNED;

  p = ep::LayoutParams{};
  char* ws = static_cast<char*>(workspace);
  p.idx = topk_idx;
  p.expert_count = expert_count;
  p.expert_offset = expert_offset;
  p.rank_count = rank_count;
  p.rank_offset = rank_offset;
  p.slot = slot;
  p.src_pair = src_pair;
  p.diag = diag;
  p.ws_tile = reinterpret_cast<int32_t*>(ws + pl.ws_tile_off);
  p.ws_rank = reinterpret_cast<int32_t*>(ws + pl.ws_rank_off);
  p.ws_bad = reinterpret_cast<int32_t*>(ws + pl.ws_bad_off);
  p.T = T;
  p.k = shape->num_topk;
  p.E = shape->num_experts;
  p.R = shape->num_ranks;
  p.A = shape->expert_alignment;
  p.C = shape->capacity;
  p.rows = recv_rows_of(shape);
  return EP_OK;
}

// Checks of ep_dispatch's arguments (shape already checked) and its parameters.
ep_status_t dispatch_args(const ep_shape_t* shape, const void* x, const int32_t* slot, ep_dtype_t recv_dtype,
                          void* recv_x, void* recv_scale, ep::RowParams& p) {
  const bool mx = recv_dtype == EP_MXFP8_E4M3 || recv_dtype == EP_MXFP4_E2M1;
  if (recv_dtype != EP_BF16 && recv_dtype != EP_FP8_E4M3 && !mx) return EP_ERR_INVALID_ARG;
  if (recv_dtype == EP_FP8_E4M3 && shape->hidden % 128 != 0) return EP_ERR_UNSUPPORTED;
  if (mx && shape->hidden % 32 != 0) return EP_ERR_UNSUPPORTED;
  const int T = shape->num_tokens;
  p = ep::RowParams{};
  if (T == 0) return EP_OK;
  if (!x || !slot || !recv_x) return EP_ERR_INVALID_ARG;
  if (recv_dtype != EP_BF16 && !recv_scale) return EP_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(slot, 4) || !aligned(recv_scale, 4))
    return EP_ERR_MISALIGNED;
  p.src = x;
  p.slot = slot;
  p.dst = recv_x;
  p.recv_scale = recv_scale;
  p.T = T;
  p.H = shape->hidden;
  p.k = shape->num_topk;
  p.rows = recv_rows_of(shape);
  p.num_cus = shape->num_cus;
  return EP_OK;
}

hipError_t launch_dispatch(const ep::RowParams& p, ep_dtype_t recv_dtype, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  switch (recv_dtype) {
    case EP_BF16: return ep::launch_dispatch_bf16(p, stream);
    case EP_FP8_E4M3: return ep::launch_dispatch_fp8(p, stream);
    case EP_MXFP8_E4M3: return ep::launch_dispatch_mx(p, 8, stream);
    default: return ep::launch_dispatch_mx(p, 4, stream);
  }
}

}  // namespace

EP_EXPORT ep_status_t ep_layout(const ep_shape_t* shape, const int32_t* topk_idx, int32_t* expert_count,
                                int32_t* expert_offset, int32_t* rank_count, int32_t* rank_offset, int32_t* slot,
                                int32_t* src_pair, int32_t* diag, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  const ep_status_t st = check_shape(shape);
  if (st != EP_OK) return st;
  ep::LayoutPlan pl;
  ep::LayoutParams p;
  const ep_status_t st2 = layout_args(shape, topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot,
                                      src_pair, diag, workspace, workspace_bytes, pl, p);
  if (st2 != EP_OK) return st2;
  return hip_status(ep::launch_layout(pl, p, stream));
}

EP_EXPORT ep_status_t ep_dispatch(const ep_shape_t* shape, const void* x, const int32_t* slot,
                                  ep_dtype_t recv_dtype, void* recv_x, void* recv_scale, hipStream_t stream) {
  const ep_status_t st = check_shape(shape);
  if (st != EP_OK) return st;
  ep::RowParams p;
  const ep_status_t st2 = dispatch_args(shape, x, slot, recv_dtype, recv_x, recv_scale, p);
  if (st2 != EP_OK) return st2;
  return hip_status(launch_dispatch(p, recv_dtype, stream));
}

EP_EXPORT ep_status_t ep_layout_dispatch(const ep_shape_t* shape, const int32_t* topk_idx, int32_t* expert_count,
                                         int32_t* expert_offset, int32_t* rank_count, int32_t* rank_offset,
                                         int32_t* slot, int32_t* src_pair, int32_t* diag, void* workspace,
                                         size_t workspace_bytes, const void* x, ep_dtype_t recv_dtype, void* recv_x,
                                         void* recv_scale, hipStream_t stream) {
  const ep_status_t st = check_shape(shape);
  if (st != EP_OK) return st;
  ep::LayoutPlan pl;
  ep::LayoutParams lp;
  ep_status_t st2 = layout_args(shape, topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot,
                                src_pair, diag, workspace, workspace_bytes, pl, lp);
  if (st2 != EP_OK) return st2;
  ep::RowParams rp;
  st2 = dispatch_args(shape, x, slot, recv_dtype, recv_x, recv_scale, rp);
  if (st2 != EP_OK) return st2;
  if (shape->num_tokens > 0 && shape->num_cus == 0 && (recv_dtype == EP_BF16 || recv_dtype == EP_FP8_E4M3) &&
      ep::layout_dispatch_fusable(pl, lp))
    return hip_status(ep::launch_layout_dispatch(pl, lp, rp, recv_dtype == EP_FP8_E4M3, stream));
  const hipError_t err = ep::launch_layout(pl, lp, stream);
  if (err != hipSuccess) return hip_status(err);
  return hip_status(launch_dispatch(rp, recv_dtype, stream));
}

EP_EXPORT ep_status_t ep_dispatch_prequantized(const ep_shape_t* shape, const void* x_q, const float* x_scale,
                                               const int32_t* slot, void* recv_x, float* recv_scale,
                                               hipStream_t stream) {
  const ep_status_t st = check_shape(shape);
  if (st != EP_OK) return st;
  if (shape->hidden % 128 != 0) return EP_ERR_UNSUPPORTED;
  const int T = shape->num_tokens;
  if (T == 0) return EP_OK;
  if (!x_q || !x_scale || !slot || !recv_x || !recv_scale) return EP_ERR_INVALID_ARG;
  if (!aligned(x_q, 16) || !aligned(recv_x, 16) || !aligned(x_scale, 4) || !aligned(slot, 4) ||
      !aligned(recv_scale, 4))
    return EP_ERR_MISALIGNED;
  ep::RowParams p{};
  p.src = x_q;
  p.src_scale = x_scale;
  p.slot = slot;
  p.dst = recv_x;
  p.recv_scale = recv_scale;
  p.T = T;
  p.H = shape->hidden;
  p.k = shape->num_topk;
  p.rows = recv_rows_of(shape);
  p.num_cus = shape->num_cus;
  return hip_status(ep::launch_dispatch_prequantized(p, stream));
}

EP_EXPORT ep_status_t ep_combine(const ep_shape_t* shape, const void* y, const int32_t* slot,
                                 const float* topk_weights, void* out, hipStream_t stream) {
  const ep_status_t st = check_shape(shape);
  if (st != EP_OK) return st;
  const int T = shape->num_tokens;
  if (T == 0) return EP_OK;
  if (!y || !slot || !topk_weights || !out) return EP_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(slot, 4) || !aligned(topk_weights, 4))
    return EP_ERR_MISALIGNED;
  ep::RowParams p{};
  p.src = y;
  p.slot = slot;
  p.weights = topk_weights;
  p.dst = out;
  p.T = T;
  p.H = shape->hidden;
  p.k = shape->num_topk;
  p.rows = recv_rows_of(shape);
  p.num_cus = shape->num_cus;
  return hip_status(ep::launch_combine(p, stream));
}

EP_EXPORT ep_status_t ep_dispatch_backward(const ep_shape_t* shape, const void* grad_recv_x, const int32_t* slot,
                                           void* grad_x, hipStream_t stream) {
  const ep_status_t st = check_shape(shape);
  if (st != EP_OK) return st;
  const int T = shape->num_tokens;
  if (T == 0) return EP_OK;
  if (!grad_recv_x || !slot || !grad_x) return EP_ERR_INVALID_ARG;
  if (!aligned(grad_recv_x, 16) || !aligned(grad_x, 16) || !aligned(slot, 4)) return EP_ERR_MISALIGNED;
  ep::RowParams p{};
  p.src = grad_recv_x;
  p.slot = slot;
  p.weights = nullptr;  // unit weights
  p.dst = grad_x;
  p.T = T;
  p.H = shape->hidden;
  p.k = shape->num_topk;
  p.rows = recv_rows_of(shape);
  p.num_cus = shape->num_cus;
  return hip_status(ep::launch_combine(p, stream));
}

EP_EXPORT ep_status_t ep_combine_backward(const ep_shape_t* shape, const void* grad_out, const void* y,
                                          const int32_t* slot, const float* topk_weights, void* grad_y,
                                          float* grad_weights, hipStream_t stream) {
  const ep_status_t st = check_shape(shape);
  if (st != EP_OK) return st;
  const int T = shape->num_tokens;
  if (T == 0) return EP_OK;
  if (!grad_out || !slot || !topk_weights || !grad_y) return EP_ERR_INVALID_ARG;
  if (grad_weights && !y) return EP_ERR_INVALID_ARG;
  if (!aligned(grad_out, 16) || !aligned(y, 16) || !aligned(grad_y, 16) || !aligned(slot, 4) ||
      !aligned(topk_weights, 4) || !aligned(grad_weights, 4))
    return EP_ERR_MISALIGNED;
  ep::BackParams p{};
  p.g = grad_out;
  p.y = y;
  p.slot = slot;
  p.weights = topk_weights;
  p.grad_y = grad_y;
  p.grad_w = grad_weights;
  p.T = T;
  p.H = shape->hidden;
  p.k = shape->num_topk;
  p.rows = recv_rows_of(shape);
  p.num_cus = shape->num_cus;
  return hip_status(ep::launch_combine_backward(p, stream));
}

EP_EXPORT ep_status_t ep_check_cvt_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n < 0) return EP_ERR_INVALID_ARG;
  if (n > 0 && (!in || !out)) return EP_ERR_INVALID_ARG;
  if (!aligned(in, 4)) return EP_ERR_MISALIGNED;
  return hip_status(ep::launch_check_cvt_e4m3(in, out, n, stream));
}

EP_EXPORT ep_status_t ep_check_cvt_e2m1(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n < 0) return EP_ERR_INVALID_ARG;
  if (n > 0 && (!in || !out)) return EP_ERR_INVALID_ARG;
  if (!aligned(in, 4)) return EP_ERR_MISALIGNED;
  return hip_status(ep::launch_check_cvt_e2m1(in, out, n, stream));
}

EP_EXPORT ep_status_t ep_check_quant_e4m3(const uint16_t* x, const float* s, uint8_t* out, int64_t n,
                                          hipStream_t stream) {
  if (n < 0) return EP_ERR_INVALID_ARG;
  if (n > 0 && (!x || !s || !out)) return EP_ERR_INVALID_ARG;
  if (!aligned(x, 2) || !aligned(s, 4)) return EP_ERR_MISALIGNED;
  return hip_status(ep::launch_check_quant_e4m3(x, s, out, n, stream));
}

EP_EXPORT ep_status_t ep_probe_stream(const void* src, void* dst, int64_t units, int read_chunks, int write_chunks,
                                      int policy, hipStream_t stream) {
  if (units < 0 || write_chunks < 1 || write_chunks > 64 || policy < 0 || policy > 7) return EP_ERR_INVALID_ARG;
  if (read_chunks != 1 && read_chunks != 2 && read_chunks != 4 && read_chunks != 8 && read_chunks != 16)
    return EP_ERR_INVALID_ARG;
  if (units > 0 && (!src || !dst)) return EP_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return EP_ERR_MISALIGNED;
  return hip_status(ep::launch_probe_stream(src, dst, units, read_chunks, write_chunks, policy, stream));
}

EP_EXPORT ep_status_t ep_check_cvt_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream) {
  if (n < 0) return EP_ERR_INVALID_ARG;
  if (n > 0 && (!in || !out)) return EP_ERR_INVALID_ARG;
  if (!aligned(in, 4) || !aligned(out, 2)) return EP_ERR_MISALIGNED;
  return hip_status(ep::launch_check_cvt_bf16(in, out, n, stream));
}
