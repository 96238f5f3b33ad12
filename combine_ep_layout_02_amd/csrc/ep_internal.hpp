// Internal interfaces between the C ABI (ep_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

struct LayoutParams {
  const int32_t* idx;
  int32_t* expert_count;
  int32_t* expert_offset;
  int32_t* rank_count;
  int32_t* rank_offset;
  int32_t* slot;
  int32_t* src_pair;  // may be null
  int32_t* diag;      // may be null
  int32_t* ws_tile;   // [ntiles][E] pairs per (tile, expert)
  int32_t* ws_rank;   // [ntiles][R] distinct tokens per (tile, rank)
  int32_t* ws_bad;    // [ntiles] invalid ids per tile
  int T, k, E, R, A, C;
  int W;       // 64-pair windows (wavefronts) per tile
  int TT;      // tokens per tile
  int ntiles;
  int G;       // tile groups per expert in the finalize kernel
  // n / d == __umulhi(n, magic_d) for the n that occur (n * d < 2^32):
  uint32_t magic_k;    // d = k
  uint32_t magic_per;  // d = E / R
  uint32_t magic_E;    // d = E
  uint32_t magic_R;    // d = R
  int64_t rows;  // worst-case receive rows (length of src_pair)
};

struct LayoutPlan {
  int W, TT, ntiles, threads, G, fin_threads;
  size_t lds_bytes, fin_lds_bytes;
  size_t ws_tile_off, ws_rank_off, ws_bad_off, ws_bytes;
};

LayoutPlan plan_layout(int T, int k, int E, int R);
void prepare_layout_params(const LayoutPlan& plan, LayoutParams& p);  // tile shape and division constants
hipError_t launch_layout(const LayoutPlan& plan, LayoutParams p, hipStream_t stream);

struct RowParams {
  const void* src;          // x (dispatch) or y (combine)
  const int32_t* slot;
  const float* weights;     // combine: null = every weight 1 (dispatch backward);
                            // BF16 dispatch: non-null = copy j scaled by w[t,j] (combine backward)
  void* dst;                // recv_x (dispatch) or out (combine)
  void* recv_scale;         // FP8: fp32 [rows, H/128]; MX: E8M0 bytes [rows, H/32]
  const float* src_scale;   // pre-quantised dispatch: the caller's fp32 scales [T, H/128]
  int T, H, k;
  int64_t rows;             // receive rows (bounds for slot values)
  int num_cus;              // 0: whole GPU; n > 0: n persistent workgroups of kBudgetWaves wavefronts
};

// Combine backward: g [T, H] and y [rows, H] BF16, grad_y [rows, H] BF16,
// grad_w [T, k] fp32 or null (then y is not read).
struct BackParams {
  const void* g;
  const void* y;
  const int32_t* slot;
  const float* weights;
  void* grad_y;
  float* grad_w;
  int T, H, k;
  int64_t rows;
  int num_cus;  // as in RowParams
};

// Wavefronts per workgroup of a launch limited to a CU budget: one 1024-thread
// workgroup per CU of the budget.
constexpr int kBudgetWaves = 16;

// Upper bound of num_topk (the C ABI's EP_MAX_TOPK), for LDS sizing.
constexpr int kMaxTopk = 64;

// Dispatch work split: wavefronts per token (wpt) and even chunks per
// wavefront (cpw) for hidden size H, and the launch shape.
struct DispatchSplit {
  int nchunks, wpt, cpw, blocks;
  bool budget;  // persistent kBudgetWaves-wavefront workgroups, one per CU of the budget
};
DispatchSplit dispatch_split(const RowParams& p);

hipError_t launch_dispatch_bf16(const RowParams& p, hipStream_t stream);  // weights non-null: scaled copies
hipError_t launch_dispatch_fp8(const RowParams& p, hipStream_t stream);
hipError_t launch_dispatch_mx(const RowParams& p, int elem_bits, hipStream_t stream);  // 8: MXFP8, 4: MXFP4
hipError_t launch_dispatch_prequantized(const RowParams& p, hipStream_t stream);     // src = E4M3 codes
// Layout and BF16 / FP8 dispatch in one launch for batches of at most 1024
// pairs (see ep_layout_dispatch.hip).
bool layout_dispatch_fusable(const LayoutPlan& plan, const LayoutParams& lp);
hipError_t launch_layout_dispatch(const LayoutPlan& plan, LayoutParams lp, const RowParams& rp, bool fp8,
                                  hipStream_t stream);
hipError_t launch_combine(const RowParams& p, hipStream_t stream);  // weights null: unit weights
hipError_t launch_combine_backward(const BackParams& p, hipStream_t stream);

hipError_t launch_check_cvt_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream);
hipError_t launch_check_cvt_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream);
hipError_t launch_check_cvt_e2m1(const float* in, uint8_t* out, int64_t n, hipStream_t stream);
hipError_t launch_check_quant_e4m3(const uint16_t* x, const float* s, uint8_t* out, int64_t n, hipStream_t stream);
hipError_t launch_probe_stream(const void* src, void* dst, int64_t units, int read_chunks, int write_chunks,
                               int policy, hipStream_t stream);

}  // namespace ep
