// Combine backward for gfx950: the gradient of the gate-weighted combine
// with respect to the expert outputs y and the gate weights w.
//
// DeepEP runs the backward of combine as a dispatch over the same routing
// handle (DeepEP documentation item 10, "Backward Pass"; GeekNews "DeepSeek
// publica DeepEP ...", section "Patrones de uso en entrenamiento, prefill y
// decoding").  With out[t] = sum over valid j of w[t,j] * y[slot[t,j]] and
// g = d loss / d out:
//   grad_y[slot[t,j], h] = BF16_RNE(w[t,j] * g[t,h])   (fp32 product)
//   grad_w[t,j]          = sum_h g[t,h] * y[slot[t,j], h]   (fp32)
// grad_y is a dispatch of g with a different scale per copy: the BF16
// dispatch kernel's scaled mode writes it (ep_dispatch.hip).  grad_w is a
// gather of the rows combine reads: the kernel below.  They run as two
// kernels, the read-only gather first and then the write-mostly scatter: on
// MI355X that is ~14% faster at 8192 tokens than one fused kernel that reads
// g and y and writes grad_y in the same pass (400 us fused vs 160 + 185 us),
// although the scatter reads g a second time (mostly from the 256 MB
// Infinity Cache, where the gather left it).  DRAM pays for every switch
// between reading and writing; the fused kernel mixes them throughout.
//
// grad_w work unit: one workgroup per token, one wavefront per 512-column
// chunk (up to 16 wavefronts; wider rows loop).  Every lane holds 8 columns:
// it loads g and the k rows of y for them (all loads issued before any
// arithmetic) and keeps one fp32 dot partial per row.  The partials are
// summed in a fixed tree: 8 columns serially in the lane, 16-lane DPP rows,
// the 4 rows of the wavefront, then the wavefronts in ascending order
// through LDS.  The result is deterministic; its error is that of a
// summation tree of depth at most 8*ceil(chunks/16) + 6 + 15 over exact
// BF16 x BF16 products.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kChunkCols = 512;  // 64 lanes x 8 BF16 columns
constexpr int kMaxWaves = 16;

// Sum of a float over each 16-lane DPP row; every lane of the row ends with
// the same value (the pairwise additions are commutative).
__device__ __forceinline__ float row16_sum(float v) {
  v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0xB1, 0xF, 0xF, false));
  v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x4E, 0xF, 0xF, false));
  v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x141, 0xF, 0xF, false));
  v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x140, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float lane_f(float v, int lane) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), lane));
}

// Wave-uniform sum over the 64 lanes: ((row0 + row1) + (row2 + row3)).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ void widen8(u32x4 v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// The gate-weight gradients of token t.  K > 0: exactly K pairs per token,
// one batch.  K == 0: any k, in batches of 8 pairs (g is re-read per batch,
// from L2).  g is loaded with the default policy so that it stays cached for
// the grad_y scatter that follows; the rows of y are streamed (AUX_Y).
// Ends with a barrier after which `part` may be reused.
template <int K, int AUX_Y>
__device__ __forceinline__ void grad_weights_token(const BackParams& p, int chunks, int t,
                                                   float (&part)[kMaxWaves][kMaxTopk]) {
  constexpr int NB = K > 0 ? K : 8;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int waves = uniform(blockDim.x >> 6);
  const int H = p.H;
  const int k = K > 0 ? K : p.k;
  const uint32_t row_bytes = (uint32_t)H * 2u;

  const int sl = lane < k ? p.slot[(int64_t)t * k + lane] : -1;
  const uint16_t* y = static_cast<const uint16_t*>(p.y);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(static_cast<const uint16_t*>(p.g) + (int64_t)t * H, row_bytes);

  for (int j0 = 0; j0 < k; j0 += NB) {
    int s[NB];
    bool ok[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = j0 + i;
      s[i] = __builtin_amdgcn_readlane(sl, j & 63);
      ok[i] = j < k && s[i] >= 0 && (int64_t)s[i] < p.rows;
    }
    float dot[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) dot[i] = 0.0f;

    for (int c = wave; c < chunks; c += waves) {
      const uint32_t off = (uint32_t)(c * kChunkCols + lane * 8) * 2u;
      const u32x4 gv = load16<kAuxDefault>(rg, off);
      u32x4 yv[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i)
        yv[i] = load16<AUX_Y>(make_rsrc(y + (ok[i] ? (int64_t)s[i] * H : 0), ok[i] ? row_bytes : 0u), off);
      float gf[8];
      widen8(gv, gf);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        float yf[8];
        widen8(yv[i], yf);  // an invalid row reads zeros: its partial stays 0
#pragma unroll
        for (int m = 0; m < 8; ++m) dot[i] = __builtin_fmaf(gf[m], yf[m], dot[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (j0 + i >= k) break;
      const float total = wave_sum(dot[i]);
      if (lane == 0) part[wave][j0 + i] = total;
    }
  }
  __syncthreads();
  const int j = threadIdx.x;
  if (j < k) {
    float acc = part[0][j];
    for (int w = 1; w < waves; ++w) acc += part[w][j];
    p.grad_w[(int64_t)t * k + j] = acc;
  }
}

// Whole-GPU launch: one workgroup per token.  (A token loop in this kernel
// costs 20% here: 150 -> 182 us at 8192 tokens.)
template <int K, int AUX_Y>
__global__ __launch_bounds__(64 * kMaxWaves) void grad_weights_kernel(BackParams p, int chunks) {
  __shared__ float part[kMaxWaves][kMaxTopk];
  grad_weights_token<K, AUX_Y>(p, chunks, blockIdx.x, part);
}

// Launch limited to a CU budget: gridDim.x persistent workgroups loop over
// the tokens.
template <int K, int AUX_Y>
__global__ __launch_bounds__(64 * kMaxWaves) void grad_weights_budget_kernel(BackParams p, int chunks) {
  __shared__ float part[kMaxWaves][kMaxTopk];
  for (int t = blockIdx.x; t < p.T; t += gridDim.x) {
    grad_weights_token<K, AUX_Y>(p, chunks, t, part);
    __syncthreads();  // part is rewritten by the next token
  }
}

template <int K, int AUX_Y>
void launch_gw_aux(const BackParams& p, int waves, int chunks, hipStream_t stream) {
  const dim3 block(64 * waves);
  if (p.num_cus > 0)
    hipLaunchKernelGGL((grad_weights_budget_kernel<K, AUX_Y>), dim3(p.num_cus < p.T ? p.num_cus : p.T), block, 0,
                       stream, p, chunks);
  else
    hipLaunchKernelGGL((grad_weights_kernel<K, AUX_Y>), dim3(p.T), block, 0, stream, p, chunks);
}

template <int K>
hipError_t launch_gw(const BackParams& p, int waves, int chunks, hipStream_t stream) {
  if ((int64_t)p.T * p.k * p.H * 2 < kStreamingBytes)
    launch_gw_aux<K, kAuxDefault>(p, waves, chunks, stream);
  else
    launch_gw_aux<K, kAuxNT>(p, waves, chunks, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_backward(const BackParams& p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  if (p.grad_w) {
    const int chunks = (p.H + kChunkCols - 1) / kChunkCols;
    const int waves = chunks < kMaxWaves ? chunks : kMaxWaves;
    hipError_t err;
    switch (p.k) {
      case 1: err = launch_gw<1>(p, waves, chunks, stream); break;
      case 2: err = launch_gw<2>(p, waves, chunks, stream); break;
      case 4: err = launch_gw<4>(p, waves, chunks, stream); break;
      case 6: err = launch_gw<6>(p, waves, chunks, stream); break;
      case 8: err = launch_gw<8>(p, waves, chunks, stream); break;
      default: err = launch_gw<0>(p, waves, chunks, stream); break;
    }
    if (err != hipSuccess) return err;
  }
  RowParams r{};
  r.src = p.g;
  r.slot = p.slot;
  r.weights = p.weights;
  r.dst = p.grad_y;
  r.T = p.T;
  r.H = p.H;
  r.k = p.k;
  r.rows = p.rows;
  r.num_cus = p.num_cus;
  return launch_dispatch_bf16(r, stream);
}

}  // namespace ep
