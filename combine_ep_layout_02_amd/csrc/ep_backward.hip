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
// so grad_y is a dispatch of g with a different scale per copy, and grad_w
// is a gather of the same rows combine reads.  One kernel does both: it
// reads g[t] once, reads each of the token's k rows of y once and writes each
// of its k rows of grad_y once.  (The backward of dispatch is the combine
// kernel with unit weights: it lives in ep_combine.hip.)
//
// Work unit: one workgroup per token, one wavefront per 512-column chunk
// (up to 16 wavefronts; wider rows loop).  Every lane holds 8 columns: it
// loads g and the k rows of y for them (all loads issued before any
// arithmetic), stores the k scaled grad_y vectors, and keeps one fp32 dot
// partial per row.  The partials are summed in a fixed tree: 8 columns
// serially in the lane, 16-lane DPP rows, the 4 rows of the wavefront, then
// the wavefronts in ascending order through LDS.  The result is
// deterministic; its error is that of a summation tree of depth at most
// 8*ceil(chunks/16) + 6 + 15 over exact BF16 x BF16 products.
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

__device__ __forceinline__ u32x4 scale_pack8(float w, const float* g) {
  u32x4 o;
  o.x = pack_bf16x2(w * g[0], w * g[1]);
  o.y = pack_bf16x2(w * g[2], w * g[3]);
  o.z = pack_bf16x2(w * g[4], w * g[5]);
  o.w = pack_bf16x2(w * g[6], w * g[7]);
  return o;
}

// K > 0: exactly K pairs per token, one batch.  K == 0: any k, in batches
// of 8 pairs (g is re-read per batch, from L2).
template <int K, bool GW, int AUX_LD, int AUX_ST>
__global__ __launch_bounds__(64 * kMaxWaves) void combine_backward_kernel(BackParams p, int chunks) {
  constexpr int NB = K > 0 ? K : 8;
  __shared__ float part[kMaxWaves][kMaxTopk];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int waves = uniform(blockDim.x >> 6);
  const int t = blockIdx.x;
  const int H = p.H;
  const int k = K > 0 ? K : p.k;
  const uint32_t row_bytes = (uint32_t)H * 2u;

  int sl = -1, wl = 0;
  if (lane < k) {
    sl = p.slot[(int64_t)t * k + lane];
    wl = (int)__float_as_uint(p.weights[(int64_t)t * k + lane]);
  }
  const uint16_t* y = static_cast<const uint16_t*>(p.y);
  uint16_t* gy = static_cast<uint16_t*>(p.grad_y);
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
      const u32x4 gv = load16<AUX_LD>(rg, off);
      u32x4 yv[NB];
      if constexpr (GW) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
          yv[i] = load16<AUX_LD>(make_rsrc(y + (ok[i] ? (int64_t)s[i] * H : 0), ok[i] ? row_bytes : 0u), off);
      }
      float gf[8];
      widen8(gv, gf);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (!ok[i]) continue;
        const float w = __uint_as_float((uint32_t)__builtin_amdgcn_readlane(wl, (j0 + i) & 63));
        store16<AUX_ST>(make_rsrc(gy + (int64_t)s[i] * H, row_bytes), off, scale_pack8(w, gf));
        if constexpr (GW) {
          float yf[8];
          widen8(yv[i], yf);
#pragma unroll
          for (int m = 0; m < 8; ++m) dot[i] = __builtin_fmaf(gf[m], yf[m], dot[i]);
        }
      }
    }
    if constexpr (GW) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (j0 + i >= k) break;
        const float total = wave_sum(dot[i]);
        if (lane == 0) part[wave][j0 + i] = total;
      }
    }
  }
  if constexpr (GW) {
    __syncthreads();
    const int j = threadIdx.x;
    if (j < k) {
      float acc = part[0][j];
      for (int w = 1; w < waves; ++w) acc += part[w][j];
      p.grad_w[(int64_t)t * k + j] = acc;
    }
  }
}

template <int K, bool GW>
hipError_t launch_kg(const BackParams& p, int waves, int chunks, hipStream_t stream) {
  const dim3 grid(p.T), block(64 * waves);
  if ((int64_t)p.T * p.k * p.H * 2 < kStreamingBytes)
    hipLaunchKernelGGL((combine_backward_kernel<K, GW, kAuxDefault, kAuxDefault>), grid, block, 0, stream, p, chunks);
  else
    hipLaunchKernelGGL((combine_backward_kernel<K, GW, kAuxNT, kAuxNT>), grid, block, 0, stream, p, chunks);
  return hipGetLastError();
}

template <bool GW>
hipError_t launch_g(const BackParams& p, int waves, int chunks, hipStream_t stream) {
  switch (p.k) {
    case 1: return launch_kg<1, GW>(p, waves, chunks, stream);
    case 2: return launch_kg<2, GW>(p, waves, chunks, stream);
    case 4: return launch_kg<4, GW>(p, waves, chunks, stream);
    case 6: return launch_kg<6, GW>(p, waves, chunks, stream);
    case 8: return launch_kg<8, GW>(p, waves, chunks, stream);
    default: return launch_kg<0, GW>(p, waves, chunks, stream);
  }
}

}  // namespace

hipError_t launch_combine_backward(const BackParams& p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const int chunks = (p.H + kChunkCols - 1) / kChunkCols;
  const int waves = chunks < kMaxWaves ? chunks : kMaxWaves;
  return p.grad_w ? launch_g<true>(p, waves, chunks, stream) : launch_g<false>(p, waves, chunks, stream);
}

}  // namespace ep
