// Combine for gfx950: gather each token's k expert-output rows and write the
// gate-weighted fp32 sum as BF16.
//
// Combine reduces the expert outputs back to the tokens' origin (DeepEP
// documentation item 10; GeekNews "DeepSeek publica DeepEP ...", section
// "Patrones de uso en entrenamiento, prefill y decoding"); here the origin
// rows are local.  The sum is a fixed chain: acc = +0, then for j = 0..k-1
// over valid slots acc = fmaf(w[t,j], y[slot[t,j], h], acc), then one BF16
// round to nearest even (v_cvt_pk_bf16_f32).  A fixed order keeps the result
// deterministic and equal to a scalar evaluation of the same chain.
//
// With no weights (every weight 1) the same kernel is the backward of
// dispatch: the gradient of a token is the sum of the gradients of its
// received copies (DeepEP runs the backward of dispatch as a combine:
// documentation item 10, "Backward Pass"), and fmaf(1, v, acc) == acc + v.
//
// Work unit: one wavefront per (token, column chunk).  All k row loads
// (16 bytes per lane and column group each) are issued before the first FMA,
// so a wavefront keeps k * groups independent 1 KiB reads in flight.  Slots
// and weights arrive with one vector load (lane j holds pair j) and are made
// wave-uniform with v_readlane; an invalid slot gets an empty buffer range,
// so its loads return zeros without touching memory and the FMA is skipped.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

// 16-byte column groups per lane per row (NG): a work item covers 512 * NG
// columns.  Two groups (1024 columns, 16 loads in flight per wavefront) for
// large batches; one group for small ones, where twice the wavefronts spread
// the latency-bound gather over more CUs (128 decode tokens: 3.4 vs 3.7 us).
constexpr int kSmallItems = 4096;  // (token, 1024-column) items below which NG = 1
constexpr int kWavesPerBlock = 1;  // whole-GPU launches: 64-thread blocks, measured ~3% faster than 256 at the 8K step

__device__ __forceinline__ void fma8(float* acc, float w, u32x4 v) {
  acc[0] = __builtin_fmaf(w, bf16_lo(v.x), acc[0]);
  acc[1] = __builtin_fmaf(w, bf16_hi(v.x), acc[1]);
  acc[2] = __builtin_fmaf(w, bf16_lo(v.y), acc[2]);
  acc[3] = __builtin_fmaf(w, bf16_hi(v.y), acc[3]);
  acc[4] = __builtin_fmaf(w, bf16_lo(v.z), acc[4]);
  acc[5] = __builtin_fmaf(w, bf16_hi(v.z), acc[5]);
  acc[6] = __builtin_fmaf(w, bf16_lo(v.w), acc[6]);
  acc[7] = __builtin_fmaf(w, bf16_hi(v.w), acc[7]);
}

__device__ __forceinline__ u32x4 pack8(const float* acc) {
  u32x4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  return o;
}

// Rows j0 .. j0+NB-1 of the chain (NB known at compile time; rows >= k are
// empty).  All loads first, then the FMAs in j order.
template <int NB, int NG, int AUX_LD>
__device__ __forceinline__ void accumulate(const uint16_t* y, int64_t rows, int H, int k, int j0, int sl,
                                           int wl, uint32_t col0, float (&acc)[NG][8]) {
  u32x4 v[NB][NG];
  bool ok[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int j = j0 + i;
    const int s = __builtin_amdgcn_readlane(sl, j & 63);
    ok[i] = j < k && s >= 0 && (int64_t)s < rows;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(y + (ok[i] ? (int64_t)s * H : 0), ok[i] ? (uint32_t)H * 2u : 0u);
#pragma unroll
    for (int g = 0; g < NG; ++g) v[i][g] = load16<AUX_LD>(r, (col0 + 512u * g) * 2u);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (!ok[i]) continue;
    const float w = __uint_as_float((uint32_t)__builtin_amdgcn_readlane(wl, (j0 + i) & 63));
#pragma unroll
    for (int g = 0; g < NG; ++g) fma8(acc[g], w, v[i][g]);
  }
}

// Items (token, chunk) are handed out grid-stride: a whole-GPU launch has one
// wavefront per item and runs the loop once; a launch limited to a CU budget
// runs that many persistent workgroups of WPB wavefronts.
template <int K, int AUX_LD, int AUX_ST, int WPB, int NG>
__global__ __launch_bounds__(64 * WPB) void combine_kernel(RowParams p, int chunks) {
  const int lane = threadIdx.x & 63;
  const int items = p.T * chunks;
  for (int item = uniform((int)blockIdx.x * WPB + (int)(threadIdx.x >> 6)); item < items;
       item += (int)gridDim.x * WPB) {
  const int t = item / chunks;
  const int c = item - t * chunks;
  const int H = p.H;
  const int k = K > 0 ? K : p.k;
  const uint32_t col0 = (uint32_t)(c * 512 * NG + lane * 8);

  int sl = -1, wl = 0;
  if (lane < k) {
    sl = p.slot[(int64_t)t * k + lane];
    wl = (int)__float_as_uint(p.weights ? p.weights[(int64_t)t * k + lane] : 1.0f);
  }
  const uint16_t* y = static_cast<const uint16_t*>(p.src);
  float acc[NG][8];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;

  if constexpr (K > 0) {
    accumulate<K, NG, AUX_LD>(y, p.rows, H, k, 0, sl, wl, col0, acc);
  } else {
    for (int j0 = 0; j0 < k; j0 += 8) accumulate<8, NG, AUX_LD>(y, p.rows, H, k, j0, sl, wl, col0, acc);
  }

  uint16_t* out = static_cast<uint16_t*>(p.dst) + (int64_t)t * H;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, (uint32_t)H * 2u);
#pragma unroll
  for (int g = 0; g < NG; ++g) store16<AUX_ST>(ro, (col0 + 512u * g) * 2u, pack8(acc[g]));
  }
}

template <int K, int WPB, int NG>
void launch_kw(const RowParams& p, int blocks, int chunks, hipStream_t stream) {
  const dim3 block(64 * WPB);
  if ((int64_t)p.T * p.k * p.H * 2 < kStreamingBytes)
    hipLaunchKernelGGL((combine_kernel<K, kAuxDefault, kAuxSmallStore, WPB, NG>), dim3(blocks), block, 0, stream, p,
                       chunks);
  else if ((int64_t)p.T * p.H * 2 <= kCacheableOutputBytes)
    hipLaunchKernelGGL((combine_kernel<K, kAuxNT, kAuxSC1, WPB, NG>), dim3(blocks), block, 0, stream, p, chunks);
  else
    hipLaunchKernelGGL((combine_kernel<K, kAuxNT, kAuxNT, WPB, NG>), dim3(blocks), block, 0, stream, p, chunks);
}

template <int K>
hipError_t launch_k(const RowParams& p, hipStream_t stream) {
  const int chunks2 = (p.H + 1023) / 1024;
  if (p.num_cus > 0) {
    const int64_t need = ((int64_t)p.T * chunks2 + kBudgetWaves - 1) / kBudgetWaves;
    launch_kw<K, kBudgetWaves, 2>(p, (int)(need < p.num_cus ? need : p.num_cus), chunks2, stream);
  } else if ((int64_t)p.T * chunks2 < kSmallItems) {
    const int chunks1 = (p.H + 511) / 512;
    launch_kw<K, kWavesPerBlock, 1>(p, (int)(((int64_t)p.T * chunks1 + kWavesPerBlock - 1) / kWavesPerBlock),
                                    chunks1, stream);
  } else {
    launch_kw<K, kWavesPerBlock, 2>(p, (int)(((int64_t)p.T * chunks2 + kWavesPerBlock - 1) / kWavesPerBlock),
                                    chunks2, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const RowParams& p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  switch (p.k) {
    case 1: return launch_k<1>(p, stream);
    case 2: return launch_k<2>(p, stream);
    case 4: return launch_k<4>(p, stream);
    case 6: return launch_k<6>(p, stream);
    case 8: return launch_k<8>(p, stream);
    default: return launch_k<0>(p, stream);
  }
}

}  // namespace ep
