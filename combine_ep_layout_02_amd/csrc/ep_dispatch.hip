// Dispatch for gfx950: scatter BF16 token rows into the expert-major receive
// buffer, as BF16 copies or as OCP E4M3FN codes with one fp32 scale per
// 128-column block.
//
// Dispatch sends every token to each of its top-k experts, BF16 or FP8
// (DeepEP documentation item 10; GeekNews "DeepSeek publica DeepEP ...",
// section "Resultados de medición de rendimiento": FP8 dispatch, BF16
// combine).  This is one GPU's share: the receive buffer is local HBM.
//
// Work unit: one wavefront per (token, 1024-column chunk).  Each lane owns
// two 8-column groups, columns [c*1024 + 8*lane, +8) and the same +512, so
// both 16-byte loads of a wavefront are fully coalesced 1 KiB reads.  The
// token row is read once and written to all of its k slots.  For FP8, a
// 128-column block is exactly one 16-lane DPP row, so the block amax is four
// DPP max steps on the magnitude bits, with no LDS and no barrier.
//
// Out-of-range columns of the last chunk are handled by raw buffer
// addressing: loads past the row return 0 and stores past it are dropped.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kChunk = 1024;       // columns per work unit
constexpr int kWavesPerBlock = 4;  // 256 threads

// Loads the pair slots of token t into lanes 0..k-1 (one vector load), so a
// wave-uniform slot is one v_readlane away.
__device__ __forceinline__ int load_lane_slot(const int32_t* slot, int64_t t, int k, int lane) {
  return lane < k ? slot[t * k + lane] : -1;
}

__device__ __forceinline__ bool slot_ok(int s, int64_t rows) { return s >= 0 && (int64_t)s < rows; }

template <int AUX_LD, int AUX_ST>
__global__ __launch_bounds__(256) void dispatch_bf16_kernel(RowParams p, int chunks) {
  const int lane = threadIdx.x & 63;
  const int item = uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int t = item / chunks;
  if (t >= p.T) return;
  const int c = item - t * chunks;
  const int H = p.H, k = p.k;
  const uint32_t colA = (uint32_t)(c * kChunk + lane * 8), colB = colA + 512;

  const uint16_t* xrow = static_cast<const uint16_t*>(p.src) + (int64_t)t * H;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xrow, (uint32_t)H * 2u);
  const u32x4 a = load16<AUX_LD>(rx, colA * 2u);
  const u32x4 b = load16<AUX_LD>(rx, colB * 2u);
  const int sl = load_lane_slot(p.slot, t, k, lane);

  uint16_t* dst = static_cast<uint16_t*>(p.dst);
  for (int j = 0; j < k; ++j) {
    const int s = __builtin_amdgcn_readlane(sl, j);
    if (!slot_ok(s, p.rows)) continue;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + (int64_t)s * H, (uint32_t)H * 2u);
    store16<AUX_ST>(rd, colA * 2u, a);
    store16<AUX_ST>(rd, colB * 2u, b);
  }
}

// Eight BF16 values -> eight E4M3 codes with scale s: code = E4M3(x / s),
// one correctly rounded fp32 division per element.
__device__ __forceinline__ u32x2 quantize8(u32x4 v, float s) {
  u32x2 q;
  q.x = pack_e4m3x4(bf16_lo(v.x) / s, bf16_hi(v.x) / s, bf16_lo(v.y) / s, bf16_hi(v.y) / s);
  q.y = pack_e4m3x4(bf16_lo(v.z) / s, bf16_hi(v.z) / s, bf16_lo(v.w) / s, bf16_hi(v.w) / s);
  return q;
}

// Block scale: s = max(amax, 1e-4) / 448 (fp32, correctly rounded).  The
// floor keeps an all-zero block finite; 448 is E4M3's largest magnitude, so
// the block's largest element lands on the top code.
__device__ __forceinline__ float block_scale(uint32_t amax_bits16) {
  return fmaxf(__uint_as_float(amax_bits16 << 16), 1e-4f) / 448.0f;
}

template <int AUX_LD, int AUX_ST>
__global__ __launch_bounds__(256) void dispatch_fp8_kernel(RowParams p, int chunks) {
  const int lane = threadIdx.x & 63;
  const int item = uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int t = item / chunks;
  if (t >= p.T) return;
  const int c = item - t * chunks;
  const int H = p.H, k = p.k, nb = H >> 7;
  const uint32_t colA = (uint32_t)(c * kChunk + lane * 8), colB = colA + 512;

  const uint16_t* xrow = static_cast<const uint16_t*>(p.src) + (int64_t)t * H;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xrow, (uint32_t)H * 2u);
  const u32x4 a = load16<AUX_LD>(rx, colA * 2u);
  const u32x4 b = load16<AUX_LD>(rx, colB * 2u);
  const int sl = load_lane_slot(p.slot, t, k, lane);

  // lanes 16r..16r+15 hold one 128-column block: reduce over the DPP row
  const float sa = block_scale(row16_max_u32(absmax_bits8(a)));
  const float sb = block_scale(row16_max_u32(absmax_bits8(b)));
  const u32x2 qa = quantize8(a, sa);
  const u32x2 qb = quantize8(b, sb);

  uint8_t* dst = static_cast<uint8_t*>(p.dst);
  const bool scale_lane = (lane & 15) == 0;
  for (int j = 0; j < k; ++j) {
    const int s = __builtin_amdgcn_readlane(sl, j);
    if (!slot_ok(s, p.rows)) continue;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + (int64_t)s * H, (uint32_t)H);
    store8<AUX_ST>(rd, colA, qa);
    store8<AUX_ST>(rd, colB, qb);
    if (scale_lane) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.recv_scale + (int64_t)s * nb, (uint32_t)nb * 4u);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sa), rs, (int)((colA >> 7) * 4u), 0, AUX_ST);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sb), rs, (int)((colB >> 7) * 4u), 0, AUX_ST);
    }
  }
}

__global__ __launch_bounds__(256) void check_cvt_e4m3_kernel(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n;
       i += (int64_t)gridDim.x * blockDim.x * 4) {
    float v[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) v[m] = (i + m < n) ? in[i + m] : 0.0f;
    const uint32_t q = pack_e4m3x4(v[0], v[1], v[2], v[3]);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (i + m < n) out[i + m] = (uint8_t)(q >> (8 * m));
  }
}

__global__ __launch_bounds__(256) void check_cvt_bf16_kernel(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 2; i < n;
       i += (int64_t)gridDim.x * blockDim.x * 2) {
    const float a = in[i];
    const float b = (i + 1 < n) ? in[i + 1] : 0.0f;
    const uint32_t q = pack_bf16x2(a, b);
    out[i] = (uint16_t)q;
    if (i + 1 < n) out[i + 1] = (uint16_t)(q >> 16);
  }
}

int blocks_for(const RowParams& p, int* chunks) {
  *chunks = (p.H + kChunk - 1) / kChunk;
  const int64_t items = (int64_t)p.T * *chunks;
  return (int)((items + kWavesPerBlock - 1) / kWavesPerBlock);
}

}  // namespace

hipError_t launch_dispatch_bf16(const RowParams& p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  int chunks;
  const int blocks = blocks_for(p, &chunks);
  hipLaunchKernelGGL((dispatch_bf16_kernel<kAuxDefault, kAuxDefault>), dim3(blocks), dim3(256), 0, stream,
                     p, chunks);
  return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const RowParams& p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  int chunks;
  const int blocks = blocks_for(p, &chunks);
  hipLaunchKernelGGL((dispatch_fp8_kernel<kAuxDefault, kAuxDefault>), dim3(blocks), dim3(256), 0, stream,
                     p, chunks);
  return hipGetLastError();
}

hipError_t launch_check_cvt_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 1023) / 1024;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(check_cvt_e4m3_kernel, dim3(blocks), dim3(256), 0, stream, in, out, n);
  return hipGetLastError();
}

hipError_t launch_check_cvt_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 511) / 512;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(check_cvt_bf16_kernel, dim3(blocks), dim3(256), 0, stream, in, out, n);
  return hipGetLastError();
}

}  // namespace ep
