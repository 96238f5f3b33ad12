// Streaming probe: the practical HBM ceiling of a given read:write mix.
//
// Not part of the method.  The dispatch and combine kernels move bytes in
// very different proportions (combine at 8192 tokens reads 8 bytes for every
// one it writes, FP8 dispatch writes 4 for every one it reads), and DRAM
// delivers a different bandwidth for each mix.  This kernel moves the same
// mix with the simplest possible access pattern, contiguous 1 KiB chunks
// streamed through, so a measured kernel can be set against the rate its own
// byte mix allows on the same machine.  The cache policy is a parameter (policy 0: non-temporal loads and stores;
// 1: default loads and stores; 2: non-temporal loads, device-scope sc1
// stores; 3: default loads, non-temporal stores), so a caller can take the
// best of them as the ceiling.  Policy + 4: the same, with units taken in
// XCD-contiguous order (each XCD one contiguous eighth of them), the order
// the scaled dispatch kernels use.
//
// Unit u (one wavefront each, grid-stride over units): reads chunks
// [u*r, (u+1)*r) of src, XORs them lane-wise into one 16-byte value per lane
// and writes that value to chunks [u*w, (u+1)*w) of dst.  All r loads are
// issued before the first XOR.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kChunk = 1024;           // bytes per chunk: 64 lanes x 16 bytes
constexpr int kProbeWaves = 4;         // wavefronts per workgroup

template <int R, int AUX_LD, int AUX_ST>
__global__ __launch_bounds__(64 * kProbeWaves) void probe_stream_kernel(const uint8_t* src, uint8_t* dst,
                                                                         int64_t units, int w, int xcd) {
  const int lane = threadIdx.x & 63;
  const int blk = xcd ? xcd_contiguous((int)blockIdx.x, (int)gridDim.x) : (int)blockIdx.x;
  for (int64_t u = (int64_t)blk * kProbeWaves + (threadIdx.x >> 6); u < units;
       u += (int64_t)gridDim.x * kProbeWaves) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + u * R * kChunk, (uint32_t)(R * kChunk));
    u32x4 v[R];
#pragma unroll
    for (int c = 0; c < R; ++c) v[c] = load16<AUX_LD>(rs, (uint32_t)(c * kChunk + lane * 16));
    u32x4 x = v[0];
#pragma unroll
    for (int c = 1; c < R; ++c) x ^= v[c];
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + u * w * kChunk, (uint32_t)w * kChunk);
    for (int c = 0; c < w; ++c) store16<AUX_ST>(rd, (uint32_t)(c * kChunk + lane * 16), x);
  }
}

template <int R, int AUX_LD, int AUX_ST>
void launch_rp(const void* src, void* dst, int64_t units, int w, int xcd, hipStream_t stream) {
  const int64_t blocks = (units + kProbeWaves - 1) / kProbeWaves;
  const unsigned grid = (unsigned)(blocks < 65536 * 8 ? blocks : 65536 * 8);
  hipLaunchKernelGGL((probe_stream_kernel<R, AUX_LD, AUX_ST>), dim3(grid), dim3(64 * kProbeWaves), 0, stream,
                     static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), units, w, xcd);
}

template <int R>
void launch_r(const void* src, void* dst, int64_t units, int w, int policy, hipStream_t stream) {
  const int xcd = policy >> 2;
  switch (policy & 3) {
    case 0: launch_rp<R, kAuxNT, kAuxNT>(src, dst, units, w, xcd, stream); break;
    case 1: launch_rp<R, kAuxDefault, kAuxDefault>(src, dst, units, w, xcd, stream); break;
    case 2: launch_rp<R, kAuxNT, kAuxSC1>(src, dst, units, w, xcd, stream); break;
    default: launch_rp<R, kAuxDefault, kAuxNT>(src, dst, units, w, xcd, stream); break;
  }
}

}  // namespace

hipError_t launch_probe_stream(const void* src, void* dst, int64_t units, int read_chunks, int write_chunks,
                               int policy, hipStream_t stream) {
  if (units == 0) return hipSuccess;
  switch (read_chunks) {
    case 1: launch_r<1>(src, dst, units, write_chunks, policy, stream); break;
    case 2: launch_r<2>(src, dst, units, write_chunks, policy, stream); break;
    case 4: launch_r<4>(src, dst, units, write_chunks, policy, stream); break;
    case 8: launch_r<8>(src, dst, units, write_chunks, policy, stream); break;
    default: launch_r<16>(src, dst, units, write_chunks, policy, stream); break;
  }
  return hipGetLastError();
}

}  // namespace ep
