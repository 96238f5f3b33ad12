// Device helpers shared by the gfx950 layout / dispatch / combine kernels.
//
// Everything here is written for CDNA4 (gfx950): 64-lane wavefronts, DPP
// row operations for 16-lane reductions, raw buffer loads whose range check
// turns out-of-range reads into zeros, and the gfx950 conversion
// instructions v_cvt_pk_fp8_f32 (OCP E4M3FN on this target) and
// v_cvt_pk_bf16_f32 (round to nearest even).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource word 3 for gfx9-family targets (32-bit data format,
// no swizzle).  A load whose offset is at or past num_bytes returns 0.
constexpr int kBufferWord3 = 0x00020000;

// Cache-policy bits of the buffer instructions' aux operand on gfx94x/gfx950.
constexpr int kAuxDefault = 0;
constexpr int kAuxNT = 2;    // nt: non-temporal, stream through
constexpr int kAuxSC1 = 16;  // sc1: device-scope store

// Receive-buffer traffic above which dispatch / combine switch to streaming
// cache policies.  Small (decode-sized) calls load through the caches and
// store with sc1 (kAuxSmallStore): their rows stay in the 256 MB Infinity
// Cache, and device-scope stores leave no dirty L2 lines to be written back
// when the kernel ends (measured at 128 decode tokens: layout + FP8 dispatch
// in one launch 5.87 -> 5.29 us, with combine 9.3 -> 8.6 us per call; nt
// stores 5.56 us).  Large ones, as measured on MI355X for the 8192-token
// step:
//   - dispatch stores its receive rows with nt, so they do not sit dirty in
//     the caches and get written back during the next kernel;
//   - combine gathers its rows with nt loads, so they do not evict anything;
//   - combine stores its output with sc1 while the output fits in half of the
//     256 MB Infinity Cache (the writes then interleave far less with the
//     gathered reads at the DRAM: at 8192 tokens the output costs ~36 us with
//     sc1 vs 46 us with nt beside 137 us of reads), and with nt beyond that
//     (a 235 MB output thrashes the cache and sc1 loses 5% at 16384 tokens).
constexpr int64_t kStreamingBytes = (int64_t)64 << 20;
constexpr int kAuxSmallStore = kAuxSC1;

// Workgroups are dealt to the chip's 8 XCDs round robin (workgroup b to XCD
// b mod 8).  This renumbering, a bijection on [0, nb), gives XCD x one
// contiguous eighth of the logical workgroups [x*q + min(x, r), ...) with
// q = nb / 8, r = nb % 8, instead of every eighth one.
__device__ __forceinline__ int xcd_contiguous(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}
constexpr int64_t kCacheableOutputBytes = (int64_t)128 << 20;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)num_bytes, kBufferWord3);
}

template <int AUX>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)byte_off, 0, AUX);
}

// Exact widening of the two BF16 halves of a dword.
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Two fp32 -> two BF16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Four fp32 -> four OCP E4M3FN codes (round to nearest even), a in byte 0.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Maximum of an unsigned value over each 16-lane DPP row of the wavefront.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// Largest |x| of the 8 BF16 values in a 16-byte vector, as a 15-bit
// magnitude pattern (|x| bits >> 16).  For non-negative floats the bit
// pattern orders like the value, so integer max is exact.
__device__ __forceinline__ uint32_t absmax_bits8(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, v[i] & 0x7FFFu);
    m = max(m, (v[i] >> 16) & 0x7FFFu);
  }
  return m;
}

// Wave-uniform value (lets the compiler keep it in scalar registers).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace ep
