// Device building blocks of dispatch, shared by the dispatch kernels
// (ep_dispatch.hip) and the fused layout + dispatch kernel
// (ep_layout_dispatch.hip).  See ep_dispatch.hip for the design.
#pragma once

#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace dsp {

constexpr uint32_t kNoColumn = 0xFFFFFFF0u;  // a load offset past any row: reads 0

// Loads the pair slots of token t into lanes 0..k-1 (one vector load), so a
// wave-uniform slot is one v_readlane away.
static __device__ __forceinline__ int load_lane_slot(const int32_t* slot, int64_t t, int k, int lane) {
  return lane < k ? slot[t * k + lane] : -1;
}

static __device__ __forceinline__ bool slot_ok(int s, int64_t rows) { return s >= 0 && (int64_t)s < rows; }

// Token and first chunk of slice `wave` (token-major: wpt slices per token).
struct Slice {
  int t, c0, nc;
};

static __device__ __forceinline__ Slice slice_of(int wave, int wpt, int cpw, int nchunks) {
  Slice sl;
  sl.t = wave / wpt;
  sl.c0 = (wave - sl.t * wpt) * cpw;
  sl.nc = min(cpw, nchunks - sl.c0);
  return sl;
}

template <int NC, int AUX_LD>
static __device__ __forceinline__ void load_row(const RowParams& p, const Slice& sl, int lane, u32x4 (&v)[NC]) {
  const uint16_t* xrow = static_cast<const uint16_t*>(p.src) + (int64_t)sl.t * p.H;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xrow, (uint32_t)p.H * 2u);
#pragma unroll
  for (int c = 0; c < NC; ++c)
    v[c] = load16<AUX_LD>(rx, c < sl.nc ? (uint32_t)((sl.c0 + c) * 512 + lane * 8) * 2u : kNoColumn);
}

// Eight BF16 values times w, each product rounded to fp32 and then to BF16
// (nearest even).
static __device__ __forceinline__ u32x4 scale8(u32x4 v, float w) {
  u32x4 o;
  o.x = pack_bf16x2(w * bf16_lo(v.x), w * bf16_hi(v.x));
  o.y = pack_bf16x2(w * bf16_lo(v.y), w * bf16_hi(v.y));
  o.z = pack_bf16x2(w * bf16_lo(v.z), w * bf16_hi(v.z));
  o.w = pack_bf16x2(w * bf16_lo(v.w), w * bf16_hi(v.w));
  return o;
}

// Eight BF16 values -> eight E4M3 codes with scale s: code = E4M3(x / s),
// one correctly rounded fp32 division per element.  (Measured at 8192
// tokens: a multiplication by 1/s with the division kept only for quotients
// near an E4M3 rounding threshold gives the same codes, but is no faster
// when the compiler evaluates both sides, and 2% slower when the divisions
// sit behind a wave-uniform branch, which raises register use from 82 to 115
// VGPRs.)
static __device__ __forceinline__ u32x2 quantize8(u32x4 v, float s) {
  u32x2 q;
  q.x = pack_e4m3x4(bf16_lo(v.x) / s, bf16_hi(v.x) / s, bf16_lo(v.y) / s, bf16_hi(v.y) / s);
  q.y = pack_e4m3x4(bf16_lo(v.z) / s, bf16_hi(v.z) / s, bf16_lo(v.w) / s, bf16_hi(v.w) / s);
  return q;
}

// Block scale: s = max(amax, 1e-4) / 448 (fp32, correctly rounded).  The
// floor keeps an all-zero block finite; 448 is E4M3's largest magnitude, so
// the block's largest element lands on the top code.
static __device__ __forceinline__ float block_scale(uint32_t amax_bits16) {
  return fmaxf(__uint_as_float(amax_bits16 << 16), 1e-4f) / 448.0f;
}

// Stores the slice's row (NC chunks in v) to every valid slot of its token;
// slots holds slot[t, lane] in lanes 0..k-1.  SCALED: copy j is
// BF16_RNE(w[t,j] * x[t]) instead of x[t] (the output-row gradients of the
// combine backward: a dispatch scaled per copy).
template <int NC, int AUX_ST, bool SCALED>
static __device__ __forceinline__ void store_bf16_row(const RowParams& p, const Slice& sl, int lane, const u32x4 (&v)[NC],
                                               int slots) {
  int wl = 0;
  if (SCALED && lane < p.k) wl = (int)__float_as_uint(p.weights[(int64_t)sl.t * p.k + lane]);
  uint16_t* dst = static_cast<uint16_t*>(p.dst);
  const uint32_t col = (uint32_t)(sl.c0 * 512 + lane * 8) * 2u;
  for (int j = 0; j < p.k; ++j) {
    const int s = __builtin_amdgcn_readlane(slots, j);
    if (!slot_ok(s, p.rows)) continue;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + (int64_t)s * p.H, (uint32_t)p.H * 2u);
    if constexpr (SCALED) {
      const float w = __uint_as_float((uint32_t)__builtin_amdgcn_readlane(wl, j));
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        // Re-widen the row for every copy: an empty asm makes the register
        // opaque, so the compiler does not keep 8 * NC widened floats live
        // across the j loop (which halves occupancy at NC = 14).
        u32x4 vc = v[c];
        asm volatile("" : "+v"(vc));
        if (c < sl.nc) store16<AUX_ST>(rd, col + 1024u * c, scale8(vc, w));
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c < sl.nc) store16<AUX_ST>(rd, col + 1024u * c, v[c]);
    }
  }
}

// Quantises the slice's row (NC chunks in v) and stores the codes and block
// scales to every valid slot of its token (slots as in store_bf16_row).
// cpw (chunks per wavefront) is even, so chunks pair up as (2m, 2m+1): the
// even lane of a lane pair stores 16 bytes of chunk 2m, the odd lane the same
// bytes of chunk 2m+1.  A pair whose second chunk lies past the row stores
// that half out of range, where the store is dropped.
template <int NC, int AUX_ST>
static __device__ __forceinline__ void store_fp8_row(const RowParams& p, const Slice& sl, int lane, const u32x4 (&v)[NC],
                                              int slots) {
  static_assert(NC % 2 == 0, "chunks pair up");
  float sc[NC];
  u32x2 q[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    sc[c] = block_scale(row16_max_u32(absmax_bits8(v[c])));
    q[c] = quantize8(v[c], sc[c]);
  }
  const bool odd = lane & 1;
  u32x4 out[NC / 2];
#pragma unroll
  for (int m = 0; m < NC / 2; ++m) {
    const u32x2 a = q[2 * m], b = q[2 * m + 1];
    const u32x2 send = odd ? a : b;
    u32x2 recv;
    recv.x = (uint32_t)__builtin_amdgcn_mov_dpp((int)send.x, 0xB1, 0xF, 0xF, false);
    recv.y = (uint32_t)__builtin_amdgcn_mov_dpp((int)send.y, 0xB1, 0xF, 0xF, false);
    out[m].x = odd ? recv.x : a.x;
    out[m].y = odd ? recv.y : a.y;
    out[m].z = odd ? b.x : recv.x;
    out[m].w = odd ? b.y : recv.y;
  }
  // lane l < 4*nc takes the scale of block 4*c0 + l (chunk l/4, DPP row l%4)
  float my_scale = 0.0f;
  const int owner = (lane & 3) << 4;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float g = __shfl(sc[c], owner, 64);
    if ((lane >> 2) == c) my_scale = g;
  }

  const int H = p.H, nb = H >> 7;
  uint8_t* dst = static_cast<uint8_t*>(p.dst);
  const uint32_t ocol = (uint32_t)(sl.c0 * 512) + (odd ? 512u : 0u) + 16u * (uint32_t)(lane >> 1);
  const uint32_t scol = (uint32_t)(sl.c0 * 4 + lane) * 4u;
  for (int j = 0; j < p.k; ++j) {
    const int s = __builtin_amdgcn_readlane(slots, j);
    if (!slot_ok(s, p.rows)) continue;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + (int64_t)s * H, (uint32_t)H);
#pragma unroll
    for (int m = 0; m < NC / 2; ++m)
      if (2 * m < sl.nc) store16<AUX_ST>(rd, ocol + 1024u * m, out[m]);
    if (lane < 4 * sl.nc) {
      // The scales of consecutive receive rows are neighbours in recv_scale
      // but come from different tokens: stored through the caches, the
      // partial lines merge before they reach HBM (streamed as the rows are,
      // they cost 10 us of the 113 us dispatch at 8192 tokens).
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(static_cast<float*>(p.recv_scale) + (int64_t)s * nb, (uint32_t)nb * 4u);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(my_scale), rs, (int)scol, 0, kAuxDefault);
    }
  }
}

}  // namespace dsp
}  // namespace ep
