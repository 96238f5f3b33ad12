// Dispatch for gfx950: scatter BF16 token rows into the expert-major receive
// buffer, as BF16 copies or as OCP E4M3FN codes with one fp32 scale per
// 128-column block.
//
// Dispatch sends every token to each of its top-k experts, BF16 or FP8
// (DeepEP documentation item 10; GeekNews "DeepSeek publica DeepEP ...",
// section "Resultados de medición de rendimiento": FP8 dispatch, BF16
// combine).  This is one GPU's share: the receive buffer is local HBM.
//
// Work unit: one wavefront per slice of a token's row: two 512-column chunks
// (1024 columns; one chunk for BF16 copies) in a whole-GPU launch; whole
// rows of up to kMaxChunks chunks in a launch limited to a CU budget, whose
// persistent wavefronts loop.  Lane l owns columns [512c + 8l, +8) of every chunk c, so each
// 16-byte load of the wavefront is a fully coalesced 1 KiB read.  The
// wavefront reads its slice once, keeps it in registers (quantised, for FP8)
// and then writes it to each of the token's k receive rows.  Measured at
// 8192 tokens x 7168 columns: two-chunk slices (7 wavefronts per token)
// against whole rows (1 per token), FP8 100.7 vs 106.3 us, BF16 185.3 vs
// 187.0, MXFP4 58.3 vs 60.6, and 280-281 vs 284-285 us for the whole
// layout + dispatch + combine step; a streaming probe with the same 1:4
// read:write mix likewise runs 8% faster with 2-4 KiB units per wavefront
// than with 16 KiB ones (more, smaller units keep more DRAM banks busy).
//
// FP8: a 128-column block is one 16-lane DPP row, so the block amax is four
// DPP max steps on the magnitude bits.  Neighbouring lanes swap halves of
// their quantised bytes (DPP quad_perm 1,0,3,2) so every lane stores 16
// bytes; the block scales are gathered into lanes 0..4*chunks-1 and stored
// as one contiguous run per receive row.
//
// Out-of-range columns are handled by raw buffer addressing: loads past the
// row return 0 and stores past it are dropped.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "ep_dispatch_device.hpp"

namespace ep {
namespace {

using namespace dsp;

constexpr int kMaxChunks = 16;     // most 512-column chunks a wavefront holds (8192 columns)
constexpr int kWavesPerBlock = 4;  // 256 threads (whole-GPU launches)

// Slices are handed out grid-stride: a whole-GPU launch has one wavefront per
// slice and runs the loop once; a launch limited to a CU budget runs that many
// persistent workgroups, each wavefront taking every (grid * WPB)-th
// slice.  The loop starts at workgroup index `blk`: the hardware index, or
// its XCD-contiguous renumbering (first_block, below).
#define EP_FOR_EACH_SLICE(WPB, total, wave, blk)                                     \
  for (int wave = uniform((blk) * (WPB) + (int)(threadIdx.x >> 6)); wave < (total); \
       wave += (int)gridDim.x * (WPB))

// xcd_contiguous (ep_device.hpp) gives XCD x one contiguous eighth of the
// slices instead of every eighth workgroup.  Measured at 8192 tokens x 7168
// in whole-GPU launches: FP8 93.2-93.7 vs 100.3-100.7 us, MXFP8 92.6 vs
// 100.4, MXFP4 55.7 vs 57.6, and FP8 at 4096 x 4096 x top-6 23.5 vs 24.1;
// runs of 16 to 256 workgroups per XCD instead of one eighth gain little or
// nothing.  It is applied to the formats with block scales in whole-GPU
// launches above the streaming threshold: BF16 dispatch (188.0 vs 188.4 us;
// 42.4 vs 41.5 at 4096 x 4096), combine (187.9 vs 175.3), decode-sized
// launches and CU-budget launches do not gain from it.
__device__ __forceinline__ int first_block(int xcd) {
  return xcd ? xcd_contiguous((int)blockIdx.x, (int)gridDim.x) : (int)blockIdx.x;
}

// NC: chunk capacity of the instantiation (>= chunks per wavefront).
template <int NC, int AUX_LD, int AUX_ST, bool SCALED, int WPB>
__global__ __launch_bounds__(64 * WPB) void dispatch_bf16_kernel(RowParams p, int wpt, int cpw, int nchunks) {
  const int lane = threadIdx.x & 63;
  EP_FOR_EACH_SLICE(WPB, p.T * wpt, wave, (int)blockIdx.x) {
    const Slice sl = slice_of(wave, wpt, cpw, nchunks);
    u32x4 v[NC];
    load_row<NC, AUX_LD>(p, sl, lane, v);
    store_bf16_row<NC, AUX_ST, SCALED>(p, sl, lane, v, load_lane_slot(p.slot, sl.t, p.k, lane));
  }
}

template <int NC, int AUX_LD, int AUX_ST, int WPB>
__global__ __launch_bounds__(64 * WPB) void dispatch_fp8_kernel(RowParams p, int wpt, int cpw, int nchunks,
                                                                int xcd) {
  const int lane = threadIdx.x & 63;
  EP_FOR_EACH_SLICE(WPB, p.T * wpt, wave, first_block(xcd)) {
    const Slice sl = slice_of(wave, wpt, cpw, nchunks);
    u32x4 v[NC];
    load_row<NC, AUX_LD>(p, sl, lane, v);
    store_fp8_row<NC, AUX_ST>(p, sl, lane, v, load_lane_slot(p.slot, sl.t, p.k, lane));
  }
}

// ---------------------------------------------------------------------------
// MX dispatch: OCP Microscaling blocks of 32 columns with one E8M0 scale.
// The 4-bit dispatch of DeepEP's Hybrid-EP branch (GeekNews "DeepSeek publica
// DeepEP ...", section "Ramas experimentales y forks de la comunidad") maps
// on MI355X to the MX formats its matrix cores read natively.  Per block:
// e = floor(log2 amax) - emax (clamped to [-127, 127]; an all-zero block gets
// -127), element = RNE(x * 2^-e) saturated to the element's largest normal,
// stored scale byte e + 127.  MXFP8 elements are E4M3 (emax 8), MXFP4 E2M1
// (emax 2, two per byte, the even column in the low nibble).
//
// A 32-column block is one lane quad (8 columns per lane), so the block amax
// is two DPP max steps.  For a BF16 amax with biased exponent E,
// floor(log2 amax) = E - 127 (E = 0, zero or subnormal, clamps to -127), so
// the scale byte is max(E - emax, 0) and 2^-e is built from its exponent
// bits; x * 2^-e is exact.
// ---------------------------------------------------------------------------

// E2M1 code of v (4 bits), nearest with ties to the even code, saturating at
// 6, sign kept.  The magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 are codes 0..7, so
// the code is the number of rounding thresholds |v| has passed; a threshold
// that is a tie counts as passed only when the upper code is even.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float m = fabsf(v);
  const uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
                     (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 0x8u);
}

// Maximum over each lane quad (one 32-column MX block).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  return v;
}

template <int ELEM>
struct MxFormat;
template <>
struct MxFormat<8> {
  static constexpr int kEmax = 8;
  static constexpr float kMaxNorm = 448.0f;
};
template <>
struct MxFormat<4> {
  static constexpr int kEmax = 2;
  static constexpr float kMaxNorm = 6.0f;
};

// ELEM 8: 8 E4M3 codes per lane and chunk (8 bytes); ELEM 4: 8 E2M1 codes
// (4 bytes).  The 16 scale bytes of a chunk are gathered into 4 dwords, and
// lane L < 4 * nc holds dword L % 4 of chunk L / 4, so one store per receive
// row writes the slice's scales as one contiguous run.
template <int NC, int AUX_LD, int AUX_ST, int WPB, int ELEM>
__global__ __launch_bounds__(64 * WPB) void dispatch_mx_kernel(RowParams p, int wpt, int cpw, int nchunks,
                                                               int xcd) {
  using F = MxFormat<ELEM>;
  const int lane = threadIdx.x & 63;
  EP_FOR_EACH_SLICE(WPB, p.T * wpt, wave, first_block(xcd)) {
  const Slice sl = slice_of(wave, wpt, cpw, nchunks);
  u32x4 v[NC];
  load_row<NC, AUX_LD>(p, sl, lane, v);
  const int slots = load_lane_slot(p.slot, sl.t, p.k, lane);

  uint32_t code[NC][ELEM == 8 ? 2 : 1];
  uint32_t sdw[NC];  // scale dword of lanes 0, 16, 32, 48: quads 4r .. 4r+3 of the chunk
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t E = quad_max_u32(absmax_bits8(v[c])) >> 7;           // biased exponent of the block amax
    const uint32_t sbyte = E > (uint32_t)F::kEmax ? E - F::kEmax : 0u;  // e + 127
    const float inv = __uint_as_float((254u - sbyte) << 23);             // 2^-e
    float q[8];
    q[0] = bf16_lo(v[c].x) * inv; q[1] = bf16_hi(v[c].x) * inv;
    q[2] = bf16_lo(v[c].y) * inv; q[3] = bf16_hi(v[c].y) * inv;
    q[4] = bf16_lo(v[c].z) * inv; q[5] = bf16_hi(v[c].z) * inv;
    q[6] = bf16_lo(v[c].w) * inv; q[7] = bf16_hi(v[c].w) * inv;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(q[i], -F::kMaxNorm), F::kMaxNorm);
    if constexpr (ELEM == 8) {
      code[c][0] = pack_e4m3x4(q[0], q[1], q[2], q[3]);
      code[c][1] = pack_e4m3x4(q[4], q[5], q[6], q[7]);
    } else {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= e2m1_code(q[i]) << (4 * i);
      code[c][0] = w;
    }
    // scale bytes of quads 4r..4r+3 into lane 16r (every lane of a quad holds its byte)
    const uint32_t b1 = (uint32_t)__shfl((int)sbyte, lane + 4, 64);
    const uint32_t b2 = (uint32_t)__shfl((int)sbyte, lane + 8, 64);
    const uint32_t b3 = (uint32_t)__shfl((int)sbyte, lane + 12, 64);
    sdw[c] = sbyte | (b1 << 8) | (b2 << 16) | (b3 << 24);
  }
  uint32_t my_sdw = 0;
  const int owner = (lane & 3) << 4;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t g = (uint32_t)__shfl((int)sdw[c], owner, 64);
    if ((lane >> 2) == c) my_sdw = g;
  }

  const int H = p.H, nb = H >> 5;
  const uint32_t row_bytes = ELEM == 8 ? (uint32_t)H : (uint32_t)H / 2u;
  const uint32_t ocol = (uint32_t)(sl.c0 * 512 + lane * 8) * (uint32_t)ELEM / 8u;
  const uint32_t chunk_bytes = 512u * (uint32_t)ELEM / 8u;
  const uint32_t scol = (uint32_t)(sl.c0 * 16 + lane * 4);
  uint8_t* dst = static_cast<uint8_t*>(p.dst);
  uint8_t* sdst = static_cast<uint8_t*>(p.recv_scale);
  for (int j = 0; j < p.k; ++j) {
    const int s = __builtin_amdgcn_readlane(slots, j);
    if (!slot_ok(s, p.rows)) continue;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + (int64_t)s * row_bytes, row_bytes);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c >= sl.nc) continue;
      if constexpr (ELEM == 8) {
        u32x2 w2 = {code[c][0], code[c][1]};
        store8<AUX_ST>(rd, ocol + chunk_bytes * c, w2);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(code[c][0], rd, (int)(ocol + chunk_bytes * c), 0, AUX_ST);
      }
    }
    if (lane < 4 * sl.nc) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(sdst + (int64_t)s * nb, (uint32_t)nb);
      // through the caches, as the FP8 scales (partial lines of neighbouring rows merge there)
      if (scol + 4u <= (uint32_t)nb) {
        __builtin_amdgcn_raw_buffer_store_b32(my_sdw, rs, (int)scol, 0, kAuxDefault);
      } else {
        // the row's last scales when H / 32 is not a multiple of 4: a dword
        // reaching past the row would be dropped whole by the range check,
        // so store byte by byte (bytes past the row are dropped)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(my_sdw >> (8 * b)), rs, (int)scol + b, 0, kAuxDefault);
      }
    }
  }
  }
}

// ---------------------------------------------------------------------------
// Pre-quantised FP8 dispatch: DeepEP's dispatch also takes FP8 input as a
// (data, scale factors) pair (DeepEP documentation item 10).  The caller's
// E4M3 codes [T, H] and fp32 scales [T, H/128] go to every valid slot as
// they are: a byte scatter.  The launch treats a code row as H/2 two-byte
// columns, so a 512-column chunk here is 1024 code bytes (16 per lane) and
// carries 8 block scales.
// ---------------------------------------------------------------------------
template <int NC, int AUX_LD, int AUX_ST, int WPB>
__global__ __launch_bounds__(64 * WPB) void dispatch_prequantized_kernel(RowParams p, int wpt, int cpw,
                                                                         int nchunks, int xcd) {
  const int lane = threadIdx.x & 63;
  EP_FOR_EACH_SLICE(WPB, p.T * wpt, wave, first_block(xcd)) {
  const Slice sl = slice_of(wave, wpt, cpw, nchunks);
  u32x4 v[NC];
  load_row<NC, AUX_LD>(p, sl, lane, v);  // p.H counts two-byte columns
  const int slots = load_lane_slot(p.slot, sl.t, p.k, lane);
  const int nb = p.H >> 6;               // scales per row: (2 H) / 128
  const int sc0 = sl.c0 * 8, nsc = min(8 * sl.nc, nb - sc0);
  // lane L holds scales sc0 + L and sc0 + 64 + L of the slice (8 per chunk)
  const __amdgpu_buffer_rsrc_t rsi = make_rsrc(p.src_scale + (int64_t)sl.t * nb, (uint32_t)nb * 4u);
  uint32_t scale[NC > 8 ? 2 : 1];
#pragma unroll
  for (int m = 0; m < (NC > 8 ? 2 : 1); ++m) {
    const int i = 64 * m + lane;
    scale[m] = __builtin_amdgcn_raw_buffer_load_b32(rsi, i < nsc ? (int)((sc0 + i) * 4) : (int)kNoColumn, 0, 0);
  }

  uint8_t* dst = static_cast<uint8_t*>(p.dst);
  float* sdst = static_cast<float*>(p.recv_scale);
  const uint32_t row_bytes = (uint32_t)p.H * 2u;
  const uint32_t col = (uint32_t)(sl.c0 * 512 + lane * 8) * 2u;
  for (int j = 0; j < p.k; ++j) {
    const int s = __builtin_amdgcn_readlane(slots, j);
    if (!slot_ok(s, p.rows)) continue;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + (int64_t)s * row_bytes, row_bytes);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (c < sl.nc) store16<AUX_ST>(rd, col + 1024u * c, v[c]);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sdst + (int64_t)s * nb, (uint32_t)nb * 4u);
#pragma unroll
    for (int m = 0; m < (NC > 8 ? 2 : 1); ++m) {
      const int i = 64 * m + lane;
      if (i < nsc) __builtin_amdgcn_raw_buffer_store_b32(scale[m], rs, (sc0 + i) * 4, 0, kAuxDefault);
    }
  }
  }
}

#undef EP_FOR_EACH_SLICE

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

__global__ __launch_bounds__(256) void check_quant_e4m3_kernel(const uint16_t* x, const float* sc, uint8_t* out,
                                                               int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 v = {(uint32_t)x[i], 0u, 0u, 0u};  // the value in the low half of the first dword
    out[i] = (uint8_t)quantize8(v, sc[i]).x;
  }
}

__global__ __launch_bounds__(256) void check_cvt_e2m1_kernel(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (uint8_t)e2m1_code(in[i]);
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


}  // namespace

namespace {

template <int NC, bool SCALED, int WPB>
void launch_bf16_ncsw(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  if (streaming)
    hipLaunchKernelGGL((dispatch_bf16_kernel<NC, kAuxDefault, kAuxNT, SCALED, WPB>), dim3(s.blocks), dim3(64 * WPB),
                       0, stream, p, s.wpt, s.cpw, s.nchunks);
  else
    hipLaunchKernelGGL((dispatch_bf16_kernel<NC, kAuxDefault, kAuxSmallStore, SCALED, WPB>), dim3(s.blocks),
                       dim3(64 * WPB), 0, stream, p, s.wpt, s.cpw, s.nchunks);
}

template <int NC, bool SCALED>
void launch_bf16_ncs(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  if (s.budget)
    launch_bf16_ncsw<NC, SCALED, kBudgetWaves>(s, p, streaming, stream);
  else
    launch_bf16_ncsw<NC, SCALED, kWavesPerBlock>(s, p, streaming, stream);
}

template <int NC>
void launch_bf16_nc(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  if (p.weights)
    launch_bf16_ncs<NC, true>(s, p, streaming, stream);
  else
    launch_bf16_ncs<NC, false>(s, p, streaming, stream);
}

template <int NC, int WPB>
void launch_fp8_ncw(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  if (streaming)
    hipLaunchKernelGGL((dispatch_fp8_kernel<NC, kAuxDefault, kAuxNT, WPB>), dim3(s.blocks), dim3(64 * WPB), 0, stream,
                       p, s.wpt, s.cpw, s.nchunks, (int)!s.budget);
  else
    hipLaunchKernelGGL((dispatch_fp8_kernel<NC, kAuxDefault, kAuxSmallStore, WPB>), dim3(s.blocks), dim3(64 * WPB), 0,
                       stream, p, s.wpt, s.cpw, s.nchunks, 0);
}

template <int NC, int WPB, int ELEM>
void launch_mx_ncw(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  if (streaming)
    hipLaunchKernelGGL((dispatch_mx_kernel<NC, kAuxDefault, kAuxNT, WPB, ELEM>), dim3(s.blocks), dim3(64 * WPB), 0,
                       stream, p, s.wpt, s.cpw, s.nchunks, (int)!s.budget);
  else
    hipLaunchKernelGGL((dispatch_mx_kernel<NC, kAuxDefault, kAuxSmallStore, WPB, ELEM>), dim3(s.blocks),
                       dim3(64 * WPB), 0, stream, p, s.wpt, s.cpw, s.nchunks, 0);
}

template <int NC, int ELEM>
void launch_mx_nce(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  if (s.budget)
    launch_mx_ncw<NC, kBudgetWaves, ELEM>(s, p, streaming, stream);
  else
    launch_mx_ncw<NC, kWavesPerBlock, ELEM>(s, p, streaming, stream);
}

template <int NC>
void launch_mx8_nc(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  launch_mx_nce<NC, 8>(s, p, streaming, stream);
}

template <int NC>
void launch_mx4_nc(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  launch_mx_nce<NC, 4>(s, p, streaming, stream);
}

template <int NC, int WPB>
void launch_pq_ncw(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  if (streaming)
    hipLaunchKernelGGL((dispatch_prequantized_kernel<NC, kAuxDefault, kAuxNT, WPB>), dim3(s.blocks), dim3(64 * WPB),
                       0, stream, p, s.wpt, s.cpw, s.nchunks, (int)!s.budget);
  else
    hipLaunchKernelGGL((dispatch_prequantized_kernel<NC, kAuxDefault, kAuxSmallStore, WPB>), dim3(s.blocks),
                       dim3(64 * WPB), 0, stream, p, s.wpt, s.cpw, s.nchunks, 0);
}

template <int NC>
void launch_pq_nc(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  if (s.budget)
    launch_pq_ncw<NC, kBudgetWaves>(s, p, streaming, stream);
  else
    launch_pq_ncw<NC, kWavesPerBlock>(s, p, streaming, stream);
}

template <int NC>
void launch_fp8_nc(const DispatchSplit& s, const RowParams& p, bool streaming, hipStream_t stream) {
  if (s.budget)
    launch_fp8_ncw<NC, kBudgetWaves>(s, p, streaming, stream);
  else
    launch_fp8_ncw<NC, kWavesPerBlock>(s, p, streaming, stream);
}

}  // namespace

DispatchSplit dispatch_split(const RowParams& p) {
  DispatchSplit s;
  s.nchunks = (p.H + 511) / 512;
  s.budget = p.num_cus > 0;
  // Whole-GPU launch: two-chunk slices.  Budget: whole rows per wavefront
  // (measured at 8192 tokens: 278 vs 373 us with two-chunk slices at 32 CUs,
  // 149 vs 189 at 64), unless the batch is too small to give every wavefront
  // of the budget some work; then rows split into 2-chunk slices.
  const int min_wpt = (s.nchunks + kMaxChunks - 1) / kMaxChunks;
  if (s.budget) {
    const int want_wpt = (p.num_cus * kBudgetWaves + p.T - 1) / p.T;
    s.wpt = max(min_wpt, min(want_wpt, (s.nchunks + 1) / 2));
  } else {
    s.wpt = max(min_wpt, (s.nchunks + 1) / 2);
  }
  s.cpw = (s.nchunks + s.wpt - 1) / s.wpt;
  s.cpw += s.cpw & 1;
  s.wpt = (s.nchunks + s.cpw - 1) / s.cpw;
  const int64_t waves = (int64_t)p.T * s.wpt;
  if (s.budget) {
    const int64_t need = (waves + kBudgetWaves - 1) / kBudgetWaves;
    s.blocks = (int)(need < p.num_cus ? need : p.num_cus);
  } else {
    s.blocks = (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
  }
  return s;
}

// The instantiation's chunk capacity equals the (even) chunks per wavefront,
// so no slice carries dead registers or instructions.
#define EP_BY_CAPACITY(FN, s, ...)                  \
  switch (s.cpw) {                                  \
    case 2: FN<2>(s, __VA_ARGS__); break;           \
    case 4: FN<4>(s, __VA_ARGS__); break;           \
    case 6: FN<6>(s, __VA_ARGS__); break;           \
    case 8: FN<8>(s, __VA_ARGS__); break;           \
    case 10: FN<10>(s, __VA_ARGS__); break;         \
    case 12: FN<12>(s, __VA_ARGS__); break;         \
    case 14: FN<14>(s, __VA_ARGS__); break;         \
    default: FN<16>(s, __VA_ARGS__); break;         \
  }

hipError_t launch_dispatch_bf16(const RowParams& p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  DispatchSplit s = dispatch_split(p);
  const bool streaming = (int64_t)p.T * p.k * p.H * 2 >= kStreamingBytes;
  if (!s.budget) {
    // BF16 copies have no 128-column blocks to pair up: a whole-GPU launch
    // takes one-chunk slices (512 columns, 1 KiB per copy).  Measured against
    // two-chunk slices: 184.7 vs 188.9 us at 8192 tokens x 7168 x top-8,
    // 39.8 vs 41.6 at 4096 x 4096 x top-6.
    s.cpw = 1;
    s.wpt = s.nchunks;
    s.blocks = (int)(((int64_t)p.T * s.wpt + kWavesPerBlock - 1) / kWavesPerBlock);
    launch_bf16_nc<1>(s, p, streaming, stream);
    return hipGetLastError();
  }
  EP_BY_CAPACITY(launch_bf16_nc, s, p, streaming, stream);
  return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const RowParams& p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const DispatchSplit s = dispatch_split(p);
  const bool streaming = (int64_t)p.T * p.k * p.H >= kStreamingBytes;
  EP_BY_CAPACITY(launch_fp8_nc, s, p, streaming, stream);
  return hipGetLastError();
}

hipError_t launch_dispatch_mx(const RowParams& p, int elem_bits, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const DispatchSplit s = dispatch_split(p);
  const bool streaming = (int64_t)p.T * p.k * p.H * elem_bits / 8 >= kStreamingBytes;
  if (elem_bits == 8) {
    EP_BY_CAPACITY(launch_mx8_nc, s, p, streaming, stream);
  } else {
    EP_BY_CAPACITY(launch_mx4_nc, s, p, streaming, stream);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch_prequantized(const RowParams& p_in, hipStream_t stream) {
  if (p_in.T == 0) return hipSuccess;
  RowParams p = p_in;
  p.H = p_in.H / 2;  // code rows as two-byte columns
  const DispatchSplit s = dispatch_split(p);
  const bool streaming = (int64_t)p.T * p.k * p_in.H >= kStreamingBytes;
  EP_BY_CAPACITY(launch_pq_nc, s, p, streaming, stream);
  return hipGetLastError();
}

#undef EP_BY_CAPACITY

hipError_t launch_check_cvt_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 1023) / 1024;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(check_cvt_e4m3_kernel, dim3(blocks), dim3(256), 0, stream, in, out, n);
  return hipGetLastError();
}

hipError_t launch_check_quant_e4m3(const uint16_t* x, const float* s, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(check_quant_e4m3_kernel, dim3(blocks), dim3(256), 0, stream, x, s, out, n);
  return hipGetLastError();
}

hipError_t launch_check_cvt_e2m1(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(check_cvt_e2m1_kernel, dim3(blocks), dim3(256), 0, stream, in, out, n);
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
