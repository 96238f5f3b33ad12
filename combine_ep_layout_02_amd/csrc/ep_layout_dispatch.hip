// Layout fused into dispatch, for batches whose pairs fit one layout tile
// (at most 1024 pairs: the decode shape, e.g. 128 tokens x top-8).
//
// The layout is the routing metadata dispatch needs; the decode path re-runs
// it every step, and DeepEP's low-latency path is built to keep exactly this
// step cheap (DeepEP documentation item 3; GeekNews "DeepSeek publica DeepEP
// ...", section "Patrones de uso en entrenamiento, prefill y decoding").  One
// tile's layout is a few microseconds of LDS work for one workgroup, so
// every workgroup of the dispatch recomputes it instead of waiting for a
// separate layout launch and reading the slots back from memory:
//   1. each wavefront issues the loads of its token slice (x does not depend
//      on the layout), so they are in flight during steps 2-3;
//   2. the workgroup's 1024 threads run the tile pass and the offset scan of
//      ep_layout (ep_layout_device.hpp) and keep every pair's slot in LDS;
//   3. workgroup 0 writes the layout outputs exactly as ep_layout does, and
//      all workgroups share the src_pair padding rows;
//   4. each wavefront writes its slice's copies (BF16 or FP8) to the slots
//      read from LDS, with the dispatch kernels' row code
//      (ep_dispatch_device.hpp).
// Results are bit-identical to ep_layout followed by ep_dispatch.
#include <algorithm>

#include "ep_device.hpp"
#include "ep_dispatch_device.hpp"
#include "ep_internal.hpp"
#include "ep_layout_device.hpp"

namespace ep {
namespace {

using namespace lay;
using namespace dsp;

constexpr int kW = 16;  // layout windows per tile = wavefronts per workgroup (1024 threads)
// Wavefronts per workgroup that also dispatch.  All 16 build the layout;
// giving only 4 of them a slice spreads the dispatch over 4x more CUs (the
// quantisation is ALU work that 16 slices on one CU serialise): measured at
// 128 tokens x top-8, 9.2 us per fused call with 16, 8.1 with 8, 7.5 with 4,
// 8.4 with 2.
constexpr int kD = 4;

// One workgroup of kW wavefronts; wavefront w < kD of workgroup b takes
// dispatch slice b * kD + w (at most one each).
template <int NC, bool FP8>
__global__ __launch_bounds__(64 * kW) void layout_dispatch_kernel(LayoutParams lp, RowParams rp, int wpt, int cpw,
                                                                  int nchunks) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_bad;
  __shared__ int s_part[20];
  const TileLds<kW> L(smem, lp.E, lp.R);
  const int tid = threadIdx.x, lane = tid & 63, nthr = 64 * kW;
  const int wave = uniform(tid >> 6);

  // 1. this wavefront's slice: start its loads now
  const int sidx = uniform((int)blockIdx.x * kD + wave);
  const bool has = wave < kD && sidx < rp.T * wpt;
  const Slice sl = slice_of(has ? sidx : 0, wpt, cpw, nchunks);
  u32x4 v[NC];
  if (has) load_row<NC, kAuxDefault>(rp, sl, lane, v);

  // 2. the tile's layout in LDS (one pair per thread)
  int e, local;
  tile_pass<kW>(lp, L, 0, &s_bad, e, local);
  const bool lead = blockIdx.x == 0;
  if (lead && tid == 0 && lp.diag) { lp.diag[0] = s_bad; lp.diag[1] = 0; }
  scan_offsets(L.cnt_s, L.offs, lp.E, lp.A, lp.C, s_part);  // barrier: diag[1] is zero before the adds
  const int np = lp.T * lp.k;
  int s = -1;
  if (tid < np && e >= 0) s = slot_of(lp, e, local, L.offs);
  int* slot_s = L.idx_s;  // the tile pass is done with idx_s: reuse it for the slots
  slot_s[tid] = s;

  // 3. the layout outputs
  if (lead) {
    write_outputs(lp, L.cnt_s, L.offs, L.rank_hist);
    if (tid < np) {
      if (s >= 0 && lp.src_pair) lp.src_pair[s] = tid;
      lp.slot[tid] = s;
    }
  }
  fill_padding_rows(lp, L.cnt_s, L.offs, (int)blockIdx.x * kW + wave, (int)gridDim.x * kW, lane,
                    (int64_t)blockIdx.x * nthr + tid, (int64_t)gridDim.x * nthr);
  __syncthreads();  // slot_s complete

  // 4. the slice's copies
  if (has) {
    const int slots = lane < rp.k ? slot_s[sl.t * rp.k + lane] : -1;
    if constexpr (FP8)
      store_fp8_row<NC, kAuxDefault>(rp, sl, lane, v, slots);
    else
      store_bf16_row<NC, kAuxDefault, false>(rp, sl, lane, v, slots);
  }
}

template <int NC, bool FP8>
void launch_nc(int blocks, size_t lds, const LayoutParams& lp, const RowParams& rp, int wpt, int cpw, int nchunks,
               hipStream_t stream) {
  hipLaunchKernelGGL((layout_dispatch_kernel<NC, FP8>), dim3(blocks), dim3(64 * kW), lds, stream, lp, rp, wpt, cpw,
                     nchunks);
}

template <bool FP8>
void launch_fp(int cpw, int blocks, size_t lds, const LayoutParams& lp, const RowParams& rp, int wpt, int nchunks,
               hipStream_t stream) {
  switch (cpw) {
    case 2: launch_nc<2, FP8>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 4: launch_nc<4, FP8>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 6: launch_nc<6, FP8>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 8: launch_nc<8, FP8>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 10: launch_nc<10, FP8>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 12: launch_nc<12, FP8>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 14: launch_nc<14, FP8>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    default: launch_nc<16, FP8>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
  }
}

}  // namespace

bool layout_dispatch_fusable(const LayoutPlan& pl) { return pl.ntiles == 1 && pl.W == kW; }

hipError_t launch_layout_dispatch(const LayoutPlan& pl, LayoutParams lp, const RowParams& rp, bool fp8,
                                  hipStream_t stream) {
  prepare_layout_params(pl, lp);
  const DispatchSplit s = dispatch_split(rp);  // rp.num_cus is 0 here: one wavefront per slice
  const int64_t slices = (int64_t)rp.T * s.wpt;
  const int blocks = (int)std::max<int64_t>(1, (slices + kD - 1) / kD);
  if (fp8)
    launch_fp<true>(s.cpw, blocks, pl.lds_bytes, lp, rp, s.wpt, s.nchunks, stream);
  else
    launch_fp<false>(s.cpw, blocks, pl.lds_bytes, lp, rp, s.wpt, s.nchunks, stream);
  return hipGetLastError();
}

}  // namespace ep
