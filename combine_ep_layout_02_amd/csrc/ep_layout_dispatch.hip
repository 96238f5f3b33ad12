// Layout fused into dispatch, for batches of at most 1024 pairs (the decode
// shape, e.g. 128 tokens x top-8).
//
// The layout is the routing metadata dispatch needs; the decode path re-runs
// it every step, and DeepEP's low-latency path is built to keep exactly this
// step cheap (DeepEP documentation item 3; GeekNews "DeepSeek publica DeepEP
// ...", section "Patrones de uso en entrenamiento, prefill y decoding").
// Rather than wait for a separate layout launch and read the slots back from
// memory, the dispatch works them out itself.  Two forms; both give results
// bit-identical to ep_layout followed by ep_dispatch.
//
// Direct form (flat layouts with expert_alignment 1, and padded layouts).
// Each receive row then has a closed form in the ids: for pair (t, j) of
// expert e,
//   flat:   slot = #{valid pairs with id < e} + #{pairs before (t, j) with id e}
//   padded: pos  = #{pairs before (t, j) with id e},  slot = e*C + pos if pos < C
// ("before" in (token, k-index) order: the stable counting sort).  Each
// workgroup of 4 wavefronts stages the batch's ids in LDS once (16 per lane
// of each wavefront); after that no wavefront waits for another:
//   * dispatch wavefronts (one per token slice) issue the loads of their row,
//     count their token's k slots with a small LDS histogram of their own
//     (atomic adds, order independent), write the token's slot / src_pair
//     entries (first slice only) and store the row's copies with the
//     dispatch kernels' row code (ep_dispatch_device.hpp);
//   * job wavefronts after them take the other outputs, each a count over
//     the ids: one job per expert (its count, offset, the rank offset it
//     starts, its padding rows), one per rank (distinct tokens, through a
//     token bit set in LDS) and one for the totals (offset end, diag, the
//     flat layout's tail rows).
//
// Tile form (expert_alignment > 1, whose offsets need every expert's
// rounded-up count): every workgroup of 16 wavefronts rebuilds the one-tile
// layout in LDS with the tile pass and offset scan of ep_layout
// (ep_layout_device.hpp) while 4 of its wavefronts have their row loads in
// flight; workgroup 0 writes the layout outputs and all share the padding
// rows; the 4 wavefronts then store their copies to the slots held in LDS.
#include <algorithm>

#include "ep_device.hpp"
#include "ep_dispatch_device.hpp"
#include "ep_internal.hpp"
#include "ep_layout_device.hpp"

namespace ep {
namespace {

using namespace lay;
using namespace dsp;

constexpr int kMaxPairs = 1024;         // pairs a fused batch may hold
constexpr int kIds = kMaxPairs / 64;    // ids per lane in the direct form

// ---------------------------------------------------------------------------
// direct form
// ---------------------------------------------------------------------------

constexpr int kDirectWaves = 4;  // wavefronts per workgroup
static_assert(4 * 64 * kDirectWaves == kMaxPairs, "each thread stages four ids");
// LDS a direct-form workgroup may take for its wavefronts' histograms;
// larger expert counts take the other paths.
constexpr size_t kDirectLdsMax = 32768;

// Staged ids: the expert id when valid, else one of two markers above any
// expert id.
constexpr uint32_t kMasked = 0xFFFFFFFFu;  // -1, or past the batch's pairs
constexpr uint32_t kBad = 0xFFFFFFFEu;     // neither -1 nor in [0, E)

// Histogram ints per wavefront (a multiple of 4, for 16-byte accesses):
// padded layout, E (pairs ahead of the token per expert); flat, 2E (pairs
// per key, below).
__host__ __device__ constexpr int direct_hist_ints(int E, bool padded) { return ((padded ? E : 2 * E) + 3) & ~3; }

// Orders LDS accesses of different lanes of one wavefront (a wavefront's LDS
// operations complete in issue order; this keeps the compiler from moving
// them across the point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Wave-uniform sum of an int over the 64 lanes: DPP sums within each 16-lane
// row, then the four row sums.
__device__ __forceinline__ int wave_sum_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}

// The batch's ids are staged in LDS once per workgroup, four per thread,
// already classified: were every wavefront to read the same few KB from L2,
// its requests would queue on the few L2 channels that hold them.
// stage_load issues the loads before a wavefront's row loads, so that
// waiting for the ids does not wait for the row; stage_commit writes them
// and ends with a barrier.
struct Staged {
  uint32_t raw[4];
};

__device__ __forceinline__ void stage_load(const LayoutParams& p, int np, Staged& s) {
  const int q0 = 4 * (int)threadIdx.x;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // unconditional loads (clamped into the batch), so that the wait for
    // them is a count of the loads issued after them
    const uint32_t raw = (uint32_t)p.idx[min(q0 + c, np - 1)];
    s.raw[c] = q0 + c < np ? raw : kMasked;
  }
}

__device__ __forceinline__ void stage_commit(const LayoutParams& p, const Staged& s, uint32_t* ids_s) {
  uint32_t u[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) u[c] = s.raw[c] < (uint32_t)p.E ? s.raw[c] : s.raw[c] == kMasked ? kMasked : kBad;
  *reinterpret_cast<u32x4*>(&ids_s[4 * threadIdx.x]) = u32x4{u[0], u[1], u[2], u[3]};
  // A workgroup barrier ordering LDS only: __syncthreads() would also wait
  // for the wavefront's row loads still in flight.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A wavefront's copy of the staged ids: element i of lane l holds pair
// 256*(i/4) + 4*l + i%4.
struct Ids {
  uint32_t u[kIds];
};

__device__ __forceinline__ int pair_of(int i, int lane) { return 256 * (i >> 2) + 4 * lane + (i & 3); }

__device__ __forceinline__ void load_ids(const uint32_t* ids_s, int lane, Ids& ids) {
#pragma unroll
  for (int m = 0; m < kIds / 4; ++m) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(&ids_s[256 * m + 4 * lane]);
    ids.u[4 * m] = v.x;
    ids.u[4 * m + 1] = v.y;
    ids.u[4 * m + 2] = v.z;
    ids.u[4 * m + 3] = v.w;
  }
}

// Wave-uniform number of pairs whose element satisfies pred (elements past
// the batch hold kMasked, which no caller's test counts).  Each lane counts
// its own elements with independent vector compares and adds (a ballot per
// element would chain every compare to a scalar popcount), then one
// reduction sums the lanes.
template <typename Pred>
__device__ __forceinline__ int count_ids(Pred pred) {
  int c = 0;
#pragma unroll
  for (int i = 0; i < kIds; ++i) c += pred(i) ? 1 : 0;
  return wave_sum_i(c);
}

// Zeroes n ints (a multiple of 4) of this wavefront's LDS, then syncs.
__device__ __forceinline__ void wave_clear_lds(int* h, int n, int lane) {
  for (int e = 4 * lane; e < n; e += 256) *reinterpret_cast<u32x4*>(&h[e]) = u32x4{0u, 0u, 0u, 0u};
  wave_lds_sync();
}

// Exclusive prefix sum, in place, of h[0..n) in this wavefront's LDS: each
// lane sums a run of entries, one wavefront scan, then each lane rewrites
// its run.  Ends synchronised.
__device__ void wave_exclusive_scan_lds(int* h, int n, int lane) {
  const int per = (n + 63) >> 6;
  const int lo = min(n, lane * per), hi = min(n, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += h[e];
  int run = wave_inclusive_scan(sum) - sum;
  for (int e = lo; e < hi; ++e) {
    const int c = h[e];
    h[e] = run;
    run += c;
  }
  wave_lds_sync();
}

// Slots of token t's pairs, slot[t, j] in lane j (-1 in lanes >= k); lane_e
// holds the lane's own pair's staged id (lanes < k).  h: this wavefront's
// histogram LDS.  Counts are LDS atomic adds, which are order independent
// (an element that counts nothing adds 0 to entry 0, so no lane branches):
//   padded: h[e] = pairs of expert e ahead of the token; pos = h[e] + the
//           token's own earlier pairs of e; slot = e*C + pos if pos < C
//   flat:   h[2e + (pair at or after the token)] = pairs per key; after an
//           exclusive scan h[2e + 1] = valid pairs with id < e + pairs of e
//           ahead of the token; slot = h[2e + 1] + the token's own earlier
//           pairs of e
template <bool PADDED>
__device__ __forceinline__ int token_slots(const LayoutParams& p, const Ids& ids, uint32_t lane_e, int t, int lane,
                                           int* h) {
  const uint32_t E = (uint32_t)p.E;
  const int tk = t * p.k;
  wave_clear_lds(h, direct_hist_ints(p.E, PADDED), lane);
#pragma unroll
  for (int i = 0; i < kIds; ++i) {
    const uint32_t e = ids.u[i];
    const bool valid = e < E;
    const bool ahead = pair_of(i, lane) < tk;
    if constexpr (PADDED) {
      if (256 * (i >> 2) < tk) atomicAdd(&h[valid ? e : 0u], valid && ahead ? 1 : 0);  // wave-uniform test
    } else {
      atomicAdd(&h[valid ? 2u * e + (ahead ? 0u : 1u) : 0u], valid ? 1 : 0);
    }
  }
  wave_lds_sync();
  if (!PADDED) wave_exclusive_scan_lds(h, 2 * p.E, lane);
  int own_before = 0;
  for (int j = 0; j < p.k; ++j) {
    const uint32_t ej = (uint32_t)__builtin_amdgcn_readlane((int)lane_e, j);
    own_before += (j < lane && ej == lane_e) ? 1 : 0;
  }
  if (lane_e >= E) return -1;
  if constexpr (PADDED) {
    const int pos = h[lane_e] + own_before;
    return pos < p.C ? (int)lane_e * p.C + pos : -1;
  }
  return h[2u * lane_e + 1u] + own_before;
}

// Job q of the layout outputs: q < E expert q, q < E + R rank q - E, else the
// totals.  bits: this wavefront's 32-word token set; h: this wavefront's
// histogram LDS (the totals job of a padded layout with diag uses it).
template <bool PADDED>
__device__ void layout_job(const LayoutParams& p, const Ids& ids, int q, int lane, uint32_t* bits, int* h) {
  const int E = p.E, R = p.R, C = p.C, per = E / R;
  if (q < E) {
    const uint32_t e = (uint32_t)q;
    const int cnt = count_ids([&](int i) { return ids.u[i] == e; });
    const int off = PADDED ? q * C : count_ids([&](int i) { return ids.u[i] < e; });
    if (lane == 0) {
      p.expert_count[q] = cnt;
      p.expert_offset[q] = off;
    }
    const int r = udiv(e, p.magic_per);
    if (lane == 0 && r * per == q) p.rank_offset[r] = off;
    if (PADDED && p.src_pair)
      for (int row = q * C + min(cnt, C) + lane; row < (q + 1) * C; row += 64) p.src_pair[row] = -1;
    return;
  }
  if (q < E + R) {
    // distinct tokens with a pair on rank r: a bit per token, set by its pairs
    const int r = q - E;
    const uint32_t lo = (uint32_t)(r * per);
    const int words = (p.T + 31) >> 5;
    if (lane < words) bits[lane] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < kIds; ++i) {
      if (ids.u[i] - lo < (uint32_t)per) {  // the markers lie above every rank's range
        const int t = udiv((uint32_t)pair_of(i, lane), p.magic_k);
        atomicOr(&bits[t >> 5], 1u << (t & 31));
      }
    }
    wave_lds_sync();
    const int n = wave_sum_i(lane < words ? (int)__popc(bits[lane]) : 0);
    if (lane == 0) p.rank_count[r] = n;
    return;
  }
  // totals
  const int nvalid = count_ids([&](int i) { return ids.u[i] < (uint32_t)E; });
  const int end = PADDED ? E * C : nvalid;
  if (lane == 0) {
    p.expert_offset[E] = end;
    p.rank_offset[R] = end;
  }
  if (p.diag) {
    const int nbad = count_ids([&](int i) { return ids.u[i] == kBad; });
    int drop = 0;
    if constexpr (PADDED) {
      // pairs past their expert's capacity: sum over experts of (count - C)+
      wave_clear_lds(h, direct_hist_ints(E, true), lane);
#pragma unroll
      for (int i = 0; i < kIds; ++i) {
        const bool valid = ids.u[i] < (uint32_t)E;
        atomicAdd(&h[valid ? ids.u[i] : 0u], valid ? 1 : 0);
      }
      wave_lds_sync();
      int d = 0;
      for (int e = lane; e < E; e += 64) d += max(0, h[e] - C);
      drop = wave_sum_i(d);
    }
    if (lane == 0) {
      p.diag[0] = nbad;
      p.diag[1] = drop;
    }
  }
  // flat layout: rows past the last pair (one per masked or invalid pair)
  if (!PADDED && p.src_pair)
    for (int64_t row = (int64_t)nvalid + lane; row < p.rows; row += 64) p.src_pair[row] = -1;
}

// Wavefront gw < slices takes dispatch slice gw; the next E + R + 1 take the
// layout jobs.
template <int NC, bool FP8, bool PADDED>
__global__ __launch_bounds__(64 * kDirectWaves) void layout_dispatch_direct_kernel(LayoutParams lp, RowParams rp,
                                                                                    int wpt, int cpw, int nchunks) {
  extern __shared__ __align__(16) int lds_h[];  // per wavefront: direct_hist_ints(E, PADDED)
  __shared__ __align__(16) uint32_t ids_s[kMaxPairs];
  __shared__ uint32_t bits[kDirectWaves][32];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int gw = uniform((int)blockIdx.x * kDirectWaves + wave);
  const int slices = rp.T * wpt;
  const int np = lp.T * lp.k;
  int* h = lds_h + (size_t)wave * direct_hist_ints(lp.E, PADDED);

  // ids first, then a dispatch wavefront's row (x does not depend on the layout)
  Staged st;
  stage_load(lp, np, st);
  const bool dispatching = gw < slices;
  Slice sl = slice_of(dispatching ? gw : 0, wpt, cpw, nchunks);
  if (!dispatching) sl.nc = 0;  // its loads fall outside the row and read nothing
  u32x4 v[NC];
  load_row<NC, kAuxDefault>(rp, sl, lane, v);  // unconditional: the wait for the ids counts past it
  stage_commit(lp, st, ids_s);
  Ids ids;
  load_ids(ids_s, lane, ids);
  if (!dispatching) {
    const int q = gw - slices;
    if (q <= lp.E + lp.R) layout_job<PADDED>(lp, ids, q, lane, bits[wave], h);
    return;
  }

  const int tk = sl.t * lp.k;
  const uint32_t lane_e = lane < lp.k ? ids_s[tk + lane] : kMasked;
  const int slots = token_slots<PADDED>(lp, ids, lane_e, sl.t, lane, h);
  if (sl.c0 == 0 && lane < lp.k) {
    lp.slot[tk + lane] = slots;
    if (slots >= 0 && lp.src_pair) lp.src_pair[slots] = tk + lane;
  }
  if constexpr (FP8)
    store_fp8_row<NC, kAuxSmallStore>(rp, sl, lane, v, slots);
  else
    store_bf16_row<NC, kAuxSmallStore, false>(rp, sl, lane, v, slots);
}

template <int NC, bool FP8, bool PADDED>
void launch_direct_nc(int blocks, size_t lds, const LayoutParams& lp, const RowParams& rp, int wpt, int cpw,
                      int nchunks, hipStream_t stream) {
  hipLaunchKernelGGL((layout_dispatch_direct_kernel<NC, FP8, PADDED>), dim3(blocks), dim3(64 * kDirectWaves), lds,
                     stream, lp, rp, wpt, cpw, nchunks);
}

template <bool FP8, bool PADDED>
void launch_direct(int cpw, int blocks, size_t lds, const LayoutParams& lp, const RowParams& rp, int wpt,
                   int nchunks, hipStream_t stream) {
  switch (cpw) {
    case 2: launch_direct_nc<2, FP8, PADDED>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 4: launch_direct_nc<4, FP8, PADDED>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 6: launch_direct_nc<6, FP8, PADDED>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 8: launch_direct_nc<8, FP8, PADDED>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 10: launch_direct_nc<10, FP8, PADDED>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 12: launch_direct_nc<12, FP8, PADDED>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    case 14: launch_direct_nc<14, FP8, PADDED>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
    default: launch_direct_nc<16, FP8, PADDED>(blocks, lds, lp, rp, wpt, cpw, nchunks, stream); break;
  }
}

// ---------------------------------------------------------------------------
// tile form
// ---------------------------------------------------------------------------

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
      store_fp8_row<NC, kAuxSmallStore>(rp, sl, lane, v, slots);
    else
      store_bf16_row<NC, kAuxSmallStore, false>(rp, sl, lane, v, slots);
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

size_t direct_lds(const LayoutParams& lp) { return (size_t)kDirectWaves * direct_hist_ints(lp.E, lp.C > 0) * 4; }

bool direct_form(const LayoutParams& lp) {
  return (lp.C > 0 || lp.A == 1) && (int64_t)lp.T * lp.k <= kMaxPairs && direct_lds(lp) <= kDirectLdsMax;
}

}  // namespace

bool layout_dispatch_fusable(const LayoutPlan& pl, const LayoutParams& lp) {
  return direct_form(lp) || (pl.ntiles == 1 && pl.W == kW);
}

hipError_t launch_layout_dispatch(const LayoutPlan& pl, LayoutParams lp, const RowParams& rp, bool fp8,
                                  hipStream_t stream) {
  prepare_layout_params(pl, lp);
  const DispatchSplit s = dispatch_split(rp);  // rp.num_cus is 0 here: one wavefront per slice
  const int64_t slices = (int64_t)rp.T * s.wpt;
  if (direct_form(lp)) {
    const int64_t waves = slices + lp.E + lp.R + 1;
    const int blocks = (int)((waves + kDirectWaves - 1) / kDirectWaves);
    const size_t lds = direct_lds(lp);
    const bool padded = lp.C > 0;
    if (fp8) {
      if (padded) launch_direct<true, true>(s.cpw, blocks, lds, lp, rp, s.wpt, s.nchunks, stream);
      else launch_direct<true, false>(s.cpw, blocks, lds, lp, rp, s.wpt, s.nchunks, stream);
    } else {
      if (padded) launch_direct<false, true>(s.cpw, blocks, lds, lp, rp, s.wpt, s.nchunks, stream);
      else launch_direct<false, false>(s.cpw, blocks, lds, lp, rp, s.wpt, s.nchunks, stream);
    }
    return hipGetLastError();
  }
  const int blocks = (int)std::max<int64_t>(1, (slices + kD - 1) / kD);
  if (fp8)
    launch_fp<true>(s.cpw, blocks, pl.lds_bytes, lp, rp, s.wpt, s.nchunks, stream);
  else
    launch_fp<false>(s.cpw, blocks, pl.lds_bytes, lp, rp, s.wpt, s.nchunks, stream);
  return hipGetLastError();
}

}  // namespace ep
