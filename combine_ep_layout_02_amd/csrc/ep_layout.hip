// Routing layout for gfx950: top-k expert ids -> per-expert and per-rank
// counts, prefix offsets and a deterministic token->slot map.
//
// The layout is the routing metadata a DeepEP dispatch hands to combine and
// the per-expert receive counts the expert GEMM needs (GeekNews "DeepSeek
// publica DeepEP ...", section "Patrones de uso en entrenamiento, prefill y
// decoding"; DeepEP documentation item 10).  Slots inside an expert are in
// ascending (token, k-index) order: a stable counting sort.
//
// Design (no global atomics, nothing depends on arrival order):
//   * The pairs (t, j) are cut into tiles of whole tokens, at most 64*W pairs
//     per tile, one pair per thread, one 64-pair window per wavefront.
//   * Each wavefront sets bit `lane` of an LDS 64-bit mask per (window,
//     expert) with ds_or_b64.  OR is order independent, so the masks are
//     deterministic.  A pair's rank inside its tile is the popcount of its
//     expert's mask below its lane plus the popcounts of the earlier windows.
//   * A batch that fits one tile (e.g. 128 decode tokens x top-8) is done by
//     that one block: one launch.
//   * Otherwise the tile kernel stores per-tile counts and in-tile ranks, and
//     a finalize kernel runs one block per tile: every block reads the whole
//     (small) [tiles x experts] count matrix with independent coalesced loads,
//     derives the expert totals, the exclusive scan over experts (offsets) and
//     its own tile's prefix, and writes its tile's slots.  There is no ticket,
//     no inter-block wait and no serial scan over tiles.
//   * Divisions by k, E/R and E use host-computed multiply-high constants.
#include <algorithm>

#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "ep_layout_device.hpp"

namespace ep {
namespace {

using namespace lay;

// Per-expert totals over all tiles and the part before `tile`, from the
// [tiles x E] count matrix: (tile group, expert) jobs, loads in batches of
// 16 independent reads, then a reduction over groups.  Ends with a barrier.
__device__ void reduce_tiles(const LayoutParams& p, int tile, int G, int* part_tot, int* part_pre, int* tot,
                             int* pre) {
  const int E = p.E, ntiles = p.ntiles;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int gE = max(G * E, E);
  for (int job = tid; job < gE; job += nthr) {
    int g = 0, e = job;
    if (G > 1) { g = udiv((uint32_t)job, p.magic_E); e = job - g * E; }
    const int a = (int)((int64_t)ntiles * g / G), b = (int)((int64_t)ntiles * (g + 1) / G);
    int st = 0, sp = 0;
    int t = a;
    for (; t + 16 <= b; t += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = p.ws_tile[(size_t)(t + u) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) { st += c[u]; sp += (t + u) < tile ? c[u] : 0; }
    }
    for (; t < b; ++t) {
      const int c = p.ws_tile[(size_t)t * E + e];
      st += c;
      sp += t < tile ? c : 0;
    }
    part_tot[g * E + e] = st;
    part_pre[g * E + e] = sp;
  }
  __syncthreads();
  for (int e = tid; e < E; e += nthr) {
    int st = 0, sp = 0;
    for (int g = 0; g < G; ++g) { st += part_tot[g * E + e]; sp += part_pre[g * E + e]; }
    tot[e] = st;
    pre[e] = sp;
  }
  __syncthreads();
}

// Block 0 only: rank counts and invalid ids summed over tiles (coalesced
// sweeps, LDS atomics); rank_tot must be zero.  Entries tid of both arrays
// arrive preloaded in rank0 / bad0.  Ends with a barrier.
__device__ void reduce_ranks(const LayoutParams& p, int* rank_tot, int* s_bad, int rank0, int bad0) {
  const int R = p.R, ntiles = p.ntiles;
  const int tid = threadIdx.x, nthr = blockDim.x;
  if (rank0) atomicAdd(&rank_tot[tid - udiv((uint32_t)tid, p.magic_R) * R], rank0);
  for (int i = tid + nthr; i < ntiles * R; i += nthr) {
    const int v = p.ws_rank[i];
    if (v) atomicAdd(&rank_tot[i - udiv((uint32_t)i, p.magic_R) * R], v);
  }
  int bad = bad0;
  for (int t = tid + nthr; t < ntiles; t += nthr) bad += p.ws_bad[t];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) bad += __shfl_xor(bad, d, 64);
  if ((tid & 63) == 0 && bad) atomicAdd(s_bad, bad);
  __syncthreads();
}

// Tile pass.  With a single tile, gridDim.x blocks each rebuild the (small)
// layout in LDS and share the output writes, so no block waits for another.
// With several tiles it publishes the tile's counts and in-tile ranks for
// layout_finalize_kernel.
template <int W>
__global__ __launch_bounds__(64 * W) void layout_tiles_kernel(LayoutParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_bad;
  __shared__ int s_part[20];
  const TileLds<W> L(smem, p.E, p.R);
  const int tid = threadIdx.x, nthr = 64 * W;
  const bool single = p.ntiles == 1;
  const int tile = single ? 0 : blockIdx.x;
  const int64_t g0 = (int64_t)tile * p.TT * p.k;
  const int np = max(0, min(p.TT, p.T - tile * p.TT)) * p.k;
  int e, local;
  tile_pass<W>(p, L, tile, &s_bad, e, local);

  if (single) {
    // Block 0 writes outputs and slots; all blocks share the padding rows.
    const bool lead = blockIdx.x == 0;
    if (lead && tid == 0 && p.diag) { p.diag[0] = s_bad; p.diag[1] = 0; }
    scan_offsets(L.cnt_s, L.offs, p.E, p.A, p.C, s_part);  // barrier: diag[1] is zero before the adds
    if (lead) {
      write_outputs(p, L.cnt_s, L.offs, L.rank_hist);
      if (tid < np) {
        int s = -1;
        if (e >= 0) {
          s = slot_of(p, e, local, L.offs);
          if (s >= 0 && p.src_pair) p.src_pair[s] = (int)(g0 + tid);
        }
        p.slot[g0 + tid] = s;
      }
    }
    fill_padding_rows(p, L.cnt_s, L.offs, blockIdx.x * W + (tid >> 6), gridDim.x * W, tid & 63,
                      (int64_t)blockIdx.x * nthr + tid, (int64_t)gridDim.x * nthr);
    return;
  }

  for (int ee = tid; ee < p.E; ee += nthr) p.ws_tile[(size_t)tile * p.E + ee] = L.cnt_s[ee];
  for (int r = tid; r < p.R; r += nthr) p.ws_rank[(size_t)tile * p.R + r] = L.rank_hist[r];
  if (tid == 0) p.ws_bad[tile] = s_bad;
  if (tid < np) p.slot[g0 + tid] = local;
}

// Finalize LDS, carved from the front of the dynamic shared memory.
struct FinLds {
  int *part_tot, *part_pre, *tot, *pre, *offs, *rank_tot;
  __device__ FinLds(unsigned char* smem, int G, int E) {
    const int gE = max(G * E, E);
    part_tot = reinterpret_cast<int*>(smem);
    part_pre = part_tot + gE;
    tot = part_pre + gE;
    pre = tot + E;
    offs = pre + E;
    rank_tot = offs + E + 1;
  }
};

// One block per tile.  Rebuilds totals, offsets and this tile's prefix from
// the per-tile counts, then turns the tile's in-tile ranks into slots.
__global__ __launch_bounds__(1024) void layout_finalize_kernel(LayoutParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_bad;
  __shared__ int s_part[20];
  const int E = p.E, R = p.R;
  const FinLds F(smem, p.G, E);
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int tile = blockIdx.x;
  // this thread's pair (a tile has at most 1024 pairs, one per thread),
  // loaded up front so its latency overlaps the reductions
  const int t0 = tile * p.TT;
  const int np = max(0, min(p.TT, p.T - t0)) * p.k;
  const int64_t g0 = (int64_t)t0 * p.k;
  int v = -1, local = 0;
  if (tid < np) {
    v = p.idx[g0 + tid];
    local = p.slot[g0 + tid];
  }
  // block 0 also sums the per-tile rank counts and invalid ids; its first
  // share of them is loaded here too
  const bool lead = tile == 0;
  const int nrank = p.ntiles * R;
  const int rank0 = lead && tid < nrank ? p.ws_rank[tid] : 0;
  const int bad0 = lead && tid < p.ntiles ? p.ws_bad[tid] : 0;
  for (int r = tid; r < R; r += nthr) F.rank_tot[r] = 0;
  if (tid == 0) s_bad = 0;
  reduce_tiles(p, tile, p.G, F.part_tot, F.part_pre, F.tot, F.pre);
  if (lead) reduce_ranks(p, F.rank_tot, &s_bad, rank0, bad0);
  if (tile == 0 && tid == 0 && p.diag) { p.diag[0] = s_bad; p.diag[1] = 0; }
  scan_offsets(F.tot, F.offs, E, p.A, p.C, s_part);  // barrier: diag[1] is zero before the adds

  // this tile's slots (an invalid id's slot is already -1)
  if (tid < np && v >= 0 && v < E) {
    int s = slot_of(p, v, F.pre[v] + local, F.offs);
    if ((int64_t)s >= p.rows) s = -1;  // cannot happen; keeps every write in bounds
    p.slot[g0 + tid] = s;
    if (s >= 0 && p.src_pair) p.src_pair[s] = (int)(g0 + tid);
  }
  if (tile == 0) write_outputs(p, F.tot, F.offs, F.rank_tot);
  const int nw = nthr >> 6;
  fill_padding_rows(p, F.tot, F.offs, tile * nw + (tid >> 6), gridDim.x * nw, tid & 63,
                    (int64_t)tile * nthr + tid, (int64_t)gridDim.x * nthr);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// ceil(2^32 / d): for n * d < 2^32, n / d == (n * magic) >> 32.  For d = 1
// that is 2^32, which does not fit: 0 stands for it (udiv returns n).
uint32_t magic_for(uint32_t d) { return d == 1 ? 0u : (uint32_t)(0xFFFFFFFFull / d + 1ull); }

}  // namespace

LayoutPlan plan_layout(int T, int k, int E, int R) {
  LayoutPlan pl;
  // W = 16 windows (1024 pairs) per tile where the LDS allows it, within 64 KiB;
  // a power of two so the kernel's window loops unroll.
  auto tile_lds = [&](int W) {
    return (size_t)12 * W * E + (size_t)768 * W + (size_t)12 * E + (size_t)4 * R + 4;
  };
  pl.W = 16;
  while (pl.W > 1 && (64 * pl.W > 64 * 4096 / E || tile_lds(pl.W) > 65536)) pl.W /= 2;
  pl.TT = max(1, (64 * pl.W) / k);
  pl.ntiles = max(1, (T + pl.TT - 1) / pl.TT);
  pl.threads = 64 * pl.W;
  pl.lds_bytes = tile_lds(pl.W);
  pl.fin_threads = 1024;
  pl.G = E <= pl.fin_threads ? max(1, min(pl.fin_threads / E, pl.ntiles)) : 1;
  auto fin_lds = [&](int G) {
    const size_t gE = (size_t)(G * E > E ? G * E : E);
    return (size_t)4 * (2 * gE + 3 * (size_t)E + 1 + R);
  };
  pl.fin_lds_bytes = fin_lds(pl.G);
  pl.ws_tile_off = 0;
  pl.ws_rank_off = pl.ws_tile_off + (((size_t)pl.ntiles * E * 4 + 255) & ~(size_t)255);
  pl.ws_bad_off = pl.ws_rank_off + (((size_t)pl.ntiles * R * 4 + 255) & ~(size_t)255);
  pl.ws_bytes = pl.ws_bad_off + (((size_t)pl.ntiles * 4 + 255) & ~(size_t)255);
  return pl;
}

namespace {

template <int W>
hipError_t launch_tiles(const LayoutPlan& pl, LayoutParams& p, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(layout_tiles_kernel<W>, dim3(blocks), dim3(pl.threads), pl.lds_bytes, stream, p);
  return hipGetLastError();
}

}  // namespace

void prepare_layout_params(const LayoutPlan& pl, LayoutParams& p) {
  p.W = pl.W;
  p.TT = pl.TT;
  p.ntiles = pl.ntiles;
  p.G = pl.G;
  // Exact for every quotient taken: pair index < 1024 over k <= 64, expert id
  // < 2048 over E/R <= 2048, job index < 2048 over E <= 2048, workspace index
  // < 2^22 over R <= 2048 (n * d < 2^32 in each case).
  p.magic_k = magic_for((uint32_t)p.k);
  p.magic_per = magic_for((uint32_t)(p.E / p.R));
  p.magic_E = magic_for((uint32_t)p.E);
  p.magic_R = magic_for((uint32_t)p.R);
}

hipError_t launch_layout(const LayoutPlan& pl, LayoutParams p, hipStream_t stream) {
  prepare_layout_params(pl, p);
  // One tile: several blocks rebuild it and share the padding rows of src_pair.
  int blocks = pl.ntiles;
  if (pl.ntiles == 1 && p.src_pair) blocks = (int)std::min<int64_t>(16, std::max<int64_t>(1, p.rows / 4096));
  hipError_t err;
  switch (pl.W) {
    case 16: err = launch_tiles<16>(pl, p, blocks, stream); break;
    case 8: err = launch_tiles<8>(pl, p, blocks, stream); break;
    case 4: err = launch_tiles<4>(pl, p, blocks, stream); break;
    case 2: err = launch_tiles<2>(pl, p, blocks, stream); break;
    default: err = launch_tiles<1>(pl, p, blocks, stream); break;
  }
  if (err != hipSuccess || pl.ntiles == 1) return err;
  hipLaunchKernelGGL(layout_finalize_kernel, dim3(pl.ntiles), dim3(pl.fin_threads), pl.fin_lds_bytes, stream, p);
  return hipGetLastError();
}

}  // namespace ep
