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

namespace ep {
namespace {

__device__ __forceinline__ int aligned_count(int c, int A) { return ((c + A - 1) / A) * A; }

__device__ __forceinline__ int udiv(uint32_t n, uint32_t magic) { return (int)__umulhi(n, magic); }

// Exclusive scan over experts of the (aligned) counts in cnt[0..E): offs[e]
// for e <= E.  Padded layouts use e*C directly.  Each thread takes a run of
// experts, wavefronts scan their runs with shuffles, and every thread adds
// the totals of the wavefronts before it (no serial step).  Ends with a
// barrier.
__device__ void scan_offsets(const int* cnt, int* offs, int E, int A, int C, int* s_part) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  if (C > 0) {
    for (int e = tid; e <= E; e += nthr) offs[e] = e * C;
    __syncthreads();
    return;
  }
  const int per = (E + nthr - 1) / nthr;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += aligned_count(cnt[e], A);
  const int lane = tid & 63, wv = tid >> 6, nw = (nthr + 63) >> 6;
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) s_part[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int i = 0; i < nw; ++i) {
    const int v = s_part[i];
    before += i < wv ? v : 0;
    total += v;
  }
  int run = before + incl - sum;
  for (int e = lo; e < hi; ++e) { offs[e] = run; run += aligned_count(cnt[e], A); }
  if (tid == 0) offs[E] = total;
  __syncthreads();
}

// Layout outputs that depend only on totals and offsets (one block writes
// them).  diag[1] must already be zero.
__device__ void write_outputs(const LayoutParams& p, const int* tot, const int* offs, const int* rank_cnt) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int E = p.E, R = p.R, per = p.E / p.R;
  for (int e = tid; e < E; e += nthr) {
    p.expert_count[e] = tot[e];
    p.expert_offset[e] = offs[e];
  }
  if (tid == 0) p.expert_offset[E] = offs[E];
  for (int r = tid; r <= R; r += nthr) p.rank_offset[r] = offs[r * per];
  for (int r = tid; r < R; r += nthr) p.rank_count[r] = rank_cnt[r];
  if (p.diag && p.C > 0) {
    // pairs past a padded expert's capacity: sum over experts of (count - C)+
    int drop = 0;
    for (int e = tid; e < E; e += nthr) drop += max(0, tot[e] - p.C);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) drop += __shfl_xor(drop, d, 64);
    if ((tid & 63) == 0 && drop) atomicAdd(&p.diag[1], drop);
  }
}

// Receive row of a valid pair of expert v whose position in v's segment is
// pos; -1 if the padded layout has no room.
__device__ __forceinline__ int slot_of(const LayoutParams& p, int v, int pos, const int* offs) {
  if (p.C > 0) return pos < p.C ? v * p.C + pos : -1;
  return offs[v] + pos;
}

// src_pair = -1 on padding rows: rows of each expert segment past its count,
// and (flat layout) rows past the layout's end up to the worst case.
// Experts go to work units of 64 lanes (wavefronts), `unit` of `nunits`.
__device__ void fill_padding_rows(const LayoutParams& p, const int* tot, const int* offs, int unit, int nunits,
                                  int lane, int64_t gtid, int64_t gthreads) {
  if (!p.src_pair) return;
  const int E = p.E, C = p.C;
  for (int e = unit; e < E; e += nunits) {
    const int c = tot[e];
    const int lo = C > 0 ? e * C + min(c, C) : offs[e] + c;
    const int hi = C > 0 ? (e + 1) * C : offs[e + 1];
    for (int r = lo + lane; r < hi; r += 64) p.src_pair[r] = -1;
  }
  if (C == 0)
    for (int64_t r = (int64_t)offs[E] + gtid; r < p.rows; r += gthreads) p.src_pair[r] = -1;
}

}  // namespace

// One block per tile of tokens, 64*W threads, one pair per thread.  With a
// single tile, `gridDim.x` blocks each rebuild the (small) layout in LDS and
// share the output writes, so no block waits for another.
template <int W>
__global__ __launch_bounds__(64 * W) void layout_tiles_kernel(LayoutParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int E = p.E, R = p.R, k = p.k;
  uint64_t* masks = reinterpret_cast<uint64_t*>(smem);     // [W][E]
  uint64_t* tokrank = masks + (size_t)W * E;               // [64*W] ranks hit per token (R <= 64)
  int* pref = reinterpret_cast<int*>(tokrank + 64 * W);    // [W][E] pairs of e in earlier windows
  int* idx_s = pref + (size_t)W * E;                       // [64*W]
  int* rank_of = idx_s + 64 * W;                           // [E]
  int* rank_hist = rank_of + E;                            // [R]
  int* cnt_s = rank_hist + R;                              // [E]
  int* offs = cnt_s + E;                                   // [E+1]
  __shared__ int s_bad;
  __shared__ int s_part[20];

  const int tid = threadIdx.x, nthr = 64 * W;
  const bool single = p.ntiles == 1;
  const int tile = single ? 0 : blockIdx.x;
  const int t0 = tile * p.TT;
  const int nt = max(0, min(p.TT, p.T - t0));
  const int np = nt * k;
  const int64_t g0 = (int64_t)t0 * k;
  const bool small_r = R <= 64;

  for (int i = tid; i < W * E; i += nthr) masks[i] = 0;
  tokrank[tid] = 0;
  for (int i = tid; i < E; i += nthr) rank_of[i] = udiv((uint32_t)i, p.magic_per);
  for (int i = tid; i < R; i += nthr) rank_hist[i] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  int e = -1;
  bool bad = false;
  if (tid < np) {
    const int v = p.idx[g0 + tid];
    if (v >= 0 && v < E) e = v;
    else bad = (v != -1);
  }
  idx_s[tid] = e;
  const int w = tid >> 6, lane = tid & 63;
  const int tl = udiv((uint32_t)tid, p.magic_k);  // token of the pair inside the tile
  if (e >= 0) {
    atomicOr(reinterpret_cast<unsigned long long*>(&masks[w * E + e]), 1ull << lane);
    if (small_r) atomicOr(reinterpret_cast<unsigned long long*>(&tokrank[tl]), 1ull << rank_of[e]);
  }
  {
    const uint64_t bb = __ballot(bad);
    if (lane == 0 && bb) atomicAdd(&s_bad, (int)__popcll(bb));
  }
  __syncthreads();

  // per expert: pairs in earlier windows (prefix over windows) and tile total
  for (int ee = tid; ee < E; ee += nthr) {
    int c[W];
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) c[w2] = (int)__popcll(masks[w2 * E + ee]);
    int run = 0;
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) { pref[w2 * E + ee] = run; run += c[w2]; }
    cnt_s[ee] = run;
  }
  // distinct tokens per rank
  if (small_r) {
    if (tid < nt) {
      uint64_t m = tokrank[tid];
      while (m) {
        atomicAdd(&rank_hist[__builtin_ctzll(m)], 1);
        m &= m - 1;
      }
    }
  } else if (e >= 0) {
    // the token's first pair on a rank counts the token once for it
    const int r = rank_of[e];
    bool first = true;
    for (int q = tl * k; q < tid; ++q) {
      const int e2 = idx_s[q];
      if (e2 >= 0 && rank_of[e2] == r) { first = false; break; }
    }
    if (first) atomicAdd(&rank_hist[r], 1);
  }
  __syncthreads();

  // rank of the pair among the tile's pairs of the same expert
  const int local =
      e >= 0 ? pref[w * E + e] + (int)__popcll(masks[w * E + e] & ((1ull << lane) - 1ull)) : -1;

  if (single) {
    // The whole batch is this tile.  Block 0 writes outputs and slots; all
    // blocks share the padding rows.
    const bool lead = blockIdx.x == 0;
    if (lead && tid == 0 && p.diag) { p.diag[0] = s_bad; p.diag[1] = 0; }
    scan_offsets(cnt_s, offs, E, p.A, p.C, s_part);  // barrier: diag[1] is zero before the adds
    if (lead) {
      write_outputs(p, cnt_s, offs, rank_hist);
      if (tid < np) {
        int s = -1;
        if (e >= 0) {
          s = slot_of(p, e, local, offs);
          if (s >= 0 && p.src_pair) p.src_pair[s] = (int)(g0 + tid);
        }
        p.slot[g0 + tid] = s;
      }
    }
    fill_padding_rows(p, cnt_s, offs, blockIdx.x * W + w, gridDim.x * W, lane,
                      (int64_t)blockIdx.x * nthr + tid, (int64_t)gridDim.x * nthr);
    return;
  }

  // Publish this tile's counts and in-tile ranks for the finalize kernel.
  for (int ee = tid; ee < E; ee += nthr) p.ws_tile[(size_t)tile * E + ee] = cnt_s[ee];
  for (int r = tid; r < R; r += nthr) p.ws_rank[(size_t)tile * R + r] = rank_hist[r];
  if (tid == 0) p.ws_bad[tile] = s_bad;
  if (tid < np) p.slot[g0 + tid] = local;
}

// One block per tile.  Rebuilds totals, offsets and this tile's prefix from
// the per-tile counts, then turns the tile's in-tile ranks into slots.
__global__ __launch_bounds__(1024) void layout_finalize_kernel(LayoutParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int E = p.E, R = p.R, G = p.G, ntiles = p.ntiles;
  const int gE = max(G * E, E);
  int* part_tot = reinterpret_cast<int*>(smem);  // [G][E]
  int* part_pre = part_tot + gE;                 // [G][E]
  int* tot = part_pre + gE;                      // [E]
  int* pre = tot + E;                            // [E]
  int* offs = pre + E;                           // [E+1]
  int* rank_tot = offs + E + 1;                  // [R]
  __shared__ int s_bad;
  __shared__ int s_part[20];

  const int tid = threadIdx.x, nthr = blockDim.x;
  const int tile = blockIdx.x;
  for (int r = tid; r < R; r += nthr) rank_tot[r] = 0;

  // (a) per (tile group, expert): sum of the group's tile counts, and the
  //     part of it that lies before this block's tile.  Loads go out in
  //     batches of 16 independent reads.
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
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int e = tid; e < E; e += nthr) {
    int st = 0, sp = 0;
    for (int g = 0; g < G; ++g) { st += part_tot[g * E + e]; sp += part_pre[g * E + e]; }
    tot[e] = st;
    pre[e] = sp;
  }
  if (tile == 0) {
    // rank counts and invalid ids: coalesced sweeps, LDS atomics
    for (int i = tid; i < ntiles * R; i += nthr) {
      const int v = p.ws_rank[i];
      if (v) atomicAdd(&rank_tot[i - udiv((uint32_t)i, p.magic_R) * R], v);
    }
    int bad = 0;
    for (int t = tid; t < ntiles; t += nthr) bad += p.ws_bad[t];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) bad += __shfl_xor(bad, d, 64);
    if ((tid & 63) == 0 && bad) atomicAdd(&s_bad, bad);
  }
  __syncthreads();
  if (tile == 0 && tid == 0 && p.diag) { p.diag[0] = s_bad; p.diag[1] = 0; }
  scan_offsets(tot, offs, E, p.A, p.C, s_part);  // barrier: diag[1] is zero before the adds

  // (b) this tile's slots
  {
    const int t0 = tile * p.TT;
    const int np = max(0, min(p.TT, p.T - t0)) * p.k;
    const int64_t g0 = (int64_t)t0 * p.k;
    for (int i = tid; i < np; i += nthr) {
      const int v = p.idx[g0 + i];
      if (!(v >= 0 && v < E)) continue;  // slot already -1
      int s = slot_of(p, v, pre[v] + p.slot[g0 + i], offs);
      if ((int64_t)s >= p.rows) s = -1;  // cannot happen; keeps every write in bounds
      p.slot[g0 + i] = s;
      if (s >= 0 && p.src_pair) p.src_pair[s] = (int)(g0 + i);
    }
  }

  // (c) block 0: counts, offsets, rank counts, dropped pairs
  if (tile == 0) write_outputs(p, tot, offs, rank_tot);

  // (d) padding rows, experts spread over all wavefronts of the grid
  const int nw = nthr >> 6;
  fill_padding_rows(p, tot, offs, tile * nw + (tid >> 6), gridDim.x * nw, tid & 63,
                    (int64_t)tile * nthr + tid, (int64_t)gridDim.x * nthr);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {
// ceil(2^32 / d): for n * d < 2^32, n / d == (n * magic) >> 32.
uint32_t magic_for(uint32_t d) { return (uint32_t)(0xFFFFFFFFull / d + 1ull); }
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
  const size_t gE = (size_t)(pl.G * E > E ? pl.G * E : E);
  pl.fin_lds_bytes = (size_t)4 * (2 * gE + 3 * (size_t)E + 1 + R);
  pl.ws_tile_off = 0;
  pl.ws_rank_off = pl.ws_tile_off + (((size_t)pl.ntiles * E * 4 + 255) & ~(size_t)255);
  pl.ws_bad_off = pl.ws_rank_off + (((size_t)pl.ntiles * R * 4 + 255) & ~(size_t)255);
  pl.ws_bytes = pl.ws_bad_off + (((size_t)pl.ntiles * 4 + 255) & ~(size_t)255);
  return pl;
}

hipError_t launch_layout(const LayoutPlan& pl, LayoutParams p, hipStream_t stream) {
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
  // One tile: several blocks rebuild it and share the padding rows of src_pair.
  int blocks = pl.ntiles;
  if (pl.ntiles == 1 && p.src_pair) blocks = (int)std::min<int64_t>(16, std::max<int64_t>(1, p.rows / 4096));
  switch (pl.W) {
    case 16: hipLaunchKernelGGL(layout_tiles_kernel<16>, dim3(blocks), dim3(pl.threads), pl.lds_bytes, stream, p); break;
    case 8: hipLaunchKernelGGL(layout_tiles_kernel<8>, dim3(blocks), dim3(pl.threads), pl.lds_bytes, stream, p); break;
    case 4: hipLaunchKernelGGL(layout_tiles_kernel<4>, dim3(blocks), dim3(pl.threads), pl.lds_bytes, stream, p); break;
    case 2: hipLaunchKernelGGL(layout_tiles_kernel<2>, dim3(blocks), dim3(pl.threads), pl.lds_bytes, stream, p); break;
    default: hipLaunchKernelGGL(layout_tiles_kernel<1>, dim3(blocks), dim3(pl.threads), pl.lds_bytes, stream, p); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || pl.ntiles == 1) return err;
  hipLaunchKernelGGL(layout_finalize_kernel, dim3(pl.ntiles), dim3(pl.fin_threads), pl.fin_lds_bytes, stream, p);
  return hipGetLastError();
}

}  // namespace ep
