// Routing layout for gfx950: top-k expert ids -> per-expert and per-rank
// counts, prefix offsets and a deterministic token->slot map.
//
// The layout is the routing metadata a DeepEP dispatch hands to combine and
// the per-expert receive counts the expert GEMM needs (GeekNews "DeepSeek
// publica DeepEP ...", section "Patrones de uso en entrenamiento, prefill y
// decoding"; DeepEP documentation item 10).  Slots inside an expert are in
// ascending (token, k-index) order: a stable counting sort.
//
// Design (no global atomics on hot counters, no dependence on arrival order):
//   * The pairs (t, j) are cut into tiles of whole tokens, at most 64*W pairs
//     per tile, one pair per thread, one 64-pair window per wavefront.
//   * Each wavefront sets bit `lane` of an LDS 64-bit mask per (window,
//     expert) with ds_or_b64.  OR is order independent, so the masks are
//     deterministic.  A pair's rank inside its tile is the popcount of its
//     expert's mask below its lane plus the popcounts of the earlier windows.
//   * Tile counts go to the workspace.  The last tile block to finish
//     (atomic ticket) scans them: per-expert totals -> aligned exclusive scan
//     over experts -> offsets, and per-expert exclusive scans over tiles ->
//     tile bases.  A second, light kernel adds the bases to the in-tile
//     ranks and writes slot / src_pair.
//   * A batch that fits one tile (e.g. 128 decode tokens x top-8) is done by
//     one block in one launch.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

__device__ __forceinline__ int aligned_count(int c, int A) { return ((c + A - 1) / A) * A; }

// Exclusive scan over experts of the (aligned) counts in cnt_s[0..E):
// offs[e] for e <= E.  Padded layouts use e*C directly.
__device__ void scan_offsets(const int* cnt_s, int* offs, int E, int A, int C, int* s_part) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  if (C > 0) {
    for (int e = tid; e <= E; e += nthr) offs[e] = e * C;
    __syncthreads();
    return;
  }
  const int per = (E + nthr - 1) / nthr;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += aligned_count(cnt_s[e], A);
  // inclusive scan inside the wavefront
  const int lane = tid & 63, wv = tid >> 6, nw = (nthr + 63) >> 6;
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) s_part[wv] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < nw; ++i) { int v = s_part[i]; s_part[i] = run; run += v; }
    s_part[nw] = run;
  }
  __syncthreads();
  int run = s_part[wv] + incl - sum;
  for (int e = lo; e < hi; ++e) { offs[e] = run; run += aligned_count(cnt_s[e], A); }
  if (tid == 0) offs[E] = s_part[nw];
  __syncthreads();
}

// Writes the layout outputs that only depend on counts and offsets, and the
// src_pair padding rows (rows of each segment past its count, and rows past
// the end of the flat layout up to the worst case).
__device__ void write_count_outputs(const LayoutParams& p, const int* cnt_s, const int* offs,
                                    const int* rank_cnt, int bad) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int E = p.E, R = p.R, per = p.E / p.R;
  for (int e = tid; e < E; e += nthr) {
    p.expert_count[e] = cnt_s[e];
    p.expert_offset[e] = offs[e];
  }
  if (tid == 0) p.expert_offset[E] = offs[E];
  for (int r = tid; r <= R; r += nthr) p.rank_offset[r] = offs[r * per];
  for (int r = tid; r < R; r += nthr) p.rank_count[r] = rank_cnt[r];
  if (tid == 0 && p.diag) { p.diag[0] = bad; p.diag[1] = 0; }
}

// Sets src_pair = -1 on padding rows: rows of each expert segment past its
// count, and (flat layout) rows past the layout's end up to the worst case.
// Experts are spread over `nunits` work units of `width` lanes each.
__device__ void fill_padding_rows(const LayoutParams& p, const int* cnt, const int* offs,
                                  int unit, int nunits, int lane, int width,
                                  int gtid, int gthreads) {
  if (!p.src_pair) return;
  const int E = p.E, C = p.C;
  for (int e = unit; e < E; e += nunits) {
    const int c = cnt[e];
    const int lo = C > 0 ? e * C + min(c, C) : offs[e] + c;
    const int hi = C > 0 ? (e + 1) * C : offs[e + 1];
    for (int r = lo + lane; r < hi; r += width) p.src_pair[r] = -1;
  }
  if (C == 0) {
    for (int64_t r = (int64_t)offs[E] + gtid; r < p.rows; r += gthreads) p.src_pair[r] = -1;
  }
}

__device__ int block_sum(int v, int* s_red) {
  // s_red[0] must be zero on entry (callers clear it before a barrier).
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if (lane == 0 && v) atomicAdd(s_red, v);
  __syncthreads();
  return *s_red;
}

}  // namespace

// One block per tile of tokens, 64*W threads, one pair per thread.
__global__ __launch_bounds__(1024) void layout_tiles_kernel(LayoutParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int W = p.W, E = p.E, R = p.R, k = p.k;
  uint64_t* masks = reinterpret_cast<uint64_t*>(smem);   // [W][E]
  int* idx_s = reinterpret_cast<int*>(masks + (size_t)W * E);  // [64*W]
  int* rank_hist = idx_s + 64 * W;                        // [R]
  int* cnt_s = rank_hist + R;                             // [E]
  int* offs = cnt_s + E;                                  // [E+1]
  __shared__ int s_bad, s_last, s_drop;
  __shared__ int s_part[20];

  const int tid = threadIdx.x, nthr = blockDim.x;
  const int tile = blockIdx.x;
  const int t0 = tile * p.TT;
  const int nt = max(0, min(p.TT, p.T - t0));
  const int np = nt * k;
  const int64_t g0 = (int64_t)t0 * k;

  for (int i = tid; i < W * E; i += nthr) masks[i] = 0;
  for (int i = tid; i < R; i += nthr) rank_hist[i] = 0;
  if (tid == 0) { s_bad = 0; s_drop = 0; }
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
  if (e >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&masks[w * E + e]), 1ull << lane);
  {
    const uint64_t bb = __ballot(bad);
    if (lane == 0 && bb) atomicAdd(&s_bad, (int)__popcll(bb));
  }
  __syncthreads();

  // rank of the pair among the tile's pairs of the same expert
  int local = -1;
  if (e >= 0) {
    local = (int)__popcll(masks[w * E + e] & ((1ull << lane) - 1ull));
    for (int w2 = 0; w2 < w; ++w2) local += (int)__popcll(masks[w2 * E + e]);
    // first pair of its token on this rank -> one distinct token for the rank
    const int per = E / R, r = e / per;
    const int tl = tid / k, j = tid - tl * k;
    bool first = true;
    for (int jj = 0; jj < j; ++jj) {
      const int e2 = idx_s[tl * k + jj];
      if (e2 >= 0 && e2 / per == r) { first = false; break; }
    }
    if (first) atomicAdd(&rank_hist[r], 1);
  }
  for (int ee = tid; ee < E; ee += nthr) {
    int c = 0;
    for (int w2 = 0; w2 < W; ++w2) c += (int)__popcll(masks[w2 * E + ee]);
    cnt_s[ee] = c;
  }
  __syncthreads();

  if (p.ntiles == 1) {
    // Whole batch in this block: finish here.
    scan_offsets(cnt_s, offs, E, p.A, p.C, s_part);
    write_count_outputs(p, cnt_s, offs, rank_hist, s_bad);
    int drop = 0;
    if (tid < np) {
      int s = -1;
      if (e >= 0) {
        if (p.C > 0) {
          if (local < p.C) s = e * p.C + local;
          else drop = 1;
        } else {
          s = offs[e] + local;
        }
        if (s >= 0 && p.src_pair) p.src_pair[s] = (int)(g0 + tid);
      }
      p.slot[g0 + tid] = s;
    }
    fill_padding_rows(p, cnt_s, offs, tid >> 6, nthr >> 6, tid & 63, 64, tid, nthr);
    if (p.diag && p.C > 0) {
      const int total = block_sum(drop, &s_drop);
      if (tid == 0) p.diag[1] = total;
    }
    return;
  }

  // Publish this tile's counts and in-tile ranks.
  for (int ee = tid; ee < E; ee += nthr) p.ws_tile[(size_t)tile * E + ee] = cnt_s[ee];
  for (int r = tid; r < R; r += nthr) p.ws_rank[(size_t)tile * R + r] = rank_hist[r];
  if (tid == 0) p.ws_bad[tile] = s_bad;
  if (tid < np) p.slot[g0 + tid] = local;
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(p.ticket, 1u) == (unsigned)(p.ntiles - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- last block: scans over all tiles ----
  const int ntiles = p.ntiles;
  for (int i = tid; i < E; i += nthr) cnt_s[i] = 0;
  for (int i = tid; i < R; i += nthr) rank_hist[i] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // totals: coalesced sweep of the [tile][E] and [tile][R] matrices
  for (int i = tid; i < ntiles * E; i += nthr) {
    const int c = p.ws_tile[i];
    if (c) atomicAdd(&cnt_s[i % E], c);
  }
  for (int i = tid; i < ntiles * R; i += nthr) {
    const int c = p.ws_rank[i];
    if (c) atomicAdd(&rank_hist[i % R], c);
  }
  for (int i = tid; i < ntiles; i += nthr) {
    const int c = p.ws_bad[i];
    if (c) atomicAdd(&s_bad, c);
  }
  __syncthreads();
  scan_offsets(cnt_s, offs, E, p.A, p.C, s_part);
  write_count_outputs(p, cnt_s, offs, rank_hist, s_bad);

  // tile bases: exclusive scan over tiles per expert, G tile groups per expert
  int G = nthr / E;
  G = max(1, min(G, 2 * W));
  int* gsum = reinterpret_cast<int*>(masks);  // [G][E], fits in the mask area
  for (int job = tid; job < G * E; job += nthr) {
    const int g = job / E, ee = job - g * E;
    const int a = (int)((int64_t)ntiles * g / G), b = (int)((int64_t)ntiles * (g + 1) / G);
    int s = 0;
    for (int t = a; t < b; ++t) s += p.ws_tile[(size_t)t * E + ee];
    gsum[g * E + ee] = s;
  }
  __syncthreads();
  for (int ee = tid; ee < E; ee += nthr) {
    int run = p.C > 0 ? 0 : offs[ee];
    for (int g = 0; g < G; ++g) { const int v = gsum[g * E + ee]; gsum[g * E + ee] = run; run += v; }
  }
  __syncthreads();
  for (int job = tid; job < G * E; job += nthr) {
    const int g = job / E, ee = job - g * E;
    const int a = (int)((int64_t)ntiles * g / G), b = (int)((int64_t)ntiles * (g + 1) / G);
    int run = gsum[g * E + ee];
    for (int t = a; t < b; ++t) {
      const int c = p.ws_tile[(size_t)t * E + ee];
      p.ws_tile[(size_t)t * E + ee] = run;
      run += c;
    }
  }
  if (tid == 0) *p.ticket = 0u;  // leave the workspace ready for the next call
}

// Adds tile bases to the in-tile ranks, writes src_pair, fills padding rows.
__global__ __launch_bounds__(256) void layout_finalize_kernel(LayoutParams p) {
  __shared__ int s_drop;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int b = blockIdx.x;
  if (tid == 0) s_drop = 0;
  __syncthreads();
  int drop = 0;
  if (b < p.ntiles) {
    const int t0 = b * p.TT;
    const int np = max(0, min(p.TT, p.T - t0)) * p.k;
    const int64_t g0 = (int64_t)t0 * p.k;
    const int* base = p.ws_tile + (size_t)b * p.E;
    for (int i = tid; i < np; i += nthr) {
      const int v = p.idx[g0 + i];
      if (!(v >= 0 && v < p.E)) continue;  // slot already -1
      const int pos = base[v] + p.slot[g0 + i];
      int s;
      if (p.C > 0) {
        if (pos >= p.C) { p.slot[g0 + i] = -1; ++drop; continue; }
        s = v * p.C + pos;
      } else {
        s = pos;
      }
      // A workspace that was not zero-filled before its first use breaks the
      // tile scan; keep even that case inside the buffers.
      if (s < 0 || (int64_t)s >= p.rows) { p.slot[g0 + i] = -1; continue; }
      p.slot[g0 + i] = s;
      if (p.src_pair) p.src_pair[s] = (int)(g0 + i);
    }
  }
  fill_padding_rows(p, p.expert_count, p.expert_offset, b * (nthr >> 6) + (tid >> 6),
                    gridDim.x * (nthr >> 6), tid & 63, 64, b * nthr + tid, gridDim.x * nthr);
  if (p.diag && p.C > 0) {
    const int total = block_sum(drop, &s_drop);
    if (tid == 0 && total) atomicAdd(&p.diag[1], total);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

LayoutPlan plan_layout(int T, int k, int E, int R) {
  LayoutPlan pl;
  pl.W = max(1, min(16, 4096 / E));
  pl.TT = max(1, (64 * pl.W) / k);
  pl.ntiles = max(1, (T + pl.TT - 1) / pl.TT);
  pl.threads = 64 * pl.W;
  pl.lds_bytes = (size_t)8 * pl.W * E + (size_t)4 * (64 * pl.W + R + E + E + 1);
  pl.ws_tile_off = 256;
  pl.ws_rank_off = pl.ws_tile_off + (((size_t)pl.ntiles * E * 4 + 255) & ~(size_t)255);
  pl.ws_bad_off = pl.ws_rank_off + (((size_t)pl.ntiles * R * 4 + 255) & ~(size_t)255);
  pl.ws_bytes = pl.ws_bad_off + (((size_t)pl.ntiles * 4 + 255) & ~(size_t)255);
  return pl;
}

hipError_t launch_layout(const LayoutPlan& pl, LayoutParams p, hipStream_t stream) {
  p.W = pl.W;
  p.TT = pl.TT;
  p.ntiles = pl.ntiles;
  hipLaunchKernelGGL(layout_tiles_kernel, dim3(pl.ntiles), dim3(pl.threads), pl.lds_bytes, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || pl.ntiles == 1) return err;
  const int fin_blocks = max(pl.ntiles, min(p.E, 1024));
  hipLaunchKernelGGL(layout_finalize_kernel, dim3(fin_blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ep
