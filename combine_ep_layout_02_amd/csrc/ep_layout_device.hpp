// Device building blocks of the routing layout, shared by the layout
// kernels (ep_layout.hip) and the fused layout + dispatch kernel
// (ep_layout_dispatch.hip).  See ep_layout.hip for the design.
#pragma once

#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace lay {

static __device__ __forceinline__ int aligned_count(int c, int A) { return ((c + A - 1) / A) * A; }

// n / d from magic = ceil(2^32 / d) (exact for n * d < 2^32); d = 1 has no
// 32-bit magic and is encoded as 0.
static __device__ __forceinline__ int udiv(uint32_t n, uint32_t magic) {
  return magic ? (int)__umulhi(n, magic) : (int)n;
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP: four
// row_shr steps scan each 16-lane row, then two row broadcasts carry row
// totals into the rows above (lanes without a source add 0).
static __device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Exclusive scan over experts of the (aligned) counts in cnt[0..E): offs[e]
// for e <= E.  Padded layouts use e*C directly.  Each thread takes a run of
// experts, wavefronts scan their runs with DPP, and every thread adds the
// totals of the wavefronts before it (no serial step).  Ends with a barrier.
static __device__ void scan_offsets(const int* cnt, int* offs, int E, int A, int C, int* s_part) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  if (C > 0) {
    for (int e = tid; e <= E; e += nthr) offs[e] = e * C;
    __syncthreads();
    return;
  }
  const int per = (E + nthr - 1) / nthr;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int sum = 0;
  if (A == 1) {
    for (int e = lo; e < hi; ++e) sum += cnt[e];
  } else {
    for (int e = lo; e < hi; ++e) sum += aligned_count(cnt[e], A);
  }
  const int lane = tid & 63, wv = tid >> 6, nw = (nthr + 63) >> 6;
  const int incl = wave_inclusive_scan(sum);
  if (lane == 63) s_part[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int v = i < nw ? s_part[i] : 0;
    before += i < wv ? v : 0;
    total += v;
  }
  int run = before + incl - sum;
  if (A == 1) {
    for (int e = lo; e < hi; ++e) { offs[e] = run; run += cnt[e]; }
  } else {
    for (int e = lo; e < hi; ++e) { offs[e] = run; run += aligned_count(cnt[e], A); }
  }
  if (tid == 0) offs[E] = total;
  __syncthreads();
}

// Layout outputs that depend only on totals and offsets (one block writes
// them).  diag[1] must already be zero.
static __device__ void write_outputs(const LayoutParams& p, const int* tot, const int* offs, const int* rank_cnt) {
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
static __device__ __forceinline__ int slot_of(const LayoutParams& p, int v, int pos, const int* offs) {
  if (p.C > 0) return pos < p.C ? v * p.C + pos : -1;
  return offs[v] + pos;
}

// src_pair = -1 on padding rows: rows of each expert segment past its count,
// and (flat layout) rows past the layout's end up to the worst case.
// Experts go to work units of 64 lanes (wavefronts), `unit` of `nunits`.
static __device__ void fill_padding_rows(const LayoutParams& p, const int* tot, const int* offs, int unit, int nunits,
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

// LDS of the tile pass (dynamic shared memory, carved in this order).
template <int W>
struct TileLds {
  uint64_t* masks;    // [W][E]   pairs of expert e in window w, one bit per lane
  uint64_t* tokrank;  // [64*W]   ranks hit by each token of the tile (R <= 64)
  int* pref;          // [W][E]   pairs of expert e in earlier windows
  int* idx_s;         // [64*W]   expert of each pair (-1 if none)
  int* rank_of;       // [E]      rank owning each expert
  int* rank_hist;     // [R]      distinct tokens per rank
  int* cnt_s;         // [E]      pairs per expert
  int* offs;          // [E+1]    offsets (single-tile path)
  __device__ TileLds(unsigned char* smem, int E, int R) {
    masks = reinterpret_cast<uint64_t*>(smem);
    tokrank = masks + (size_t)W * E;
    pref = reinterpret_cast<int*>(tokrank + 64 * W);
    idx_s = pref + (size_t)W * E;
    rank_of = idx_s + 64 * W;
    rank_hist = rank_of + E;
    cnt_s = rank_hist + R;
    offs = cnt_s + E;
  }
};

// Counts and stable in-tile ranks of one tile, one pair per thread.  Leaves
// cnt_s / rank_hist / *s_bad in LDS and returns the thread's expert (or -1)
// and in-tile rank.  Ends with a barrier.
template <int W>
static __device__ void tile_pass(const LayoutParams& p, const TileLds<W>& L, int tile, int* s_bad, int& e_out,
                          int& local_out) {
  const int E = p.E, R = p.R, k = p.k;
  const int tid = threadIdx.x, nthr = 64 * W;
  const int t0 = tile * p.TT;
  const int nt = max(0, min(p.TT, p.T - t0));
  const int np = nt * k;
  const int64_t g0 = (int64_t)t0 * k;
  const bool small_r = R <= 64;

  // the pair's id is loaded first; its latency overlaps the LDS set-up
  const int v = tid < np ? p.idx[g0 + tid] : -1;
  for (int i = tid; i < W * E; i += nthr) L.masks[i] = 0;
  L.tokrank[tid] = 0;
  for (int i = tid; i < E; i += nthr) L.rank_of[i] = udiv((uint32_t)i, p.magic_per);
  for (int i = tid; i < R; i += nthr) L.rank_hist[i] = 0;
  if (tid == 0) *s_bad = 0;
  __syncthreads();

  int e = -1;
  bool bad = false;
  if (tid < np) {
    if (v >= 0 && v < E) e = v;
    else bad = (v != -1);
  }
  L.idx_s[tid] = e;
  const int w = tid >> 6, lane = tid & 63;
  const int tl = udiv((uint32_t)tid, p.magic_k);  // token of the pair inside the tile
  if (e >= 0) {
    atomicOr(reinterpret_cast<unsigned long long*>(&L.masks[w * E + e]), 1ull << lane);
    if (small_r) atomicOr(reinterpret_cast<unsigned long long*>(&L.tokrank[tl]), 1ull << L.rank_of[e]);
  }
  {
    const uint64_t bb = __ballot(bad);
    if (lane == 0 && bb) atomicAdd(s_bad, (int)__popcll(bb));
  }
  __syncthreads();

  // per expert: pairs in earlier windows (prefix over windows) and tile total
  for (int ee = tid; ee < E; ee += nthr) {
    int c[W];
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) c[w2] = (int)__popcll(L.masks[w2 * E + ee]);
    int run = 0;
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) { L.pref[w2 * E + ee] = run; run += c[w2]; }
    L.cnt_s[ee] = run;
  }
  // distinct tokens per rank
  if (small_r) {
    if (tid < nt) {
      uint64_t m = L.tokrank[tid];
      while (m) {
        atomicAdd(&L.rank_hist[__builtin_ctzll(m)], 1);
        m &= m - 1;
      }
    }
  } else if (e >= 0) {
    // the token's first pair on a rank counts the token once for it
    const int r = L.rank_of[e];
    bool first = true;
    for (int q = tl * k; q < tid; ++q) {
      const int e2 = L.idx_s[q];
      if (e2 >= 0 && L.rank_of[e2] == r) { first = false; break; }
    }
    if (first) atomicAdd(&L.rank_hist[r], 1);
  }
  __syncthreads();

  // rank of the pair among the tile's pairs of the same expert
  e_out = e;
  local_out = e >= 0 ? L.pref[w * E + e] + (int)__popcll(L.masks[w * E + e] & ((1ull << lane) - 1ull)) : -1;
}

}  // namespace lay
}  // namespace ep
