// Split-KV work plan, built on the device from the device-resident kv_lens.
//
// The pages motivate long contexts (128K) but say nothing about how one
// query's softmax is spread over many compute units; this plan is the usual
// split into token ranges whose partial softmax statistics are merged by
// log-sum-exp afterwards.
//
// Auto mode (num_splits == 0): the tiles (tile = 64 tokens) of all valid
// sequences are laid end to end, each sequence preceded by kSegCost virtual
// tiles that stand for the fixed cost of starting a segment (its query, its
// partial write), and this line is cut into G equal ranges, one per
// work-group: every work-group gets the same cache bytes plus segment
// overheads, whatever the length mix.  A range that crosses a sequence
// boundary becomes several segments; a cut that falls on a sequence's
// virtual tiles moves to the sequence's first tile.  Forced mode
// (num_splits = S): every sequence is cut into at most S ranges and each
// segment gets its own work-group.
//
// plan_build is the planner of one work-group; it runs in a launch of its
// own, or as one extra work-group of a launch that precedes the attention.
#pragma once

#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kPlanThreads = 256;   // one chunk of sequences per pass (4 waves)
constexpr int kSegCost = 1;         // virtual tiles per segment start
constexpr int kMaxAutoWg = 1024;    // work-groups an auto plan may use

// Exclusive prefix sum over the work-group (wave scans + 4 wave totals).
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kPlanThreads / 64; ++i) {
    base += i < w ? wsum[i] : 0;
    tot += wsum[i];
  }
  __syncthreads();   // wsum is reused by the next scan
  *total = tot;
  return base + x - v;
}

__device__ inline bool len_valid(int len, int max_kv_len, int cap) {
  return len >= 1 && len <= max_kv_len && len <= cap;
}

// floor(a / b) for 0 <= a < 2^53, b > 0: a double estimate, corrected to the
// exact quotient (64-bit integer division is a long software routine here)
__device__ inline long div_floor(long a, long b) {
  long q = (long)((double)a / (double)b);
  if (q * b > a) --q;
  else if ((q + 1) * b <= a) ++q;
  return q;
}
// Work-group g (of G) owns tiles [w(g), w(g+1)), w(g) = floor(g T / G).
__device__ inline long wg_first_tile(long g, long T, long G) { return div_floor(g * T, G); }
// the work-group owning tile x: the largest g with w(g) <= x, ceil((x+1) G / T) - 1
__device__ inline long wg_of_tile(long x, long T, long G) {
  return div_floor((x + 1) * G + T - 1, T) - 1;
}

// The plan, built by one work-group of kPlanThreads threads.
__device__ void plan_build(const PlanJob& job) {
  const PlanPtrs& p = job.p;
  const int32_t* __restrict__ kv_lens = job.kv_lens;
  const int B = job.B, max_kv_len = job.max_kv_len, max_pages = job.max_pages;
  const int page = job.page, tile = job.tile, num_splits = job.num_splits, max_wg = job.max_wg;
  __shared__ int wsum[kPlanThreads / 64];
  __shared__ int s_kseq[kPlanThreads + 1];   // first segment of each sequence of the chunk
  __shared__ long s_sb[kPlanThreads];        // first tile (global) of each sequence
  __shared__ int s_len[kPlanThreads], s_tiles[kPlanThreads];
  __shared__ long s_g0[kPlanThreads];        // work-group owning each sequence's first tile
  __shared__ int s_wgs[kMaxAutoWg + 1];       // first segment of each work-group (auto mode)
  const int t = threadIdx.x;
  const long cap = (long)max_pages * page;
  const int capi = cap > 0x7fffffffL ? 0x7fffffff : (int)cap;
  auto tiles_of = [&](int b, int* len) {
    int l = b < B ? kv_lens[b] : 0;
    if (!len_valid(l, max_kv_len, capi)) l = 0;
    *len = l;
    return (l + tile - 1) / tile;
  };

  // a valid sequence's length on the virtual line
  auto vtiles = [](int tiles) { return tiles > 0 ? tiles + kSegCost : 0; };

  // ---- total tiles and virtual tiles over the valid sequences (one chunk:
  // kept for pass 2)
  const bool one_chunk = B <= kPlanThreads;
  int len0 = 0, tiles0 = 0, off0 = 0;
  long T = 0, V = 0;
  for (int c0 = 0; c0 < B; c0 += kPlanThreads) {
    int len, tot, vtot;
    const int tl = tiles_of(c0 + t, &len);
    block_exclusive_scan(tl, wsum, &tot);
    const int off = block_exclusive_scan(vtiles(tl), wsum, &vtot);
    if (one_chunk) {
      len0 = len;
      tiles0 = tl;
      off0 = off;
    }
    T += tot;
    V += vtot;
  }
  long G = 0;
  if (num_splits == 0) {
    G = T < max_wg ? T : max_wg;
    if (G > kMaxAutoWg) G = kMaxAutoWg;
    for (int g = t; g <= G; g += kPlanThreads) s_wgs[g] = -1;
    __syncthreads();
  }

  // ---- per chunk: segments per sequence, their prefix sums, then the list
  long tile_base = 0;
  int seg_base = 0;
  for (int c0 = 0; c0 < B; c0 += kPlanThreads) {
    const int b = c0 + t;
    int len = len0, tiles = tiles0, off = off0, tot_vt = (int)V;
    if (!one_chunk) {
      tiles = tiles_of(b, &len);
      off = block_exclusive_scan(vtiles(tiles), wsum, &tot_vt);
    }
    // the sequence's virtual tiles start at s_b, its real tiles at s_b + kSegCost
    const long s_b = tile_base + off;
    int nseg = 0, per = 1;
    long g0 = 0;
    if (tiles > 0) {
      if (num_splits == 0) {
        g0 = wg_of_tile(s_b + kSegCost, V, G);
        nseg = (int)(wg_of_tile(s_b + kSegCost + tiles - 1, V, G) - g0) + 1;
      } else {
        per = (tiles + num_splits - 1) / num_splits;
        nseg = (tiles + per - 1) / per;
      }
    }
    int tot_segs;
    const int k0 = seg_base + block_exclusive_scan(nseg, wsum, &tot_segs);
    if (b < B) {
      p.seq_seg_start[b] = k0;
      p.seq_seg_count[b] = nseg;
    }
    s_kseq[t] = k0;
    s_sb[t] = s_b;
    s_len[t] = len;
    s_tiles[t] = per;   // forced mode: tiles per segment
    s_g0[t] = g0;
    if (t == 0) s_kseq[kPlanThreads] = seg_base + tot_segs;
    __syncthreads();
    // emit the chunk's segments, spread over all threads
    for (int k = seg_base + t; k < seg_base + tot_segs; k += kPlanThreads) {
      int lo = 0, hi = kPlanThreads;   // the sequence i with kseq[i] <= k < kseq[i+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_kseq[mid] <= k) lo = mid;
        else hi = mid;
      }
      while (lo + 1 < kPlanThreads && s_kseq[lo + 1] <= k) ++lo;   // skip empty sequences
      const int i = lo, j = k - s_kseq[i];
      const int slen = s_len[i];
      Seg sg;
      sg.b = c0 + i;
      if (num_splits == 0) {
        const long vb = s_sb[i], sb = vb + kSegCost, eb = sb + (slen + tile - 1) / tile;
        const long g = s_g0[i] + j;
        const long w0 = wg_first_tile(g, V, G), w1 = wg_first_tile(g + 1, V, G);
        const long a = w0 > sb ? w0 : sb, e = w1 < eb ? w1 : eb;
        sg.t0 = (int)((a - sb) * tile);
        const long t1 = (e - sb) * tile;
        sg.t1 = (int)(t1 < slen ? t1 : slen);
        sg.pad = (int)g;
        // a work-group's first segment: every later segment of a sequence,
        // and its first one when the work-group's range starts within the
        // sequence's virtual tiles
        if (j > 0 || w0 >= vb) s_wgs[g] = k;
      } else {
        const int per_i = s_tiles[i];
        sg.t0 = j * per_i * tile;
        const int t1 = (j + 1) * per_i * tile;
        sg.t1 = t1 < slen ? t1 : slen;
        sg.pad = k;
        p.wg_seg_start[k] = k;
      }
      p.segs[k] = sg;
    }
    __syncthreads();   // the chunk's shared arrays are rewritten next
    tile_base += tot_vt;
    seg_base += tot_segs;
  }
  if (num_splits == 0) {
    // a work-group whose range holds only virtual tiles has no segment: its
    // list is empty (it starts where the next one does)
    if (t == 0) s_wgs[G] = seg_base;
    __syncthreads();
    for (int g = t; g <= G; g += kPlanThreads) {
      int gg = g;
      while (s_wgs[gg] < 0) ++gg;
      p.wg_seg_start[g] = s_wgs[gg];
    }
  }
  if (t == 0) {
    const int n_wg = num_splits == 0 ? (int)G : seg_base;
    if (num_splits != 0) p.wg_seg_start[n_wg] = seg_base;
    p.counts[0] = seg_base;
    p.counts[1] = n_wg;
  }
}

}  // namespace

}  // namespace mla
