// Split-KV work plan, built on the device from the device-resident kv_lens.
//
// The pages motivate long contexts (128K) but say nothing about how one
// query's softmax is spread over many compute units; this plan is the usual
// split into token ranges whose partial softmax statistics are merged by
// log-sum-exp afterwards.
//
// Auto mode (num_splits == 0): the tiles (tile = 64 tokens) of all valid
// sequences are laid end to end and cut into G equal ranges, one per
// work-group, so every work-group streams the same number of cache bytes
// whatever the length mix.  A range that crosses a sequence boundary becomes
// several segments.  Forced mode (num_splits = S): every sequence is cut into
// at most S ranges and each segment gets its own work-group.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kPlanThreads = 1024;

__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  // Hillis-Steele over 1024 threads in LDS.
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    int add = (t >= off) ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  int incl = tmp[t];
  *total = tmp[kPlanThreads - 1];
  __syncthreads();
  return incl - v;
}

__device__ inline bool len_valid(int len, int max_kv_len, int cap) {
  return len >= 1 && len <= max_kv_len && len <= cap;
}

// number of g in [0, G] with floor(g*T/G) <= y   (T >= G >= 1, y >= 0)
__device__ inline long count_le(long y, long T, long G) {
  long c = ((y + 1) * G + T - 1) / T;  // ceil((y+1)G/T) = #g with g*T < (y+1)*G
  return c > G + 1 ? G + 1 : c;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    PlanPtrs p, const int32_t* __restrict__ kv_lens, int B, int max_kv_len, int max_pages,
    int page, int tile, int num_splits, int max_wg) {
  __shared__ int tmp[kPlanThreads];
  __shared__ long s_tile_base;
  __shared__ int s_seg_base;
  const int t = threadIdx.x;
  const long cap = (long)max_pages * page;
  const int capi = cap > 0x7fffffffL ? 0x7fffffff : (int)cap;

  // ---- pass 1: total tiles over valid sequences
  if (t == 0) s_tile_base = 0;
  __syncthreads();
  long total_tiles = 0;
  for (int c0 = 0; c0 < B; c0 += kPlanThreads) {
    int b = c0 + t;
    int tiles = 0;
    if (b < B) {
      int len = kv_lens[b];
      if (len_valid(len, max_kv_len, capi)) tiles = (len + tile - 1) / tile;
    }
    int tot;
    block_exclusive_scan(tiles, tmp, &tot);
    total_tiles += tot;
  }

  long G = 0;
  if (num_splits == 0) {
    G = max_wg;
    if (G > total_tiles) G = total_tiles;
  }

  // ---- pass 2: segments per sequence, prefix sums, and the segment list
  long tile_base = 0;
  int seg_base = 0;
  for (int c0 = 0; c0 < B; c0 += kPlanThreads) {
    int b = c0 + t;
    int len = 0, tiles = 0;
    if (b < B) {
      len = kv_lens[b];
      if (len_valid(len, max_kv_len, capi)) tiles = (len + tile - 1) / tile;
      else len = 0;
    }
    int tot_tiles;
    int my_tile_off = block_exclusive_scan(tiles, tmp, &tot_tiles);
    long s_b = tile_base + my_tile_off;
    long e_b = s_b + tiles;
    int nseg = 0;
    long g_first = 0;
    int per = 1;
    if (tiles > 0) {
      if (num_splits == 0) {
        // WG boundaries w_g = floor(g*T/G); interior ones cut the sequence.
        g_first = count_le(s_b, total_tiles, G);  // first g with w_g > s_b
        long g = g_first;
        nseg = 1;
        while (g < G && (g * total_tiles) / G < e_b) {
          ++nseg;
          ++g;
        }
      } else {
        per = (tiles + num_splits - 1) / num_splits;
        nseg = (tiles + per - 1) / per;
      }
    }
    int tot_segs;
    int my_seg_off = block_exclusive_scan(nseg, tmp, &tot_segs);
    int k0 = seg_base + my_seg_off;
    if (b < B) {
      p.seq_seg_start[b] = k0;
      p.seq_seg_count[b] = nseg;
    }
    if (nseg > 0) {
      if (num_splits == 0) {
        long cur = s_b;
        long g = g_first;
        long owner = g_first - 1;  // WG owning tile s_b
        for (int k = 0; k < nseg; ++k) {
          long nxt = e_b;
          if (k + 1 < nseg) nxt = (g * total_tiles) / G;
          Seg sg;
          sg.b = b;
          sg.t0 = (int)((cur - s_b) * tile);
          long t1 = (nxt - s_b) * tile;
          sg.t1 = (int)(t1 < len ? t1 : len);
          sg.pad = (int)owner;
          p.segs[k0 + k] = sg;
          // a segment that starts exactly on a WG boundary opens that WG's list
          if ((owner * total_tiles) / G == cur) p.wg_seg_start[owner] = k0 + k;
          cur = nxt;
          owner = g;
          ++g;
        }
      } else {
        for (int k = 0; k < nseg; ++k) {
          Seg sg;
          sg.b = b;
          sg.t0 = k * per * tile;
          int t1 = (k + 1) * per * tile;
          sg.t1 = t1 < len ? t1 : len;
          sg.pad = k0 + k;
          p.segs[k0 + k] = sg;
          p.wg_seg_start[k0 + k] = k0 + k;
        }
      }
    }
    tile_base += tot_tiles;
    seg_base += tot_segs;
  }
  if (t == 0) {
    int n_wg = (num_splits == 0) ? (int)G : seg_base;
    p.wg_seg_start[n_wg] = seg_base;
    p.counts[0] = seg_base;
    p.counts[1] = n_wg;
  }
  (void)s_tile_base;
  (void)s_seg_base;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int auto_wg_budget() {
  static int cached = 0;
  if (cached > 0) return cached;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0) {
    cached = cus;
  } else {
    (void)hipGetLastError();
    return 256;
  }
  return cached;
}

PlanDims plan_dims(int B, int num_splits) {
  PlanDims d;
  if (num_splits > 0) {
    d.max_segs = B * num_splits;
    d.max_wg = B * num_splits;
  } else {
    d.max_wg = auto_wg_budget();
    d.max_segs = d.max_wg + B;
  }
  return d;
}

size_t plan_bytes(int B, int num_splits) {
  PlanDims d = plan_dims(B, num_splits);
  return align256(sizeof(Seg) * (size_t)d.max_segs) + align256(sizeof(int) * (size_t)B) * 2 +
         align256(sizeof(int) * (size_t)(d.max_wg + 1)) + 256;
}

void carve_plan(void* base, int B, int num_splits, PlanPtrs* p) {
  PlanDims d = plan_dims(B, num_splits);
  char* c = (char*)base;
  p->segs = (Seg*)c;
  c += align256(sizeof(Seg) * (size_t)d.max_segs);
  p->seq_seg_start = (int*)c;
  c += align256(sizeof(int) * (size_t)B);
  p->seq_seg_count = (int*)c;
  c += align256(sizeof(int) * (size_t)B);
  p->wg_seg_start = (int*)c;
  c += align256(sizeof(int) * (size_t)(d.max_wg + 1));
  p->counts = (int*)c;
}

hipError_t launch_plan(const PlanPtrs& p, const int32_t* kv_lens, int B, int max_kv_len,
                       int max_pages, int page, int tile, int num_splits, hipStream_t s) {
  PlanDims d = plan_dims(B, num_splits);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, p, kv_lens, B, max_kv_len,
                     max_pages, page, tile, num_splits, d.max_wg);
  return hipGetLastError();
}

}  // namespace mla
