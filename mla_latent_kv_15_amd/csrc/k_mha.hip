// MHA-equivalent decode attention: the multi-head cache the pages weigh MLA
// against ([formulas] §一 and §三; [walkthrough] §2).  Every cached token
// holds a key and a value for each head, 2 n_h d_h numbers (32768 at the V2
// shape, against MLA's 576), and head i attends with its own keys:
//   o_i = sum_j softmax_j(scale * q_i . k_ij) v_ij.
// A token's cache row is [k_0 .. k_{n_h-1} | v_0 .. v_{n_h-1}], each d_h wide,
// in the same paging as the latent cache.
//
// The step reads every cached number once for two flops, so HBM bounds it and
// it runs on the vector ALUs: a work-group takes one split-KV segment (the
// plan of k_plan.hip) and a group of heads; the tph = d_h / 16 threads of a
// head each hold 16 dims of q and of the output, and a run of tokens' keys
// and values (8 tokens in bf16, 4 in fp32) is loaded before any is used.
#include <math.h>

#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kDpt = 16;   // dims per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline void unpack(const u32x4* p, float* x, const float*) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 v = p[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * c + e] = __uint_as_float(v[e]);
  }
}
__device__ inline void unpack(const u32x4* p, float* x, const __bf16*) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4 v = p[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * c + 2 * e] = __uint_as_float(v[e] << 16);
      x[8 * c + 2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  }
}
__device__ inline float ldf(const float* p) { return *p; }
__device__ inline float ldf(const __bf16* p) { return (float)*p; }
__device__ inline void stf(float* p, float v) { *p = v; }
__device__ inline void stf(__bf16* p, float v) { *p = (__bf16)v; }

// 16-byte pieces holding kDpt elements of T
template <typename T>
constexpr int pieces() { return kDpt * (int)sizeof(T) / 16; }

template <typename T, int U>
__global__ __launch_bounds__(256) void mha_decode_kernel(
    int n_h, int d_h, int tph, float scale, const T* __restrict__ q, const T* __restrict__ cache,
    int num_pages, const int32_t* __restrict__ page_table, int max_pages, int page, PlanPtrs plan,
    float* __restrict__ part_o, float* __restrict__ part_ml, T* __restrict__ out) {
  const int k = blockIdx.x;
  if (k >= plan.counts[0]) return;
  const Seg sg = plan.segs[k];
  const int hpw = 256 / tph;
  const int h = blockIdx.y * hpw + (int)threadIdx.x / tph;
  const int c = (int)threadIdx.x % tph;
  // the tph threads of a head are consecutive lanes of one wave (tph divides
  // 64), so a head's threads leave together and its shuffles stay whole
  if (h >= n_h) return;
  const int b = sg.b;
  const long rowlen = 2L * n_h * d_h;
  const long koff = (long)h * d_h + c * kDpt, voff = (long)n_h * d_h + koff;
  float qv[kDpt], o[kDpt];
  const T* qp = q + ((long)b * n_h + h) * d_h + c * kDpt;
#pragma unroll
  for (int i = 0; i < kDpt; ++i) {
    qv[i] = ldf(qp + i) * scale;
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  bool bad = false;
  for (int t0 = sg.t0; t0 < sg.t1; t0 += U) {
    u32x4 kb[U][pieces<T>()], vb[U][pieces<T>()];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + u, sg.t1 - 1);
      live[u] = t0 + u < sg.t1;
      int pg = page_table[(long)b * max_pages + t / page];
      if (pg < 0 || pg >= num_pages) {
        bad = true;
        pg = 0;   // read a valid row; the segment's result is NaN
      }
      const T* row = cache + ((long)pg * page + t % page) * rowlen;
#pragma unroll
      for (int p = 0; p < pieces<T>(); ++p) {
        kb[u][p] = ((const u32x4*)(row + koff))[p];
        vb[u][p] = ((const u32x4*)(row + voff))[p];
      }
    }
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[kDpt];
      unpack(kb[u], x, (const T*)nullptr);
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < kDpt; ++i) a = fmaf(qv[i], x[i], a);
      for (int off = tph >> 1; off > 0; off >>= 1) a += __shfl_xor(a, off);
      sc[u] = live[u] ? a : -INFINITY;
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, sc[u]);
    const float alpha = mn == -INFINITY ? 1.f : expf(m - mn);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < kDpt; ++i) o[i] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = live[u] ? expf(sc[u] - mn) : 0.f;
      l += p;
      float x[kDpt];
      unpack(vb[u], x, (const T*)nullptr);
#pragma unroll
      for (int i = 0; i < kDpt; ++i) o[i] = fmaf(p, x[i], o[i]);
    }
    m = mn;
  }
  const float nanv = __builtin_nanf("");
  if (plan.seq_seg_count[b] == 1) {
    const float inv = 1.f / l;
    T* op = out + ((long)b * n_h + h) * d_h + c * kDpt;
#pragma unroll
    for (int i = 0; i < kDpt; ++i) stf(op + i, bad ? nanv : o[i] * inv);
  } else {
    float* pp = part_o + ((long)k * n_h + h) * d_h + c * kDpt;
#pragma unroll
    for (int i = 0; i < kDpt; ++i) pp[i] = bad ? nanv : o[i];
    if (c == 0) {
      part_ml[((long)k * n_h + h) * 2] = m;
      part_ml[((long)k * n_h + h) * 2 + 1] = bad ? nanv : l;
    }
  }
}

}  // namespace

bool mha_supported(const Geo& g) {
  const int tph = g.d_h / kDpt;
  return g.d_h % kDpt == 0 && tph >= 1 && tph <= 64 && (tph & (tph - 1)) == 0 && g.d_h <= 1024;
}

hipError_t mha_decode(const Geo& g, const void* q, const void* cache, int num_pages,
                      const int32_t* page_table, int max_pages, const PlanPtrs& plan, int max_segs,
                      float scale, float* part_o, float* part_ml, void* out, hipStream_t s) {
  if (max_segs <= 0) return hipSuccess;
  if (!mha_supported(g)) return hipErrorInvalidValue;
  const int tph = g.d_h / kDpt, hpw = 256 / tph;
  const dim3 grid(max_segs, (g.n_h + hpw - 1) / hpw);
  if (g.bf16)
    hipLaunchKernelGGL((mha_decode_kernel<__bf16, 8>), grid, dim3(256), 0, s, g.n_h, g.d_h, tph,
                       scale, (const __bf16*)q, (const __bf16*)cache, num_pages, page_table,
                       max_pages, g.page, plan, part_o, part_ml, (__bf16*)out);
  else
    hipLaunchKernelGGL((mha_decode_kernel<float, 4>), grid, dim3(256), 0, s, g.n_h, g.d_h, tph,
                       scale, (const float*)q, (const float*)cache, num_pages, page_table,
                       max_pages, g.page, plan, part_o, part_ml, (float*)out);
  return hipGetLastError();
}

}  // namespace mla
