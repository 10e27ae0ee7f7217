// Generic HIP kernels: any layer geometry, fp32 or bf16 storage, fp32 math.
//
// They serve shapes the MFMA kernels do not specialise for (for example the
// tiny fp32 layer) and the prefill path.  Each kernel computes one step of the
// MLA layer as the pages define it; the citations sit with the host calls.
#include <math.h>

#include "mla_internal.h"

namespace mla {

namespace {

__device__ inline float ld(const float* p) { return *p; }
__device__ inline float ld(const __bf16* p) { return (float)(*p); }
__device__ inline void st(float* p, float v) { *p = v; }
__device__ inline void st(__bf16* p, float v) { *p = (__bf16)v; }

__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// 256-thread block reductions (4 waves); `red` holds >= 4 floats.
__device__ inline float block_max256(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ inline float block_sum256(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// tiled SIMT GEMM: C = alpha * A * B^T (B(n,k) as BLayout BL says)
// ---------------------------------------------------------------------------
template <int BL>
__device__ inline long b_index(int n, int k, long ldb) {
  if constexpr (BL == B_NK) return (long)n * ldb + k;
  if constexpr (BL == B_KN) return (long)k * ldb + n;
  if constexpr (BL == B_NK_TILES) return tile_index(n, k, ldb);
  return tile_index(k, n, ldb);
}

// a_kmajor: A(m, k) = A[k * lda + m] instead of A[m * lda + k]; c_tiled: C in
// the tiled layout with ldc columns (sC then counts elements of that layout)
template <typename TA, typename TB, typename TC, int BL>
__global__ __launch_bounds__(256) void gemm_generic_kernel(int M, int N, int K,
                                                           const TA* __restrict__ A, long lda,
                                                           long sA, const TB* __restrict__ B,
                                                           long ldb, long sB, TC* __restrict__ C,
                                                           long ldc, long sC, float alpha,
                                                           int a_kmajor, int c_tiled) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const long z = blockIdx.z;
  A += z * sA;
  B += z * sB;
  C += z * sC;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = threadIdx.x; e < 1024; e += 256) {
      int mm = e >> 4, kk = e & 15;
      int gm = m0 + mm, gk = k0 + kk;
      As[kk][mm] = (gm < M && gk < K)
                       ? ld(A + (a_kmajor ? (long)gk * lda + gm : (long)gm * lda + gk))
                       : 0.f;
    }
    for (int e = threadIdx.x; e < 1024; e += 256) {
      int nn, kk;
      if (BL == B_KN || BL == B_KN_TILES) {
        kk = e >> 6;
        nn = e & 63;
      } else {
        nn = e >> 4;
        kk = e & 15;
      }
      int gn = n0 + nn, gk = k0 + kk;
      float v = 0.f;
      if (gn < N && gk < K) v = ld(B + b_index<BL>(gn, gk, ldb));
      Bs[kk][nn] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty + 16 * i];
        bb[i] = Bs[kk][tx + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int gm = m0 + ty + 16 * i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int gn = n0 + tx + 16 * j;
      if (gn < N)
        st(C + (c_tiled ? tile_index(gm, gn, ldc) : (long)gm * ldc + gn), alpha * acc[i][j]);
    }
  }
}

template <typename TA, typename TB, typename TC>
hipError_t gemm_launch(BLayout bl, int M, int N, int K, const void* A, long lda, long sA,
                       const void* B, long ldb, long sB, void* C, long ldc, long sC, int batch,
                       float alpha, hipStream_t s, int a_kmajor, int c_tiled) {
  dim3 grid((N + 63) / 64, (M + 63) / 64, batch);
#define MLA_GG(BL)                                                                              \
  hipLaunchKernelGGL((gemm_generic_kernel<TA, TB, TC, BL>), grid, dim3(256), 0, s, M, N, K,     \
                     (const TA*)A, lda, sA, (const TB*)B, ldb, sB, (TC*)C, ldc, sC, alpha,      \
                     a_kmajor, c_tiled)
  switch (bl) {
    case B_NK: MLA_GG(B_NK); break;
    case B_KN: MLA_GG(B_KN); break;
    case B_NK_TILES: MLA_GG(B_NK_TILES); break;
    case B_KN_TILES: MLA_GG(B_KN_TILES); break;
    default: return hipErrorInvalidValue;
  }
#undef MLA_GG
  return hipGetLastError();
}

// row-major [R][C] -> tiled layout, one thread per 8-element piece of dst
template <typename T>
__global__ void pack_tiles_kernel(const T* __restrict__ src, long R, long C, T* __restrict__ dst) {
  struct Piece { T v[8]; };
  const long p = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= R * C / 8) return;
  const long tile = p >> 6, tiles_per_row = C >> 5;
  const int l = (int)(p & 63);
  const long r = (tile / tiles_per_row) * 16 + (l & 15);
  const long c = (tile % tiles_per_row) * 32 + 8 * (l >> 4);
  ((Piece*)dst)[p] = *(const Piece*)(src + r * C + c);
}

// ---------------------------------------------------------------------------
// RoPE table: angles in fp64
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(float* table, int max_pos, int d_r, double base) {
  long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  int half = d_r / 2;
  if (idx >= (long)max_pos * half) return;
  int pos = (int)(idx / half);
  int k = (int)(idx % half);
  double theta = pow(base, -2.0 * (double)k / (double)d_r);
  double ang = (double)pos * theta;
  table[2 * idx] = (float)cos(ang);
  table[2 * idx + 1] = (float)sin(ang);
}

// q_abs[b][i][d_c + 2k, 2k+1] = rotate(q_r[b][i][2k, 2k+1]) * scale
template <typename T>
__global__ void pack_query_rope_kernel(int n_h, int d_c, int d_r, int row, float scale,
                                       const float* __restrict__ q_r,
                                       const int32_t* __restrict__ positions, int B,
                                       const float* __restrict__ rope, int rope_len,
                                       T* __restrict__ q_abs) {
  long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  int half = d_r / 2;
  long total = (long)B * n_h * half;
  if (idx >= total) return;
  int k = (int)(idx % half);
  long bi = idx / half;  // b * n_h + i
  int b = (int)(bi / n_h);
  int pos = positions[b];
  float x = q_r[bi * d_r + 2 * k], y = q_r[bi * d_r + 2 * k + 1];
  float o0, o1;
  if (pos >= 0 && pos < rope_len) {
    float c = rope[((long)pos * half + k) * 2], sn = rope[((long)pos * half + k) * 2 + 1];
    o0 = (x * c - y * sn) * scale;
    o1 = (x * sn + y * c) * scale;
  } else {
    o0 = o1 = __builtin_nanf("");
  }
  st(q_abs + bi * row + d_c + 2 * k, o0);
  st(q_abs + bi * row + d_c + 2 * k + 1, o1);
}

// ---------------------------------------------------------------------------
// decode attention core (order B), one work-group per (segment, head)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_decode_generic_kernel(
    int n_h, int d_c, int row, int page, const T* __restrict__ q_abs, const T* __restrict__ cache,
    int num_pages, const int32_t* __restrict__ page_table, int max_pages, PlanPtrs plan,
    float* __restrict__ part_o, float* __restrict__ part_ml, T* __restrict__ lat_out) {
  extern __shared__ float sm[];
  float* qs = sm;                         // [row]
  float* ps = qs + row;                   // [256]
  long* offs = (long*)(sm + ((row + 256 + 1) & ~1));  // [256], 8-byte aligned
  __shared__ float red[4];
  __shared__ int bad;
  const int k = blockIdx.x;
  if (k >= plan.counts[0]) return;
  const Seg sg = plan.segs[k];
  const int i = blockIdx.y;
  const int b = sg.b;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  for (int e = tid; e < row; e += 256) qs[e] = ld(q_abs + ((long)b * n_h + i) * row + e);
  __syncthreads();
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  for (int j0 = sg.t0; j0 < sg.t1; j0 += 256) {
    const int j = j0 + tid;
    float sc = -INFINITY;
    long off = -1;
    if (j < sg.t1) {
      int pg = page_table[(long)b * max_pages + j / page];
      if (pg < 0 || pg >= num_pages) {
        bad = 1;
      } else {
        off = ((long)pg * page + j % page) * row;
        float a = 0.f;
        for (int e = 0; e < row; ++e) a = fmaf(qs[e], ld(cache + off + e), a);
        sc = a;
      }
    }
    offs[tid] = off;
    float cm = block_max256(sc, red);
    float mn = fmaxf(m, cm);
    float alpha = (mn == -INFINITY) ? 1.f : expf(m - mn);
    float p = (off >= 0) ? expf(sc - mn) : 0.f;
    ps[tid] = p;
    float cs = block_sum256(p, red);  // contains a barrier: ps/offs visible
    l = l * alpha + cs;
    m = mn;
    const int nj = min(256, sg.t1 - j0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int dim = tid + 256 * r;
      if (dim >= d_c) break;
      float a = acc[r] * alpha;
      for (int jj = 0; jj < nj; ++jj) {
        long o = offs[jj];
        if (o >= 0) a = fmaf(ps[jj], ld(cache + o + dim), a);
      }
      acc[r] = a;
    }
    __syncthreads();
  }
  const bool is_bad = bad != 0;
  const float nanv = __builtin_nanf("");
  if (plan.seq_seg_count[b] == 1) {
    float inv = 1.f / l;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int dim = tid + 256 * r;
      if (dim >= d_c) break;
      st(lat_out + ((long)b * n_h + i) * d_c + dim, is_bad ? nanv : acc[r] * inv);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int dim = tid + 256 * r;
      if (dim >= d_c) break;
      part_o[((long)k * n_h + i) * d_c + dim] = is_bad ? nanv : acc[r];
    }
    if (tid == 0) {
      part_ml[((long)k * n_h + i) * 2] = m;
      part_ml[((long)k * n_h + i) * 2 + 1] = is_bad ? nanv : l;
    }
  }
}

// ---------------------------------------------------------------------------
// log-sum-exp merge of split partials: one work-group per (sequence, head)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(int n_h, int d_c, PlanPtrs plan,
                                                      const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      T* __restrict__ lat_out) {
  __shared__ float wts[1024];
  __shared__ float red[4];
  const int b = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const int cnt = plan.seq_seg_count[b];
  if (cnt == 1) return;
  T* out = lat_out + ((long)b * n_h + i) * d_c;
  if (cnt == 0) {
    for (int e = tid; e < d_c; e += 256) st(out + e, __builtin_nanf(""));
    return;
  }
  const int k0 = plan.seq_seg_start[b];
  float M = -INFINITY;
  for (int s = tid; s < cnt; s += 256) M = fmaxf(M, part_ml[((long)(k0 + s) * n_h + i) * 2]);
  M = block_max256(M, red);
  float L = 0.f;
  for (int s = tid; s < cnt; s += 256) {
    const float* ml = part_ml + ((long)(k0 + s) * n_h + i) * 2;
    L += ml[1] * expf(ml[0] - M);
  }
  L = block_sum256(L, red);
  const float invL = 1.f / L;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < cnt; c0 += 1024) {
    int nc = min(1024, cnt - c0);
    for (int s = tid; s < nc; s += 256) {
      const float* ml = part_ml + ((long)(k0 + c0 + s) * n_h + i) * 2;
      wts[s] = expf(ml[0] - M) * invL;
    }
    __syncthreads();
    for (int s = 0; s < nc; ++s) {
      const float w = wts[s];
      const float* po = part_o + ((long)(k0 + c0 + s) * n_h + i) * d_c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int dim = tid + 256 * r;
        if (dim < d_c) acc[r] = fmaf(w, po[dim], acc[r]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int dim = tid + 256 * r;
    if (dim < d_c) st(out + dim, acc[r]);
  }
}

// ---------------------------------------------------------------------------
// append: RoPE on the k^R columns, round, scatter to the slot
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void append_finish_kernel(int d_c, int d_r, int row, int page,
                                                            const float* __restrict__ y,
                                                            const int32_t* __restrict__ positions,
                                                            const int32_t* __restrict__ slots,
                                                            const float* __restrict__ rope,
                                                            int rope_len, T* __restrict__ cache,
                                                            long n_slots) {
  const int t = blockIdx.x;
  const int slot = slots[t];
  const int pos = positions[t];
  if (slot < 0 || (long)slot >= n_slots || pos < 0 || pos >= rope_len) return;
  const float* yr = y + (long)t * row;
  T* dst = cache + (long)slot * row;
  for (int e = threadIdx.x; e < d_c; e += 256) st(dst + e, yr[e]);
  const int half = d_r / 2;
  for (int k = threadIdx.x; k < half; k += 256) {
    float x = yr[d_c + 2 * k], z = yr[d_c + 2 * k + 1];
    float c = rope[((long)pos * half + k) * 2], sn = rope[((long)pos * half + k) * 2 + 1];
    st(dst + d_c + 2 * k, x * c - z * sn);
    st(dst + d_c + 2 * k + 1, x * sn + z * c);
  }
}

// ---------------------------------------------------------------------------
// prefill helpers (fp32 intermediates)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void gather_rows_kernel(int row, int page, const T* __restrict__ cache,
                                                          int num_pages,
                                                          const int32_t* __restrict__ page_table,
                                                          float* __restrict__ rows) {
  const int j = blockIdx.x;
  const int pg = page_table[j / page];
  const bool ok = pg >= 0 && pg < num_pages;
  const T* src = cache + ((long)pg * page + j % page) * row;
  for (int e = threadIdx.x; e < row; e += 256)
    rows[(long)j * row + e] = ok ? ld(src + e) : __builtin_nanf("");
}

__global__ void broadcast_kr_kernel(int n_h, int d_h, int d_c, int d_r, int row,
                                    const float* __restrict__ rows, float* __restrict__ kbuf) {
  const int j = blockIdx.x;
  const int w = d_h + d_r;
  for (int e = threadIdx.x; e < n_h * d_r; e += blockDim.x) {
    int i = e / d_r, k = e % d_r;
    kbuf[((long)j * n_h + i) * w + d_h + k] = rows[(long)j * row + d_c + k];
  }
}

__global__ void rope_inplace_kernel(int n_h, int d_r, float* __restrict__ q, long ld_row, int off,
                                    const int32_t* __restrict__ positions, int T,
                                    const float* __restrict__ rope, int rope_len, int head_stride) {
  long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  int half = d_r / 2;
  long total = (long)T * n_h * half;
  if (idx >= total) return;
  int k = (int)(idx % half);
  long ti = idx / half;
  int i = (int)(ti % n_h);
  int t = (int)(ti / n_h);
  int pos = positions[t];
  float* p = q + (long)t * ld_row + (long)i * head_stride + off + 2 * k;
  float x = p[0], y = p[1];
  if (pos >= 0 && pos < rope_len) {
    float c = rope[((long)pos * half + k) * 2], sn = rope[((long)pos * half + k) * 2 + 1];
    p[0] = x * c - y * sn;
    p[1] = x * sn + y * c;
  } else {
    p[0] = p[1] = __builtin_nanf("");
  }
}

// causal attention in order A: query t, head i over keys j <= positions[t]
__global__ __launch_bounds__(256) void attn_prefill_generic_kernel(
    int n_h, int d_h, int d_r, const float* __restrict__ q, const float* __restrict__ kbuf,
    const float* __restrict__ vbuf, const int32_t* __restrict__ positions, int kv_len,
    float* __restrict__ o) {
  extern __shared__ float sm[];
  const int w = d_h + d_r;
  float* qs = sm;          // [w]
  float* ps = qs + w;      // [256]
  __shared__ float red[4];
  const int t = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const int pos = positions[t];
  float* dst = o + ((long)t * n_h + i) * d_h;
  if (pos < 0 || pos >= kv_len) {
    for (int e = tid; e < d_h; e += 256) dst[e] = __builtin_nanf("");
    return;
  }
  for (int e = tid; e < w; e += 256) qs[e] = q[((long)t * n_h + i) * w + e];
  __syncthreads();
  const int n = pos + 1;
  float acc[2] = {0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 < n; j0 += 256) {
    int j = j0 + tid;
    float sc = -INFINITY;
    if (j < n) {
      const float* kr = kbuf + ((long)j * n_h + i) * w;
      float a = 0.f;
      for (int e = 0; e < w; ++e) a = fmaf(qs[e], kr[e], a);
      sc = a;
    }
    float cm = block_max256(sc, red);
    float mn = fmaxf(m, cm);
    float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
    float p = (j < n) ? expf(sc - mn) : 0.f;
    ps[tid] = p;
    float cs = block_sum256(p, red);
    l = l * alpha + cs;
    m = mn;
    int nj = min(256, n - j0);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      int dim = tid + 256 * r;
      if (dim >= d_h) break;
      float a = acc[r] * alpha;
      for (int jj = 0; jj < nj; ++jj) a = fmaf(ps[jj], vbuf[((long)(j0 + jj) * n_h + i) * d_h + dim], a);
      acc[r] = a;
    }
    __syncthreads();
  }
  for (int r = 0; r < 2; ++r) {
    int dim = tid + 256 * r;
    if (dim < d_h) dst[dim] = acc[r] / l;
  }
}

}  // namespace

hipError_t pack_tiles(const void* src, long R, long C, int elem_bytes, void* dst, hipStream_t s) {
  if (R % 16 != 0 || C % 32 != 0 || (elem_bytes != 2 && elem_bytes != 4)) return hipErrorInvalidValue;
  const long pieces = R * C / 8;
  if (pieces == 0) return hipSuccess;
  const dim3 grid((unsigned)((pieces + 255) / 256));
  if (elem_bytes == 2)
    hipLaunchKernelGGL(pack_tiles_kernel<__bf16>, grid, dim3(256), 0, s, (const __bf16*)src, R, C,
                       (__bf16*)dst);
  else
    hipLaunchKernelGGL(pack_tiles_kernel<float>, grid, dim3(256), 0, s, (const float*)src, R, C,
                       (float*)dst);
  return hipGetLastError();
}

hipError_t gemm_generic(GType ta, GType tb, GType tc, BLayout bk, int M, int N, int K,
                        const void* A, long lda, long sA, const void* B, long ldb, long sB,
                        void* C, long ldc, long sC, int batch, float alpha, hipStream_t s,
                        bool a_kmajor, bool c_tiled) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
#define MLA_G(TA_, TB_, TC_) \
  return gemm_launch<TA_, TB_, TC_>(bk, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch, alpha, \
                                    s, a_kmajor ? 1 : 0, c_tiled ? 1 : 0)
  if (ta == G_F32 && tb == G_F32 && tc == G_F32) MLA_G(float, float, float);
  if (ta == G_BF16 && tb == G_BF16 && tc == G_F32) MLA_G(__bf16, __bf16, float);
  if (ta == G_BF16 && tb == G_BF16 && tc == G_BF16) MLA_G(__bf16, __bf16, __bf16);
  if (ta == G_F32 && tb == G_BF16 && tc == G_F32) MLA_G(float, __bf16, float);
  if (ta == G_F32 && tb == G_BF16 && tc == G_BF16) MLA_G(float, __bf16, __bf16);
  if (ta == G_BF16 && tb == G_F32 && tc == G_F32) MLA_G(__bf16, float, float);
#undef MLA_G
  return hipErrorInvalidValue;
}

hipError_t rope_table_fill(float* table, int max_pos, int d_r, double base, hipStream_t s) {
  long n = (long)max_pos * (d_r / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, table,
                     max_pos, d_r, base);
  return hipGetLastError();
}

hipError_t pack_query_rope(const Geo& g, const float* q_r, const int32_t* positions, int B,
                           const float* rope, int rope_len, void* q_abs, hipStream_t s) {
  long n = (long)B * g.n_h * (g.d_r / 2);
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  if (g.bf16)
    hipLaunchKernelGGL(pack_query_rope_kernel<__bf16>, grid, dim3(256), 0, s, g.n_h, g.d_c, g.d_r,
                       g.row, g.scale, q_r, positions, B, rope, rope_len, (__bf16*)q_abs);
  else
    hipLaunchKernelGGL(pack_query_rope_kernel<float>, grid, dim3(256), 0, s, g.n_h, g.d_c, g.d_r,
                       g.row, g.scale, q_r, positions, B, rope, rope_len, (float*)q_abs);
  return hipGetLastError();
}

hipError_t attn_decode_generic(const Geo& g, const void* q_abs, const void* cache, int num_pages,
                               const int32_t* page_table, int max_pages, const PlanPtrs& plan,
                               int max_segs, float* part_o, float* part_ml, void* lat_out,
                               hipStream_t s) {
  if (max_segs <= 0) return hipSuccess;
  dim3 grid(max_segs, g.n_h);
  size_t shm = sizeof(float) * ((g.row + 256 + 1) & ~1) + sizeof(long) * 256;
  if (g.bf16)
    hipLaunchKernelGGL(attn_decode_generic_kernel<__bf16>, grid, dim3(256), shm, s, g.n_h, g.d_c,
                       g.row, g.page, (const __bf16*)q_abs, (const __bf16*)cache, num_pages,
                       page_table, max_pages, plan, part_o, part_ml, (__bf16*)lat_out);
  else
    hipLaunchKernelGGL(attn_decode_generic_kernel<float>, grid, dim3(256), shm, s, g.n_h, g.d_c,
                       g.row, g.page, (const float*)q_abs, (const float*)cache, num_pages,
                       page_table, max_pages, plan, part_o, part_ml, (float*)lat_out);
  return hipGetLastError();
}

hipError_t combine_partials(const Geo& g, const PlanPtrs& plan, int B, const float* part_o,
                            const float* part_ml, void* lat_out, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  dim3 grid(B, g.n_h);
  if (g.bf16)
    hipLaunchKernelGGL(combine_kernel<__bf16>, grid, dim3(256), 0, s, g.n_h, g.d_c, plan, part_o,
                       part_ml, (__bf16*)lat_out);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, g.n_h, g.d_c, plan, part_o,
                       part_ml, (float*)lat_out);
  return hipGetLastError();
}

hipError_t append_finish(const Geo& g, const float* y, const int32_t* positions,
                         const int32_t* slots, int T, const float* rope, int rope_len,
                         void* cache, int num_pages, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  long n_slots = (long)num_pages * g.page;
  if (g.bf16)
    hipLaunchKernelGGL(append_finish_kernel<__bf16>, dim3(T), dim3(256), 0, s, g.d_c, g.d_r, g.row,
                       g.page, y, positions, slots, rope, rope_len, (__bf16*)cache, n_slots);
  else
    hipLaunchKernelGGL(append_finish_kernel<float>, dim3(T), dim3(256), 0, s, g.d_c, g.d_r, g.row,
                       g.page, y, positions, slots, rope, rope_len, (float*)cache, n_slots);
  return hipGetLastError();
}

hipError_t gather_rows_f32(const Geo& g, const void* cache, int num_pages, const int32_t* page_table,
                           int max_pages, int kv_len, float* rows, hipStream_t s) {
  (void)max_pages;
  if (kv_len <= 0) return hipSuccess;
  if (g.bf16)
    hipLaunchKernelGGL(gather_rows_kernel<__bf16>, dim3(kv_len), dim3(256), 0, s, g.row, g.page,
                       (const __bf16*)cache, num_pages, page_table, rows);
  else
    hipLaunchKernelGGL(gather_rows_kernel<float>, dim3(kv_len), dim3(256), 0, s, g.row, g.page,
                       (const float*)cache, num_pages, page_table, rows);
  return hipGetLastError();
}

hipError_t broadcast_kr(const Geo& g, const float* rows, int kv_len, float* kbuf, hipStream_t s) {
  if (kv_len <= 0) return hipSuccess;
  hipLaunchKernelGGL(broadcast_kr_kernel, dim3(kv_len), dim3(256), 0, s, g.n_h, g.d_h, g.d_c,
                     g.d_r, g.row, rows, kbuf);
  return hipGetLastError();
}

hipError_t rope_inplace_heads(const Geo& g, float* q, int T, long ld_row, int off,
                              const int32_t* positions, const float* rope, int rope_len,
                              hipStream_t s) {
  long n = (long)T * g.n_h * (g.d_r / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_inplace_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g.n_h,
                     g.d_r, q, ld_row, off, positions, T, rope, rope_len, g.d_h + g.d_r);
  return hipGetLastError();
}

hipError_t attn_prefill_generic(const Geo& g, const float* q, const float* kbuf, const float* vbuf,
                                const int32_t* positions, int T, int kv_len, int rope_len,
                                float* o, hipStream_t s) {
  (void)rope_len;
  if (T <= 0) return hipSuccess;
  size_t shm = sizeof(float) * (g.d_h + g.d_r + 256);
  hipLaunchKernelGGL(attn_prefill_generic_kernel, dim3(T, g.n_h), dim3(256), shm, s, g.n_h, g.d_h,
                     g.d_r, q, kbuf, vbuf, positions, kv_len, o);
  return hipGetLastError();
}

}  // namespace mla
