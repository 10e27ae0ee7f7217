// Order-A attention backward ([walkthrough] §3 顺序 A: training keeps W_UK and
// W_UV as two matrices, so each gets its own gradient).  The products of the
// chain rule run on the generic GEMM; this file holds the two steps that are
// not products:
//   * per (query t, head i): the causal scores, the softmax p_tij and
//     ds_tij = p_tij (dp_tij - sum_j' p_tij' dp_tij'), dp_tij = dO_ti . v_ij,
//     stored as [n_h][T][N] (zero past the query's position);
//   * the assembly of dC = [dc_j | dk^R_j] from the per-head pieces.
// fp32 throughout; sized for training-step checks, not tuned.
#include <math.h>

#include "mla_internal.h"

namespace mla {

namespace {

__device__ inline float bwd_block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ inline float bwd_block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// one work-group (256 threads) per (query t, head i); dynamic LDS holds q_ti
// (d_h + d_r) and dO_ti (d_h)
__global__ __launch_bounds__(256) void attn_bwd_ps_kernel(
    int n_h, int d_h, int d_r, int d_c, int row, int N, int T, float scale,
    const float* __restrict__ q, const int32_t* __restrict__ positions,
    const float* __restrict__ K, const float* __restrict__ V, const float* __restrict__ rows,
    const float* __restrict__ dO, float* __restrict__ P, float* __restrict__ dS) {
  extern __shared__ float sm[];
  __shared__ float red[4];
  const int t = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const int dq = d_h + d_r;
  float* qs = sm;
  float* ds = sm + dq;
  for (int e = tid; e < dq; e += 256) qs[e] = q[((long)t * n_h + i) * dq + e];
  for (int e = tid; e < d_h; e += 256) ds[e] = dO[((long)t * n_h + i) * d_h + e];
  __syncthreads();
  const int pos = positions[t];
  const bool valid = pos >= 0 && pos < N;
  const int last = valid ? pos : -1;
  float* Pr = P + ((long)i * T + t) * N;
  float* Dr = dS + ((long)i * T + t) * N;
  // scores (kept in P for the next pass) and their max
  float mx = -INFINITY;
  for (int j = tid; j < N; j += 256) {
    float s = -INFINITY;
    if (j <= last) {
      const float* kj = K + ((long)j * n_h + i) * d_h;
      const float* rj = rows + (long)j * row + d_c;
      float a = 0.f;
      for (int e = 0; e < d_h; ++e) a = fmaf(qs[e], kj[e], a);
      for (int e = 0; e < d_r; ++e) a = fmaf(qs[d_h + e], rj[e], a);
      s = scale * a;
    }
    Pr[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = bwd_block_max(mx, red);
  // numerators and dp
  float sum = 0.f;
  for (int j = tid; j < N; j += 256) {
    float p = 0.f, dp = 0.f;
    if (j <= last) {
      p = expf(Pr[j] - mx);
      const float* vj = V + ((long)j * n_h + i) * d_h;
      for (int e = 0; e < d_h; ++e) dp = fmaf(ds[e], vj[e], dp);
    }
    Pr[j] = p;
    Dr[j] = dp;
    sum += p;
  }
  sum = bwd_block_sum(sum, red);
  const float inv = 1.f / sum;
  float D = 0.f;
  for (int j = tid; j < N; j += 256) {
    const float p = Pr[j] * inv;
    Pr[j] = p;
    D = fmaf(p, Dr[j], D);
  }
  D = bwd_block_sum(D, red);
  const float nanv = __builtin_nanf("");
  for (int j = tid; j < N; j += 256) {
    const float p = Pr[j];
    Dr[j] = valid ? p * (Dr[j] - D) : nanv;
    if (!valid) Pr[j] = nanv;
  }
}

// dC[j] = [lat_k[j] + lat_v[j] | sum_i dkr[i][j]]
__global__ void attn_bwd_dc_kernel(int N, int d_c, int d_r, int n_h, const float* __restrict__ lat_k,
                                   const float* __restrict__ lat_v, const float* __restrict__ dkr,
                                   float* __restrict__ dC) {
  const int row = d_c + d_r;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)N * row) return;
  const int j = (int)(idx / row), e = (int)(idx % row);
  if (e < d_c) {
    dC[idx] = lat_k[(long)j * d_c + e] + lat_v[(long)j * d_c + e];
  } else {
    float a = 0.f;
    for (int i = 0; i < n_h; ++i) a += dkr[((long)i * N + j) * d_r + (e - d_c)];
    dC[idx] = a;
  }
}

}  // namespace

hipError_t attn_bwd_ps(const Geo& g, int N, int T, float scale, const float* q,
                       const int32_t* positions, const float* K, const float* V,
                       const float* rows, const float* dO, float* P, float* dS, hipStream_t s) {
  if (N <= 0 || T <= 0) return hipSuccess;
  const size_t shm = sizeof(float) * (size_t)(2 * g.d_h + g.d_r);
  hipLaunchKernelGGL(attn_bwd_ps_kernel, dim3(T, g.n_h), dim3(256), shm, s, g.n_h, g.d_h, g.d_r,
                     g.d_c, g.row, N, T, scale, q, positions, K, V, rows, dO, P, dS);
  return hipGetLastError();
}

hipError_t attn_bwd_dc(const Geo& g, int N, const float* lat_k, const float* lat_v,
                       const float* dkr, float* dC, hipStream_t s) {
  const long n = (long)N * g.row;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_bwd_dc_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, N,
                     g.d_c, g.d_r, g.n_h, lat_k, lat_v, dkr, dC);
  return hipGetLastError();
}

}  // namespace mla
