// Weight-streaming MFMA GEMMs of the decode step (bf16 weights, fp32 accumulate).
//
// At decode every projection is a skinny product Y[B][N] = X[B][K] . W[N][K]^T
// with B <= 64 rows of activations against a large weight matrix, so each
// kernel is bound by streaming W from HBM once.  Layer steps served here:
//   c^Q = W_DQ h                  formula page eq. (12)
//   q^C = W_UQ c^Q, W_QR c^Q      formula page eq. (13); walkthrough step 3
//   q~_i = W_UK,i^T q^C_i         walkthrough §3 顺序 B (absorption)
//   o_i = W_UV,i o~_i             walkthrough §3 顺序 B (decompress once)
//   u = W_O [o_0 | ... | o_127]   walkthrough step 5
//
// wgemm: a work-group owns 64 weight rows and a K slice; its four waves split
// that slice four ways, each streaming 16-byte pieces of W straight into the
// B operand of v_mfma_f32_16x16x32_bf16 (lane = weight row, 8 consecutive k),
// with the activation rows as the A operand, then the four partial tiles are
// summed in LDS in a fixed order.  Split-K across work-groups writes fp32
// partials that a small kernel reduces in a fixed order (deterministic).
#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNT = 64;   // weight rows per work-group
constexpr int kMT = 64;   // activation rows per work-group (4 MFMA blocks of 16)

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Y = alpha * X . W^T over one K split.  X row m of the n-th weight-row group
// lives at X + (n / n_group) * x_group_stride + m * ldx.
template <bool OUT_F32>
__global__ __launch_bounds__(256, 2) void wgemm_kernel(int M, int N, int K, int k_split,
                                                       const __bf16* __restrict__ X, long ldx,
                                                       long x_group_stride, int n_group,
                                                       const __bf16* __restrict__ W,
                                                       void* __restrict__ Y, long ldy,
                                                       long y_split_stride, float alpha) {
  __shared__ f32x4 red[4][4][4][64];  // [wave][mb][nb][lane]
  const int n0 = blockIdx.x * kNT;
  const int split = blockIdx.y;
  const int m0 = blockIdx.z * kMT;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int kt = K / k_split;
  const int kw = kt >> 2;
  const int kbeg = split * kt + wave * kw + 8 * g;
  const int nmb = min(4, (M - m0 + 15) >> 4);
  const __bf16* xb = X + (long)(n0 / n_group) * x_group_stride;
  const bf16x8* xr[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = min(m0 + mb * 16 + r16, M - 1);
    xr[mb] = (const bf16x8*)(xb + (long)m * ldx + kbeg);
  }
  const bf16x8* wr[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) wr[nb] = (const bf16x8*)(W + (long)(n0 + nb * 16 + r16) * K + kbeg);

  f32x4 acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{};

#pragma unroll 4
  for (int k = 0; k < kw; k += 32) {
    bf16x8 b[4], a[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) b[nb] = wr[nb][k >> 3];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) a[mb] = xr[mb][k >> 3];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb < nmb) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma16(a[mb], b[nb], acc[mb][nb]);
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) red[wave][mb][nb][lane] = acc[mb][nb];
  __syncthreads();
  // wave w finishes activation block w: fixed-order sum over the four waves
  const int mb = wave;
  if (mb >= nmb) return;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    f32x4 v = red[0][mb][nb][lane];
    v += red[1][mb][nb][lane];
    v += red[2][mb][nb][lane];
    v += red[3][mb][nb][lane];
    const int n = n0 + nb * 16 + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + mb * 16 + 4 * g + i;
      if (m < M) {
        if (OUT_F32)
          ((float*)Y)[split * y_split_stride + (long)m * ldy + n] = alpha * v[i];
        else
          ((__bf16*)Y)[(long)m * ldy + n] = (__bf16)(alpha * v[i]);
      }
    }
  }
}

// out[m][n] = sum_s part[s][m][n] (fixed order), as bf16
__global__ void splitk_reduce_kernel(int M, int N, int S, const float* __restrict__ part,
                                     long split_stride, __bf16* __restrict__ out, long ldo) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[s * split_stride + (long)m * N + n];
  out[(long)m * ldo + n] = (__bf16)v;
}

// q~_i = scale * W_UK,i^T q^C_i for one head i (grid.x) and 64 batch rows
// (grid.y).  W_UK,i is [128 d][512 c]; the contraction runs over its row index,
// so each lane reads eight consecutive rows (d) of one 16-byte column chunk and
// transposes them in registers into eight B operands: N block j covers
// c = 128 * wave + 8 * r16 + j.
__global__ __launch_bounds__(256, 1) void absorb_kernel(int M, const __bf16* __restrict__ qc,
                                                        const __bf16* __restrict__ W_UK,
                                                        __bf16* __restrict__ q_abs, float scale) {
  const int head = blockIdx.x;
  const int m0 = blockIdx.y * kMT;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int nmb = min(4, (M - m0 + 15) >> 4);
  const __bf16* w = W_UK + (long)head * 128 * 512 + 128 * wave + 8 * r16;
  f32x4 acc[4][8];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[mb][j] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = *(const u32x4*)(w + (long)(32 * ks + 8 * g + r) * 512);
    bf16x8 a[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = min(m0 + mb * 16 + r16, M - 1);
      a[mb] = *(const bf16x8*)(qc + (long)m * 16384 + head * 128 + 32 * ks + 8 * g);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x4 lo, hi;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        lo[f] = __builtin_amdgcn_perm(v[2 * f + 1][e], v[2 * f][e], 0x05040100u);
        hi[f] = __builtin_amdgcn_perm(v[2 * f + 1][e], v[2 * f][e], 0x07060302u);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < nmb) {
          acc[mb][2 * e] = mfma16(a[mb], __builtin_bit_cast(bf16x8, lo), acc[mb][2 * e]);
          acc[mb][2 * e + 1] = mfma16(a[mb], __builtin_bit_cast(bf16x8, hi), acc[mb][2 * e + 1]);
        }
      }
    }
  }
  // D: lane holds column r16 (c = 128 wave + 8 r16 + j) and rows 4g + i
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb >= nmb) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + mb * 16 + 4 * g + i;
      if (m >= M) continue;
      bf16x8 o;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = (__bf16)(scale * acc[mb][j][i]);
      *(bf16x8*)(q_abs + ((long)m * 128 + head) * 576 + 128 * wave + 8 * r16) = o;
    }
  }
}

}  // namespace

bool wgemm_shape_ok(int N, int K, int k_split) {
  return N % kNT == 0 && k_split > 0 && K % (k_split * 128) == 0;
}

hipError_t wgemm(int M, int N, int K, int k_split, const void* X, long ldx, long x_group_stride,
                 int n_group, const void* W, void* Y, long ldy, long y_split_stride, bool out_f32,
                 float alpha, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  dim3 grid(N / kNT, k_split, (M + kMT - 1) / kMT);
  if (out_f32)
    hipLaunchKernelGGL(wgemm_kernel<true>, grid, dim3(256), 0, s, M, N, K, k_split,
                       (const __bf16*)X, ldx, x_group_stride, n_group, (const __bf16*)W, Y, ldy,
                       y_split_stride, alpha);
  else
    hipLaunchKernelGGL(wgemm_kernel<false>, grid, dim3(256), 0, s, M, N, K, k_split,
                       (const __bf16*)X, ldx, x_group_stride, n_group, (const __bf16*)W, Y, ldy,
                       y_split_stride, alpha);
  return hipGetLastError();
}

hipError_t splitk_reduce(int M, int N, int S, const float* part, long split_stride, void* out,
                         long ldo, hipStream_t s) {
  long n = (long)M * N;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, M,
                     N, S, part, split_stride, (__bf16*)out, ldo);
  return hipGetLastError();
}

hipError_t absorb_v2(int M, const void* qc, const void* W_UK, void* q_abs, float scale,
                     hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(absorb_kernel, dim3(128, (M + kMT - 1) / kMT), dim3(256), 0, s, M,
                     (const __bf16*)qc, (const __bf16*)W_UK, (__bf16*)q_abs, scale);
  return hipGetLastError();
}

}  // namespace mla
