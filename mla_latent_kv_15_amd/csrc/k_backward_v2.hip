// Order-A attention backward for the DeepSeek-V2 heads (n_h = 128, scores
// over 192 numbers, values of 128) on bf16 MFMA, flash style: the softmax
// probabilities are recomputed per block of 32 queries x 32 keys and never
// stored ([walkthrough] §3 顺序 A: training keeps W_UK and W_UV as two
// matrices, so the attention's gradients are taken per head in order A).
//
// For head i, with Q = scale * q (bf16), K = [W_UK,i c | k^R], V = W_UV,i c,
// S = Q K^T, P = softmax_causal(S), O = P V and the incoming dO:
//   dP = dO V^T,  D_t = sum_j P_tj dP_tj (= dO_t . O_t),
//   dS = P o (dP - D),  dV = P^T dO,  dK = dS^T Q,  dq = scale * dS K.
// A query whose position lies outside [0, kv_len) gets NaN rows of P and dS
// over every key, so its dq row and every key's dK and dV are NaN (the
// generic path's rule).
//
// Two kernels, both four waves per work-group and one MFMA tile of 32 x 32
// per wave (v_mfma_f32_32x32x16_bf16):
//  * the query side (one wave per 32 queries of a head, key blocks staged in
//    LDS once for the four waves): pass 1 recomputes S^T = K Q^T and
//    dP^T = V dO^T per key block and keeps, per query, the running maximum,
//    the sum of exponentials l and the sum z of exponentials times dP (all
//    rescaled together), so that LSE = m + log2 l and D = z / l come out
//    without forming O; pass 2 recomputes S^T and dP^T, forms dS^T and
//    accumulates dQ^T += K^T dS^T (K^T by transposing LDS reads).  It
//    writes dq, LSE and D, and each query block's furthest visible key.
//  * the key side (one wave per 32 keys of a head, query blocks staged in
//    LDS once for the four waves): with keys as the MFMA columns, S = Q K^T
//    and dP = dO V^T give P and dS per (query, key) from the stored LSE and
//    D; dV^T += dO^T P and dK^T += Q^T dS (dO^T and Q^T by transposing LDS
//    reads).  Query blocks that see none of the work-group's keys are
//    skipped.  It writes dk^R per head in fp32 and the latent parts dk^C and
//    dv in bf16 twice: as rows [key][dk^C of every head | dv of every head]
//    (the left operand of dc = sum_i W_UK,i^T dk^C_i + W_UV,i^T dv_i) and
//    key-contiguous [head, dim][key] (the left operand of dW_UK,i =
//    sum_j dk^C_ij c_j^T and dW_UV,i), both for the MFMA GEMMs that follow.
// The numerators enter the second products as bf16 (the B operand), with
// fp32 accumulation throughout.
#include <math.h>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) v4bf16 lds_v4bf16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kH = 128;          // heads
constexpr int kW = 192;          // query and key width
constexpr int kDv = 128;         // value width
constexpr int kB = 32;           // queries or keys per wave tile
constexpr int kWv = 4;           // waves per work-group
constexpr int kQK = kW / 16;     // K-steps of the 192-wide products (12)
constexpr int kVK = kDv / 16;    // K-steps of the 128-wide products (8)
constexpr float kLog2e = 1.4426950408889634f;
// LDS rows: 192-wide rows padded to 200 bf16 (the 16 rows a row read serves
// at once start at distinct 16-byte bank groups); 128-wide rows read only
// as rows padded to 136; 128-wide rows read mostly by transposing reads
// padded to 160 (the four rows such a read serves at once start 64 banks
// apart).
constexpr int kRow192 = kW + 8;
constexpr int kRowRd = kDv + 8;
constexpr int kRowTr = kDv + 32;

__device__ inline uint32_t pack2(float x, float y) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x, (__bf16)y});
}

// MFMA operand layouts (32 x 32 x 16): lane l = (c, h), c = l & 31,
// h = l >> 5.  A[m][k]: lane holds row m = c, k = 8h .. 8h + 7.  B[k][n]:
// lane holds column n = c, k = 8h .. 8h + 7.  D[m][n]: lane holds column
// n = c, rows 8 (r >> 2) + 4h + (r & 3) for r = 0 .. 15.

// A D-layout tile X (rows 8 (r >> 2) + 4h + (r & 3) of column c) as two B
// operands over its rows: pb[kap] holds rows 16 kap + 8h .. + 7 of column
// c, rounded to bf16.  A lane holds rows 4h .. 4h + 3 (+ 8, 16, 24); the lane
// 32 apart holds the other four of each eight.
__device__ inline void rows_as_b(const f32x16& X, bf16x8 (&pb)[2]) {
  uint32_t R[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) R[k] = pack2(X[2 * k], X[2 * k + 1]);
#pragma unroll
  for (int k = 0; k < 8; k += 4) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(R[k], R[k + 2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(R[k + 1], R[k + 3], false, false);
    R[k] = s0[0];
    R[k + 2] = s0[1];
    R[k + 1] = s1[0];
    R[k + 3] = s1[1];
  }
  pb[0] = __builtin_bit_cast(bf16x8, u32x4{R[0], R[1], R[2], R[3]});
  pb[1] = __builtin_bit_cast(bf16x8, u32x4{R[4], R[5], R[6], R[7]});
}

// The A operand "columns D0 .. D0 + 31 of rows k0 + 8h .. + 7" of a
// row-major LDS block (byte base `base`, `pitch` bf16 per row), transposed:
// lane (c, h) receives column D0 + c of those eight rows.  Two transposing
// reads of four rows each: in each 16-lane group lane s supplies the 8-byte
// chunk of row k0 + 8h + s / 4, columns D0 + 16 (group & 1) + 4 (s % 4), and
// output lane i receives, as its element r, element i % 4 of lane
// 4 r + i / 4's chunk.
__device__ inline bf16x8 tr_operand(lds_char* lds, int base, int pitch, int k0, int D0) {
  const int lane = threadIdx.x & 63;
  const int row = k0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = D0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int b = base + 2 * (row * pitch + col);
  const v4bf16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(lds + b));
  const v4bf16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(lds + b + 2 * 4 * pitch));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline float swap_max(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float swap_sum(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// ---------------------------------------------------------------------------
// query side: LSE, D and dq
// ---------------------------------------------------------------------------
constexpr int kKElemsA = kB * kRow192;             // K block
constexpr int kBufA = kKElemsA + kB * kRowRd;      // + V block (rows)

__global__ __launch_bounds__(256, 1) void attn_bwd_dq_v2_kernel(
    const __bf16* __restrict__ q16, const __bf16* __restrict__ do16,
    const __bf16* __restrict__ k16, const __bf16* __restrict__ v16,
    const int32_t* __restrict__ positions, int T, int N, float scale, float* __restrict__ lse_out,
    float* __restrict__ d_out, int* __restrict__ qblk_far, float* __restrict__ dq) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][kBufA];
  __shared__ int s_far[kWv];
  const int i = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
  const int qb = blockIdx.x * kWv + wave;   // this wave's block of 32 queries
  const int t = qb * kB + c;
  const bool t_ok = t < T;
  const int pos = t_ok ? positions[t] : -1;
  const bool valid = pos >= 0 && pos < N;
  // keys this query sees: 0 .. last (an invalid position: all of them, NaN)
  const int last = t_ok ? (valid ? pos : N - 1) : -1;
  int far = last;
  for (int off = 32; off >= 1; off >>= 1) far = max(far, __shfl_xor(far, off));
  if (lane == 0) {
    s_far[wave] = far;
    if (i == 0 && qb * kB < T) qblk_far[qb] = far;
  }
  __syncthreads();
  const int far_wg = max(max(s_far[0], s_far[1]), max(s_far[2], s_far[3]));
  const int nkb = (far_wg + kB) / kB;   // key blocks the work-group stages

  // Q^T and dO^T as B operands: K-step ks holds dims 16 ks + 8h .. + 7
  bf16x8 qv[kQK], dv[kVK];
  {
    const long row = (long)(t_ok ? t : 0) * kH + i;
#pragma unroll
    for (int ks = 0; ks < kQK; ++ks) qv[ks] = *(const bf16x8*)(q16 + row * kW + 16 * ks + 8 * h);
#pragma unroll
    for (int ks = 0; ks < kVK; ++ks)
      dv[ks] = *(const bf16x8*)(do16 + row * kDv + 16 * ks + 8 * h);
  }
  // staging: K pieces p = tid + 256 r (key p / 24, piece p % 24), V pieces
  // (key p / 16, dims 8 (p % 16) ..); keys past N repeat the last one
  uint4 k0r, k1r, k2r, v0r, v1r;
  auto kpiece = [&](int kb, int r) {
    const int p = tid + 256 * r, key = p / (kW / 8), pc = p % (kW / 8);
    return *(const uint4*)(k16 + ((long)min(kb * kB + key, N - 1) * kH + i) * kW + 8 * pc);
  };
  auto vpiece = [&](int kb, int r) {
    const int p = tid + 256 * r, key = p / (kDv / 8), pc = p % (kDv / 8);
    return *(const uint4*)(v16 + ((long)min(kb * kB + key, N - 1) * kH + i) * kDv + 8 * pc);
  };
  auto gload = [&](int kb) {
    k0r = kpiece(kb, 0);
    k1r = kpiece(kb, 1);
    k2r = kpiece(kb, 2);
    v0r = vpiece(kb, 0);
    v1r = vpiece(kb, 1);
  };
  auto lstore = [&](int buf) {
    __bf16* K = lds[buf];
    auto ks_ = [&](int r, uint4 x) {
      const int p = tid + 256 * r, key = p / (kW / 8), pc = p % (kW / 8);
      *(uint4*)(K + key * kRow192 + 8 * pc) = x;
    };
    auto vs_ = [&](int r, uint4 x) {
      const int p = tid + 256 * r, key = p / (kDv / 8), pc = p % (kDv / 8);
      *(uint4*)(K + kKElemsA + key * kRowRd + 8 * pc) = x;
    };
    ks_(0, k0r);
    ks_(1, k1r);
    ks_(2, k2r);
    vs_(0, v0r);
    vs_(1, v1r);
  };
  // S^T = K Q^T and dP^T = V dO^T of key block kb (rows: keys, column: query)
  auto scores = [&](const __bf16* K, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kQK; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *(const bf16x8*)(K + c * kRow192 + 16 * ks + 8 * h), qv[ks], s, 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < kVK; ++ks)
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *(const bf16x8*)(K + kKElemsA + c * kRowRd + 16 * ks + 8 * h), dv[ks], dp, 0, 0, 0);
  };

  // ---- pass 1: m, l, z of this lane's query (log2 units)
  float m = -INFINITY, l = 0.f, z = 0.f;
  if (nkb > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) gload(kb + 1);
    const int j0 = kb * kB;
    if (j0 <= far) {
      f32x16 s, dp;
      scores(lds[kb & 1], s, dp);
      float bm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
        s[r] = key <= last ? s[r] * kLog2e : -INFINITY;
        bm = fmaxf(bm, s[r]);
      }
      const float mn = fmaxf(m, swap_max(bm));
      const float ref = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m - ref);
      float ps = 0.f, zs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[r] - ref);
        ps += p;
        zs = fmaf(p, dp[r], zs);
      }
      l = l * alpha + swap_sum(ps);
      z = z * alpha + swap_sum(zs);
      m = mn;
    }
    if (kb + 1 < nkb) lstore((kb + 1) & 1);
    __syncthreads();
  }
  const float nanv = __builtin_nanf("");
  const float lse = valid ? m + __log2f(l) : nanv;
  const float dd = valid ? z / l : nanv;
  if (t_ok && h == 0) {
    lse_out[(long)i * T + t] = lse;
    d_out[(long)i * T + t] = dd;
  }

  // ---- pass 2: dQ^T += K^T dS^T
  f32x16 acc[kW / 32];
#pragma unroll
  for (int dt = 0; dt < kW / 32; ++dt) acc[dt] = f32x16{};
  if (nkb > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) gload(kb + 1);
    const int j0 = kb * kB;
    if (j0 <= far) {
      f32x16 s, dp;
      scores(lds[kb & 1], s, dp);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
        const float p = key <= last ? __builtin_amdgcn_exp2f(fmaf(s[r], kLog2e, -lse)) : 0.f;
        s[r] = p * (dp[r] - dd);   // dS^T
      }
      bf16x8 pb[2];
      rows_as_b(s, pb);
      const int base = (kb & 1) * 2 * kBufA;
#pragma unroll
      for (int kap = 0; kap < 2; ++kap)
#pragma unroll
        for (int dt = 0; dt < kW / 32; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_operand((lds_char*)lds, base, kRow192, 16 * kap, 32 * dt), pb[kap], acc[dt], 0,
              0, 0);
    }
    if (kb + 1 < nkb) lstore((kb + 1) & 1);
    __syncthreads();
  }
  if (!t_ok) return;
  // lane (c, h) holds dims 32 dt + 8 g + 4h .. + 3 (g = r >> 2) of query t
  float* dst = dq + ((long)t * kH + i) * kW + 4 * h;
#pragma unroll
  for (int dt = 0; dt < kW / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(dst + 32 * dt + 8 * g) =
          f32x4{scale * acc[dt][4 * g], scale * acc[dt][4 * g + 1], scale * acc[dt][4 * g + 2],
                scale * acc[dt][4 * g + 3]};
}

// ---------------------------------------------------------------------------
// key side: dK (its latent part per head, its RoPE part per head) and dV
// ---------------------------------------------------------------------------
constexpr int kQElemsB = kB * kRow192;             // Q block
constexpr int kBufB = kQElemsB + kB * kRowTr;      // + dO block
constexpr int kMaxQbLds = 1024;                    // query blocks whose far key sits in LDS
constexpr int kTrPitch = kB + 8;                   // keys per LDS row of the transposed tiles
static_assert(kWv * kDv * kTrPitch * 2 <= 2 * kBufB * 2, "transposed tiles fit the ring");

__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_v2_kernel(
    const __bf16* __restrict__ q16, const __bf16* __restrict__ do16,
    const __bf16* __restrict__ k16, const __bf16* __restrict__ v16,
    const int32_t* __restrict__ positions, const float* __restrict__ lse_in,
    const float* __restrict__ d_in, const int* __restrict__ qblk_far, int T, int N, int Npad,
    __bf16* __restrict__ dkv16, __bf16* __restrict__ dkT16, __bf16* __restrict__ dvT16,
    float* __restrict__ dkr) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][kBufB];
  __shared__ __attribute__((aligned(16))) float s_lse[2][kB];
  __shared__ __attribute__((aligned(16))) float s_d[2][kB];
  __shared__ __attribute__((aligned(16))) int s_last[2][kB];
  __shared__ int s_qf[kMaxQbLds];
  const int i = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
  const int wg_j0 = blockIdx.x * kWv * kB;
  const int j0 = wg_j0 + wave * kB;   // this wave's block of 32 keys
  const int key = j0 + c;
  const bool key_ok = key < N;

  // K^T and V^T as B operands (column: key c, K-step ks: dims 16 ks + 8h ..)
  bf16x8 kv[kQK], vv[kVK];
  {
    const long row = (long)min(key, N - 1) * kH + i;
#pragma unroll
    for (int ks = 0; ks < kQK; ++ks) kv[ks] = *(const bf16x8*)(k16 + row * kW + 16 * ks + 8 * h);
#pragma unroll
    for (int ks = 0; ks < kVK; ++ks) vv[ks] = *(const bf16x8*)(v16 + row * kDv + 16 * ks + 8 * h);
  }
  // staging of query block qb: Q pieces (query p / 24, piece p % 24), dO
  // pieces (query p / 16, dims 8 (p % 16) ..), queries past T repeat the
  // last one; per query LSE, D and the last key it sees (-1 past T)
  uint4 q0r, q1r, q2r, d0r, d1r;
  float lse_r = 0.f, d_r = 0.f;
  int last_r = -1;
  auto qpiece = [&](int qb, int r) {
    const int p = tid + 256 * r, qq = p / (kW / 8), pc = p % (kW / 8);
    return *(const uint4*)(q16 + ((long)min(qb * kB + qq, T - 1) * kH + i) * kW + 8 * pc);
  };
  auto dpiece = [&](int qb, int r) {
    const int p = tid + 256 * r, qq = p / (kDv / 8), pc = p % (kDv / 8);
    return *(const uint4*)(do16 + ((long)min(qb * kB + qq, T - 1) * kH + i) * kDv + 8 * pc);
  };
  auto gload = [&](int qb) {
    q0r = qpiece(qb, 0);
    q1r = qpiece(qb, 1);
    q2r = qpiece(qb, 2);
    d0r = dpiece(qb, 0);
    d1r = dpiece(qb, 1);
    if (tid < kB) {
      const int t = qb * kB + tid;
      if (t < T) {
        const int p = positions[t];
        const bool valid = p >= 0 && p < N;
        last_r = valid ? p : N - 1;
        lse_r = lse_in[(long)i * T + t];
        d_r = d_in[(long)i * T + t];
      } else {
        last_r = -1;
        lse_r = 0.f;
        d_r = 0.f;
      }
    }
  };
  auto lstore = [&](int buf) {
    __bf16* Q = lds[buf];
    auto qs_ = [&](int r, uint4 x) {
      const int p = tid + 256 * r, qq = p / (kW / 8), pc = p % (kW / 8);
      *(uint4*)(Q + qq * kRow192 + 8 * pc) = x;
    };
    auto ds_ = [&](int r, uint4 x) {
      const int p = tid + 256 * r, qq = p / (kDv / 8), pc = p % (kDv / 8);
      *(uint4*)(Q + kQElemsB + qq * kRowTr + 8 * pc) = x;
    };
    qs_(0, q0r);
    qs_(1, q1r);
    qs_(2, q2r);
    ds_(0, d0r);
    ds_(1, d1r);
    if (tid < kB) {
      s_lse[buf][tid] = lse_r;
      s_d[buf][tid] = d_r;
      s_last[buf][tid] = last_r;
    }
  };

  f32x16 accK[kW / 32], accV[kDv / 32];
#pragma unroll
  for (int dt = 0; dt < kW / 32; ++dt) accK[dt] = f32x16{};
#pragma unroll
  for (int dt = 0; dt < kDv / 32; ++dt) accV[dt] = f32x16{};

  // the query blocks that see at least one key of the work-group; the
  // decision is the same for every thread (qblk_far is per query block).
  // The first kMaxQbLds blocks' far keys are read once into LDS, so that the
  // scan below costs no memory round trips.
  const int nqb = (T + kB - 1) / kB;
  for (int e = tid; e < min(nqb, kMaxQbLds); e += 256) s_qf[e] = qblk_far[e];
  __syncthreads();
  auto qfar = [&](int qb) { return qb < kMaxQbLds ? s_qf[qb] : qblk_far[qb]; };
  auto next_active = [&](int qb) {
    while (qb < nqb && qfar(qb) < wg_j0) ++qb;
    return qb;
  };
  int qb = next_active(0);
  if (qb < nqb) {
    gload(qb);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;
  while (qb < nqb) {
    const int qn = next_active(qb + 1);
    if (qn < nqb) gload(qn);
    if (qfar(qb) >= j0) {   // this wave's keys: some query of the block sees one
      const __bf16* Q = lds[buf];
      // S = Q K^T and dP = dO V^T (rows: queries, column: key c)
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < kQK; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *(const bf16x8*)(Q + c * kRow192 + 16 * ks + 8 * h), kv[ks], s, 0, 0, 0);
#pragma unroll
      for (int ks = 0; ks < kVK; ++ks)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *(const bf16x8*)(Q + kQElemsB + c * kRowTr + 16 * ks + 8 * h), vv[ks], dp, 0, 0, 0);
      // rows 8 g + 4h .. + 3: the statistics of those four queries
      f32x16 ds;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)&s_lse[buf][8 * g + 4 * h];
        const f32x4 d4 = *(const f32x4*)&s_d[buf][8 * g + 4 * h];
        const i32x4 t4 = *(const i32x4*)&s_last[buf][8 * g + 4 * h];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          // (a key past N stays exactly zero even beside a NaN query row)
          const bool seen = key_ok && key <= t4[e];
          const float p = seen ? __builtin_amdgcn_exp2f(fmaf(s[r], kLog2e, -l4[e])) : 0.f;
          s[r] = p;                                   // P
          ds[r] = seen ? p * (dp[r] - d4[e]) : 0.f;   // dS
        }
      }
      bf16x8 pbP[2], pbS[2];
      rows_as_b(s, pbP);
      rows_as_b(ds, pbS);
      const int base = buf * 2 * kBufB;
#pragma unroll
      for (int kap = 0; kap < 2; ++kap) {
#pragma unroll
        for (int dt = 0; dt < kDv / 32; ++dt)
          accV[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_operand((lds_char*)lds, base + 2 * kQElemsB, kRowTr, 16 * kap, 32 * dt),
              pbP[kap], accV[dt], 0, 0, 0);
#pragma unroll
        for (int dt = 0; dt < kW / 32; ++dt)
          accK[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_operand((lds_char*)lds, base, kRow192, 16 * kap, 32 * dt), pbS[kap], accK[dt],
              0, 0, 0);
      }
    }
    if (qn < nqb) lstore(buf ^ 1);   // that buffer was last read one block ago
    __syncthreads();
    buf ^= 1;
    qb = qn;
  }
  // lane (c, h) holds dims 32 dt + 8 g + 4h .. + 3 (g = r >> 2) of key `key`
  if (key_ok) {
    __bf16* rowk = dkv16 + (long)key * (2 * kH * kDv) + i * kDv + 4 * h;
    __bf16* rowv = rowk + kH * kDv;
#pragma unroll
    for (int dt = 0; dt < kDv / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = accK[dt];
        const f32x16& b = accV[dt];
        *(uint2*)(rowk + 32 * dt + 8 * g) =
            uint2{pack2(a[4 * g], a[4 * g + 1]), pack2(a[4 * g + 2], a[4 * g + 3])};
        *(uint2*)(rowv + 32 * dt + 8 * g) =
            uint2{pack2(b[4 * g], b[4 * g + 1]), pack2(b[4 * g + 2], b[4 * g + 3])};
      }
#pragma unroll
    for (int dt = kDv / 32; dt < kW / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(dkr + ((long)i * N + key) * (kW - kDv) + 32 * (dt - kDv / 32) + 8 * g + 4 * h) =
            f32x4{accK[dt][4 * g], accK[dt][4 * g + 1], accK[dt][4 * g + 2], accK[dt][4 * g + 3]};
  }
  // key-contiguous copies through LDS (the ring is free after the loop's
  // last barrier): each wave puts its [128 dims][32 keys] tile at a pitch of
  // 40 keys (rows 4 apart land 16 banks apart), then stores 16-byte pieces
  // of 8 keys.  Keys past N hold zeros.
  lds_char* tile = (lds_char*)lds + wave * (kDv * kTrPitch * 2);
  auto put_t = [&](const f32x16* acc, __bf16* dstT) {
#pragma unroll
    for (int dt = 0; dt < kDv / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + 8 * (r >> 2) + 4 * h + (r & 3);
        *(__attribute__((address_space(3))) __bf16*)(tile + 2 * (d * kTrPitch + c)) =
            (__bf16)(key_ok ? acc[dt][r] : 0.f);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < kDv * kB / (8 * 64); ++q) {
      const int piece = lane + 64 * q, d = piece >> 2, k8 = 8 * (piece & 3);
      const u32x4 x = *(const lds_u32x4*)(tile + 2 * (d * kTrPitch + k8));
      *(u32x4*)(dstT + ((long)i * kDv + d) * Npad + j0 + k8) = x;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  put_t(accK, dkT16);
  put_t(accV, dvT16);
}

// A bf16 matrix transposed: dst[c][dst_off + r] = src(r, c) for r < R, zero
// for R <= r < 64 gridDim.y; src row-major (ld_src) or, tiled, in the
// 16 x 32 tile layout of an [.][C] weight.  64 x 64 blocks through LDS,
// 16-byte reads and writes.
constexpr int kTp = 64 + 8;   // LDS pitch of a block (bf16)
__global__ __launch_bounds__(256) void transpose16_kernel(const __bf16* __restrict__ src,
                                                          long ld_src, int tiled, int C, int R,
                                                          __bf16* __restrict__ dst, long ld_dst,
                                                          long dst_off) {
  __shared__ __attribute__((aligned(16))) __bf16 t[64 * kTp];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int piece = tid + 256 * k, r = piece >> 3, cc = 8 * (piece & 7);
    uint4 x = uint4{0u, 0u, 0u, 0u};
    if (r0 + r < R) {
      const long off = tiled ? tile_index(r0 + r, c0 + cc, C) : (long)(r0 + r) * ld_src + c0 + cc;
      x = *(const uint4*)(src + off);
    }
    const __bf16* e = (const __bf16*)&x;
#pragma unroll
    for (int u = 0; u < 8; ++u) t[(cc + u) * kTp + r] = e[u];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int piece = tid + 256 * k, cc = piece >> 3, r = 8 * (piece & 7);
    *(uint4*)(dst + (long)(c0 + cc) * ld_dst + dst_off + r0 + r) = *(const uint4*)&t[cc * kTp + r];
  }
}

// q (fp32, RoPE applied) times the softmax scale, and dO, as bf16 rows
__global__ __launch_bounds__(256) void bwd_inputs_v2_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ dO, long nq,
                                                            long nd, float scale,
                                                            __bf16* __restrict__ q16,
                                                            __bf16* __restrict__ do16) {
  const long idx = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (idx < nq) {
    const f32x4 x = *(const f32x4*)(q + idx);
    *(uint2*)(q16 + idx) = uint2{pack2(scale * x[0], scale * x[1]), pack2(scale * x[2], scale * x[3])};
  }
  if (idx < nd) {
    const f32x4 x = *(const f32x4*)(dO + idx);
    *(uint2*)(do16 + idx) = uint2{pack2(x[0], x[1]), pack2(x[2], x[3])};
  }
}

}  // namespace

bool attn_bwd_v2_supported(const Geo& g) { return prefill_v2_supported(g); }

int attn_bwd_v2_npad(int N) { return (N + kWv * kB - 1) / (kWv * kB) * (kWv * kB); }

hipError_t attn_bwd_v2(const Geo& g, int N, int T, const float* q, const float* dO,
                       const int32_t* positions, const void* k16, const void* v16, void* q16,
                       void* do16, float* lse, float* dd, int* qblk_far, float* dq, void* dkv16,
                       void* dkT16, void* dvT16, float* dkr, hipStream_t s) {
  if (N <= 0 || T <= 0) return hipSuccess;
  if (!attn_bwd_v2_supported(g)) return hipErrorInvalidValue;
  const long nq = (long)T * kH * kW, nd = (long)T * kH * kDv;
  hipLaunchKernelGGL(bwd_inputs_v2_kernel, dim3((unsigned)((nq / 4 + 255) / 256)), dim3(256), 0, s,
                     q, dO, nq, nd, g.scale, (__bf16*)q16, (__bf16*)do16);
  hipLaunchKernelGGL(attn_bwd_dq_v2_kernel, dim3((T + kWv * kB - 1) / (kWv * kB), kH),
                     dim3(64 * kWv), 0, s, (const __bf16*)q16, (const __bf16*)do16,
                     (const __bf16*)k16, (const __bf16*)v16, positions, T, N, g.scale, lse, dd,
                     qblk_far, dq);
  hipLaunchKernelGGL(attn_bwd_dkv_v2_kernel, dim3(attn_bwd_v2_npad(N) / (kWv * kB), kH),
                     dim3(64 * kWv), 0, s, (const __bf16*)q16, (const __bf16*)do16,
                     (const __bf16*)k16, (const __bf16*)v16, positions, lse, dd, qblk_far, T, N,
                     attn_bwd_v2_npad(N), (__bf16*)dkv16, (__bf16*)dkT16, (__bf16*)dvT16, dkr);
  return hipGetLastError();
}

hipError_t transpose16(const void* src, long ld_src, bool tiled, int C, int R, int Rpad, void* dst,
                       long ld_dst, long dst_off, hipStream_t s) {
  if (C <= 0 || Rpad <= 0) return hipSuccess;
  if (C % 64 != 0 || Rpad % 64 != 0 || R > Rpad || (tiled && C % 32 != 0) || ld_dst % 8 != 0 ||
      dst_off % 8 != 0 || (!tiled && ld_src % 8 != 0))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose16_kernel, dim3(C / 64, Rpad / 64), dim3(256), 0, s,
                     (const __bf16*)src, ld_src, tiled ? 1 : 0, C, R, (__bf16*)dst, ld_dst,
                     dst_off);
  return hipGetLastError();
}

}  // namespace mla
