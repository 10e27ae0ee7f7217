// Causal prefill attention in order A for the DeepSeek-V2 head shape
// (n_h = 128, scores over 192 numbers, values of 128), on gfx950 MFMA.
//
// What it computes ([walkthrough] §3, order A, the form training uses, with
// the keys and values decompressed per head): for query t at position p_t
// and head i,
//   o_ti = sum_{j <= p_t} softmax_j(q_ti . k_ij) v_ij,   j < kv_len,
// q_ti = [q^C_ti | RoPE(q^R_ti)] with the softmax scale folded in,
// k_ij = [W_UK,i c_j | k^R_j], v_ij = W_UV,i c_j.  A query whose position
// lies outside [0, kv_len) gets NaN.
//
// Design: one wave per (block of 32 queries, head), four such waves of one
// head per work-group, which stages each block of 32 keys in LDS once for
// all four.  The scores are formed transposed, S^T[key][query] = K . Q^T,
// with v_mfma_f32_32x32x16_bf16, so that every lane owns one query: its
// softmax statistics stay in the lane apart from one permlane32 swap with
// the lane 32 apart, which holds the other half of the block's keys.  Four
// more swaps turn the numerators into the B operand of
// O^T[dim][query] += V^T . P^T in registers.  Q, K and V arrive as bf16
// (written so by the weight-streaming MFMA GEMMs); accumulation is fp32 with
// an online softmax in the log2 domain.  Key blocks past a wave's furthest
// query position are skipped (causality).  o is written as bf16 rows
// [T][n_h * d_h], the input of the W_O product.
#include <math.h>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) v4bf16 lds_v4bf16;

constexpr int kH = 128;    // heads
constexpr int kW = 192;    // query and key width
constexpr int kDv = 128;   // value width
constexpr int kQB = 32;    // queries per wave
constexpr int kKB = 32;    // keys per block
constexpr int kKSteps = kW / 16;
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline uint32_t pack2(float x, float y) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x, (__bf16)y});
}

// MFMA operand layouts (32 x 32 x 16): lane l = (c, h), c = l & 31,
// h = l >> 5.  A[m][k]: lane holds row m = c, k = 8h .. 8h + 7.  B[k][n]:
// lane holds column n = c, k = 8h .. 8h + 7.  D[m][n]: lane holds column
// n = c, rows 8 (r >> 2) + 4h + (r & 3) for r = 0 .. 15.
//
// A work-group of four waves takes 128 consecutive queries of one head; its
// threads stage each block of 32 keys in LDS once for all four waves (K and V
// as rows, 16-byte stores), double-buffered with one barrier per block.  The
// V^T operand of the second product comes from transposing LDS reads
// (ds_read_b64_tr_b16).  K rows are padded by 16 bytes to spread the banks;
// V rows by 64 bytes, so that the four rows one transposing read serves to
// 32 lanes at once start 64 banks apart.
constexpr int kWQ = 4;                       // waves (query blocks) per work-group

// Work-groups are dispatched round-robin over the eight XCDs (linear index
// L = blockIdx.y * gridDim.x + blockIdx.x goes to XCD L % 8).  Each XCD takes
// whole heads: its s-th work-group runs block xb = s % gridDim.x of head
// 8 (s / gridDim.x) + L % 8, so all work-groups of one head stream its key
// blocks through one L2.  (gridDim.y = 128 heads.)
__device__ inline void xcd_head_block(int& head, int& xb) {
  const int gx = gridDim.x;
  const int L = blockIdx.y * gx + blockIdx.x;
  const int s = L >> 3;
  xb = s % gx;
  head = (s / gx) * 8 + (L & 7);
}
constexpr int kKRow = kW + 8;                // LDS K row: 192 + 8 bf16
constexpr int kVRow = kDv + 32;              // LDS V row: 128 + 32 bf16
constexpr int kKElems = kKB * kKRow;         // 6400
constexpr int kBufElems = kKElems + kKB * kVRow;   // + 5120
constexpr int kKPieces = kKB * kW / 8;       // 768 16-byte pieces of a K block
constexpr int kVPieces = kKB * kDv / 8;      // 512 of a V block

__global__ __launch_bounds__(256, 2) void attn_prefill_v2_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kbuf, const __bf16* __restrict__ vbuf,
    const int32_t* __restrict__ positions, int T, int kv_len, __bf16* __restrict__ o) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][kBufElems];
  __shared__ int s_far[kWQ];
  int i, xb;
  xcd_head_block(i, xb);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
  // the last query blocks see the most keys: dispatch them first
  const int t = ((gridDim.x - 1 - xb) * kWQ + wave) * kQB + c;
  const bool t_ok = t < T;
  const int pos = t_ok ? positions[t] : -1;
  const bool valid = pos >= 0 && pos < kv_len;
  const int last = valid ? pos : -1;   // this query sees keys 0 .. last
  int far = last;                      // the wave's furthest key
  for (int off = 32; off >= 1; off >>= 1) far = max(far, __shfl_xor(far, off));
  if (lane == 0) s_far[wave] = far;
  __syncthreads();
  const int far_wg = max(max(s_far[0], s_far[1]), max(s_far[2], s_far[3]));
  const int nkb = (far_wg + kKB) / kKB;   // key blocks the work-group stages

  // Q^T as the B operand: K-step ks holds dims 16 ks + 8h .. + 7 of query t
  bf16x8 qv[kKSteps];
  {
    const __bf16* qr = q + ((long)(t_ok ? t : 0) * kH + i) * kW + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qv[ks] = *(const bf16x8*)(qr + 16 * ks);
  }
  // staging: K pieces p = tid + 256 r (key p / 24, piece p % 24), V pieces
  // (key p / 16, dims 8 (p % 16) ..); rows past kv_len repeat the last one.
  // (Five named registers: an array here ends up in scratch.)
  static_assert(kKPieces == 3 * 256 && kVPieces == 2 * 256, "staging assumes 3 + 2 pieces");
  uint4 k0r, k1r, k2r, v0r, v1r;
  auto kpiece = [&](int kb, int r) {
    const int p = tid + 256 * r, key = p / (kW / 8), pc = p % (kW / 8);
    return *(const uint4*)(kbuf + ((long)min(kb * kKB + key, kv_len - 1) * kH + i) * kW + 8 * pc);
  };
  auto vpiece = [&](int kb, int r) {
    const int p = tid + 256 * r, key = p / (kDv / 8), pc = p % (kDv / 8);
    return *(const uint4*)(vbuf + ((long)min(kb * kKB + key, kv_len - 1) * kH + i) * kDv + 8 * pc);
  };
  auto gload = [&](int kb) {
    k0r = kpiece(kb, 0);
    k1r = kpiece(kb, 1);
    k2r = kpiece(kb, 2);
    v0r = vpiece(kb, 0);
    v1r = vpiece(kb, 1);
  };
  auto kstore = [&](__bf16* K, int r, uint4 x) {
    const int p = tid + 256 * r, key = p / (kW / 8), pc = p % (kW / 8);
    *(uint4*)(K + key * kKRow + 8 * pc) = x;
  };
  auto vstore = [&](__bf16* V, int r, uint4 x) {
    const int p = tid + 256 * r, key = p / (kDv / 8), pc = p % (kDv / 8);
    *(uint4*)(V + key * kVRow + 8 * pc) = x;
  };
  auto lstore = [&](int buf) {
    __bf16* K = lds[buf];
    kstore(K, 0, k0r);
    kstore(K, 1, k1r);
    kstore(K, 2, k2r);
    vstore(K + kKElems, 0, v0r);
    vstore(K + kKElems, 1, v1r);
  };

  // The V^T operand of dim tile d, K-step kap (keys 16 kap + 8h .. + 7 of dim
  // 32 d + c for lane (c, h)) by two transposing reads of four keys each.
  // In each 16-lane group, lane s supplies the 8-byte chunk of row
  // k0 + s / 4, dims D0 + 4 (s % 4) .. + 3, and output lane i receives, as
  // its element r, element i % 4 of lane 4 r + i / 4's chunk: dim D0 + i of
  // row k0 + r.  Byte offset of this lane's chunk in buffer 0, at d = kap = 0:
  const int vt_base = 2 * (kKElems + (8 * h + ((lane & 15) >> 2)) * kVRow +
                           16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  auto vt_read = [&](int buf, int kap, int d) {
    const int b = buf * 2 * kBufElems + vt_base + 2 * (16 * kap * kVRow + 32 * d);
    const v4bf16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_v4bf16*)((lds_char*)lds + b));
    const v4bf16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_v4bf16*)((lds_char*)lds + b + 2 * 4 * kVRow));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x16 acc[kDv / 32];   // O^T, dims 32 d .. 32 d + 31 x the wave's 32 queries
#pragma unroll
  for (int d = 0; d < kDv / 32; ++d) acc[d] = f32x16{};
  float m = -INFINITY, l = 0.f;   // running max (log2 units) and sum of this lane's query

  if (nkb > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) gload(kb + 1);   // in flight during this block's products
    const __bf16* K = lds[kb & 1];
    const int j0 = kb * kKB;
    if (j0 <= far) {   // the wave has a query that sees a key of this block
      // S^T = K . Q^T
      f32x16 s = {};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *(const bf16x8*)(K + c * kKRow + 16 * ks + 8 * h), qv[ks], s, 0, 0, 0);
      // causal mask and the block's max for this query (both lane halves)
      float bm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
        s[r] = key <= last ? s[r] * kLog2e : -INFINITY;
        bm = fmaxf(bm, s[r]);
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm),
                                                         __float_as_uint(bm), false, false);
        bm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float mn = fmaxf(m, bm);
      const float ref = mn == -INFINITY ? 0.f : mn;   // no key seen yet: all numerators 0
      const float alpha = __builtin_amdgcn_exp2f(m - ref);
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = __builtin_amdgcn_exp2f(s[r] - ref);
        ps += s[r];
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps),
                                                         __float_as_uint(ps), false, false);
        ps = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      l = l * alpha + ps;
      m = mn;
#pragma unroll
      for (int d = 0; d < kDv / 32; ++d) acc[d] *= alpha;
      // P^T as the B operand: K-step kap needs keys 16 kap + 8h .. + 7 of
      // this lane's query.  A lane holds keys 4h .. 4h + 3 (+ 8, 16, 24); the
      // lane 32 apart holds the other four of each eight.
      uint32_t R[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) R[k] = pack2(s[2 * k], s[2 * k + 1]);
#pragma unroll
      for (int k = 0; k < 8; k += 4) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(R[k], R[k + 2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(R[k + 1], R[k + 3], false, false);
        R[k] = s0[0];
        R[k + 2] = s0[1];
        R[k + 1] = s1[0];
        R[k + 3] = s1[1];
      }
      const bf16x8 pb[2] = {__builtin_bit_cast(bf16x8, u32x4{R[0], R[1], R[2], R[3]}),
                            __builtin_bit_cast(bf16x8, u32x4{R[4], R[5], R[6], R[7]})};
      // O^T += V^T . P^T: the A operand of dim tile d, K-step kap is dim
      // 32 d + c of the block's keys 16 kap + 8h .. + 7
#pragma unroll
      for (int kap = 0; kap < 2; ++kap)
#pragma unroll
        for (int d = 0; d < kDv / 32; ++d)
          acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_read(kb & 1, kap, d), pb[kap],
                                                           acc[d], 0, 0, 0);
    }
    if (kb + 1 < nkb) lstore((kb + 1) & 1);   // that buffer was last read in block kb - 1
    __syncthreads();
  }
  if (!t_ok) return;
  // lane (c, h) holds dims 32 d + 8 g + 4h .. + 3 (g = r >> 2) of query t
  const float inv = valid ? 1.f / l : __builtin_nanf("");
  __bf16* dst = o + ((long)t * kH + i) * kDv + 4 * h;
#pragma unroll
  for (int d = 0; d < kDv / 32; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(uint2*)(dst + 32 * d + 8 * g) =
          uint2{pack2(acc[d][4 * g] * inv, acc[d][4 * g + 1] * inv),
                pack2(acc[d][4 * g + 2] * inv, acc[d][4 * g + 3] * inv)};
}

// Cached rows [kv_len][576] (bf16, gathered through the page table; NaN
// for a page id outside the cache) and the RoPE key part of every head's
// k_ij = [W_UK,i c_j | k^R_j]: k[j][i][128 ..] = k^R_j.  One work-group per
// row, 16 bytes per thread and store.
__global__ __launch_bounds__(256) void prefill_rows_v2_kernel(
    int page, const __bf16* __restrict__ cache, int num_pages,
    const int32_t* __restrict__ page_table, __bf16* __restrict__ rows, __bf16* __restrict__ kbuf) {
  constexpr int kRow = 576, kPieces = kRow / 8, kRope = (kW - kDv) / 8;   // 72, 8
  const int j = blockIdx.x, tid = threadIdx.x;
  const int pg = page_table[j / page];
  const bool ok = pg >= 0 && pg < num_pages;
  const uint4* src = (const uint4*)(cache + ((long)(ok ? pg : 0) * page + j % page) * kRow);
  const uint4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  if (tid < kPieces) ((uint4*)(rows + (long)j * kRow))[tid] = ok ? src[tid] : nan4;
  for (int e = tid; e < kH * kRope; e += 256) {
    const int hd = e / kRope, pc = e % kRope;
    ((uint4*)(kbuf + ((long)j * kH + hd) * kW + kDv))[pc] = ok ? src[kPieces - kRope + pc] : nan4;
  }
}

// q[t][i][128 ..] = RoPE(qr[t][i][0 .. 64], p_t) as bf16 (qr fp32, already
// scaled); NaN for a position outside the table.  One thread per pair.
__global__ __launch_bounds__(256) void prefill_rope_q_v2_kernel(
    const float* __restrict__ qr, const int32_t* __restrict__ positions, long n,
    const float* __restrict__ rope, int rope_len, __bf16* __restrict__ q) {
  constexpr int kHalf = (kW - kDv) / 2;   // 32 pairs per head
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int k = (int)(idx % kHalf);
  const long ti = idx / kHalf;   // t * 128 + i
  const int pos = positions[ti / kH];
  const float2 x = *(const float2*)(qr + ti * (kW - kDv) + 2 * k);
  float o0 = __builtin_nanf(""), o1 = __builtin_nanf("");
  if (pos >= 0 && pos < rope_len) {
    const float2 cs = *(const float2*)(rope + ((long)pos * kHalf + k) * 2);
    o0 = x.x * cs.x - x.y * cs.y;
    o1 = x.x * cs.y + x.y * cs.x;
  }
  *(uint32_t*)(q + ti * kW + kDv + 2 * k) = pack2(o0, o1);
}

}  // namespace

bool prefill_v2_supported(const Geo& g) {
  return is_v2_fast(g) && g.d_h + g.d_r == kW && g.d_h == kDv && g.n_h == kH;
}

hipError_t attn_prefill_v2(const Geo& g, const void* q, const void* kbuf, const void* vbuf,
                           const int32_t* positions, int T, int kv_len, void* o, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (!prefill_v2_supported(g) || kv_len <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_prefill_v2_kernel, dim3((T + kWQ * kQB - 1) / (kWQ * kQB), kH),
                     dim3(64 * kWQ), 0, s,
                     (const __bf16*)q, (const __bf16*)kbuf, (const __bf16*)vbuf, positions, T,
                     kv_len, (__bf16*)o);
  return hipGetLastError();
}

hipError_t prefill_rows_v2(const Geo& g, const void* cache, int num_pages,
                           const int32_t* page_table, int kv_len, void* rows, void* kbuf,
                           hipStream_t s) {
  if (kv_len <= 0) return hipSuccess;
  if (!prefill_v2_supported(g)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_rows_v2_kernel, dim3(kv_len), dim3(256), 0, s, g.page,
                     (const __bf16*)cache, num_pages, page_table, (__bf16*)rows, (__bf16*)kbuf);
  return hipGetLastError();
}

hipError_t prefill_rope_q_v2(const Geo& g, const float* qr, const int32_t* positions, int T,
                             const float* rope, int rope_len, void* q, hipStream_t s) {
  const long n = (long)T * kH * ((kW - kDv) / 2);
  if (n <= 0) return hipSuccess;
  if (!prefill_v2_supported(g)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_rope_q_v2_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     qr, positions, n, rope, rope_len, (__bf16*)q);
  return hipGetLastError();
}

}  // namespace mla
