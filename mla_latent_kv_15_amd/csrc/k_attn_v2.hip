// Decode attention core for the DeepSeek-V2 geometry (n_h = 128, d_c = 512,
// d_r = 64, bf16 cache), on gfx950 MFMA.
//
// What it computes (order B of the walkthrough's §3, "顺序 B"): for each head
// i and cached row j = [c^KV_j | k^R_j] (576 bf16 numbers, no head index, the
// walkthrough's step 1), the score s_ij = Q~_i . row_j with the absorbed query
// Q~_i = [W_UK,i^T q^C_i | q^R_i] * scale, a softmax over j, and the weighted
// sum of the latents o~_i = sum_j p_ij c^KV_j in 512-d latent space.
//
// Design (gfx950):
//  * one work-group per compute unit (4 waves, one per SIMD); wave w owns
//    heads [32w, 32w+32).  Its slice of Q~ stays in VGPRs for the whole
//    segment (36 x 16 B per lane) and its 32 x 512 fp32 accumulator o~ in the
//    accumulation registers (256 per lane).  All 128 heads read each cache
//    row from LDS, so HBM sees every row exactly once.
//  * 64-token tiles (one page slice, 72 KB contiguous in HBM) are streamed
//    with 16-byte direct-to-LDS loads into a double buffer; LDS rows are
//    padded to 73 x 16 B so the 32 rows of one score MFMA hit distinct banks.
//  * scores: S^T[token][head] = C[token][dims] . Q~^T[dims][head] with
//    v_mfma_f32_32x32x16_bf16 (A = cache rows from LDS, B = Q~ from VGPRs).
//  * softmax numerators in the log2 domain against a per-segment reference:
//    the max of the segment's first 32 scores.  Later scores may exceed it by
//    up to 64 (P <= 2^64, harmless in fp32/bf16), so the 256-register
//    accumulator is never rescaled - VALU work on it would push the kernel
//    out of its 512-register budget.  If any score in the work-group exceeds
//    the reference by more than 64, the segment is redone: a scores-only pass
//    finds the exact max, then a full pass uses it (correct for any input,
//    essentially never taken).
//  * latent accumulation: o~^T[dims][head] += C^T[dims][tokens] . P^T with the
//    same MFMA.  The P operand comes straight from the score accumulators (the
//    token order inside one K-step is permuted to match their layout); the
//    C^T operand is an in-register 8x8 bf16 transpose of 8-byte LDS row reads,
//    which maps lane m to dims {8m .. 8m+7} across eight MFMAs.
//  * a work-group walks the segments the plan assigns to it and writes each
//    segment's unnormalised (m, l, o~) straight from the accumulation
//    registers, in register order; a merge kernel weighs the segments of each
//    sequence by e^(m_s - M) / sum_s l_s e^(m_s - M) and writes o~ as bf16.
#include <math.h>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeads = 128;
constexpr int kRow = 576;            // bf16 numbers per cached token
constexpr int kDc = 512;
constexpr int kChunks = kRow / 8;    // 72 x 16 B per row
constexpr int kLdsStride = 73;       // padded LDS row, in 16-byte chunks
constexpr int kTile = 64;            // tokens per tile
constexpr int kTileChunks = kTile * kLdsStride;      // 4672
constexpr int kLoadInsts = kTileChunks / 64;         // 73 wave-wide loads per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKSteps = kRow / 16;   // 36 score K-steps of 16 dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 64.0f;       // allowed score excess over the reference (log2 units)

typedef __attribute__((address_space(3))) void lds_void;

__device__ __shared__ __attribute__((aligned(16))) char g_tiles[2 * kTileChunks * 16];

// Stream one 64-token tile (rows [0, nvalid) valid) into LDS buffer `buf`;
// rows past nvalid are zero-filled so 0 * garbage never reaches an MFMA.
__device__ inline void load_tile(const u32x4* __restrict__ gtile, int nvalid, char* buf,
                                 int wave, int lane) {
  for (int inst = wave; inst < kLoadInsts; inst += kWaves) {
    const int p = inst * 64 + lane;
    const int r = p / kLdsStride;
    const int c = p - r * kLdsStride;
    if (c < kChunks) {
      if (r < nvalid) {
        __builtin_amdgcn_global_load_lds((const void*)(gtile + r * kChunks + c),
                                         (lds_void*)(buf + inst * 64 * 16), 16, 0, 0);
      } else {
        *(u32x4*)(buf + p * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
}

__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__global__ __launch_bounds__(kThreads, 1) void attn_v2_kernel(
    const __bf16* __restrict__ q_abs, const __bf16* __restrict__ cache, int num_pages,
    const int32_t* __restrict__ page_table, int max_pages, int page, PlanPtrs plan,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  const int g = blockIdx.x;
  if (g >= plan.counts[1]) return;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;     // lane half
  const int m32 = lane & 31;
  const int head = wave * 32 + m32;
  const u32x4* cache16 = (const u32x4*)cache;

  const int k_begin = plan.wg_seg_start[g];
  const int k_end = plan.wg_seg_start[g + 1];
  for (int k = k_begin; k < k_end; ++k) {
    const Seg sg = plan.segs[k];
    const int b = sg.b;
    const int ntiles = (sg.t1 - sg.t0 + kTile - 1) / kTile;

    // absorbed query slice -> VGPRs (B operand: lane = head, 8 dims per K-step half)
    bf16x8 qreg[kKSteps];
    {
      const bf16x8* qs = (const bf16x8*)(q_abs + ((long)b * kHeads + head) * kRow + 8 * h);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = qs[2 * ks];
    }
    f32x16 acc[16];
    float m_ref = -INFINITY;  // exponent reference (log2 units), fixed within a pass
    float l_run = 0.f;
    bool bad = false;
    // mode 0: reference = max of the first 32 tokens; mode 1: exact max only;
    // mode 2: full pass with the exact max (after a mode-0 overflow)
    int mode = 0;
    for (;;) {
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[x] = f32x16{};
      l_run = 0.f;
      float m_seen = -INFINITY;
      bool over = false;

      __syncthreads();  // every wave is done with both tile buffers
      {
        const int tt = sg.t0;
        const int pg = page_table[(long)b * max_pages + tt / page];
        const bool ok = pg >= 0 && pg < num_pages;
        bad |= !ok;
        const long slot0 = ok ? (long)pg * page + tt % page : 0;
        load_tile(cache16 + slot0 * kChunks, ok ? min(kTile, sg.t1 - tt) : 0, g_tiles, wave, lane);
      }

      for (int it = 0; it < ntiles; ++it) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // tile `it` landed everywhere; buffer (it+1)&1 is free
        if (it + 1 < ntiles) {
          const int tt = sg.t0 + (it + 1) * kTile;
          const int pg = page_table[(long)b * max_pages + tt / page];
          const bool ok = pg >= 0 && pg < num_pages;
          bad |= !ok;
          const long slot0 = ok ? (long)pg * page + tt % page : 0;
          load_tile(cache16 + slot0 * kChunks, ok ? min(kTile, sg.t1 - tt) : 0,
                    g_tiles + ((it + 1) & 1) * kTileChunks * 16, wave, lane);
        }
        const char* buf = g_tiles + (it & 1) * kTileChunks * 16;
        const int nvalid = min(kTile, sg.t1 - (sg.t0 + it * kTile));

#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          if (32 * blk >= nvalid) break;
          // ---- scores for 32 tokens x 32 heads
          f32x16 S = f32x16{};
          const char* arow = buf + ((32 * blk + m32) * kLdsStride + h) * 16;
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) {
            const bf16x8 a = *(const bf16x8*)(arow + 2 * ks * 16);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], S, 0, 0, 0);
          }
          // ---- softmax numerators (log2 domain), lane = head, 16 of the 32 tokens
          float bm = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = 32 * blk + 8 * (i >> 2) + 4 * h + (i & 3);
            S[i] = tok < nvalid ? S[i] * kLog2e : -INFINITY;
            bm = fmaxf(bm, S[i]);
          }
          bm = fmaxf(bm, __shfl_xor(bm, 32));
          m_seen = fmaxf(m_seen, bm);
          if (mode == 1) continue;
          if (mode == 0 && it == 0 && blk == 0) m_ref = bm;
          over |= bm > m_ref + kLazy;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            S[i] = __builtin_amdgcn_exp2f(S[i] - m_ref);
            l_run += S[i];
          }
          // ---- latent accumulation, two K-steps of 16 tokens
#pragma unroll
          for (int kap = 0; kap < 2; ++kap) {
            if (32 * blk + 16 * kap >= nvalid) break;
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = (__bf16)S[8 * kap + e];
            // token rows of this lane's K slots: 16kap + 8a + 4h + c (a = 0..1, c = 0..3)
            const char* vrow = buf + ((32 * blk + 16 * kap + 4 * h) * kLdsStride + m32) * 16;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                uint2 v[8];
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                  for (int c = 0; c < 4; ++c)
                    v[4 * a + c] =
                        *(const uint2*)(vrow + ((8 * a + c) * kLdsStride + 32 * q) * 16 + 8 * hh);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                  u32x4 lo, hi;
#pragma unroll
                  for (int f = 0; f < 4; ++f) {
                    const uint32_t x0 = e ? v[2 * f].y : v[2 * f].x;
                    const uint32_t x1 = e ? v[2 * f + 1].y : v[2 * f + 1].x;
                    lo[f] = perm(x1, x0, 0x05040100u);
                    hi[f] = perm(x1, x0, 0x07060302u);
                  }
                  const int j = 4 * hh + 2 * e;
                  acc[8 * q + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                      __builtin_bit_cast(bf16x8, lo), pb, acc[8 * q + j], 0, 0, 0);
                  acc[8 * q + j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                      __builtin_bit_cast(bf16x8, hi), pb, acc[8 * q + j + 1], 0, 0, 0);
                }
              }
            }
          }
        }
      }
      if (mode == 1) {
        m_ref = m_seen;
        mode = 2;
        continue;
      }
      // a score more than kLazy above the reference anywhere in the work-group:
      // find the exact maximum and redo the segment with it (rare)
      if (mode == 0 && __syncthreads_or(over ? 1 : 0)) {
        mode = 1;
        continue;
      }
      break;
    }

    // ---- unnormalised partial (m, l, o~) in register order; merged later
    {
      f32x4* dst = (f32x4*)(part_o + (long)k * kHeads * kDc) + wave * 64 + lane;
#pragma unroll
      for (int x = 0; x < 16; ++x)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          dst[(x * 4 + a) * kThreads] =
              f32x4{acc[x][4 * a], acc[x][4 * a + 1], acc[x][4 * a + 2], acc[x][4 * a + 3]};
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      if (h == 0) {
        part_ml[((long)k * kHeads + head) * 2] = m_ref * kLn2;
        part_ml[((long)k * kHeads + head) * 2 + 1] = bad ? __builtin_nanf("") : l_tot;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// merge of the register-order partials: one work-group per (sequence, wave
// slice of 32 heads).  o~ = sum_s e^(m_s - M) o~_s / sum_s e^(m_s - M) l_s.
// ---------------------------------------------------------------------------
constexpr int kCombSegs = 64;   // segments weighed per pass

__global__ __launch_bounds__(256) void combine_v2_kernel(PlanPtrs plan,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         __bf16* __restrict__ lat_out) {
  __shared__ float w[kCombSegs][32];
  __shared__ float s_M[32], s_inv[32];
  __shared__ __bf16 stage[32][kDc + 8];
  const int b = blockIdx.x, wv = blockIdx.y, t = threadIdx.x;
  const int cnt = plan.seq_seg_count[b];
  const int k0 = plan.seq_seg_start[b];
  __bf16* out = lat_out + ((long)b * kHeads + wv * 32) * kDc;
  if (cnt == 0) {
    for (int e = t; e < 32 * kDc; e += 256) out[e] = (__bf16)__builtin_nanf("");
    return;
  }
  // per-head max and normaliser
  if (t < 32) {
    const int hd = wv * 32 + t;
    float M = -INFINITY;
    for (int s = 0; s < cnt; ++s) M = fmaxf(M, part_ml[((long)(k0 + s) * kHeads + hd) * 2]);
    float L = 0.f;
    for (int s = 0; s < cnt; ++s) {
      const float* ml = part_ml + ((long)(k0 + s) * kHeads + hd) * 2;
      L += ml[1] * __expf(ml[0] - M);
    }
    s_M[t] = M;
    s_inv[t] = 1.f / L;
  }
  __syncthreads();
  const int lane = t & 63;
  const int r0 = t >> 6;              // (x, a) combos r0 + 4r, r = 0..15
  const int hd_l = lane & 31;
  f32x4 acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = f32x4{};
  for (int c0 = 0; c0 < cnt; c0 += kCombSegs) {
    const int nc = min(kCombSegs, cnt - c0);
    __syncthreads();
    for (int e = t; e < nc * 32; e += 256) {
      const int s = e >> 5, hh = e & 31;
      const float* ml = part_ml + ((long)(k0 + c0 + s) * kHeads + wv * 32 + hh) * 2;
      w[s][hh] = __expf(ml[0] - s_M[hh]) * s_inv[hh];
    }
    __syncthreads();
    for (int s = 0; s < nc; ++s) {
      const float ws = w[s][hd_l];
      const f32x4* src = (const f32x4*)(part_o + (long)(k0 + c0 + s) * kHeads * kDc) + wv * 64 + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += ws * src[(r0 + 4 * r) * kThreads];
    }
  }
  // register order -> [head][dim]: x = 8q + j, i = 4a + c, row m' = 8a + 4h + c
  const int hf = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int xa = r0 + 4 * r;
    const int x = xa >> 2, a = xa & 3;
    const int q = x >> 3, j = x & 7;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int dim = 256 * q + 8 * (8 * a + 4 * hf + c) + j;
      stage[hd_l][dim] = (__bf16)acc[r][c];
    }
  }
  __syncthreads();
  for (int e = t; e < 32 * (kDc / 8); e += 256) {
    const int hh = e / (kDc / 8), c8 = e % (kDc / 8);
    *(uint4*)(out + (long)hh * kDc + 8 * c8) = *(const uint4*)(&stage[hh][8 * c8]);
  }
}

}  // namespace

hipError_t attn_decode_v2(const Geo& g, const void* q_abs, const void* cache, int num_pages,
                          const int32_t* page_table, int max_pages, const PlanPtrs& plan,
                          int n_wg_launch, float* part_o, float* part_ml, hipStream_t s) {
  if (n_wg_launch <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_v2_kernel, dim3(n_wg_launch), dim3(kThreads), 0, s,
                     (const __bf16*)q_abs, (const __bf16*)cache, num_pages, page_table, max_pages,
                     g.page, plan, part_o, part_ml);
  return hipGetLastError();
}

hipError_t combine_decode_v2(const PlanPtrs& plan, int B, const float* part_o,
                             const float* part_ml, void* lat_out, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_v2_kernel, dim3(B, kHeads / 32), dim3(256), 0, s, plan, part_o,
                     part_ml, (__bf16*)lat_out);
  return hipGetLastError();
}

}  // namespace mla
