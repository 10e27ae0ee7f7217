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
//    heads [32w, 32w+32).  Its slice of Q~ stays in registers for the whole
//    segment (the 512 latent dims: 32 x 16 B per lane; the 64 RoPE dims of all
//    heads sit in LDS) and its 32 x 512 fp32 accumulator o~ fills the
//    accumulation registers (256 per lane).  All 128 heads read each cache row
//    from LDS, so HBM sees every row once.
//  * 32-token sub-tiles (36 KB, contiguous inside a page) stream through a
//    four-slot LDS ring with 16-byte direct-to-LDS loads, three sub-tiles in
//    flight.  Every wave issues the same number of loads per sub-tile, so the
//    waits are static vmcnt counts; barriers skip __syncthreads' fence, which
//    would drain the ring.  LDS rows are 1152 B with the 16-byte chunks of row
//    r XOR-permuted by a 3-bit function of r, which makes both read patterns
//    below free of bank conflicts.
//  * scores: S^T[token][head] = C[token][dims] . Q~^T[dims][head] with
//    v_mfma_f32_32x32x16_bf16 (A = cache rows from LDS, B = Q~), 36 K-steps.
//  * softmax numerators in the log2 domain against a per-segment reference:
//    the max of the segment's first 32 scores.  Later scores may exceed it by
//    up to 64 (P <= 2^64, harmless in fp32/bf16), so the 256-register
//    accumulator is never rescaled - VALU work on it would push the kernel
//    out of its 512-register budget.  If any score in the work-group exceeds
//    the reference by more than 64, the segment is redone once with the exact
//    maximum, which the first pass tracks (correct for any input, essentially
//    never taken).
//  * latent accumulation: o~^T[dims][head] += C^T[dims][tokens] . P^T with the
//    same MFMA.  P comes straight from the score accumulators (rounded to
//    bf16); C^T is read from the same LDS tile with ds_read_b128 and
//    transposed in registers with v_perm_b32.
//  * a work-group walks the segments the plan assigns to it and writes each
//    segment's unnormalised (m, l, o~) from the accumulation registers, o~ as
//    bf16 in register order; a merge kernel weighs the segments of each
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
constexpr int kRowBytes = kRow * 2;  // 1152
constexpr int kSub = 32;             // tokens per sub-tile (one MFMA block)
constexpr int kSlots = 4;            // LDS ring: one sub-tile computed, three in flight
constexpr int kSubChunks = kSub * kChunks;           // 2304
constexpr int kSubBytes = kSubChunks * 16;           // 36864
constexpr int kSubInsts = kSubChunks / 64;           // 36 wave-wide loads per sub-tile
constexpr int kInstsPerWave = kSubInsts / 4;         // 9
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKSteps = kRow / 16;   // 36 score K-steps of 16 dims
constexpr int kKReg = kDc / 16;      // 32 K-steps whose Q~ slice stays in VGPRs
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 64.0f;       // allowed score excess over the reference (log2 units)

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// one LDS object: the cache ring, then the query's RoPE slice
constexpr int kQropeOff = kSlots * kSubBytes;        // 147456
constexpr int kQropeBytes = kHeads * 64 * 2;         // 16384
__device__ __shared__ __attribute__((aligned(16))) char g_tiles[kQropeOff + kQropeBytes];
// rope part of the absorbed query (dims 512..575) for all 128 heads at
// g_tiles + kQropeOff; chunk c of head i sits at chunk position c ^ swz(i)

// Work-group barrier without __syncthreads' release fence: that fence waits
// for every outstanding vector memory operation, which would drain the
// in-flight cache sub-tiles of the ring at each barrier.  LDS ordering is
// established by the explicit s_waitcnt that precedes each use; the asm
// memory clobbers keep the compiler from moving LDS accesses across it.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte chunk c of tile row r sits at chunk position c ^ swz(r) of that row
__device__ inline int swz(int r) {
  return ((((r & 3) << 1) | ((r >> 2) & 1)) ^ (((r >> 3) & 1) << 1)) & 7;
}

// Stream one 32-token sub-tile into LDS slot `buf`.  Rows at or past nvalid
// re-read the last valid row (nvalid = 0: row 0 of the page passed in): their
// scores are masked to zero weight, and the data stays finite, so
// 0 * row never turns into NaN.  Every wave issues exactly kInstsPerWave loads
// per sub-tile whatever nvalid is; the ring's vmcnt bookkeeping relies on it.
__device__ inline void load_sub(const u32x4* __restrict__ gsub, int nvalid, char* buf, int wave,
                                int lane) {
  // recompute the per-lane addresses at every call instead of keeping nine
  // loop-invariant offsets live across the compute loop (VGPRs are scarce)
  asm volatile("" : "+v"(lane));
  const int rmax = max(nvalid - 1, 0);
  // wave w fills rows [8w, 8w+8): its i-th load covers chunks [64i, 64i+64)
  // of those 576, i.e. rows k_i and k_i + 1 with the switch at lane b_i
#pragma unroll
  for (int i = 0; i < kInstsPerWave; ++i) {
    const int k = (64 * i) / kChunks;
    const int bnd = kChunks * (k + 1) - 64 * i;
    const bool second = lane >= bnd;
    const int r = 8 * wave + k + (second ? 1 : 0);
    const int cp = 64 * i - kChunks * k + lane - (second ? kChunks : 0);
    __builtin_amdgcn_global_load_lds((const void*)(gsub + min(r, rmax) * kChunks + (cp ^ swz(r))),
                                     (lds_void*)(buf + (8 * wave * kChunks + 64 * i) * 16), 16, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads, 1) void attn_v2_kernel(
    const __bf16* __restrict__ q_abs, const __bf16* __restrict__ cache, int num_pages,
    const int32_t* __restrict__ page_table, int max_pages, int page, PlanPtrs plan,
    __bf16* __restrict__ part_o, float* __restrict__ part_ml) {
  // Work-groups are dispatched round-robin over the eight XCDs.  Give the
  // work-groups of one XCD consecutive plan slots: consecutive slots share
  // sequences, so a sequence's absorbed query is fetched into one L2.
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int g = xcd * (G >> 3) + min(xcd, G & 7) + (blockIdx.x >> 3);
  if (g >= plan.counts[1]) return;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;     // lane half
  const int m32 = lane & 31;
  const int head = wave * 32 + m32;
  const u32x4* cache16 = (const u32x4*)cache;
  lds_char* const lds = (lds_char*)g_tiles;

  // Per-lane LDS byte offsets inside a 32-token block (row 0 of the block is
  // a multiple of 16, so the swizzle only sees the low 4 row bits).
  // scores: row m32, chunk 2ks + h   -> qoff[ks & 3] + 128 * (ks >> 2)
  int qoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qoff[j] = m32 * kRowBytes + (((2 * j + h) ^ swz(m32)) << 4);
  // latent accumulation: element e = 4a + c of lane (m32, h) is token row
  // 8a + 4h + c of the K-step; it reads 16-byte chunk m32 (+32 per quarter)
  int voff[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = 8 * (e >> 2) + 4 * h + (e & 3);
    voff[e] = row * kRowBytes + ((m32 ^ swz(row)) << 4);
  }

  const int k_begin = plan.wg_seg_start[g];
  const int k_end = plan.wg_seg_start[g + 1];
  for (int k = k_begin; k < k_end; ++k) {
    const Seg sg = plan.segs[k];
    const int b = sg.b;

    // absorbed query slice -> VGPRs (B operand: lane = head, 8 dims per K-step half)
    bf16x8 qreg[kKReg];
    {
      int hd = head, hh = h;
      asm volatile("" : "+v"(hd), "+v"(hh));
      const bf16x8* qs = (const bf16x8*)(q_abs + ((long)b * kHeads + hd) * kRow + 8 * hh);
#pragma unroll
      for (int ks = 0; ks < kKReg; ++ks) qreg[ks] = qs[2 * ks];
    }
    f32x16 acc[16];
    float m_ref = -INFINITY;  // exponent reference (log2 units), fixed within a pass
    float l_run = 0.f;
    bool bad = false;
    // pass 0: reference = max of the first 32 tokens; every sub-tile's max is
    // tracked, so after a pass-0 overflow the exact segment max is known and
    // pass 1 redoes the segment with it as the reference
    int mode = 0;
    for (;;) {
      // opaque to the optimiser: one copy of the sub-tile loop serves both passes
      asm volatile("" : "+v"(mode));
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[x] = f32x16{};
      l_run = 0.f;
      float m_seen = -INFINITY;
      bool over = false;

      __syncthreads();  // every wave is done with the ring and the query buffer
      {
        // rope part of Q~ for all heads -> LDS: 1024 chunks, 4 per thread
        int tl = threadIdx.x;
        asm volatile("" : "+v"(tl));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = tl + kThreads * u;
          const int hd = e >> 3, c = e & 7;
          const u32x4 v = *(const u32x4*)(q_abs + ((long)b * kHeads + hd) * kRow + kDc + 8 * c);
          *(u32x4*)(g_tiles + kQropeOff + hd * 128 + ((c ^ swz(hd)) << 4)) = v;
        }
      }
      const int nsub = (sg.t1 - sg.t0 + kSub - 1) / kSub;
      // sub-tile j of the segment: tokens [t0 + 32j, ...) inside one page
      auto issue = [&](int j) {
        const int tt = sg.t0 + j * kSub;
        const int pg = page_table[(long)b * max_pages + tt / page];
        const bool ok = pg >= 0 && pg < num_pages;
        bad |= !ok;
        const long slot0 = ok ? (long)pg * page + tt % page : 0;
        load_sub(cache16 + slot0 * kChunks, ok ? min(kSub, sg.t1 - tt) : 0,
                 g_tiles + (j % kSlots) * kSubBytes, wave, lane);
      };
      for (int j = 0; j < kSlots - 1 && j < nsub; ++j) issue(j);

#pragma clang loop unroll(disable)
      for (int j = 0; j < nsub; ++j) {
        // sub-tile j is complete once at most the loads of the sub-tiles
        // issued after it are outstanding
        const int later = min(kSlots - 2, nsub - 1 - j);
        static_assert(kInstsPerWave == 9, "vmcnt immediates below assume 9 loads per sub-tile");
        if (later >= 2)
          asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
        else if (later == 1)
          asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // the ring slot after the last sub-tile is free at the last iteration;
        // it carries the work-group's redo flag
        if (j == nsub - 1 && threadIdx.x == 0) {
          *(int __attribute__((address_space(3)))*)(lds + (nsub % kSlots) * kSubBytes) = 0;
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        lds_barrier();  // sub-tile j landed everywhere; slot (j+3)%4 is free
        const int nvalid = min(kSub, sg.t1 - (sg.t0 + j * kSub));
        lds_char* bb = lds + (j % kSlots) * kSubBytes;
        {
          // ---- scores for 32 tokens x 32 heads, A operand prefetched 4 deep.
          // The MFMA chain is written as inline asm with a VGPR ("v")
          // accumulator: with the builtin the compiler puts S in the
          // accumulation registers, which the 32 x 512 o~ accumulator already
          // fills, and then spills o~.  Back-to-back accumulation into the
          // same registers needs no wait states; the s_nop after the chain
          // covers the MFMA-result -> VALU-read hazard.
          f32x16 S;
          bf16x8 abuf[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) abuf[ks] = *(const bf16x8 __attribute__((address_space(3)))*)(bb + qoff[ks & 3] + 128 * (ks >> 2));
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) {
            const bf16x8 a = abuf[ks & 3];
            if (ks + 4 < kKSteps)
              abuf[ks & 3] = *(const bf16x8 __attribute__((address_space(3)))*)(bb + qoff[(ks + 4) & 3] + 128 * ((ks + 4) >> 2));
            const bf16x8 q = ks < kKReg
                ? qreg[ks]
                : *(const bf16x8 __attribute__((address_space(3)))*)(
                      lds + kQropeOff + head * 128 + (((2 * (ks - kKReg) + h) ^ swz(head)) << 4));
            if (ks == 0)
              // early clobber: the destination must not overlap the A/B operands
              asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(S) : "v"(a), "v"(q));
            else
              asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(S) : "v"(a), "v"(q));
          }
          asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(S));
          // ---- softmax numerators (log2 domain), lane = head, 16 of the 32 tokens
          if (nvalid < kSub) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int tok = 8 * (i >> 2) + 4 * h + (i & 3);
              S[i] = tok < nvalid ? S[i] : -INFINITY;
            }
          }
          float bm = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) bm = fmaxf(bm, S[i]);
          bm = fmaxf(bm, __shfl_xor(bm, 32)) * kLog2e;
          m_seen = fmaxf(m_seen, bm);
          // pass 0 takes its reference from the first sub-tile (m_ref is -inf
          // until then); the redo pass starts with the exact maximum
          m_ref = (m_ref == -INFINITY) ? bm : m_ref;
          over |= bm > m_ref + kLazy;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            S[i] = __builtin_amdgcn_exp2f(fmaf(S[i], kLog2e, -m_ref));
            l_run += S[i];
          }
          // ---- latent accumulation: o~^T[dims][head] += C^T . P^T, two K-steps
          // of 16 tokens.  Lane (m32, h) reads the 16-byte chunk m32 of each
          // quarter-row for its eight token rows and transposes the 8 x 8 bf16
          // block in registers: M-block (q, j) holds dims 256q + 8m + j.
          bf16x8 pb[2];
#pragma unroll
          for (int kap = 0; kap < 2; ++kap)
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[kap][e] = (__bf16)S[8 * kap + e];
          // (a K-step past nvalid adds P = 0 times finite re-read rows)
#pragma unroll
          for (int g8 = 0; g8 < 4; ++g8) {       // (kap, q) groups of 8 MFMAs
            const int kap = g8 >> 1, q = g8 & 1;
            u32x4 v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              v[e] = *(const u32x4 __attribute__((address_space(3)))*)(
                  bb + 16 * kap * kRowBytes + voff[e] + 512 * q);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              u32x4 lo, hi;
#pragma unroll
              for (int f = 0; f < 4; ++f) {
                lo[f] = __builtin_amdgcn_perm(v[2 * f + 1][d], v[2 * f][d], 0x05040100u);
                hi[f] = __builtin_amdgcn_perm(v[2 * f + 1][d], v[2 * f][d], 0x07060302u);
              }
              acc[8 * q + 2 * d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, lo), pb[kap], acc[8 * q + 2 * d], 0, 0, 0);
              acc[8 * q + 2 * d + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, hi), pb[kap], acc[8 * q + 2 * d + 1], 0, 0, 0);
            }
          }
          // refill the ring after this iteration's last LDS read (the
          // compiler places a full vmcnt wait before LDS reads that follow a
          // direct-to-LDS load in program order)
          if (j + kSlots - 1 < nsub) issue(j + kSlots - 1);
        }
      }
      // a score more than kLazy above the reference anywhere in the work-group:
      // redo the segment with the exact maximum seen in this pass (rare)
      if (mode == 0) {
        int __attribute__((address_space(3)))* flag =
            (int __attribute__((address_space(3)))*)(lds + (nsub % kSlots) * kSubBytes);
        if (over) *flag = 1;
        __syncthreads();
        const int redo = *flag;
        if (redo) {
          m_ref = m_seen;
          mode = 1;
          continue;
        }
      }
      break;
    }

    // ---- unnormalised partial (m, l, o~): o~ rounded to bf16, in register
    // order (8-byte piece 4x + a of a lane holds elements 4a .. 4a + 3 of
    // accumulator x); merged later
    {
      int tl = threadIdx.x;
      asm volatile("" : "+v"(tl));  // form the per-lane address here, not at kernel entry
      uint2* dst = (uint2*)(part_o + (long)k * kHeads * kDc) + tl;
#pragma unroll
      for (int x = 0; x < 16; ++x)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float f0 = acc[x][4 * a], f1 = acc[x][4 * a + 1];
          const float f2 = acc[x][4 * a + 2], f3 = acc[x][4 * a + 3];
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          const bf16x2 p0 = {(__bf16)f0, (__bf16)f1}, p1 = {(__bf16)f2, (__bf16)f3};
          dst[(x * 4 + a) * kThreads] =
              uint2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
        }
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      if (h == 0) {
        int hd = head;
        asm volatile("" : "+v"(hd));
        float2* ml = (float2*)(part_ml + ((long)k * kHeads + hd) * 2);
        *ml = float2{m_ref * kLn2, bad ? __builtin_nanf("") : l_tot};
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
                                                         const __bf16* __restrict__ part_o,
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
  const int r0 = t >> 6;              // 8-byte pieces p = 4x + a = r0 + 4r, r = 0..15
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
      const uint2* src = (const uint2*)(part_o + (long)(k0 + c0 + s) * kHeads * kDc) + wv * 64 + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint2 v = src[(r0 + 4 * r) * kThreads];
        acc[r] += ws * f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                             __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
      }
    }
  }
  // register order -> [head][dim]: accumulator x = 8q + j holds dims
  // 256q + 8m + j with row m = 8a + 4h + c for element i = 4a + c
  const int hf = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int xa = r0 + 4 * r;
    const int x = xa >> 2, a = xa & 3;
    const int q = x >> 3, j = x & 7;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      stage[hd_l][256 * q + 8 * (8 * a + 4 * hf + c) + j] = (__bf16)acc[r][c];
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
                          int n_wg_launch, void* part_o, float* part_ml, hipStream_t s) {
  if (n_wg_launch <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_v2_kernel, dim3(n_wg_launch), dim3(kThreads), 0, s,
                     (const __bf16*)q_abs, (const __bf16*)cache, num_pages, page_table, max_pages,
                     g.page, plan, (__bf16*)part_o, part_ml);
  return hipGetLastError();
}

hipError_t combine_decode_v2(const PlanPtrs& plan, int B, const void* part_o,
                             const float* part_ml, void* lat_out, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_v2_kernel, dim3(B, kHeads / 32), dim3(256), 0, s, plan,
                     (const __bf16*)part_o, part_ml, (__bf16*)lat_out);
  return hipGetLastError();
}

}  // namespace mla
