// Causal prefill attention in order A for the DeepSeek-V2 head shape
// (n_h = 128, scores over 192 numbers, values of 128), on gfx950 MFMA.
//
// What it computes ([walkthrough] §3, order A, the form training uses, with
// the keys and values decompressed per head): for query t at position p_t
// and head i,
//   o_ti = sum_{j <= p_t} softmax_j(q_ti . k_ij) v_ij,   j < kv_len,
// q_ti = [q^C_ti | RoPE(q^R_ti)] with the softmax scale and log2(e) folded
// in (the scores come out in log2 units),
// k_ij = [W_UK,i c_j | k^R_j], v_ij = W_UV,i c_j.  A query whose position
// lies outside [0, kv_len) gets NaN.
//
// Design: one wave per (block of 32 queries, head), four such waves of one
// head per work-group, two work-groups per compute unit.  The work-group
// streams the blocks of 32 keys (K and V rows) through a ring of four LDS
// slots by direct-to-LDS loads, rows swizzled so that row reads and
// transposing reads are free of bank conflicts (head_blocks.h).  Each wave
// forms block kb + 1's scores between the exp2s of block kb's softmax,
// one MFMA at a time, then block kb's O update.  The scores
// are formed transposed, S^T[key][query] = K . Q^T, with
// v_mfma_f32_32x32x16_bf16, so that every lane owns one query: its softmax
// statistics stay in the lane apart from one permlane32 swap with the lane
// 32 apart, which holds the other half of the block's keys.  Four more swaps
// turn the numerators into the B operand of O^T[dim][query] += V^T . P^T,
// whose V^T operand comes from transposing LDS reads.  Accumulation is fp32
// with an online softmax in the log2 domain; O is rescaled only in the
// blocks where some query's maximum passes its reference by more than 8.  Key blocks past a wave's
// furthest query position are skipped (causality).  Q, K and V arrive as
// bf16 (written so by the MFMA GEMMs); o is written as bf16 rows
// [T][n_h * d_h], the input of the W_O product.
#include <math.h>

#include "head_blocks.h"
#include "mla_internal.h"

namespace mla {

namespace {

using namespace dev;

// ring slots: block kb (its V rows for P.V), block kb + 1 (its K rows for
// the scores formed beside block kb's softmax), kb + 2 and kb + 3 in flight
constexpr int kPSlots = 4;
template <int I>
using ic = std::integral_constant<int, I>;
constexpr int kPLoads = (kUnitsW + kUnitsV) / 64 / kWv;    // 5 loads per wave per block
constexpr int kPSlot = (kUnitsW + kUnitsV) * 16;           // 20 KB: K rows, then V rows
static_assert(kPLoads * (kPSlots - 2) < 64, "vmcnt range");

// The four O accumulators as the operands of one asm: 24 wait states after
// the last MFMA that wrote them, before VALU reads them (one statement, so
// that no MFMA can be placed between the wait and the reads), and more than
// the 2 wait states an MFMA read needs after a VALU write of them.
__device__ __forceinline__ void drain_o(f32x16 (&o)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
}
__device__ __forceinline__ void settle_o(f32x16 (&o)[4]) {
  asm volatile("s_nop 4" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
}

constexpr float kLazy = 8.f;   // log2 units a block's maximum may exceed the reference

__global__ __launch_bounds__(256, 2) void attn_prefill_v2_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kbuf, const __bf16* __restrict__ vbuf,
    const int32_t* __restrict__ positions, int T, int kv_len, __bf16* __restrict__ o) {
  __shared__ __attribute__((aligned(16))) char ring[kPSlots * kPSlot];
  // (80 KB: two work-groups fill a compute unit's LDS.  The waves' furthest
  // keys pass through the last slot, which no load writes before every wave
  // has read them.)
  int* const s_far = (int*)(ring + (kPSlots - 1) * kPSlot);
  lds_char* const lds = (lds_char*)ring;
  int i, xb;
  xcd_head_block(i, xb);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
  // the last query blocks see the most keys: dispatch them first
  const int t = ((gridDim.x - 1 - xb) * kWv + wave) * kB + c;
  const bool t_ok = t < T;
  const int pos = t_ok ? positions[t] : -1;
  const bool valid = pos >= 0 && pos < kv_len;
  const int last = valid ? pos : -1;   // this query sees keys 0 .. last
  int far = last, near = last;         // the wave's furthest and nearest last keys
  for (int off = 32; off >= 1; off >>= 1) {
    far = max(far, __shfl_xor(far, off));
    near = min(near, __shfl_xor(near, off));
  }
  if (lane == 0) s_far[wave] = far;

  // Q^T as the B operand: K-step ks holds dims 16 ks + 8h .. + 7 of query t
  bf16x8 qv[kQK];
  {
    const __bf16* qr = q + ((long)(t_ok ? t : 0) * kH + i) * kW + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kQK; ++ks) qv[ks] = *(const bf16x8*)(qr + 16 * ks);
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);   // the ring below counts its own loads
  __syncthreads();
  const int far_wg = max(max(s_far[0], s_far[1]), max(s_far[2], s_far[3]));
  const int nkb = (far_wg + kB) / kB;   // key blocks the work-group streams

  // load k of wave w carries units 64 (w + 4k) .. of a block: K rows for
  // k < 3, V rows after; blocks past nkb are padding (zero ranges)
  int voff[kPLoads];
#pragma unroll
  for (int k = 0; k < kPLoads; ++k) voff[k] = src_off(wave + 4 * k, lane);
  auto issue = [&](int b) {
    const bool real = b < nkb;
    const int kb = real ? b : 0;
    const int nv = real ? min(kB, kv_len - kb * kB) : 0;
    const i32x4 rk = make_rsrc(kbuf + ((long)kb * kB * kH + i) * kW, nv * kStrideW);
    const i32x4 rv = make_rsrc(vbuf + ((long)kb * kB * kH + i) * kDv, nv * kStrideV);
    lds_char* slot = lds + (b % kPSlots) * kPSlot + wave * 1024;
#pragma unroll
    for (int k = 0; k < kPLoads; ++k) dma16(k < 3 ? rk : rv, voff[k], slot + 4096 * k);
  };

  f32x16 acc[kDv / 32];   // O^T, dims 32 d .. 32 d + 31 x the wave's 32 queries
#pragma unroll
  for (int d = 0; d < kDv / 32; ++d) acc[d] = f32x16{};
  settle_o(acc);
  // this lane's query: the reference u (log2 units) of O and l, and l, the
  // sum of the numerators 2^(s - u).  Any reference gives the same softmax;
  // u moves only when a block's maximum exceeds it by more than kLazy, so
  // the numerators stay at most 2^kLazy and O is rarely rescaled.  The score
  // products start from -R, R = u (0 while u = -inf), so they give s - R
  // directly: a block that keeps the reference needs no subtraction.
  float u = -INFINITY, l = 0.f, R = 0.f;
  f32x16 negr = {};
  settle(negr);
  // byte offsets of the V^T operand reads (K-step kap, dim tile d), formed
  // once; the empty asm keeps each a single register, so a read is that
  // register plus the slot's immediate (left to itself the compiler shares
  // the lanes' 8-byte half between them and adds it back at every read)
  int tro[2][kDv / 32][2];
#pragma unroll
  for (int kap = 0; kap < 2; ++kap)
#pragma unroll
    for (int d = 0; d < kDv / 32; ++d) {
      tr_offsets<false>(lane, 16 * kap, 32 * d, tro[kap][d][0], tro[kap][d][1]);
      asm volatile("" : "+v"(tro[kap][d][0]), "+v"(tro[kap][d][1]));
    }

  // Software pipeline over key blocks: iteration kb runs block kb's
  // softmax and O^T += V^T . P^T, and between them block kb + 1's score
  // products, one MFMA at a time with two of block kb's exp2s (or one pair's
  // packing) issued behind each, so that the VALU work runs while the
  // MFMA pipe is busy.  Each K-step's operand is read from LDS two MFMAs
  // ahead.  Block kb's slot is an immediate in every read: the loop body is
  // instantiated once per slot.
  // block b's scores less R in sb[b % 2] (formed during iteration b - 1;
  // b % 2 is the parity of its slot, so each copy of the body names fixed
  // registers and no tile is copied)
  f32x16 sb[2];
  auto step = [&](int kb, auto slot_c) {
    constexpr int kSlot = decltype(slot_c)::value;
    constexpr int kNext = (kSlot + 1) % kPSlots;
    f32x16& s = sb[kSlot & 1];
    f32x16& sn = sb[kNext & 1];
    wait_vm<kPLoads*(kPSlots - 3)>();   // this wave's loads of block kb + 1
    __syncthreads();   // everyone's; block kb - 1's slot is free
    issue(kb + kPSlots - 1);
    const int j0 = kb * kB;
    if (j0 <= far) {   // the wave has a query that sees a key of this block
      const lds_char* slot = lds + kSlot * kPSlot;
      const lds_char* nslot = lds + kNext * kPSlot;
      mfma_drain(s);
      // causal mask (only where the block reaches past some query's last
      // key) and the block's max for this query (both lane halves)
      if (j0 + kB - 1 > near) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
          s[r] = key <= last ? s[r] : -INFINITY;
        }
      }
      float bm = s[0];   // (the block's maximum less R)
#pragma unroll
      for (int r = 1; r < 16; ++r) bm = fmaxf(bm, s[r]);
      bm = swap_max(bm);
      // a new reference where the block's maximum passes u + kLazy (the
      // first key a query sees always does: u starts at -inf, alpha = 0 with
      // O and l still 0); no key seen yet: u stays -inf, numerators 0
      const bool raise = bm > (u == -INFINITY ? -INFINITY : kLazy);
      const float nu = raise ? bm + R : u;
      const float alpha = raise ? __builtin_amdgcn_exp2f(u - nu) : 1.f;
      u = nu;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        // scores to the new reference (a shift of 0 where it stays)
        const float nr = nu == -INFINITY ? 0.f : nu;
        const float shift = nr - R;
        R = nr;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] -= shift;
#pragma unroll
        for (int r = 0; r < 16; ++r) negr[r] = -nr;
        settle(negr);
        drain_o(acc);
#pragma unroll
        for (int d = 0; d < kDv / 32; ++d) acc[d] *= alpha;
        settle_o(acc);
      }
      // block kb + 1's scores (past the wave's last block: formed, unused)
      // beside block kb's numerators 2^(s - R) and their bf16 pairs
      uint32_t pr[8];
      bf16x8 ka[3];
      ka[0] = row24(nslot, lane, 0);
      ka[1] = row24(nslot, lane, 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < kQK; ++ks) {
        if (ks + 2 < kQK) ka[(ks + 2) % 3] = row24(nslot, lane, ks + 2);
        if (ks == 0)
          mfma_from(sn, ka[0], qv[0], negr);
        else
          mfma_acc(sn, ka[ks % 3], qv[ks]);
        if (ks < 8) {
          s[2 * ks] = __builtin_amdgcn_exp2f(s[2 * ks]);
          s[2 * ks + 1] = __builtin_amdgcn_exp2f(s[2 * ks + 1]);
        } else {
          pr[2 * (ks - 8)] = pack2(s[4 * (ks - 8)], s[4 * (ks - 8) + 1]);
          pr[2 * (ks - 8) + 1] = pack2(s[4 * (ks - 8) + 2], s[4 * (ks - 8) + 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // the pairs as the B operands of P^T (rows_as_b's exchange: a lane
      // holds rows 4h .. 4h + 3 of each eight, the lane 32 apart the others)
#pragma unroll
      for (int k = 0; k < 8; k += 4) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(pr[k], pr[k + 2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(pr[k + 1], pr[k + 3], false, false);
        pr[k] = s0[0];
        pr[k + 2] = s0[1];
        pr[k + 1] = s1[0];
        pr[k + 3] = s1[1];
      }
      bf16x8 pb[2];
      pb[0] = __builtin_bit_cast(bf16x8, u32x4{pr[0], pr[1], pr[2], pr[3]});
      pb[1] = __builtin_bit_cast(bf16x8, u32x4{pr[4], pr[5], pr[6], pr[7]});
      // l sums the bf16-rounded numerators, the values the product uses:
      // pairs dotted with (1, 1); pb holds 16 of the query's 32 keys, the
      // lane 32 apart the other 16
      {
        // (constant shuffle indices: each pair is its own register)
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        float ps0 = 0.f, ps1 = 0.f;
#define MLA_PAIR_SUM(e)                                                                       \
  ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[0], pb[0], 2 * e, 2 * e + 1), \
                                        one, ps0, false);                                     \
  ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[1], pb[1], 2 * e, 2 * e + 1), \
                                        one, ps1, false);
        MLA_PAIR_SUM(0)
        MLA_PAIR_SUM(1)
        MLA_PAIR_SUM(2)
        MLA_PAIR_SUM(3)
#undef MLA_PAIR_SUM
        l = l * alpha + swap_sum(ps0 + ps1);
      }
      settle(pb);
      // O^T += V^T . P^T: the A operand of dim tile d, K-step kap is dim
      // 32 d + c of the block's keys 16 kap + 8h .. + 7
#pragma unroll
      for (int kap = 0; kap < 2; ++kap)
#pragma unroll
        for (int d = 0; d < kDv / 32; ++d)
          mfma_acc(acc[d], tr_read(slot, tro[kap][d][0], tro[kap][d][1]), pb[kap]);
    }
  };
  static_assert(kPSlots == 4, "the loop below runs four slots");
#pragma unroll
  for (int b = 0; b < kPSlots - 1; ++b) issue(b);
  wait_vm<kPLoads*(kPSlots - 2)>();   // this wave's loads of block 0
  __syncthreads();
  if (far >= 0) {   // block 0's scores
    mfma_from(sb[0], row24(lds, lane, 0), qv[0], negr);
#pragma unroll
    for (int ks = 1; ks < kQK; ++ks) mfma_acc(sb[0], row24(lds, lane, ks), qv[ks]);
  }
  int kb = 0;
  for (; kb + 4 <= nkb; kb += 4) {
    step(kb, ic<0>{});
    step(kb + 1, ic<1>{});
    step(kb + 2, ic<2>{});
    step(kb + 3, ic<3>{});
  }
  if (kb < nkb) step(kb, ic<0>{});
  if (kb + 1 < nkb) step(kb + 1, ic<1>{});
  if (kb + 2 < nkb) step(kb + 2, ic<2>{});
  wait_vm<0>();   // the padding loads of the ring's tail still write LDS
  drain_o(acc);
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
// (Prefills of fewer rows than the tiled GEMM takes; from there on that
// GEMM's epilogue rotates q^R.)
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
  hipLaunchKernelGGL(attn_prefill_v2_kernel, dim3((T + kWv * kB - 1) / (kWv * kB), kH),
                     dim3(64 * kWv), 0, s,
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
