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
// The kernels take Q times log2(e) (q16), so that S comes out in log2 units
// for exp2; dK is scaled back by ln 2 as it leaves.
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

#include "head_blocks.h"
#include "mla_internal.h"

namespace mla {

namespace {

using namespace dev;


constexpr int kSlots = 4;
constexpr int kLoadsA = (kUnitsW + kUnitsV) / 64 / kWv;   // 5 loads per wave per block
constexpr int kLoadsB = kLoadsA + 1;                       // + records (wave 0) or padding
constexpr int kSlotA = (kUnitsW + kUnitsV) * 16;           // 20 KB
constexpr int kSlotB = kSlotA + kWv * 1024;                // 24 KB
static_assert(kLoadsA * kWv * 64 == kUnitsW + kUnitsV, "whole loads per block");
static_assert(kLoadsB * (kSlots - 2) < 64, "vmcnt range");

// ---------------------------------------------------------------------------
// query side: LSE, D and dq
// ---------------------------------------------------------------------------
// rec[i * T + t] = {LSE (log2 units), D, lim, 0} of query t and head i, lim
// (an int's bits) one past the last key the query sees: a key j takes part
// iff j < lim.  Zeros (a query past T) take no part.
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_v2_kernel(
    const __bf16* __restrict__ q16, const __bf16* __restrict__ do16,
    const __bf16* __restrict__ k16, const __bf16* __restrict__ v16,
    const int32_t* __restrict__ positions, int T, int N, float scale, f32x4* __restrict__ rec,
    int* __restrict__ qblk_far, float* __restrict__ dq) {
  __shared__ __attribute__((aligned(16))) char ring[kSlots * kSlotA];
  __shared__ int s_far[kWv];
  lds_char* const lds = (lds_char*)ring;
  int i, xb;
  xcd_head_block(i, xb);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
  // the last query blocks see the most keys: dispatch them first
  const int qb = (gridDim.x - 1 - xb) * kWv + wave;   // this wave's 32 queries
  const int t = qb * kB + c;
  const bool t_ok = t < T;
  const int pos = t_ok ? positions[t] : -1;
  const bool valid = pos >= 0 && pos < N;
  // keys this query sees: 0 .. last (an invalid position: all of them, NaN)
  const int last = t_ok ? (valid ? pos : N - 1) : -1;
  int far = last, near = last;   // the block's furthest and nearest last keys
  for (int off = 32; off >= 1; off >>= 1) {
    far = max(far, __shfl_xor(far, off));
    near = min(near, __shfl_xor(near, off));
  }
  if (lane == 0) {
    s_far[wave] = far;
    if (i == 0 && qb * kB < T) {
      qblk_far[2 * qb] = far;
      qblk_far[2 * qb + 1] = near;
    }
  }
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
  // the ring below counts its own loads: none other may be in flight
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  const int far_wg = max(max(s_far[0], s_far[1]), max(s_far[2], s_far[3]));
  const int nkb = (far_wg + kB) / kB;   // key blocks the work-group streams (per pass)

  // The two passes stream the same key blocks: sequence element b < nkb is
  // block b of pass 1, nkb <= b < 2 nkb block b - nkb of pass 2; past that a
  // padding load.  Load k of wave w carries units 64 (w + 4k) .. of a block:
  // K rows for k < 3, V rows after.
  int voff[kLoadsA];
#pragma unroll
  for (int k = 0; k < kLoadsA; ++k) voff[k] = src_off(wave + 4 * k, lane);
  const int nseq = 2 * nkb;
  auto issue = [&](int b) {
    const bool real = b < nseq;
    const int kb = real ? (b < nkb ? b : b - nkb) : 0;
    const int nv = real ? min(kB, N - kb * kB) : 0;
    const i32x4 rk = make_rsrc(k16 + ((long)kb * kB * kH + i) * kW, nv * kStrideW);
    const i32x4 rv = make_rsrc(v16 + ((long)kb * kB * kH + i) * kDv, nv * kStrideV);
    lds_char* slot = lds + (b % kSlots) * kSlotA + wave * 1024;
#pragma unroll
    for (int k = 0; k < kLoadsA; ++k) dma16(k < 3 ? rk : rv, voff[k], slot + 4096 * k);
  };
  // S^T = K Q^T and dP^T = V dO^T of a block (rows: keys, column: query)
  auto scores = [&](const lds_char* slot, int ln, f32x16& s, f32x16& dp) {
    mfma_first(s, row24(slot, ln, 0), qv[0]);
#pragma unroll
    for (int ks = 1; ks < kQK; ++ks) mfma_acc(s, row24(slot, ln, ks), qv[ks]);
    mfma_first(dp, row16(slot, ln, 0), dv[0]);
#pragma unroll
    for (int ks = 1; ks < kVK; ++ks) mfma_acc(dp, row16(slot, ln, ks), dv[ks]);
    mfma_drain(s, dp);
  };

#pragma unroll
  for (int b = 0; b < kSlots - 1; ++b) issue(b);
  int b = 0;
  // ---- pass 1: m, l, z of this lane's query (log2 units)
  float m = -INFINITY, l = 0.f, z = 0.f;
  for (int kb = 0; kb < nkb; ++kb, ++b) {
    wait_vm<kLoadsA*(kSlots - 2)>();   // this wave's loads of block b
    __syncthreads();                     // everyone's; slot (b - 1) is free
    issue(b + kSlots - 1);
    const int j0 = kb * kB;
    if (j0 <= far) {
      f32x16 s, dp;
      scores(lds + (b % kSlots) * kSlotA, lane, s, dp);
      // (log2 units: q16 carries log2 e; the mask only where the block
      // reaches past some query's last key)
      if (j0 + kB - 1 > near) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
          s[r] = key <= last ? s[r] : -INFINITY;
        }
      }
      float bm = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) bm = fmaxf(bm, s[r]);
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
  }
  const float nanv = __builtin_nanf("");
  const float lse = valid ? m + __log2f(l) : nanv;
  const float dd = valid ? z / l : nanv;

  // ---- pass 2: dQ^T += K^T dS^T
  f32x16 acc[kW / 32];
#pragma unroll
  for (int dt = 0; dt < kW / 32; ++dt) acc[dt] = f32x16{};
  settle_acc(acc);
  for (int kb = 0; kb < nkb; ++kb, ++b) {
    wait_vm<kLoadsA*(kSlots - 2)>();
    __syncthreads();
    issue(b + kSlots - 1);
    const int j0 = kb * kB;
    if (j0 <= far) {
      const lds_char* slot = lds + (b % kSlots) * kSlotA;
      const int ln = lane;
      f32x16 s, dp;
      scores(slot, ln, s, dp);
      if (j0 + kB - 1 > near) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
          const float p = key <= last ? __builtin_amdgcn_exp2f(s[r] - lse) : 0.f;
          s[r] = p * (dp[r] - dd);   // dS^T
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(s[r] - lse) * (dp[r] - dd);
      }
      bf16x8 pb[2];
      rows_as_b(s, pb);
      settle(pb);
#pragma unroll
      for (int kap = 0; kap < 2; ++kap)
#pragma unroll
        for (int dt = 0; dt < kW / 32; ++dt)
          mfma_agpr(acc[dt], tr_operand<true>(slot, ln, 16 * kap, 32 * dt), pb[kap]);
    }
  }
  mfma_drain_acc(acc);
  wait_vm<0>();   // the ring's padding loads still write LDS
  if (!t_ok) return;
  if (h == 0) rec[(long)i * T + t] = f32x4{lse, dd, __int_as_float(last + 1), 0.f};
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
constexpr int kMaxQb = 2048;                       // query blocks (their far keys sit in LDS)
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTrPitch = kB + 8;                   // keys per LDS row of the transposed tiles
static_assert(kWv * kDv * kTrPitch * 2 <= kSlots * kSlotB, "transposed tiles fit the ring");

__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_v2_kernel(
    const __bf16* __restrict__ q16, const __bf16* __restrict__ do16,
    const __bf16* __restrict__ k16, const __bf16* __restrict__ v16,
    const f32x4* __restrict__ rec, const int* __restrict__ qblk_far, int T, int N, int Npad,
    __bf16* __restrict__ dkv16, __bf16* __restrict__ dkT16, __bf16* __restrict__ dvT16,
    float* __restrict__ dkr) {
  __shared__ __attribute__((aligned(16))) char ring[kSlots * kSlotB];
  __shared__ int s_qf[kMaxQb], s_qn[kMaxQb];
  lds_char* const lds = (lds_char*)ring;
  int i, xb;
  xcd_head_block(i, xb);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
  const int wg_j0 = xb * kWv * kB;   // the first key blocks see the most queries
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
  // the query blocks that see at least one key of the work-group; the
  // decision is the same for every thread (qblk_far is per query block).
  // The blocks' far keys are read once into LDS (nqb <= kMaxQb), so that the
  // scan below costs no memory round trips.
  const int nqb = (T + kB - 1) / kB;
  for (int e = tid; e < nqb; e += 256) {
    s_qf[e] = qblk_far[2 * e];
    s_qn[e] = qblk_far[2 * e + 1];
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);   // the ring below counts its own loads
  __syncthreads();
  auto qfar = [&](int qb) { return s_qf[qb]; };
  auto next_active = [&](int qb) {
    while (qb < nqb && qfar(qb) < wg_j0) ++qb;
    return qb;
  };

  // A slot: the block's Q rows, dO rows, then 32 records (wave 0's sixth
  // load; the other waves' sixth load is padding).
  int voff[kLoadsB];
#pragma unroll
  for (int k = 0; k < kLoadsA; ++k) voff[k] = src_off(wave + 4 * k, lane);
  voff[kLoadsA] = wave == 0 && lane < kB ? 16 * lane : kOob;
  int qi = next_active(0);   // the next block to load
  auto issue = [&](int b) {
    const bool real = qi < nqb;
    const int qb = real ? qi : 0;
    const int nv = real ? min(kB, T - qb * kB) : 0;
    const i32x4 rq = make_rsrc(q16 + ((long)qb * kB * kH + i) * kW, nv * kStrideW);
    const i32x4 ro = make_rsrc(do16 + ((long)qb * kB * kH + i) * kDv, nv * kStrideV);
    const i32x4 rs = make_rsrc(rec + (long)i * T + qb * kB, nv * 16);
    lds_char* slot = lds + (b % kSlots) * kSlotB + wave * 1024;
#pragma unroll
    for (int k = 0; k < kLoadsB; ++k)
      dma16(k < 3 ? rq : (k < kLoadsA ? ro : rs), voff[k], slot + 4096 * k);
    if (real) qi = next_active(qi + 1);
  };

  f32x16 accK[kW / 32], accV[kDv / 32];
#pragma unroll
  for (int dt = 0; dt < kW / 32; ++dt) accK[dt] = f32x16{};
#pragma unroll
  for (int dt = 0; dt < kDv / 32; ++dt) accV[dt] = f32x16{};
  settle_acc(accK);
  settle_acc(accV);
#pragma unroll
  for (int b = 0; b < kSlots - 1; ++b) issue(b);
  int qb = next_active(0);
  for (int b = 0; qb < nqb; ++b) {
    wait_vm<kLoadsB*(kSlots - 2)>();   // this wave's loads of block b
    __syncthreads();                     // everyone's; slot (b - 1) is free
    issue(b + kSlots - 1);
    if (qfar(qb) >= j0) {   // this wave's keys: some query of the block sees one
      const lds_char* slot = lds + (b % kSlots) * kSlotB;
      const int ln = lane;
      // S = Q K^T and dP = dO V^T (rows: queries, column: key c)
      f32x16 s, dp;
      mfma_first(s, row24(slot, ln, 0), kv[0]);
#pragma unroll
      for (int ks = 1; ks < kQK; ++ks) mfma_acc(s, row24(slot, ln, ks), kv[ks]);
      mfma_first(dp, row16(slot, ln, 0), vv[0]);
#pragma unroll
      for (int ks = 1; ks < kVK; ++ks) mfma_acc(dp, row16(slot, ln, ks), vv[ks]);
      mfma_drain(s, dp);
      // rows 8 g + 4h + e: the records of those four queries (S in log2
      // units: q16 carries log2 e).  The mask only where some (query, key)
      // pair of the block is not seen (a key past N stays exactly zero even
      // beside a NaN query row).
      f32x16 ds;
      const bool all_seen = j0 + kB - 1 <= s_qn[qb];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const f32x4 st =
              *(const lds_f32x4*)(slot + 16 * (kUnitsW + kUnitsV + 8 * g + 4 * h + e));
          if (all_seen) {
            const float p = __builtin_amdgcn_exp2f(s[r] - st[0]);
            s[r] = p;                   // P
            ds[r] = p * (dp[r] - st[1]);  // dS
          } else {
            const bool seen = key_ok && key < __float_as_int(st[2]);
            const float p = seen ? __builtin_amdgcn_exp2f(s[r] - st[0]) : 0.f;
            s[r] = p;
            ds[r] = seen ? p * (dp[r] - st[1]) : 0.f;
          }
        }
      bf16x8 pbP[2], pbS[2];
      rows_as_b(s, pbP);
      rows_as_b(ds, pbS);
      settle(pbP);
      settle(pbS);
#pragma unroll
      for (int kap = 0; kap < 2; ++kap) {
#pragma unroll
        for (int dt = 0; dt < kDv / 32; ++dt)
          mfma_agpr(accV[dt], tr_operand<false>(slot, ln, 16 * kap, 32 * dt), pbP[kap]);
#pragma unroll
        for (int dt = 0; dt < kW / 32; ++dt)
          mfma_agpr(accK[dt], tr_operand<true>(slot, ln, 16 * kap, 32 * dt), pbS[kap]);
      }
    }
    qb = next_active(qb + 1);
  }
  mfma_drain_acc(accK);
  mfma_drain_acc(accV);
  wait_vm<0>();      // the padding loads still write LDS
  // dK^T += Q16^T dS with Q16 = scale log2(e) q: dK = ln 2 . accK
#pragma unroll
  for (int dt = 0; dt < kW / 32; ++dt) accK[dt] *= kLn2;
  __syncthreads();   // and every wave is done with the ring
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

// dC[j] = [sum_z lat[z][j] | sum_i dkr[i][j]], one work-group per cached row,
// both sums in a fixed order: two latent columns per thread, and the RoPE
// part as four quarters of the heads per column, added through LDS.
__global__ __launch_bounds__(256) void bwd_dc_v2_kernel(int N, const float* __restrict__ lat,
                                                        int splits,
                                                        const float* __restrict__ dkr,
                                                        float* __restrict__ dC) {
  constexpr int kC = 512, kR = kW - kDv, kRow = kC + kR;
  __shared__ float part[4][kR];
  const int j = blockIdx.x, tid = threadIdx.x;
#pragma unroll
  for (int e = tid; e < kC; e += 256) {
    float a = 0.f;
    for (int z = 0; z < splits; ++z) a += lat[((long)z * N + j) * kC + e];
    dC[(long)j * kRow + e] = a;
  }
  const int d = tid & (kR - 1), qtr = tid >> 6;   // 64 dims x 4 quarters of the heads
  float a = 0.f;
#pragma unroll 8
  for (int i = qtr * (kH / 4); i < (qtr + 1) * (kH / 4); ++i) a += dkr[((long)i * N + j) * kR + d];
  part[qtr][d] = a;
  __syncthreads();
  if (tid < kR) dC[(long)j * kRow + kC + tid] = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
}

// q (fp32, RoPE applied) times `scale` (the softmax scale times log2 e), and
// dO, as bf16 rows
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

int attn_bwd_v2_max_queries() { return kMaxQb * kB; }

// a block's byte offsets (rows of all heads) stay within 32 bits
int attn_bwd_v2_max_keys() { return 65536; }

int attn_bwd_v2_npad(int N) { return (N + kWv * kB - 1) / (kWv * kB) * (kWv * kB); }

hipError_t attn_bwd_v2(const Geo& g, int N, int T, const float* q, const float* dO,
                       const int32_t* positions, const void* k16, const void* v16, void* q16,
                       void* do16, void* rec, int* qblk_far, float* dq, void* dkv16, void* dkT16,
                       void* dvT16, float* dkr, hipStream_t s) {
  if (N <= 0 || T <= 0) return hipSuccess;
  if (!attn_bwd_v2_supported(g) || T > attn_bwd_v2_max_queries() || N > attn_bwd_v2_max_keys())
    return hipErrorInvalidValue;
  const long nq = (long)T * kH * kW, nd = (long)T * kH * kDv;
  // q16 = scale log2(e) q: the scores come out in log2 units
  hipLaunchKernelGGL(bwd_inputs_v2_kernel, dim3((unsigned)((nq / 4 + 255) / 256)), dim3(256), 0, s,
                     q, dO, nq, nd, g.scale * kLog2e, (__bf16*)q16, (__bf16*)do16);
  hipLaunchKernelGGL(attn_bwd_dq_v2_kernel, dim3((T + kWv * kB - 1) / (kWv * kB), kH),
                     dim3(64 * kWv), 0, s, (const __bf16*)q16, (const __bf16*)do16,
                     (const __bf16*)k16, (const __bf16*)v16, positions, T, N, g.scale, (f32x4*)rec,
                     qblk_far, dq);
  hipLaunchKernelGGL(attn_bwd_dkv_v2_kernel, dim3(attn_bwd_v2_npad(N) / (kWv * kB), kH),
                     dim3(64 * kWv), 0, s, (const __bf16*)q16, (const __bf16*)do16,
                     (const __bf16*)k16, (const __bf16*)v16, (const f32x4*)rec, qblk_far, T, N,
                     attn_bwd_v2_npad(N), (__bf16*)dkv16, (__bf16*)dkT16, (__bf16*)dvT16, dkr);
  return hipGetLastError();
}

int bwd_lat_splits(int N) {
  const int units = tgemm_units(N, 512, 2 * kH * kDv);
  if (units <= 0) return 1;
  int sp = 1;
  while (sp < 32 && units * sp * 2 <= 256) sp *= 2;
  return sp;
}

hipError_t bwd_dc_v2(int N, const float* lat, int splits, const float* dkr, float* dC,
                     hipStream_t s) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dc_v2_kernel, dim3(N), dim3(256), 0, s, N, lat, splits, dkr, dC);
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
