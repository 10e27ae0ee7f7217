// Blocks of 32 rows of the DeepSeek-V2 heads (n_h = 128; query and key rows
// of 192 bf16, value rows of 128) streamed through LDS: the geometry, the
// swizzled LDS layout of a block, its loads, the MFMA operand reads of it
// (rows and transposed), and the small register shuffles the attention
// kernels of the prefill and the order-A backward share.
#pragma once

#include "lds_stream.h"

namespace mla {
namespace dev {

constexpr int kH = 128;          // heads
constexpr int kW = 192;          // query and key width
constexpr int kDv = 128;         // value width
constexpr int kB = 32;           // queries or keys per wave tile (and per block)
constexpr int kWv = 4;           // waves per work-group
constexpr int kQK = kW / 16;     // K-steps of the 192-wide products (12)
constexpr int kVK = kDv / 16;    // K-steps of the 128-wide products (8)
constexpr float kLog2e = 1.4426950408889634f;

// Blocks of 32 rows (keys, or queries) of one head stream through a ring of
// LDS slots by direct-to-LDS loads: each load moves 64 16-byte units, one
// per lane, to 1 KB of consecutive LDS.  In HBM ([row][head][width] arrays)
// consecutive rows of one head lie kStrideW (192-wide) or kStrideV (128-wide)
// bytes apart.  In a slot the 192-wide rows come first, 24 units each, then
// the 128-wide rows, 16 units each.
constexpr int kStrideW = kH * kW * 2;
constexpr int kStrideV = kH * kDv * 2;
constexpr int kUnitsW = kB * kW / 8;    // 768
constexpr int kUnitsV = kB * kDv / 8;   // 512

// A row's units are XOR-permuted so that the 16 rows one row read serves at
// once (lanes c = 0 .. 15, one unit each) and the 4 rows x 4 units that the
// 32 lanes of a transposing read served at once touch land on distinct
// banks (64 banks of 4 bytes).  192-wide rows (24 units, 96 banks apart from
// row to row): a 3-bit function of j >> 1 whose bit 2 follows bit 1 of j,
// so that rows two apart take complementary halves of each 8-unit group.
// 128-wide rows (16 units, 64 banks apart): a 4-bit function of j whose bits
// 2 and 3 follow j's two lowest bits, so that 4 consecutive rows take
// distinct 4-unit groups.
__device__ inline int sw24(int j) {
  const int v = (j >> 1) & 7;
  return ((v & 1) << 2) | ((v >> 1) & 3);
}
__device__ inline int sw16(int j) { return ((j & 3) << 2) | ((j >> 2) & 3); }
__device__ inline int unit24(int j, int p) { return j * 24 + (p ^ sw24(j)); }
__device__ inline int unit16(int j, int p) { return kUnitsW + j * 16 + (p ^ sw16(j)); }

// The source offset (from the block's first row) of the unit that lane
// `lane` of load r of a block carries: LDS unit u = 64 r + lane holds unit
// (u mod row units) ^ sw(j) of row j.
__device__ inline int src_off(int r, int lane) {
  const int u = 64 * r + lane;
  if (u < kUnitsW) {
    const int j = u / 24;
    return j * kStrideW + 16 * ((u % 24) ^ sw24(j));
  }
  const int v = u - kUnitsW, j = v / 16;
  return j * kStrideV + 16 * ((v % 16) ^ sw16(j));
}


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

// The A operand "columns D0 .. D0 + 31 of rows k0 + 8h .. + 7" of a slot's
// block, transposed: lane (c, h) receives column D0 + c of those eight rows.
// Two transposing reads of four rows each: in each 16-lane group lane s
// supplies the 8-byte piece of row k0 + 8h + s / 4 at columns D0 + 16 (group
// & 1) + 4 (s % 4), and output lane i receives, as its element r, element
// i % 4 of lane 4 r + i / 4's piece.  W24: the 192-wide rows, else the
// 128-wide ones.
template <bool W24>
__device__ inline bf16x8 tr_operand(const lds_char* slot, int lane, int k0, int D0) {
  const int j = k0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int p = D0 / 8 + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int half = 8 * (lane & 1);
  const int u0 = W24 ? unit24(j, p) : unit16(j, p);
  const int u1 = W24 ? unit24(j + 4, p) : unit16(j + 4, p);
  const v4bf16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(slot + 16 * u0 + half));
  const v4bf16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(slot + 16 * u1 + half));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// The same operand from byte offsets formed once: tr_offsets gives the two
// reads' offsets within a slot (lane-dependent, loop-invariant), tr_read
// reads them from a slot, so that a loop over blocks issues each read as a
// register plus the slot's immediate offset.
template <bool W24>
__device__ inline void tr_offsets(int lane, int k0, int D0, int& o0, int& o1) {
  const int j = k0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int p = D0 / 8 + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int half = 8 * (lane & 1);
  o0 = 16 * (W24 ? unit24(j, p) : unit16(j, p)) + half;
  o1 = 16 * (W24 ? unit24(j + 4, p) : unit16(j + 4, p)) + half;
}
__device__ inline bf16x8 tr_read(const lds_char* slot, int o0, int o1) {
  const v4bf16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(slot + o0));
  const v4bf16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(slot + o1));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Row reads: lane (c, h) gets unit 2 ks + h of row c (an A operand).
__device__ inline bf16x8 row24(const lds_char* slot, int lane, int ks) {
  const int c = lane & 31, h = lane >> 5;
  return *(const lds_bf16x8*)(slot + 16 * unit24(c, 2 * ks + h));
}
__device__ inline bf16x8 row16(const lds_char* slot, int lane, int ks) {
  const int c = lane & 31, h = lane >> 5;
  return *(const lds_bf16x8*)(slot + 16 * unit16(c, 2 * ks + h));
}


// The score products S and dP as inline-asm MFMAs with VGPR accumulators:
// with the builtin the compiler keeps them in the accumulation registers,
// which the long-lived dq, dK and dV sums fill, and copies registers between
// the two files every block.  Back-to-back accumulation into the same
// registers needs no wait states; mfma_drain's 24 wait states cover the last
// product's result before VALU reads it.
// (Not volatile: the scheduler may then hoist the LDS reads that feed them.
// Their operands come from LDS reads and from registers loaded once, never
// from a VALU write just before.)
__device__ __forceinline__ void mfma_first(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// the first product of a chain that starts from c instead of zero (c from
// registers that no VALU instruction has just written)
__device__ __forceinline__ void mfma_from(f32x16& d, bf16x8 a, bf16x8 b, const f32x16& c) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
}
__device__ __forceinline__ void mfma_drain(f32x16& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}
__device__ __forceinline__ void mfma_drain(f32x16& s, f32x16& dp) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s), "+v"(dp));
}
// The dq, dK and dV sums take mfma_agpr (AGPR accumulators); their B operands
// are the bf16 numerators, a VALU write just before: settle puts more than the
// 2 wait states an MFMA read of them needs in between.
__device__ __forceinline__ void settle(bf16x8 (&x)[2]) {
  asm volatile("s_nop 4" : "+v"(x[0]), "+v"(x[1]));
}
__device__ __forceinline__ void settle(f32x16& x) {
  asm volatile("s_nop 4" : "+v"(x));
}

// Work-groups are dispatched round-robin over the eight XCDs (linear index
// L = blockIdx.y * gridDim.x + blockIdx.x goes to XCD L % 8).  Each XCD takes
// whole heads: its s-th work-group runs block xb = s % gridDim.x of head
// 8 (s / gridDim.x) + L % 8, so all work-groups of one head stream its blocks
// through one L2.  (gridDim.y = 128 heads.)
__device__ inline void xcd_head_block(int& head, int& xb) {
  const int gx = gridDim.x;
  const int L = blockIdx.y * gx + blockIdx.x;
  const int s = L >> 3;
  xb = s % gx;
  head = (s / gx) * 8 + (L & 7);
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


}  // namespace dev
}  // namespace mla
