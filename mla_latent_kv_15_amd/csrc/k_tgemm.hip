// Tiled MFMA GEMM for many activation rows: Y = alpha * X . W^T with X
// [M][K] and W [N][K] bf16 (both K-contiguous), fp32 sums, Y bf16 or fp32.
//
// The products with hundreds to thousands of rows (prefill over T tokens,
// the order-A backward over the cached rows) are bound by MFMA, not by
// streaming W once, so they take large output tiles instead of the
// weight-streaming kernel's 64-row blocks: one work-group of eight waves per
// compute unit owns a BM x BN tile of Y and walks K in steps of 32.  Each
// step's W rows (BN x 32) and X rows (BM x 32) go to LDS by direct-to-LDS
// buffer loads through a ring of three to six stages, so that the next two
// to five steps' loads fly while this step's MFMAs run.  The products are
// v_mfma_f32_32x32x16_bf16 with the W rows as the A operand and the X rows
// as the B operand, i.e. the tile is formed as Y^T: every lane then owns one
// row of Y and four consecutive columns per result group, stored as one
// 16-byte (fp32) or 8-byte (bf16) write.  The fp32 sums stay in the
// accumulation registers (in ordinary registers for the 256 x 320 tile).
// Those four columns are two whole (2k, 2k + 1) pairs, so a bf16 Y can also
// leave the epilogue RoPE-rotated (the prefill's q^R) with no lane exchange.
#include "lds_stream.h"
#include "mla_internal.h"

namespace mla {

namespace {

using namespace dev;

constexpr int kBK = 32;   // K per step (the shapes taken need K % kBK == 0)

// BM x BN tile, K in steps of BK through a ring of S LDS stages; the eight waves form a WM x WN grid, each owning (BM / WM) x
// (BN / WN) of Y: TM x TN MFMA tiles of 32 x 32.
//
// In LDS a row's U = BK / 8 16-byte units are XOR-permuted (U = 8: by
// (row >> 1) & 7; U = 4: by (row >> 2) & 3), so that the 16 rows one operand
// read serves in one LDS cycle (lanes c = 0 .. 15, one unit each) land on
// distinct banks.
template <int U>
__device__ inline int row_swz(int r) {
  return U == 8 ? (r >> 1) & 7 : (r >> 2) & 3;
}

// K split: work-group z of the grid's third dimension takes columns
// [z kc, (z + 1) kc) and writes its fp32 partial at Y + z y_split_stride.
template <int BM, int BN, int WM, int WN, int BK, int S, bool F32, bool WT>
__global__ __launch_bounds__(512, 1) void tgemm_kernel(int M, int N, int K, int kc,
                                                       const __bf16* __restrict__ X, long ldx,
                                                       const __bf16* __restrict__ W,
                                                       void* __restrict__ Y, long ldy,
                                                       long y_split_stride, float alpha,
                                                       int y_grp, long y_grp_stride,
                                                       const int32_t* __restrict__ rope_pos,
                                                       const float* __restrict__ rope_tab,
                                                       int rope_len) {
  static_assert(WM * WN == 8, "eight waves");
  constexpr int TM = BM / (32 * WM), TN = BN / (32 * WN);
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "whole MFMA tiles");
  constexpr int U = BK / 8;                                        // 16-byte units per row
  static_assert(U == 4 || U == 8, "BK 32 or 64");
  constexpr int kUnitsW = BN * U, kUnitsX = BM * U;
  constexpr int kLoads = (kUnitsW + kUnitsX + 511) / 512;          // per wave per step
  constexpr int kStage = kLoads * 8 * 1024;                        // loads past the rows pad
  static_assert(kUnitsW % 64 == 0 && kUnitsX % 64 == 0, "whole loads per part");
  static_assert(kLoads * (S - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[S * kStage];
  lds_char* const lds = (lds_char*)smem;

  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  // (the wave index as a scalar: the loads' descriptors are picked by it)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c = lane & 31, h = lane >> 5;
  const int wm = wave % WM, wn = wave / WM;
  const int nk = kc / BK;
  const int kz = blockIdx.z * kc;   // this split's first column

  // Load k of wave w carries units 64 (w + 8k) .. of a step: W rows, then X
  // rows, then padding.  voff: the lane's source offset from the step's first
  // column of the tile's first row; part: 0 W, 1 X, 2 padding (uniform per
  // wave and load).
  int voff[kLoads], part[kLoads];
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int r = wave + 8 * k, u = 64 * r + lane;
    if (64 * r < kUnitsW) {
      const int n = u / U, p = (u % U) ^ row_swz<U>(n);
      voff[k] = WT ? 2 * (int)tile_index(n, 8 * p, K) : 2 * (n * K + 8 * p);
      part[k] = 0;
    } else if (64 * r < kUnitsW + kUnitsX) {
      const int v = u - kUnitsW, m = v / U, p = (v % U) ^ row_swz<U>(m);
      voff[k] = 2 * (m * (int)ldx + 8 * p);
      part[k] = 1;
    } else {
      voff[k] = kOob;
      part[k] = 2;
    }
  }
  const int mvalid = min(BM, M - m0);
  const __bf16* wblk =
      W + (WT ? (long)(n0 / 16) * (K / 32) * 512 + (long)(kz / 32) * 512 : (long)n0 * K + kz);
  const __bf16* xblk = X + (long)m0 * ldx + kz;
  // step kb into stage `stage` (padding past the last step: zero ranges)
  auto issue = [&](int kb, int stage) {
    const bool real = kb < nk;
    const int k0 = real ? kb * BK : 0;
    const i32x4 rw = make_rsrc(wblk + (WT ? (long)(k0 / 32) * 512 : (long)k0),
                               real ? 0x7fffffff : 0);
    const i32x4 rx = make_rsrc(xblk + k0, real ? mvalid * (int)ldx * 2 : 0);
    const i32x4 rz = make_rsrc(xblk, 0);
    lds_char* dst = lds + stage * kStage + wave * 1024;
#pragma unroll
    for (int k = 0; k < kLoads; ++k)
      dma16(part[k] == 0 ? rw : (part[k] == 1 ? rx : rz), voff[k], dst + 8192 * k);
  };

  // Up to 128 fp32 sums per lane stay in the accumulation registers.  The
  // 256 x 320 tile has 160: at two waves per SIMD the accumulation
  // registers hold at most 128 of a wave's 256, so its sums live in ordinary
  // registers (and the wait states around the MFMA chain cover all ten of
  // them in one statement, which nothing can be scheduled across).
  constexpr bool kVacc = TM * TN > 8;
  static_assert(!kVacc || TM * TN == 10, "register sums: the 256 x 320 tile only");
  f32x16 acc[TN * TM];
#pragma unroll
  for (int t = 0; t < TN * TM; ++t) acc[t] = f32x16{};
  if constexpr (kVacc)
    asm volatile("s_nop 4"
                 : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]),
                   "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7]), "+v"(acc[8]), "+v"(acc[9]));
  else
    settle_acc(acc);
  static_assert(BK == 32, "the loop below holds two K-steps of 16 per step");
  const int xc = row_swz<U>(c);
  // the operands of K-step ks (0 or 1) of the step in `stage`
  auto read = [&](int stage, int ks, bf16x8 (&a)[TN], bf16x8 (&b)[TM]) {
    const lds_char* sW = lds + stage * kStage;
    const lds_char* sX = sW + kUnitsW * 16;
    const int pu = 16 * ((2 * ks + h) ^ xc);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      a[tn] = *(const lds_bf16x8*)(sW + 16 * U * ((wn * TN + tn) * 32 + c) + pu);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      b[tm] = *(const lds_bf16x8*)(sX + 16 * U * ((wm * TM + tm) * 32 + c) + pu);
  };
  auto mult = [&](const bf16x8 (&a)[TN], const bf16x8 (&b)[TM]) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        if constexpr (kVacc)
          asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
              : "+v"(acc[tn * TM + tm])
              : "v"(a[tn]), "v"(b[tm]));
        else
          mfma_agpr(acc[tn * TM + tm], a[tn], b[tm]);
      }
  };
  // The ring holds steps kb .. kb + S - 1.  The second K-step's operands of
  // step kb stay in registers across the barrier that frees its stage, so the
  // wave has MFMAs to run while the next step's first reads are in flight
  // (both waves of a SIMD leave the barrier together).
#pragma unroll
  for (int kb = 0; kb < S; ++kb) issue(kb, kb);
  wait_vm<kLoads*(S - 1)>();   // this wave's loads of step 0
  __syncthreads();
  bf16x8 a0[TN], b0[TM], a1[TN], b1[TM];
  read(0, 0, a0, b0);
  int cur = 0;   // stage of step kb
  for (int kb = 0; kb < nk; ++kb) {
    read(cur, 1, a1, b1);
    mult(a0, b0);
    wait_vm<kLoads*(S - 2)>();                               // own loads of step kb + 1
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");     // this step's reads are done
    __syncthreads();   // everyone's loads of step kb + 1 landed; stage `cur` is free
    issue(kb + S, cur);
    const int nx = cur + 1 == S ? 0 : cur + 1;
    read(nx, 0, a0, b0);   // (past the last step: the padding's zeros, unused)
    mult(a1, b1);
    cur = nx;
  }
  if constexpr (kVacc)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]),
                   "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7]), "+v"(acc[8]), "+v"(acc[9]));
  else
    mfma_drain_acc(acc);
  wait_vm<0>();   // the padding loads of the ring's tail still write LDS

  // acc[tn][tm] is Y^T: lane (c, h) holds row m = ... + c of Y, columns
  // 8 g + 4h .. + 3 for g = 0 .. 3 (its registers 4g .. 4g + 3).
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = m0 + (wm * TM + tm) * 32 + c;
    if (m >= M) continue;
    // RoPE (bf16 Y only): row m's position, -1 where the table has no row
    int pos = -1;
    if (!F32 && rope_tab) {
      const int p = rope_pos[m];
      pos = p >= 0 && p < rope_len ? p : -1;
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + (wn * TN + tn) * 32 + 8 * g + 4 * h;
        const f32x16& a = acc[tn * TM + tm];
        f32x4 v = {alpha * a[4 * g], alpha * a[4 * g + 1], alpha * a[4 * g + 2],
                   alpha * a[4 * g + 3]};
        const long col = y_grp > 0 ? (long)(n / y_grp) * y_grp_stride + n % y_grp : n;
        if (!F32 && rope_tab) {
          // the lane's four columns are the pairs (2k, 2k + 1), (2k + 2,
          // 2k + 3) of a column group, k = (n % y_grp) / 2 even: each pair
          // turns by the angle of pair k (k + 1) at position pos, the
          // table's (cos, sin) entries k, k + 1 being one 16-byte read
          if (pos >= 0) {
            const f32x4 cs =
                *(const f32x4*)(rope_tab + ((long)pos * (y_grp / 2) + (n % y_grp) / 2) * 2);
            v = f32x4{v[0] * cs[0] - v[1] * cs[1], v[0] * cs[1] + v[1] * cs[0],
                      v[2] * cs[2] - v[3] * cs[3], v[2] * cs[3] + v[3] * cs[2]};
          } else {
            v = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                      __builtin_nanf("")};
          }
        }
        if constexpr (F32) {
          *(f32x4*)((float*)Y + blockIdx.z * y_split_stride + (long)m * ldy + col) = v;
        } else {
          const u32x2 pk = {__builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[0], (__bf16)v[1]}),
                            __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[2], (__bf16)v[3]})};
          *(u32x2*)((__bf16*)Y + (long)m * ldy + col) = pk;
        }
      }
  }
}

struct TileCfg {
  int bm, bn;
};
// The candidate tiles in order of preference (larger tiles reuse each
// operand more); the first that fills at least 90% of a round of work-groups
// on the compute units wins, else the one that fills the most.  (256 x 320:
// a 4096 x 5120 output is exactly one round of 256 tiles, and each 32-wide
// K-step moves 36 KB into LDS for 5.2 MFLOP, 142 flop/B, against 91 for
// 128 x 320.)
constexpr TileCfg kTiles[] = {{256, 320}, {256, 256}, {128, 320}, {256, 128}, {128, 192}};

int n_compute_units() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

}  // namespace

int tgemm_units(int M, int N, int K) {
  const int t = tgemm_pick(M, N, K);
  if (t < 0) return -1;
  return ((M + kTiles[t].bm - 1) / kTiles[t].bm) * (N / kTiles[t].bn);
}

int tgemm_pick(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % kBK != 0) return -1;
  const int G = n_compute_units();
  int best = -1;
  double best_eff = -1.0;
  for (int t = 0; t < (int)(sizeof(kTiles) / sizeof(kTiles[0])); ++t) {
    if (N % kTiles[t].bn != 0) continue;
    const long units = (long)((M + kTiles[t].bm - 1) / kTiles[t].bm) * (N / kTiles[t].bn);
    const long rounds = (units + G - 1) / G;
    const double eff = (double)units / (double)(rounds * G);
    if (eff >= 0.9) return t;
    if (eff > best_eff + 1e-9) {
      best = t;
      best_eff = eff;
    }
  }
  return best;
}

hipError_t tgemm(int M, int N, int K, const void* X, long ldx, const void* W, bool w_tiled,
                 void* Y, long ldy, bool out_f32, float alpha, hipStream_t s, int y_grp,
                 long y_grp_stride, int splits, long y_split_stride, const int32_t* rope_pos,
                 const float* rope_tab, int rope_len) {
  if (M <= 0) return hipSuccess;
  if (splits < 1 || K % (splits * kBK) != 0 || (splits > 1 && (!out_f32 || y_grp > 0)))
    return hipErrorNotSupported;
  if (rope_tab && (!rope_pos || out_f32 || y_grp <= 0 || rope_len <= 0))
    return hipErrorInvalidValue;
  const int kc = K / splits;
  const int t = tgemm_pick(M, N, kc);
  if (t < 0 || ldx % 8 != 0 || ldx < K || (long)256 * ldx * 2 >= 0x7fffffffL || ldy % 4 != 0 ||
      (y_grp > 0 && (y_grp % 32 != 0 || y_grp_stride % 4 != 0 || out_f32)) ||
      (w_tiled && N % 16 != 0))
    return hipErrorNotSupported;
  const dim3 block(512);
#define MLA_TG_GO(BM, BN, WM, WN, S, F32, WT)                                                  \
  hipLaunchKernelGGL((tgemm_kernel<BM, BN, WM, WN, kBK, S, F32, WT>),                          \
                     dim3(N / BN, (M + BM - 1) / BM, splits), block, 0, s, M, N, K, kc,       \
                     (const __bf16*)X, ldx, (const __bf16*)W, Y, ldy, y_split_stride, alpha,   \
                     y_grp, y_grp_stride, rope_pos, rope_tab, rope_len)
#define MLA_TG(BM, BN, WM, WN, S)                        \
  do {                                                   \
    if (out_f32 && w_tiled)                              \
      MLA_TG_GO(BM, BN, WM, WN, S, true, true);          \
    else if (out_f32)                                    \
      MLA_TG_GO(BM, BN, WM, WN, S, true, false);         \
    else if (w_tiled)                                    \
      MLA_TG_GO(BM, BN, WM, WN, S, false, true);         \
    else                                                 \
      MLA_TG_GO(BM, BN, WM, WN, S, false, false);        \
  } while (0)
  switch (t) {
    case 0: MLA_TG(256, 320, 4, 2, 3); break;
    case 1: MLA_TG(256, 256, 2, 4, 4); break;
    case 2: MLA_TG(128, 320, 4, 2, 4); break;
    case 3: MLA_TG(256, 128, 4, 2, 5); break;
    default: MLA_TG(128, 192, 4, 2, 6); break;
  }
#undef MLA_TG
#undef MLA_TG_GO
  return hipGetLastError();
}

}  // namespace mla
