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
// wgemm: one work-group per compute unit streams an equal share of W: 16 RB
// weight rows times a K chunk, with RB and the chunk chosen per shape so that
// the work-groups fill the GPU exactly (wgemm_tile).  Its four waves split the
// chunk four ways; each streams 16-byte pieces of W straight into the B
// operand of v_mfma_f32_16x16x32_bf16 (lane = weight row, 8 consecutive k) and
// reuses each activation piece (A operand) for all RB row blocks.  With W in
// the tiled layout (tile_index) each such piece of 16 rows is one contiguous
// 1 KB load, and a wave's share of a 16-row block is one contiguous run.  The four
// partial tiles are summed in LDS in a fixed order.  Split-K chunks write fp32
// partials that a small kernel reduces in a fixed order (deterministic).
#include "mla_internal.h"
#include "plan_device.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMT = 64;   // activation rows per work-group (4 MFMA blocks of 16)

// Activations may come in the "blocked" layout (blk_index): a wave then
// fetches each 16 x 32 A operand with one fully contiguous 1 KB load instead
// of touching 16 rows.  Producers of GEMM inputs write it; rows past M are
// padding.

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Y = alpha * X . W^T over one K chunk.  Work-group (row group ng, chunk sp)
// = blockIdx.x (ng fastest), activation block = blockIdx.y.  X row m of the
// weight rows n lives at X + (n / n_group) * x_group_stride + m * ldx.
// Weight rows n >= n2 come from a second matrix W2 (its row n - n2) and go to
// Y2 as fp32 (row stride ldy2): two projections of the same input in one
// launch.  n2 >= N leaves W2 unused.
// NS > 0: each wave runs exactly NS K-steps of 32, fully unrolled (the
// decode shapes); NS == 0: a loop over the steps, DEPTH dividing their count.
// WT: W (and W2) in the tiled layout, K columns.
#define MLA_WGEMM_PARAMS                                                                     \
  int M, int K, int kc, int n_groups, const __bf16 *__restrict__ X, long ldx,                \
      long x_group_stride, int n_group, const __bf16 *__restrict__ W, void *__restrict__ Y,  \
      long ldy, long y_split_stride, float alpha, int x_blocked, int y_blocked,              \
      const __bf16 *__restrict__ W2, int n2, float *__restrict__ Y2, long ldy2, int y_grp,   \
      long y_grp_stride
#define MLA_WGEMM_FWD                                                                        \
  M, K, kc, n_groups, X, ldx, x_group_stride, n_group, W, Y, ldy, y_split_stride, alpha,     \
      x_blocked, y_blocked, W2, n2, Y2, ldy2, y_grp, y_grp_stride
// the work of work-group (bx, by)
template <int RB, int NS, int DEPTH, bool OUT_F32, bool WT>
__device__ __forceinline__ void wgemm_wg(const int bx, const int by, MLA_WGEMM_PARAMS) {
  __shared__ f32x4 red[4][RB][4][64];  // [wave][rb][mb][lane]
  const int ng = bx % n_groups, sp = bx / n_groups;
  const int n0 = ng * 16 * RB;
  const int m0 = by * kMT;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int kw = kc >> 2;                       // this wave's share of the chunk
  const int kbeg = sp * kc + wave * kw + 8 * g;
  const int nmb = min(4, (M - m0 + 15) >> 4);
  const __bf16* xb = X + (long)(n0 / n_group) * x_group_stride;
  const bf16x8* xr[4];
  int xstep;   // bf16x8 units from one K-step of an A operand to the next
  if (x_blocked) {
    const long blk = ((long)(m0 >> 6) * (K >> 5) + ((kbeg - 8 * g) >> 5)) * 4;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) xr[mb] = (const bf16x8*)(xb + ((blk + mb) * 64 + lane) * 8);
    xstep = 4 * 64;
  } else {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = min(m0 + mb * 16 + r16, M - 1);
      xr[mb] = (const bf16x8*)(xb + (long)m * ldx + kbeg);
    }
    xstep = 4;
  }
  const bf16x8* wr[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // a 16-row block lies wholly on one side of n2
    const bool second = n0 + rb * 16 >= n2;
    const __bf16* wm = second ? W2 : W;
    const int nb = second ? n0 + rb * 16 - n2 : n0 + rb * 16;
    if constexpr (WT)
      wr[rb] = (const bf16x8*)(wm + ((long)(nb >> 4) * (K >> 5) + ((kbeg - 8 * g) >> 5)) * 512) +
               lane;
    else
      wr[rb] = (const bf16x8*)(wm + (long)(nb + r16) * K + kbeg);
  }
  constexpr int wstep = WT ? 64 : 4;   // bf16x8 units from one K-step of W to the next

  f32x4 acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[rb][mb] = f32x4{};

  // Register ring of DEPTH K-steps of operands: step st + DEPTH is loaded
  // while step st is multiplied, so DEPTH steps of W stay in flight.  All
  // four activation blocks are multiplied (rows past M repeat row M-1; only
  // rows < M are stored), which keeps the step free of branches.
  // The weights are read once per launch: their loads carry the nontemporal
  // hint (the decode step took about 3% less time with it); the activations,
  // re-read by every work-group of a row block, do not.
  bf16x8 bq[DEPTH][RB], aq[DEPTH][4];
  auto load = [&](int d, int st) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) bq[d][rb] = __builtin_nontemporal_load(&wr[rb][wstep * st]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) aq[d][mb] = xr[mb][xstep * st];
  };
  // inline asm with the accumulator tied in its accumulation registers: with
  // the builtin, the register allocator renames the accumulators across the
  // ring's phases and copies them back every iteration
  auto step = [&](int d) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                     : "+a"(acc[rb][mb])
                     : "v"(aq[d][mb]), "v"(bq[d][rb]));
    // the refill of slot d stays after the MFMAs that read it: hoisted above
    // them, it would need fresh registers and copies, and copying a load in
    // flight waits for it
    __builtin_amdgcn_sched_barrier(0);
  };
  // one K-step after the other: interleaved, waiting for step 0's operands
  // would also wait for parts of the later steps
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    load(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (NS > 0) {
    // straight-line code: the compiler waits for exactly the step it needs
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      step(st % DEPTH);
      if (st + DEPTH < NS) load(st % DEPTH, st + DEPTH);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // generic shapes: the loads are unconditional (the last round re-reads
    // the final step, unused); across the loop's back edge the compiler
    // drains them at the top of each round
    const int nsteps = kw >> 5;
#pragma clang loop unroll(disable)
    for (int s0 = 0; s0 < nsteps; s0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        step(d);
        load(d, min(s0 + d + DEPTH, nsteps - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // MFMA result -> read by other instructions: wait states the compiler
  // cannot see for inline-asm MFMAs
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[rb][0]), "+a"(acc[rb][1]), "+a"(acc[rb][2]), "+a"(acc[rb][3]));
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) red[wave][rb][mb][lane] = acc[rb][mb];
  __syncthreads();
  // wave w finishes activation block w: fixed-order sum over the four waves
  const int mb = wave;
  if (mb >= nmb) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    f32x4 v = red[0][rb][mb][lane];
    v += red[1][rb][mb][lane];
    v += red[2][rb][mb][lane];
    v += red[3][rb][mb][lane];
    const int n = n0 + rb * 16 + r16;
    const bool second = n0 + rb * 16 >= n2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + mb * 16 + 4 * g + i;
      if (m < M) {
        if (second)
          Y2[(long)m * ldy2 + (n - n2)] = alpha * v[i];
        else if (OUT_F32)
          ((float*)Y)[sp * y_split_stride + (long)m * ldy + n] = alpha * v[i];
        else if (y_blocked)
          ((__bf16*)Y)[blk_index(m, n, n_groups * 16 * RB)] = (__bf16)(alpha * v[i]);
        else if (y_grp > 0)
          ((__bf16*)Y)[(long)m * ldy + (long)(n / y_grp) * y_grp_stride + n % y_grp] =
              (__bf16)(alpha * v[i]);
        else
          ((__bf16*)Y)[(long)m * ldy + n] = (__bf16)(alpha * v[i]);
      }
    }
  }
}

template <int RB, int NS, int DEPTH, bool OUT_F32, bool WT>
__global__ __launch_bounds__(256, 1) void wgemm_kernel(MLA_WGEMM_PARAMS) {
  wgemm_wg<RB, NS, DEPTH, OUT_F32, WT>(blockIdx.x, blockIdx.y, MLA_WGEMM_FWD);
}

// The same GEMM and, in one extra work-group (the last of each row), the
// split-KV plan: a GEMM work-group leaves room on its compute unit for the
// planner, which then runs beside the GEMM instead of after it.
template <int RB, int NS, int DEPTH, bool OUT_F32, bool WT>
__global__ __launch_bounds__(256, 1) void wgemm_plan_kernel(MLA_WGEMM_PARAMS, PlanJob job) {
  if (blockIdx.x == gridDim.x - 1) {
    if (blockIdx.y == 0) plan_build(job);
    return;
  }
  wgemm_wg<RB, NS, DEPTH, OUT_F32, WT>(blockIdx.x, blockIdx.y, MLA_WGEMM_FWD);
}

// out[m][n] = sum_s part[s][m][n] (fixed order), as bf16
// (blocked: out in the blocked activation layout with K = N)
__global__ void splitk_reduce_kernel(int M, int N, int S, const float* __restrict__ part,
                                     long split_stride, __bf16* __restrict__ out, long ldo,
                                     int blocked) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[s * split_stride + (long)m * N + n];
  out[blocked ? blk_index(m, n, N) : (long)m * ldo + n] = (__bf16)v;
}

// the same, four consecutive outputs per thread (N, ldo multiples of 4)
__global__ void splitk_reduce4_kernel(int M, int N, int S, const float* __restrict__ part,
                                      long split_stride, __bf16* __restrict__ out, long ldo,
                                      int blocked) {
  const long idx = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (idx >= (long)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) v += *(const f32x4*)(part + s * split_stride + (long)m * N + n);
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  *(bf16x4*)(out + (blocked ? blk_index(m, n, N) : (long)m * ldo + n)) = o;
}

// The absorbed query of one head i and 64 batch rows: q~_i = scale * W_UK,i^T
// q^C_i (latent half ch of the 512 columns per work-group: grid.x = 2 i + ch,
// grid.y = row block), and the RoPE part, scale * RoPE(q^R_i) at the query's
// position, packed after q~_i (rows split between the two work-groups).
// W_UK,i is [128 d][512 c]; the contraction runs over its row index, so each
// lane reads eight consecutive rows (d) of one 8-byte column chunk and
// transposes them in registers into four B operands: N block j covers
// c = 256 ch + 64 wave + 4 r16 + j.  All loads are issued before the first
// MFMA (one memory round trip).  WT: W_UK in the tiled layout, where the four
// columns of a row stay contiguous.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <bool WT>
__global__ __launch_bounds__(256, 1) void absorb_kernel(
    int M, const __bf16* __restrict__ qc, const __bf16* __restrict__ W_UK,
    __bf16* __restrict__ q_abs, int q_tiled, float scale, const float* __restrict__ q_r,
    const int32_t* __restrict__ positions, const float* __restrict__ rope, int rope_len) {
  // Work-groups are dispatched round-robin over the eight XCDs.  In the
  // query-tile layout the eight heads 8k .. 8k + 7 share every 128-byte line
  // (16 bytes each), so all sixteen work-groups of such a group (eight heads,
  // two column halves) go to one XCD: its L2 then holds whole lines, and no
  // line reaches memory partly written from several L2s.
  const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int pair = 4 * xcd + (k >> 3);           // (head group, column half)
  const int head = 8 * (pair >> 1) + (k & 7), ch = pair & 1;
  const int m0 = blockIdx.y * kMT;
  // element (m, head, d) of the output; four (two) consecutive d from a
  // multiple of four (two) stay consecutive in both layouts
  auto qidx = [&](long m, int d) -> long {
    return q_tiled ? qtile_index(m, head, d) : (m * 128 + head) * 576 + d;
  };

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int nmb = min(4, (M - m0 + 15) >> 4);
  const int c0 = 256 * ch + 64 * wave + 4 * r16;
  // RoPE part, rows 32 ch .. 32 ch + 31 of the block: row m, rotation pair k
  // of q^R_i (NaN for a position outside the table); four per thread, stored
  // last.  The positions and q^R go out together first; the table entries
  // the positions select go out behind the W_UK loads (a position's load and
  // its table entry's load back to back would cost a memory round trip each).
  constexpr int kPer = 32 * 32 / 256;
  float2 x[kPer], cs[kPer];
  int mm[kPer], pos[kPer];
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int e = threadIdx.x + 256 * it;
    const int m = min(m0 + 32 * ch + (e >> 5), M - 1), k = e & 31;
    mm[it] = m0 + 32 * ch + (e >> 5);
    x[it] = *(const float2*)(q_r + ((long)m * 128 + head) * 64 + 2 * k);
    pos[it] = positions[m];
  }
  __builtin_amdgcn_sched_barrier(0);
  // row d of W_UK,i, columns c0 .. c0 + 3
  const __bf16* wh = W_UK + (long)head * 128 * 512;
  auto wrow = [&](int d) -> const u32x2* {
    if constexpr (WT) return (const u32x2*)(wh + tile_index(d, c0, 512));
    return (const u32x2*)(wh + (long)d * 512 + c0);
  };
  u32x2 v[4][8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int r = 0; r < 8; ++r) v[ks][r] = *wrow(32 * ks + 8 * g + r);
  bf16x8 a[4][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = min(m0 + mb * 16 + r16, M - 1);
      a[ks][mb] = *(const bf16x8*)(qc + (long)m * 16384 + head * 128 + 32 * ks + 8 * g);
    }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int k = (threadIdx.x + 256 * it) & 31;
    const bool ok = pos[it] >= 0 && pos[it] < rope_len;
    cs[it] = *(const float2*)(rope + ((long)(ok ? pos[it] : 0) * 32 + k) * 2);
    if (!ok) cs[it] = float2{__builtin_nanf(""), __builtin_nanf("")};
  }
  f32x4 acc[4][4];   // [mb][j]
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mb][j] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      u32x4 lo, hi;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        lo[f] = __builtin_amdgcn_perm(v[ks][2 * f + 1][e], v[ks][2 * f][e], 0x05040100u);
        hi[f] = __builtin_amdgcn_perm(v[ks][2 * f + 1][e], v[ks][2 * f][e], 0x07060302u);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < nmb) {
          acc[mb][2 * e] = mfma16(a[ks][mb], __builtin_bit_cast(bf16x8, lo), acc[mb][2 * e]);
          acc[mb][2 * e + 1] = mfma16(a[ks][mb], __builtin_bit_cast(bf16x8, hi), acc[mb][2 * e + 1]);
        }
      }
    }
  // D: lane holds column r16 of each N block (c = c0 + j) and rows 4g + i
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb >= nmb) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + mb * 16 + 4 * g + i;
      if (m >= M) continue;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (__bf16)(scale * acc[mb][j][i]);
      *(bf16x4*)(q_abs + qidx(m, c0)) = o;
    }
  }
  // RoPE part (its loads were issued first)
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int e = threadIdx.x + 256 * it, k = e & 31;
    if (mm[it] >= M) continue;
    const float o0 = (x[it].x * cs[it].x - x[it].y * cs[it].y) * scale;
    const float o1 = (x[it].x * cs[it].y + x[it].y * cs[it].x) * scale;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    *(bf16x2*)(q_abs + qidx(mm[it], 512 + 2 * k)) = bf16x2{(__bf16)o0, (__bf16)o1};
  }
}

}  // namespace

// Tile choice: the share of a work-group is 16 rb weight rows x K / splits.
// Among the tilings that divide the shape, take the one that keeps the most
// compute units busy (work-groups / (rounds x CUs)), then the fewest K splits
// (fewer partials to reduce), then the most rows per work-group (each
// activation piece serves more MFMAs).  A group of n_group weight rows reads
// its own activation rows, so a work-group's rows must lie in one group.
GemmTile wgemm_tile(int N, int K, int n_group, bool allow_split) {
  const int G = auto_wg_budget();
  GemmTile best{0, 0};
  double best_eff = -1.0;
  for (int rb = 5; rb >= 1; --rb) {
    const int R = 16 * rb;
    if (N % R != 0 || (n_group > 0 && n_group % R != 0)) continue;
    for (int sp = 1; sp <= (allow_split ? 64 : 1); ++sp) {
      if (K % (128 * sp) != 0) continue;
      const long units = (long)(N / R) * sp;
      const long rounds = (units + G - 1) / G;
      const double eff = (double)units / (double)(rounds * G);
      const bool better = eff > best_eff + 1e-9 ||
                          (eff > best_eff - 1e-9 && (sp < best.splits ||
                                                     (sp == best.splits && rb > best.rb)));
      if (better) {
        best = GemmTile{rb, sp};
        best_eff = eff;
      }
    }
  }
  return best;
}

hipError_t wgemm(const GemmTile& t, int M, int N, int K, const void* X, long ldx,
                 long x_group_stride, int n_group, const void* W, void* Y, long ldy,
                 long y_split_stride, bool out_f32, float alpha, hipStream_t s, bool x_blocked,
                 bool y_blocked, bool w_tiled, int y_grp, long y_grp_stride) {
  if (M <= 0) return hipSuccess;
  if (t.rb < 1 || t.rb > 5 || t.splits < 1 || N % (16 * t.rb) != 0 || K % (128 * t.splits) != 0 ||
      (t.splits > 1 && !out_f32) || (y_blocked && (out_f32 || N % 32 != 0)) ||
      (x_blocked && n_group > 0 && n_group != N) || (w_tiled && K % 32 != 0) ||
      (y_grp > 0 && (out_f32 || y_blocked)) || y_grp < 0)
    return hipErrorInvalidValue;
  const int n_groups = N / (16 * t.rb);
  const int kc = K / t.splits;
  const int nsteps = kc / 128;   // K-steps of 32 per wave
  const int depth = nsteps % 4 == 0 ? 4 : 1;
  const int xb = x_blocked ? 1 : 0, yb = y_blocked ? 1 : 0;
  const dim3 grid(n_groups * t.splits, (M + kMT - 1) / kMT);
  if (n_group <= 0) n_group = N;
#define MLA_WGEMM_GO(RB, NS, D, F32, WT)                                                       \
  hipLaunchKernelGGL((wgemm_kernel<RB, NS, D, F32, WT>), grid, dim3(256), 0, s, M, K, kc,      \
                     n_groups, (const __bf16*)X, ldx, x_group_stride, n_group,                 \
                     (const __bf16*)W, Y, ldy, y_split_stride, alpha, xb, yb,                  \
                     (const __bf16*)nullptr, N, (float*)nullptr, 0L, y_grp, y_grp_stride)
#define MLA_WGEMM_LAUNCH(RB, NS, D)                 \
  do {                                              \
    if (out_f32 && w_tiled)                         \
      MLA_WGEMM_GO(RB, NS, D, true, true);          \
    else if (out_f32)                               \
      MLA_WGEMM_GO(RB, NS, D, true, false);         \
    else if (w_tiled)                               \
      MLA_WGEMM_GO(RB, NS, D, false, true);         \
    else                                            \
      MLA_WGEMM_GO(RB, NS, D, false, false);        \
    return hipGetLastError();                       \
  } while (0)
  // fully unrolled variants for the decode projections' tiles on 256 CUs
  // (W_O, W_UQ / W_UV, W_QR, W_DQ of the DeepSeek-V2 layer)
  if (t.rb == 5 && nsteps == 32) MLA_WGEMM_LAUNCH(5, 32, 4);
  if (t.rb == 4 && nsteps == 12) MLA_WGEMM_LAUNCH(4, 12, 4);
  if (t.rb == 4 && nsteps == 4) MLA_WGEMM_LAUNCH(4, 4, 4);
  if (t.rb == 2 && nsteps == 12) MLA_WGEMM_LAUNCH(2, 12, 4);
  if (t.rb == 3 && nsteps == 5) MLA_WGEMM_LAUNCH(3, 5, 5);
#define MLA_WGEMM_CASE(RB)                                               \
  case RB:                                                               \
    if (depth == 4) MLA_WGEMM_LAUNCH(RB, 0, 4);                          \
    MLA_WGEMM_LAUNCH(RB, 0, 1);
  switch (t.rb) {
    MLA_WGEMM_CASE(1)
    MLA_WGEMM_CASE(2)
    MLA_WGEMM_CASE(3)
    MLA_WGEMM_CASE(4)
    MLA_WGEMM_CASE(5)
  }
#undef MLA_WGEMM_CASE
#undef MLA_WGEMM_LAUNCH
#undef MLA_WGEMM_GO
  return hipGetLastError();
}

hipError_t wgemm_with_plan(const GemmTile& t, int M, int N, int K, const void* X, long ldx,
                          const void* W, float* Y, long ldy, long y_split_stride, bool w_tiled,
                          const PlanJob& job, hipStream_t s) {
  // the fully unrolled tile of the W_DQ projection: 3 row blocks, 5 K-steps
  // per wave
  constexpr int RB = 3, NS = 5;
  if (M <= 0 || t.rb != RB || t.splits < 1 || N % (16 * RB) != 0 || K % (128 * t.splits) != 0 ||
      K / t.splits != 4 * 32 * NS)
    return hipErrorNotSupported;
  const int n_groups = N / (16 * RB), kc = K / t.splits;
  const dim3 grid(n_groups * t.splits + 1, (M + kMT - 1) / kMT);
#define MLA_WGEMM_PLAN(WT)                                                                      \
  hipLaunchKernelGGL((wgemm_plan_kernel<RB, NS, NS, true, WT>), grid, dim3(256), 0, s, M, K, kc, \
                     n_groups, (const __bf16*)X, ldx, 0L, N, (const __bf16*)W, (void*)Y, ldy,    \
                     y_split_stride, 1.f, 0, 0, (const __bf16*)nullptr, N, (float*)nullptr, 0L,  \
                     0, 0L, job)
  if (w_tiled)
    MLA_WGEMM_PLAN(true);
  else
    MLA_WGEMM_PLAN(false);
#undef MLA_WGEMM_PLAN
  return hipGetLastError();
}

hipError_t wgemm_pair(int M, int K, const void* X, bool x_blocked, const void* W1, int N1,
                      void* Y1, long ldy1, const void* W2, int N2, float* Y2, long ldy2,
                      bool w_tiled, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  constexpr int RB = 6, NS = 12;
  const int N = N1 + N2;
  if (N1 % 16 != 0 || N % (16 * RB) != 0 || K != 4 * 32 * NS || N / (16 * RB) > auto_wg_budget())
    return hipErrorNotSupported;
  const int n_groups = N / (16 * RB);
  const dim3 grid(n_groups, (M + kMT - 1) / kMT);
  if (w_tiled)
    hipLaunchKernelGGL((wgemm_kernel<RB, NS, 4, false, true>), grid, dim3(256), 0, s, M, K, K,
                       n_groups, (const __bf16*)X, (long)K, 0L, N, (const __bf16*)W1, Y1, ldy1,
                       0L, 1.f, x_blocked ? 1 : 0, 0, (const __bf16*)W2, N1, Y2, ldy2, 0, 0L);
  else
    hipLaunchKernelGGL((wgemm_kernel<RB, NS, 4, false, false>), grid, dim3(256), 0, s, M, K, K,
                       n_groups, (const __bf16*)X, (long)K, 0L, N, (const __bf16*)W1, Y1, ldy1,
                       0L, 1.f, x_blocked ? 1 : 0, 0, (const __bf16*)W2, N1, Y2, ldy2, 0, 0L);
  return hipGetLastError();
}

hipError_t splitk_reduce(int M, int N, int S, const float* part, long split_stride, void* out,
                         long ldo, hipStream_t s, bool blocked) {
  long n = (long)M * N;
  if (n == 0) return hipSuccess;
  if (N % 4 == 0 && split_stride % 4 == 0 && (blocked || ldo % 4 == 0) &&
      ((uintptr_t)part & 15) == 0 && ((uintptr_t)out & 7) == 0)
    hipLaunchKernelGGL(splitk_reduce4_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0,
                       s, M, N, S, part, split_stride, (__bf16*)out, ldo, blocked ? 1 : 0);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       M, N, S, part, split_stride, (__bf16*)out, ldo, blocked ? 1 : 0);
  return hipGetLastError();
}

hipError_t absorb_v2(int M, const void* qc, const void* W_UK, bool w_tiled, void* q_abs,
                     bool q_tiled, float scale, const float* q_r, const int32_t* positions,
                     const float* rope, int rope_len, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const dim3 grid(2 * 128, (M + kMT - 1) / kMT);
  if (q_tiled) scale *= kQTileLog2e;   // query tiles hold scores in log2 units
  if (w_tiled)
    hipLaunchKernelGGL(absorb_kernel<true>, grid, dim3(256), 0, s, M, (const __bf16*)qc,
                       (const __bf16*)W_UK, (__bf16*)q_abs, (int)q_tiled, scale, q_r,
                       positions, rope, rope_len);
  else
    hipLaunchKernelGGL(absorb_kernel<false>, grid, dim3(256), 0, s, M, (const __bf16*)qc,
                       (const __bf16*)W_UK, (__bf16*)q_abs, (int)q_tiled, scale, q_r,
                       positions, rope, rope_len);
  return hipGetLastError();
}

}  // namespace mla
