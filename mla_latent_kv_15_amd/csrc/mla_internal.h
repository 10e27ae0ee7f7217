// Internal declarations shared by the host API and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// Resolved layer geometry (defaults applied).
struct Geo {
  int d, n_h, d_h, d_c, d_cq, d_r, page;
  int row;        // d_c + d_r: numbers cached per token
  float scale;    // softmax scale
  double base;    // RoPE base
  bool bf16;      // storage dtype
  int esize() const { return bf16 ? 2 : 4; }
};

// The DeepSeek-V2 decode shape served by the MFMA kernels.
constexpr bool kHaveV2Attention = true;
inline bool is_v2_fast(const Geo& g) {
  return kHaveV2Attention && g.bf16 && g.n_h == 128 && g.d_c == 512 && g.d_r == 64 &&
         g.d_h == 128 && g.page % 64 == 0 && g.d % 128 == 0 && g.d_cq % 128 == 0;
}

// ---------------------------------------------------------------------------
// split-KV plan (device arrays carved from the workspace)
// ---------------------------------------------------------------------------
struct Seg {
  int b;    // sequence
  int t0;   // first token
  int t1;   // one past the last token
  int pad;
};

struct PlanPtrs {
  Seg* segs;            // [max_segs]
  int* seq_seg_start;   // [B]
  int* seq_seg_count;   // [B]; 0 marks an invalid sequence (NaN output)
  int* wg_seg_start;    // [max_wg + 1]
  int* counts;          // [0] = segments, [1] = work-groups in use
};

struct PlanDims {
  int max_segs;
  int max_wg;
};

// Work-group budget of the auto split mode for this device.
int auto_wg_budget();
PlanDims plan_dims(int B, int num_splits);
size_t plan_bytes(int B, int num_splits);
void carve_plan(void* base, int B, int num_splits, PlanPtrs* p);
hipError_t launch_plan(const PlanPtrs& p, const int32_t* kv_lens, int B, int max_kv_len,
                       int max_pages, int page, int tile, int num_splits, hipStream_t s);

// Everything the planner reads: a plan request that a launch of another kernel
// can carry (the plan then runs in one extra work-group of that launch).
struct PlanJob {
  PlanPtrs p;
  const int32_t* kv_lens;
  int B, max_kv_len, max_pages, page, tile, num_splits, max_wg;
};
PlanJob plan_job(const PlanPtrs& p, const int32_t* kv_lens, int B, int max_kv_len, int max_pages,
                 int page, int tile, int num_splits);
// out = sum_s part[s] as bf16 (splitk_reduce below) in one launch with the
// plan of `job`, built by one extra work-group beside the reduction's.
hipError_t splitk_reduce_with_plan(int M, int N, int S, const float* part, long split_stride,
                                   void* out, long ldo, bool blocked, const PlanJob& job,
                                   hipStream_t s);

// "Blocked" activation layout [M / 64][K / 32][4][64][8] of the GEMM inputs:
// the 16 x 32 A operand of one MFMA (rows 16 mb .. 16 mb + 15 of a 64-row
// group, K-step t) is 1 KB contiguous in lane order (lane 16 g + r holds row
// r, k = 32 t + 8 g .. + 7).
__device__ inline long blk_index(int m, int k, int K) {
  return ((((long)(m >> 6) * (K >> 5) + (k >> 5)) * 4 + ((m >> 4) & 3)) * 64 +
          (((k >> 3) & 3) << 4) + (m & 15)) * 8 + (k & 7);
}

// Tiled weight layout (MLA_LAYOUT_TILES): element (r, c) of a [R][C] matrix
// (R % 16 == 0, C % 32 == 0) sits in tile (r / 16, c / 32), 512 elements,
// tiles in row-major order; inside a tile at (16 ((c / 8) % 4) + r % 16) * 8
// + c % 8: the B operand of one 16x16x32 MFMA in lane order.
__host__ __device__ inline long tile_index(long r, long c, long C) {
  return (((r >> 4) * (C >> 5) + (c >> 5)) * 64 + (((c >> 3) & 3) << 4) + (r & 15)) * 8 + (c & 7);
}
// Query tiles: the absorbed query of the V2 fast path (128 heads of 576
// numbers per sequence) in the register order of the attention kernel's B
// operand, so that each of its query loads reads 1 KB contiguously instead of
// 16 B from each of 64 rows 1152 B apart.  Tiles the absorption writes hold
// the query times kQTileLog2e, so that the kernel's scores come out in log2
// units; tiles rearranged from a caller's rows hold the rows as they are.  Element (m, head, d) sits at
// [m][head / 32][d / 16][lane][d % 8] with lane = head % 32 + 32 ((d / 8) % 2):
// the 64 lanes of one wave's K-step of 16 numbers, 8 bf16 each.  A sequence's
// tiles occupy the same 147,456 bytes as its rows.
constexpr float kQTileLog2e = 1.4426950408889634f;
__host__ __device__ inline long qtile_index(long m, int head, int d) {
  return (((m * 4 + (head >> 5)) * 36 + (d >> 4)) * 64 + (head & 31) + 32 * ((d >> 3) & 1)) * 8 +
         (d & 7);
}
// The geometry admits the tiled layout for all eight matrices and their
// per-head slices (16-row aligned).
inline bool tiles_ok(const Geo& g) {
  return g.d % 32 == 0 && g.d_cq % 32 == 0 && g.d_c % 32 == 0 && (g.n_h * g.d_h) % 32 == 0 &&
         g.d_h % 16 == 0 && g.d_r % 16 == 0;
}

// ---------------------------------------------------------------------------
// generic kernels (any geometry, fp32 or bf16 storage)
// ---------------------------------------------------------------------------
enum GType { G_F32 = 0, G_BF16 = 1 };

// How the generic GEMM finds B(n, k): row-major B[n][k] or B[k][n] (ldb =
// its row length), or the same matrices in the tiled layout (ldb = columns).
enum BLayout { B_NK = 0, B_KN = 1, B_NK_TILES = 2, B_KN_TILES = 3 };
inline BLayout b_layout(bool tiled, bool kmajor) {
  return (BLayout)((tiled ? 2 : 0) + (kmajor ? 1 : 0));
}

// C[z][m][n] = alpha * sum_k A[z](m, k) * B[z](n, k), B(n, k) per bl, A(m, k)
// = A[m*lda + k] or, a_kmajor, A[k*lda + m]; c_tiled: C (ldc columns) in the
// tiled layout.  Types are element types of A, B, C.
hipError_t gemm_generic(GType ta, GType tb, GType tc, BLayout bl, int M, int N, int K,
                        const void* A, long lda, long sA, const void* B, long ldb, long sB,
                        void* C, long ldc, long sC, int batch, float alpha, hipStream_t s,
                        bool a_kmajor = false, bool c_tiled = false);

// dst = src ([R][C] row-major) in the tiled layout; elem_bytes 2 or 4.
hipError_t pack_tiles(const void* src, long R, long C, int elem_bytes, void* dst, hipStream_t s);

hipError_t rope_table_fill(float* table, int max_pos, int d_r, double base, hipStream_t s);

// q_abs[b][i][d_c + k] = RoPE(q_r[b][i][k]) * scale (fp32 source), storage out.
hipError_t pack_query_rope(const Geo& g, const float* q_r, const int32_t* positions, int B,
                           const float* rope, int rope_len, void* q_abs, hipStream_t s);

// Order-B attention core over the paged cache (generic), one WG per (segment, head).
hipError_t attn_decode_generic(const Geo& g, const void* q_abs, const void* cache, int num_pages,
                               const int32_t* page_table, int max_pages, const PlanPtrs& plan,
                               int max_segs, float* part_o, float* part_ml, void* lat_out,
                               hipStream_t s);

// Merge split partials; sequences with one segment were written directly.
hipError_t combine_partials(const Geo& g, const PlanPtrs& plan, int B, const float* part_o,
                            const float* part_ml, void* lat_out, hipStream_t s);

// Append: rotate + round + scatter rows of y [T][row] fp32.
hipError_t append_finish(const Geo& g, const float* y, const int32_t* positions,
                         const int32_t* slots, int T, const float* rope, int rope_len,
                         void* cache, int num_pages, hipStream_t s);

// Prefill helpers (generic, fp32 intermediates).
hipError_t gather_rows_f32(const Geo& g, const void* cache, int num_pages, const int32_t* page_table,
                           int max_pages, int kv_len, float* rows, hipStream_t s);
hipError_t broadcast_kr(const Geo& g, const float* rows, int kv_len, float* kbuf, hipStream_t s);
hipError_t rope_inplace_heads(const Geo& g, float* q, int T, long ld_row, int off,
                              const int32_t* positions, const float* rope, int rope_len,
                              hipStream_t s);
hipError_t attn_prefill_generic(const Geo& g, const float* q, const float* kbuf,
                                const float* vbuf, const int32_t* positions, int T, int kv_len,
                                int rope_len, float* o, hipStream_t s);
// The same causal attention on bf16 MFMA for the DeepSeek-V2 head shape:
// q [T][n_h][192] (times the softmax scale and log2 e), k [kv_len][n_h][192],
// v [kv_len][n_h][128] bf16 (p rounded to bf16, fp32 accumulation); o is bf16
// [T][n_h * d_h].
bool prefill_v2_supported(const Geo& g);
hipError_t attn_prefill_v2(const Geo& g, const void* q, const void* kbuf, const void* vbuf,
                           const int32_t* positions, int T, int kv_len, void* o, hipStream_t s);
// Its inputs besides the GEMM outputs: the cached rows [kv_len][576] bf16
// gathered through the page table (NaN for a bad page id) with k^R_j
// copied into every head's key, and RoPE of the scaled fp32 q^R into q
// (NaN for a position outside the table; the products of fewer rows than
// the tiled GEMM takes: from 128 rows on, that GEMM rotates q^R itself).
hipError_t prefill_rows_v2(const Geo& g, const void* cache, int num_pages,
                           const int32_t* page_table, int kv_len, void* rows, void* kbuf,
                           hipStream_t s);
hipError_t prefill_rope_q_v2(const Geo& g, const float* qr, const int32_t* positions, int T,
                             const float* rope, int rope_len, void* q, hipStream_t s);

// Order-A backward pieces (k_backward.hip): P and dS [n_h][T][N] per (query,
// head) from q [T][n_h][d_h + d_r], K, V [N][n_h][d_h], rows [N][row] and dO
// [T][n_h][d_h]; and dC [N][row] = [lat_k + lat_v | sum_i dkr[i]].
hipError_t attn_bwd_ps(const Geo& g, int N, int T, float scale, const float* q,
                       const int32_t* positions, const float* K, const float* V,
                       const float* rows, const float* dO, float* P, float* dS, hipStream_t s);
hipError_t attn_bwd_dc(const Geo& g, int N, const float* lat_k, const float* lat_v,
                       const float* dkr, float* dC, hipStream_t s);
// The same gradients for the DeepSeek-V2 head shape on bf16 MFMA, flash style
// (k_backward_v2.hip).  Inputs: q [T][128][192] and dO [T][128][128] fp32, k16
// [N][128][192] and v16 [N][128][128] bf16.  Scratch: q16, do16 (the bf16
// scaled query and dO), rec [128][T] x 16 bytes (LSE, D and the keys seen per
// query and head), qblk_far [ceil(T / 32)][2] (each query block's furthest and
// nearest last key).  Outputs:
// dq [T][128][192] fp32 (final), dkr [128][N][64] fp32 (per head), and dk^C,
// dv in bf16 as rows dkv16 [N][2 * 128 * 128] (all heads' dk^C, then all
// heads' dv) and key-contiguous dkT16, dvT16 [128 * 128][Npad] with zeros past
// N (Npad = attn_bwd_v2_npad(N)); T <= attn_bwd_v2_max_queries(), N <=
// attn_bwd_v2_max_keys().
bool attn_bwd_v2_supported(const Geo& g);
int attn_bwd_v2_max_queries();
int attn_bwd_v2_max_keys();
int attn_bwd_v2_npad(int N);
hipError_t attn_bwd_v2(const Geo& g, int N, int T, const float* q, const float* dO,
                       const int32_t* positions, const void* k16, const void* v16, void* q16,
                       void* do16, void* rec, int* qblk_far, float* dq, void* dkv16, void* dkT16,
                       void* dvT16, float* dkr, hipStream_t s);
// dst[c][dst_off + r] = src(r, c) (bf16) for r < R, zero for R <= r < Rpad, c
// < C; src row-major with ld_src, or tiled (tile_index with C columns).
// C and Rpad multiples of 64.
hipError_t transpose16(const void* src, long ld_src, bool tiled, int C, int R, int Rpad, void* dst,
                       long ld_dst, long dst_off, hipStream_t s);
// The K split of the latent-gradient product over N cached rows (so that its
// tiles fill the compute units), and dC [N][576] = [sum of the splits'
// partials lat [splits][N][512] | sum over the heads of dkr [128][N][64]].
int bwd_lat_splits(int N);
hipError_t bwd_dc_v2(int N, const float* lat, int splits, const float* dkr, float* dC,
                     hipStream_t s);

// MHA-equivalent decode attention over a [pages][page][2][n_h][d_h] cache
// (k_mha.hip): d_h a multiple of 16 with d_h / 16 a power of two <= 64.
bool mha_supported(const Geo& g);
// One work-group per (segment, group of heads); a sequence with one segment
// gets out directly, the others fp32 partials [segment][n_h][d_h] and
// (m, l) [segment][n_h] for combine_partials (with d_c = d_h).
hipError_t mha_decode(const Geo& g, const void* q, const void* cache, int num_pages,
                      const int32_t* page_table, int max_pages, const PlanPtrs& plan, int max_segs,
                      float scale, float* part_o, float* part_ml, void* out, hipStream_t s);

// ---------------------------------------------------------------------------
// MFMA kernels for the V2 bf16 shape
// ---------------------------------------------------------------------------
// q_tiles: the absorbed query in the query-tile layout (qtile_index).
// q_log2e: the tiles carry kQTileLog2e (as absorb_v2 writes them); else they
// are a caller's rows rearranged (pack_query_tiles).
hipError_t attn_decode_v2(const Geo& g, const void* q_tiles, bool q_log2e, const void* cache,
                          int num_pages, const int32_t* page_table, int max_pages,
                          const PlanPtrs& plan, int n_wg_launch, void* part_o, float* part_ml,
                          hipStream_t s);
// Rows [B][128][576] (bf16) rearranged into the query-tile layout (values
// unchanged).
hipError_t pack_query_tiles(const void* rows, int B, void* tiles, hipStream_t s);
// (part_o: bf16 [segments][128 * 512] in the accumulator's register order,
//  16 bytes (8 elements) of one lane per piece;
//  part_ml: fp32 [segments][128][2] = (reference max in nats, sum of numerators))
// Weight-streaming MFMA GEMM: Y = alpha * X . W^T (W [N][K] bf16, row-major
// or, w_tiled, in the tiled layout; X bf16 rows);
// X row m for weight rows n lives at X + (n / n_group) * x_group_stride + m * ldx
// (n_group <= 0: one group).  A work-group streams 16 rb rows x K / splits.
// splits > 1 requires out_f32: Y is fp32 partials [splits][M][ldy]; else Y is
// [M][ldy], bf16 or fp32 (y_grp > 0, bf16: column n lands at (n / y_grp) *
// y_grp_stride + n % y_grp of its row).  x_blocked: X (ungrouped) is in the blocked
// activation layout [ceil(M/64)][K/32][4][64][8] (1 KB per MFMA operand, rows
// padded to 64); y_blocked: bf16 Y is written in that layout with K = N.
struct GemmTile {
  int rb;       // weight rows per work-group / 16 (1..5)
  int splits;   // K chunks
};
GemmTile wgemm_tile(int N, int K, int n_group, bool allow_split);
// Split-K fp32 wgemm (row-major X) whose launch also builds the plan of `job`
// in one extra work-group; hipErrorNotSupported unless the tile is the W_DQ
// one (3 row blocks, K / splits = 640).
hipError_t wgemm_with_plan(const GemmTile& t, int M, int N, int K, const void* X, long ldx,
                          const void* W, float* Y, long ldy, long y_split_stride, bool w_tiled,
                          const PlanJob& job, hipStream_t s);
// Y1 = X . W1^T (bf16, N1 rows) and Y2 = X . W2^T (fp32, N2 rows) in one
// launch of 96-row work-groups without a K split; hipErrorNotSupported when
// the shape does not fit that tiling (K = 1536, N1 + N2 a multiple of 96
// within the compute units).
hipError_t wgemm_pair(int M, int K, const void* X, bool x_blocked, const void* W1, int N1,
                      void* Y1, long ldy1, const void* W2, int N2, float* Y2, long ldy2,
                      bool w_tiled, hipStream_t s);
hipError_t wgemm(const GemmTile& t, int M, int N, int K, const void* X, long ldx,
                 long x_group_stride, int n_group, const void* W, void* Y, long ldy,
                 long y_split_stride, bool out_f32, float alpha, hipStream_t s,
                 bool x_blocked = false, bool y_blocked = false, bool w_tiled = false,
                 int y_grp = 0, long y_grp_stride = 0);
// Tiled MFMA GEMM for many rows (k_tgemm.hip): Y = alpha * X . W^T, X [M][K]
// bf16 rows (ldx), W [N][K] bf16 row-major or tiled, Y bf16 or fp32 (ldy;
// y_grp > 0, bf16: column n at (n / y_grp) * y_grp_stride + n % y_grp).
// hipErrorNotSupported (nothing launched) when no tile fits the shape: K a
// multiple of 32, N of 128 or 192 or 320.  splits > 1 (fp32 Y only): equal K
// chunks, chunk z's partial at Y + z * y_split_stride.  tgemm_units: the
// output tiles the shape takes (-1: none).  rope_tab (bf16 Y with y_grp > 0
// only): each y_grp-column group of row m is the RoPE input, and Y receives
// it turned by position rope_pos[m] (pairs (2k, 2k + 1) by the table's
// (cos, sin) entry k of that position, y_grp / 2 entries per position; NaN
// where the position is outside [0, rope_len)).
int tgemm_pick(int M, int N, int K);
int tgemm_units(int M, int N, int K);
hipError_t tgemm(int M, int N, int K, const void* X, long ldx, const void* W, bool w_tiled,
                 void* Y, long ldy, bool out_f32, float alpha, hipStream_t s, int y_grp = 0,
                 long y_grp_stride = 0, int splits = 1, long y_split_stride = 0,
                 const int32_t* rope_pos = nullptr, const float* rope_tab = nullptr,
                 int rope_len = 0);
hipError_t splitk_reduce(int M, int N, int S, const float* part, long split_stride, void* out,
                         long ldo, hipStream_t s, bool blocked = false);
// q_abs[b][i][0:512] = scale * W_UK,i^T q^C_i and q_abs[b][i][512:576] =
// scale * RoPE(q^R_i) (V2 geometry, bf16; W_UK row-major or tiled); q_tiled:
// written in the query-tile layout (qtile_index, times kQTileLog2e) instead
// of rows.
hipError_t absorb_v2(int M, const void* qc, const void* W_UK, bool w_tiled, void* q_abs,
                     bool q_tiled, float scale, const float* q_r, const int32_t* positions,
                     const float* rope, int rope_len, hipStream_t s);
// Host-side argument checks of mla_decode; *need = its workspace bytes.
int decode_args_status(const mla_config* cfg, const mla_weights* w, const void* h,
                       const int32_t* positions, const void* kv_cache, int num_pages,
                       const int32_t* page_table, int max_pages, const int32_t* kv_lens, int B,
                       int max_kv_len, const float* rope_table, int rope_len, int num_splits,
                       const void* out, size_t* need);

// Merge of the register-order partials attn_decode_v2 writes.
hipError_t combine_decode_v2(const PlanPtrs& plan, int B, int num_splits, const void* part_o,
                             const float* part_ml, void* lat_out, hipStream_t s);

}  // namespace mla
