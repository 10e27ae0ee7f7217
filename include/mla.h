/*
 * mla.h -- C ABI of the MI355X (gfx950) Multi-head Latent Attention library.
 *
 * The layer follows the MLA pages:
 *   [walkthrough] "MLA（多头潜在注意力）" walkthrough (h.sjds.net/a/578141),
 *                 §1 steps 1-5 and §3 (orders A and B);
 *   [formulas]    DeepSeek-V2 MLA formula walk-through (modelers.csdn.net),
 *                 equations (9)-(13) and §三 (absorption);
 *   [wiki]        "MLA 多头潜在注意力" (chenshi221.pages.dev), "与 RoPE 的兼容性".
 *
 * Conventions for every call
 *  - Every pointer argument named d_* or documented as "device" is a device
 *    pointer owned by the caller.  The library never allocates, never frees
 *    and never synchronises: each call enqueues kernels on `stream` (a
 *    hipStream_t; NULL is the null stream) and returns.  Scratch memory is the
 *    caller-provided `workspace` of at least mla_workspace_size() bytes,
 *    256-byte aligned.
 *  - Matrices are row-major unless stated.  Weights are [out][in] with
 *    y = W x.  Head i owns rows [i*d_h, (i+1)*d_h) of W_UQ, W_UK, W_UV, rows
 *    [i*d_r, (i+1)*d_r) of W_QR and columns [i*d_h, (i+1)*d_h) of W_O.
 *    Weights may instead be stored tiled (mla_weights.layout,
 *    mla_pack_weights): same values, an order the decode kernels stream in
 *    contiguous 1 KB pieces.
 *  - Activations, weights and the cache share one storage dtype (cfg->dtype);
 *    all products accumulate in fp32.
 *  - The latent cache is [num_pages][page_size][d_c + d_r]: each token's row
 *    is its latent c^KV followed by its RoPE key k^R, with no head index
 *    ([walkthrough] step 1).  Token t of a sequence lives at page
 *    page_table[t / page_size], slot t % page_size.
 *  - RoPE rotates interleaved pairs (x_2k, x_2k+1) by pos * base^(-2k/d_r),
 *    with cos/sin read from a table filled by mla_rope_table_init.
 *  - Errors: host-side argument checks run before anything is enqueued and
 *    return a negative mla_status; nothing is launched then.  Device-resident
 *    indices (lengths, positions, page ids, slots) are checked inside the
 *    kernels: no kernel reads or writes outside the buffers described by the
 *    size arguments; a decode/prefill output row whose indices are invalid is
 *    filled with NaN, and an append row with an invalid slot or position is
 *    not written.  MLA_ERR_HIP reports a failed launch (hipGetLastError).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,  /* null pointer, bad size or shape */
  MLA_ERR_UNSUPPORTED = -2,  /* valid request this build does not implement */
  MLA_ERR_WORKSPACE = -3,    /* workspace missing, misaligned or too small */
  MLA_ERR_HIP = -4,          /* a HIP launch or runtime call failed */
  MLA_ERR_SCRATCH_LIMIT = -5 /* mla_decode_noalloc: needs more than its fixed buffer */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

typedef enum {
  MLA_OP_APPEND = 0,
  MLA_OP_DECODE = 1,
  MLA_OP_PREFILL = 2,
  MLA_OP_DECODE_QUERY = 3,
  MLA_OP_DECODE_ATTENTION = 4,
  MLA_OP_DECODE_OUTPUT = 5,
  MLA_OP_DECODE_MERGED = 6,
  MLA_OP_MHA_DECODE = 7,
  MLA_OP_ATTENTION_BACKWARD = 8
} mla_op;

/* Layer geometry.  DeepSeek-V2: d=5120, n_h=128, d_h=128, d_c=512,
 * d_cq=1536, d_r=64 ([walkthrough] §1). */
typedef struct mla_config {
  int d;              /* model (hidden) dim */
  int n_h;            /* heads */
  int d_h;            /* per-head content dim of q, k and v */
  int d_c;            /* KV latent dim (cached) */
  int d_cq;           /* query latent dim */
  int d_r;            /* decoupled RoPE dim (cached once per token), even */
  int page_size;      /* tokens per cache page */
  int dtype;          /* an mla_dtype: storage dtype of weights, activations and
                         cache (a plain int, so that any value a caller passes
                         reaches the library's check as a value) */
  float softmax_scale;/* <= 0 selects 1/sqrt(d_h + d_r) */
  double rope_base;   /* <= 0 selects 10000 */
} mla_config;

/* Storage order of the weight matrices.
 * MLA_LAYOUT_ROWS:  row-major [out][in].
 * MLA_LAYOUT_TILES: an [R][C] matrix is cut into 16 x 32 tiles, stored in
 *   row-major tile order, 512 elements each; element (r, c) of tile
 *   (r / 16, c / 32) sits at offset 8 * (16 * ((c / 8) % 4) + r % 16) + c % 8
 *   inside its tile, so eight consecutive columns of a row stay adjacent.
 *   Needs d, d_cq, d_c and n_h*d_h multiples of 32 and d_h, d_r multiples of
 *   16 (MLA_ERR_UNSUPPORTED otherwise).  Every entry point accepts either
 *   order and computes the same results; decode streams tiles faster. */
typedef enum { MLA_LAYOUT_ROWS = 0, MLA_LAYOUT_TILES = 1 } mla_layout;

/* Device pointers to the eight projection matrices, each [out][in]:
 * W_DKV [d_c][d], W_KR [d_r][d], W_DQ [d_cq][d], W_UQ [n_h*d_h][d_cq],
 * W_QR [n_h*d_r][d_cq], W_UK [n_h*d_h][d_c], W_UV [n_h*d_h][d_c],
 * W_O [d][n_h*d_h] ([walkthrough] steps 1-5; [formulas] eq. (9), (12),
 * (13)), all stored in `layout` (an mla_layout).  A call reads only the ones
 * it uses. */
typedef struct mla_weights {
  const void *W_DKV, *W_KR, *W_DQ, *W_UQ, *W_QR, *W_UK, *W_UV, *W_O;
  int layout;
} mla_weights;

/* Text for a status code (static storage). */
const char* mla_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int mla_version(void);

/* Fill the RoPE table d_table [max_pos][d_r/2][2] (cos, sin as fp32) for
 * positions 0..max_pos-1; angles pos * base^(-2k/d_r) are formed in fp64.
 * ([wiki] "与 RoPE 的兼容性": the decoupled RoPE part carries positions.) */
int mla_rope_table_init(const mla_config* cfg, int max_pos, float* d_table, void* stream);

/* Bytes mla_pack_weights writes: the eight matrices back to back, each
 * starting 256-byte aligned.  0 when the geometry is invalid or does not
 * admit MLA_LAYOUT_TILES. */
size_t mla_packed_weights_size(const mla_config* cfg);

/* Copy the row-major weights of `src` (src->layout == MLA_LAYOUT_ROWS) into
 * d_dst in MLA_LAYOUT_TILES, matrix by matrix in the order of mla_weights at
 * the offsets mla_packed_weights_size counts; matrices that are null in src
 * are skipped.  *out receives their device addresses (null where src has
 * null) and layout = MLA_LAYOUT_TILES.  d_dst: device, 256-byte aligned,
 * dst_bytes >= mla_packed_weights_size(cfg), not overlapping src; owned by
 * the caller, who keeps it alive while *out is in use.  Enqueued on
 * `stream`; src must stay unchanged until the copy has run.
 * Errors: MLA_ERR_INVALID_ARG (null cfg, src or out; src not row-major),
 * MLA_ERR_UNSUPPORTED (geometry without a tiled layout), MLA_ERR_WORKSPACE
 * (d_dst null, misaligned or too small). */
int mla_pack_weights(const mla_config* cfg, const mla_weights* src, void* d_dst,
                     size_t dst_bytes, mla_weights* out, void* stream);

/* Bytes of workspace `op` needs.  batch: B for decode ops, T for append and
 * prefill.  max_kv_len: longest kv_len the call may see (decode, prefill).
 * num_splits: as passed to mla_decode / mla_decode_attention (0 = auto).
 * Returns 0 for an invalid request. */
size_t mla_workspace_size(const mla_config* cfg, int op, int batch, int max_kv_len,
                          int num_splits);

/* Write memory ([walkthrough] step 1, [formulas] eq. (9)):
 *   c^KV_t = W_DKV h_t,  k^R_t = RoPE(W_KR h_t, positions[t])
 * and store [c^KV_t | k^R_t], rounded to cfg->dtype, at cache slot
 * slot_mapping[t] (= page * page_size + offset).  A row whose slot is outside
 * [0, num_pages*page_size) or whose position is outside [0, rope_len) is not
 * written.  h: device [T][d].  positions, slot_mapping: device int32 [T].
 * rope_table: device, from mla_rope_table_init with max_pos = rope_len. */
int mla_append_kv(const mla_config* cfg, const mla_weights* w, const void* h,
                  const int32_t* positions, const int32_t* slot_mapping, int T,
                  const float* rope_table, int rope_len, void* kv_cache, int num_pages,
                  void* workspace, size_t ws_bytes, void* stream);

/* Decode, order B ([walkthrough] §3 顺序 B; [formulas] §三): for each sequence
 * b, the query from h[b] at position positions[b] attends to cached tokens
 * 0..kv_lens[b]-1 (the caller appends the query's own row first, so
 * kv_lens[b] = positions[b] + 1 in the usual case) and out[b] receives
 *   u = W_O [W_UV,i o~_i]_i,  o~_i = sum_j softmax_j(Q~_i . row_j) c^KV_j,
 *   Q~_i = [W_UK,i^T q^C_i | q^R_i] * scale.
 * h: device [B][d]; positions, kv_lens: device int32 [B];
 * page_table: device int32 [B][max_pages]; out: device [B][d].
 * max_kv_len bounds every kv_lens[b] (1 <= kv_lens[b] <= max_kv_len <=
 * max_pages*page_size); a sequence outside that gets a NaN output row.
 * num_splits: 0 balances the tokens of all sequences over the GPU's compute
 * units; k > 0 cuts every sequence into k token ranges. */
int mla_decode(const mla_config* cfg, const mla_weights* w, const void* h,
               const int32_t* positions, const void* kv_cache, int num_pages,
               const int32_t* page_table, int max_pages, const int32_t* kv_lens, int B,
               int max_kv_len, const float* rope_table, int rope_len, int num_splits,
               void* workspace, size_t ws_bytes, void* out, void* stream);

/* mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same step, arguments and results, with the workspace taken from a fixed
 * 64 MiB device array that the library holds on each GPU it runs on until
 * the process ends (mla_decode's workspace at batch 64 with automatic
 * splits is 57.3 MiB at the DeepSeek-V2 shape).  It allocates nothing and
 * frees nothing; a request whose workspace (mla_workspace_size with
 * MLA_OP_DECODE) exceeds 64 MiB returns MLA_ERR_SCRATCH_LIMIT before any HIP
 * call.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind (no part of it needs to start at zero): calls that overlap
 * on one GPU - on two streams, or from two host threads - race; serialise
 * them.  The first call on a device looks the array's address up once with
 * that device current. */
int mla_decode_noalloc(const mla_config* cfg, const mla_weights* w, const void* h,
                       const int32_t* positions, const void* kv_cache, int num_pages,
                       const int32_t* page_table, int max_pages, const int32_t* kv_lens, int B,
                       int max_kv_len, const float* rope_table, int rope_len, int num_splits,
                       void* out, void* stream);

/* Decode steps 1-3 of mla_decode ([formulas] eq. (12), (13); [walkthrough]
 * step 3 and §3 顺序 B): q_abs[b][i] = [W_UK,i^T q^C_i | RoPE(q^R_i)] * scale,
 * device [B][n_h][d_c + d_r] in cfg->dtype. */
int mla_decode_query(const mla_config* cfg, const mla_weights* w, const void* h,
                     const int32_t* positions, int B, const float* rope_table, int rope_len,
                     void* workspace, size_t ws_bytes, void* q_abs, void* stream);

/* Decode steps 4-7: latent_out[b][i] = sum_j softmax_j(q_abs[b][i] . row_j) c^KV_j
 * over the cached rows j < kv_lens[b] (split over token ranges and merged by
 * log-sum-exp).  q_abs: device [B][n_h][d_c + d_r]; latent_out: device
 * [B][n_h][d_c], both cfg->dtype. */
int mla_decode_attention(const mla_config* cfg, const void* q_abs, const void* kv_cache,
                         int num_pages, const int32_t* page_table, int max_pages,
                         const int32_t* kv_lens, int B, int max_kv_len, int num_splits,
                         void* workspace, size_t ws_bytes, void* latent_out, void* stream);

/* Decode steps 8-9 ([walkthrough] step 5 and §3 顺序 B): o_i = W_UV,i o~_i,
 * out[b] = W_O [o_0 | ... | o_{n_h-1}].  latent_out: device [B][n_h][d_c];
 * out: device [B][d]. */
int mla_decode_output(const mla_config* cfg, const mla_weights* w, const void* latent_out,
                      int B, void* workspace, size_t ws_bytes, void* out, void* stream);

/* Prefill, order A ([walkthrough] §3 顺序 A and step 4): per head the cached
 * rows are decompressed into k_j = [W_UK,i c^KV_j | k^R_j] and
 * v_j = W_UV,i c^KV_j; query t (from h[t] at positions[t]) attends causally to
 * rows 0..positions[t] of the one sequence described by page_table (device
 * int32 [max_pages]) and kv_len; out: device [T][d].  Query rows with
 * positions outside [0, kv_len) get NaN outputs.  At the DeepSeek-V2 bf16
 * shape every product and the attention run on bf16 MFMA with fp32
 * accumulation and bf16 intermediates (c^Q, q, k, v, o); other shapes use
 * fp32 intermediates. */
int mla_prefill(const mla_config* cfg, const mla_weights* w, const void* h,
                const int32_t* positions, const void* kv_cache, int num_pages,
                const int32_t* page_table, int max_pages, int kv_len, int T,
                const float* rope_table, int rope_len, void* workspace, size_t ws_bytes,
                void* out, void* stream);

/* Offline-merged absorption matrices ([walkthrough] §3 顺序 B: the product
 * of the two matrices is computed once at deployment and decoding runs order
 * B on it; [formulas] §三: W^UK is absorbed into the query projection, W^UV
 * into W^O):
 *   W_UQK [n_h*d_c][d_cq]: rows [i*d_c, (i+1)*d_c) hold W_UK,i^T W_UQ,i, so
 *     that q~_i = W_UQK,i c^Q;
 *   W_OUV [d][n_h*d_c]: columns [i*d_c, (i+1)*d_c) hold W_O,i W_UV,i, W_O,i
 *     being columns [i*d_h, (i+1)*d_h) of W_O, so that u = sum_i W_OUV,i o~_i.
 * With W_DQ and W_QR as in mla_weights; all four stored in `layout`. */
typedef struct mla_merged_weights {
  const void *W_DQ, *W_QR, *W_UQK, *W_OUV;
  int layout;
} mla_merged_weights;

/* Compute W_UQK and W_OUV (sums over d_h in fp32, rounded to cfg->dtype) from
 * the row-major W_UQ, W_UK, W_UV and W_O of src (src->layout must be
 * MLA_LAYOUT_ROWS) and store them in `layout` at d_W_UQK
 * (n_h*d_c*d_cq elements) and d_W_OUV (d*n_h*d_c elements): device buffers
 * owned by the caller, overlapping nothing else.  A one-time deployment step
 * (plain SIMT kernels).  Errors: MLA_ERR_INVALID_ARG (null argument, a
 * needed matrix missing, src not row-major, unknown layout),
 * MLA_ERR_UNSUPPORTED (MLA_LAYOUT_TILES on a geometry without tiles). */
int mla_merge_weights(const mla_config* cfg, const mla_weights* src, int layout, void* d_W_UQK,
                      void* d_W_OUV, void* stream);

/* mla_decode from the merged matrices: Q~_i = [W_UQK,i c^Q | RoPE(W_QR,i
 * c^Q)] * scale, the same attention, then u = W_OUV o~.  Arguments, layouts
 * and error behaviour as mla_decode; workspace mla_workspace_size(cfg,
 * MLA_OP_DECODE_MERGED, B, max_kv_len, num_splits). */
int mla_decode_merged(const mla_config* cfg, const mla_merged_weights* w, const void* h,
                      const int32_t* positions, const void* kv_cache, int num_pages,
                      const int32_t* page_table, int max_pages, const int32_t* kv_lens, int B,
                      int max_kv_len, const float* rope_table, int rope_len, int num_splits,
                      void* workspace, size_t ws_bytes, void* out, void* stream);

/* Baseline, not MLA: decode attention over an MHA-equivalent cache, the
 * multi-head cache the pages weigh MLA against ([formulas] §一 and §三;
 * [walkthrough] §2).  Every cached token holds a key and a value for each
 * head (2*n_h*d_h numbers against MLA's d_c + d_r), and head i attends with
 * its own keys: out[b][i] = sum_j softmax_j(scale * q[b][i] . k_ij) v_ij over
 * j < kv_lens[b].  Uses cfg's n_h, d_h, page_size and dtype.
 * q: device [B][n_h][d_h]; out: device [B][n_h][d_h]; kv_cache: device
 * [num_pages][page_size][2][n_h][d_h] (the keys of all heads, then the
 * values), 16-byte aligned; page_table, kv_lens, max_kv_len, num_splits and
 * the NaN rule for invalid entries as mla_decode_attention.  scale <= 0
 * selects 1/sqrt(d_h).  d_h must be a multiple of 16 with d_h/16 a power of
 * two <= 64 (MLA_ERR_UNSUPPORTED otherwise).  Workspace:
 * mla_workspace_size(cfg, MLA_OP_MHA_DECODE, B, max_kv_len, num_splits). */
int mla_mha_decode_attention(const mla_config* cfg, const void* q, const void* kv_cache,
                             int num_pages, const int32_t* page_table, int max_pages,
                             const int32_t* kv_lens, int B, int max_kv_len, float scale,
                             int num_splits, void* workspace, size_t ws_bytes, void* out,
                             void* stream);

/* Order-A attention backward ([walkthrough] §3 顺序 A: training keeps W_UK
 * and W_UV as two matrices, each with its own gradient).  Forward, as in
 * mla_prefill: query t at positions[t] attends to the cached rows
 * j <= positions[t] (j < kv_len) of one sequence, per head i
 *   k_ij = [W_UK,i c_j | k^R_j], v_ij = W_UV,i c_j,
 *   p_tij = softmax_j(scale q_ti . k_ij), o_ti = sum_j p_tij v_ij.
 * Given dO = dL/do, writes dL/dW_UK and dL/dW_UV ([n_h*d_h][d_c] each, so
 * the two up-projections get separate gradients), dL/dq ([T][n_h][d_h+d_r]:
 * q^C then q^R per head) and dL/dC ([kv_len][d_c+d_r]: latent then RoPE key
 * per cached row).  q: device fp32 [T][n_h][d_h+d_r] (RoPE applied, not
 * scaled; scale = cfg->softmax_scale or 1/sqrt(d_h+d_r)); dO: device fp32
 * [T][n_h][d_h]; positions: device int32 [T]; cache and page_table as
 * mla_prefill; W_UK, W_UV from w in either layout; outputs device fp32.
 * A query whose position is outside [0, kv_len) makes dW_UK, dW_UV, dC and
 * its own row of dq NaN.
 * Workspace: mla_workspace_size(cfg, MLA_OP_ATTENTION_BACKWARD, T, kv_len, 0).
 * At the DeepSeek-V2 head shape with a bf16 cache and weights (n_h 128, d_h
 * 128, d_r 64, d_c 512): q (times scale) and dO are rounded to bf16 on
 * entry, k and v per head are formed in bf16 as mla_prefill forms them, the
 * attention's gradients run flash style on bf16 MFMA (the probabilities are
 * recomputed per block of 32 queries x 32 keys and never stored; fp32 sums),
 * and dW_UK, dW_UV and dC come from bf16 MFMA GEMMs over dk^C and dv rounded
 * to bf16; the workspace grows with (T + kv_len) and holds both
 * up-projections transposed (32 MB).  Other shapes: generic fp32 kernels,
 * with [n_h][T][kv_len] probabilities held twice in the workspace (a
 * training-step check, not a long-context kernel). */
int mla_attention_backward(const mla_config* cfg, const mla_weights* w, const float* q,
                           const int32_t* positions, const void* kv_cache, int num_pages,
                           const int32_t* page_table, int max_pages, int kv_len, int T,
                           const float* dO, void* workspace, size_t ws_bytes, float* dW_UK,
                           float* dW_UV, float* dq, float* dC, void* stream);

/* Kernel timing for measurement tools (not needed for computing).  While
 * enabled, every mla_decode / mla_decode_attention call records three HIP
 * events on its stream: before its cache-streaming attention kernel, after
 * it, and after the merge of the split partials.  mla_profile_read waits for
 * the recorded events and returns, summed over the recorded launches (at
 * most 4096 between two reads; later ones are not recorded), the attention
 * kernel's milliseconds, the milliseconds of attention plus merge, and the
 * number of launches; then it clears the record.  mla_profile_attention_ms
 * is the same read returning only the attention kernel's time.
 * Host-thread-unsafe; enable from one thread.  Returns MLA_ERR_HIP if an
 * event call fails, MLA_ERR_INVALID_ARG for a null pointer. */
int mla_profile_enable(int enable);
int mla_profile_read(double* attention_ms, double* attention_merge_ms, int* launches);
int mla_profile_attention_ms(double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
