// Host side of the C ABI declared in include/mla.h: argument checks,
// workspace carving and the stream-ordered launch sequence of each call.
//
// Layer steps and where the pages define them:
//   write memory    c^KV = W_DKV h, k^R = RoPE(W_KR h)   eq. (9) of the formula
//                   page; walkthrough §1 step 1
//   query side      c^Q = W_DQ h, q^C = W_UQ c^Q,        eq. (12), (13); step 3
//                   q^R = RoPE(W_QR c^Q)
//   absorption      q~_i = W_UK,i^T q^C_i (order B)      walkthrough §3 顺序 B
//   attention       softmax over [c^KV | k^R] rows       step 4, §3
//   integrate       o_i = W_UV,i o~_i, u = W_O [o_i]     step 5, §3
#include <math.h>
#include <string.h>

#include "mla_internal.h"

using namespace mla;

namespace {

constexpr size_t kAlign = 256;
inline size_t al(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Bump allocator over the caller's workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += al(bytes);
    return p;
  }
};

bool resolve(const mla_config* cfg, Geo* g) {
  if (!cfg) return false;
  if (cfg->d <= 0 || cfg->n_h <= 0 || cfg->d_h <= 0 || cfg->d_c <= 0 || cfg->d_cq <= 0 ||
      cfg->d_r <= 0 || (cfg->d_r & 1) || cfg->page_size <= 0)
    return false;
  if (cfg->dtype != MLA_F32 && cfg->dtype != MLA_BF16) return false;
  g->d = cfg->d;
  g->n_h = cfg->n_h;
  g->d_h = cfg->d_h;
  g->d_c = cfg->d_c;
  g->d_cq = cfg->d_cq;
  g->d_r = cfg->d_r;
  g->page = cfg->page_size;
  g->row = cfg->d_c + cfg->d_r;
  g->scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale
                                      : (float)(1.0 / sqrt((double)(cfg->d_h + cfg->d_r)));
  g->base = cfg->rope_base > 0.0 ? cfg->rope_base : 10000.0;
  g->bf16 = cfg->dtype == MLA_BF16;
  return true;
}

// The generic kernels hold per-thread accumulators for d_c <= 1024 and d_h <= 512.
bool generic_ok(const Geo& g) { return g.d_c <= 1024 && g.d_h <= 512; }

GType st(const Geo& g) { return g.bf16 ? G_BF16 : G_F32; }

int hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

#define MLA_TRY(expr)                         \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return MLA_ERR_HIP; \
  } while (0)

// ---------------------------------------------------------------------------
// workspace layouts
// ---------------------------------------------------------------------------
// tiles of the MFMA decode GEMMs (the same choice sizes the workspace and runs)
// rows of the blocked activation buffers (multiples of 64)
size_t pad64(int B) { return ((size_t)B + 63) / 64 * 64; }
GemmTile tile_dq(const Geo& g) { return wgemm_tile(g.d_cq, g.d, 0, true); }
GemmTile tile_uq(const Geo& g) { return wgemm_tile(g.n_h * g.d_h, g.d_cq, 0, false); }
GemmTile tile_qr(const Geo& g) { return wgemm_tile(g.n_h * g.d_r, g.d_cq, 0, false); }
GemmTile tile_uv(const Geo& g) { return wgemm_tile(g.n_h * g.d_h, g.d_c, g.d_h, false); }
GemmTile tile_o(const Geo& g) { return wgemm_tile(g.d, g.n_h * g.d_h, 0, true); }
GemmTile tile_uqk(const Geo& g) { return wgemm_tile(g.n_h * g.d_c, g.d_cq, 0, false); }
GemmTile tile_ouv(const Geo& g) { return wgemm_tile(g.d, g.n_h * g.d_c, 0, true); }

struct QueryWs {
  float *cq, *qc, *qr;   // generic: fp32 intermediates
  float* cq_part;        // MFMA path: split-K partials of c^Q
  void *cq16, *qc16;     // MFMA path: bf16 c^Q and q^C
};
void carve_query(Carver& c, const Geo& g, int B, QueryWs* w) {
  if (is_v2_fast(g)) {
    w->cq_part = (float*)c.take(sizeof(float) * (size_t)tile_dq(g).splits * B * g.d_cq);
    w->cq16 = c.take(2 * (size_t)pad64(B) * g.d_cq);   // blocked activation layout
    w->qc16 = c.take(2 * (size_t)B * g.n_h * g.d_h);
    w->qr = (float*)c.take(sizeof(float) * (size_t)B * g.n_h * g.d_r);
    w->cq = w->qc = nullptr;
    return;
  }
  w->cq = (float*)c.take(sizeof(float) * (size_t)B * g.d_cq);
  w->qc = (float*)c.take(sizeof(float) * (size_t)B * g.n_h * g.d_h);
  w->qr = (float*)c.take(sizeof(float) * (size_t)B * g.n_h * g.d_r);
  w->cq_part = nullptr;
  w->cq16 = w->qc16 = nullptr;
}

struct AttnWs {
  void* plan;
  float *part_o, *part_ml;
  void* q_tiles;   // MFMA path, query given in rows: its query-tile copy
  int max_segs, max_wg;
};
void carve_attn(Carver& c, const Geo& g, int B, int num_splits, AttnWs* w, bool q_rows = true) {
  PlanDims pd = plan_dims(B, num_splits);
  w->max_segs = pd.max_segs;
  w->max_wg = pd.max_wg;
  w->plan = c.take(plan_bytes(B, num_splits));
  w->q_tiles = (q_rows && is_v2_fast(g)) ? c.take((size_t)B * g.n_h * g.row * g.esize()) : nullptr;
  // partial o~ per segment: bf16 on the MFMA path, fp32 on the generic one
  const size_t part_elem = is_v2_fast(g) ? 2 : sizeof(float);
  w->part_o = (float*)c.take(part_elem * (size_t)pd.max_segs * g.n_h * g.d_c);
  w->part_ml = (float*)c.take(sizeof(float) * 2 * (size_t)pd.max_segs * g.n_h);
}

struct OutWs {
  float* o;        // generic: fp32 o
  void* o16;       // MFMA path: bf16 o
  float* u_part;   // MFMA path: split-K partials of u
};
void carve_out(Carver& c, const Geo& g, int B, OutWs* w) {
  if (is_v2_fast(g)) {
    w->o16 = c.take(2 * (size_t)pad64(B) * g.n_h * g.d_h);   // blocked activation layout
    w->u_part = (float*)c.take(sizeof(float) * (size_t)tile_o(g).splits * B * g.d);
    w->o = nullptr;
    return;
  }
  w->o = (float*)c.take(sizeof(float) * (size_t)B * g.n_h * g.d_h);
  w->o16 = nullptr;
  w->u_part = nullptr;
}

struct DecodeWs {
  void *q_abs, *lat;
  size_t sub_off;
};

struct PrefillWs {
  float *cq, *q, *rows, *kbuf, *vbuf, *o;
};
void carve_prefill(Carver& c, const Geo& g, int T, int kv_len, PrefillWs* w) {
  size_t wq = (size_t)g.n_h * (g.d_h + g.d_r);
  w->cq = (float*)c.take(sizeof(float) * (size_t)T * g.d_cq);
  w->q = (float*)c.take(sizeof(float) * (size_t)T * wq);
  w->rows = (float*)c.take(sizeof(float) * (size_t)kv_len * g.row);
  w->kbuf = (float*)c.take(sizeof(float) * (size_t)kv_len * wq);
  w->vbuf = (float*)c.take(sizeof(float) * (size_t)kv_len * g.n_h * g.d_h);
  w->o = (float*)c.take(sizeof(float) * (size_t)T * g.n_h * g.d_h);
}

size_t ws_query(const Geo& g, int B) {
  Carver c(nullptr);
  QueryWs w;
  carve_query(c, g, B, &w);
  return c.used;
}
size_t ws_attn(const Geo& g, int B, int ns, bool q_rows = true) {
  Carver c(nullptr);
  AttnWs w;
  carve_attn(c, g, B, ns, &w, q_rows);
  return c.used;
}
size_t ws_out(const Geo& g, int B) {
  Carver c(nullptr);
  OutWs w;
  carve_out(c, g, B, &w);
  return c.used;
}
size_t ws_decode_head(const Geo& g, int B) {
  return al((size_t)B * g.n_h * g.row * g.esize()) + al((size_t)B * g.n_h * g.d_c * g.esize());
}
size_t ws_decode(const Geo& g, int B, int ns) {
  size_t sub = ws_query(g, B);
  size_t a = ws_attn(g, B, ns, false), o = ws_out(g, B);
  if (a > sub) sub = a;
  if (o > sub) sub = o;
  // the plan has a region of its own: it is built during the query
  return ws_decode_head(g, B) + al(plan_bytes(B, ns)) + sub;
}
// merged decode: the output GEMM's split-K partials (MFMA path)
size_t ws_out_merged(const Geo& g, int B) {
  return is_v2_fast(g) ? al(sizeof(float) * (size_t)tile_ouv(g).splits * B * g.d) : 0;
}
size_t ws_decode_merged(const Geo& g, int B, int ns) {
  size_t sub = ws_query(g, B);
  size_t a = ws_attn(g, B, ns), o = ws_out_merged(g, B);
  if (a > sub) sub = a;
  if (o > sub) sub = o;
  return ws_decode_head(g, B) + al(plan_bytes(B, ns)) + sub;
}
// MHA baseline: the plan, fp32 partials and their (m, l)
size_t ws_mha(const Geo& g, int B, int ns) {
  const PlanDims pd = plan_dims(B, ns);
  return al(plan_bytes(B, ns)) + al(sizeof(float) * (size_t)pd.max_segs * g.n_h * g.d_h) +
         al(sizeof(float) * 2 * (size_t)pd.max_segs * g.n_h);
}
// order-A backward: rows, K, V, P, dS, dV, dK, per-head dk^R, two dc parts
struct BwdWs {
  float *rows, *K, *V, *P, *dS, *dV, *dK, *dkr, *lat_k, *lat_v;
};
void carve_bwd(Carver& c, const Geo& g, int T, int N, BwdWs* w) {
  const size_t hd = (size_t)g.n_h * g.d_h;
  w->rows = (float*)c.take(sizeof(float) * (size_t)N * g.row);
  w->K = (float*)c.take(sizeof(float) * (size_t)N * hd);
  w->V = (float*)c.take(sizeof(float) * (size_t)N * hd);
  w->P = (float*)c.take(sizeof(float) * (size_t)g.n_h * T * N);
  w->dS = (float*)c.take(sizeof(float) * (size_t)g.n_h * T * N);
  w->dV = (float*)c.take(sizeof(float) * (size_t)N * hd);
  w->dK = (float*)c.take(sizeof(float) * (size_t)N * hd);
  w->dkr = (float*)c.take(sizeof(float) * (size_t)g.n_h * N * g.d_r);
  w->lat_k = (float*)c.take(sizeof(float) * (size_t)N * g.d_c);
  w->lat_v = (float*)c.take(sizeof(float) * (size_t)N * g.d_c);
}
// the same at the DeepSeek-V2 head shape (bf16 MFMA, no T x N arrays): the
// gathered rows, k and v per head, the bf16 query and dO, LSE and D, the
// query blocks' furthest keys, dk^C and dv as rows and key-contiguous, the
// latent rows and both up-projections transposed, dk^R per head, and the
// two K halves of the latent gradient
struct BwdWsV2 {
  void *rows16, *k16, *v16, *q16, *do16, *rec, *dkv16, *dkT16, *dvT16, *cT16, *wT16;
  float *dkr, *lat;
  int* qblk_far;
};
void carve_bwd_v2(Carver& c, const Geo& g, int T, int N, BwdWsV2* w) {
  const size_t hd = (size_t)g.n_h * g.d_h, wq = (size_t)g.n_h * (g.d_h + g.d_r);
  const size_t Np = (size_t)attn_bwd_v2_npad(N);
  w->rows16 = c.take(2 * (size_t)N * g.row);
  w->k16 = c.take(2 * (size_t)N * wq);
  w->v16 = c.take(2 * (size_t)N * hd);
  w->q16 = c.take(2 * (size_t)T * wq);
  w->do16 = c.take(2 * (size_t)T * hd);
  w->rec = c.take(16 * (size_t)g.n_h * T);
  w->qblk_far = (int*)c.take(2 * sizeof(int) * (size_t)((T + 31) / 32));
  w->dkv16 = c.take(2 * (size_t)N * 2 * hd);
  w->dkT16 = c.take(2 * hd * Np);
  w->dvT16 = c.take(2 * hd * Np);
  w->cT16 = c.take(2 * (size_t)g.d_c * Np);
  w->wT16 = c.take(2 * (size_t)g.d_c * 2 * hd);
  w->dkr = (float*)c.take(sizeof(float) * (size_t)g.n_h * N * g.d_r);
  w->lat = (float*)c.take(sizeof(float) * (size_t)bwd_lat_splits(N) * N * g.d_c);
}
bool use_bwd_v2(const Geo& g, int T, int N) {
  return attn_bwd_v2_supported(g) && T <= attn_bwd_v2_max_queries() &&
         N <= attn_bwd_v2_max_keys();
}
size_t ws_bwd(const Geo& g, int T, int N) {
  Carver c(nullptr);
  if (use_bwd_v2(g, T, N)) {
    BwdWsV2 w;
    carve_bwd_v2(c, g, T, N, &w);
    return c.used;
  }
  BwdWs w;
  carve_bwd(c, g, T, N, &w);
  return c.used;
}
size_t ws_append(const Geo& g, int T) { return al(sizeof(float) * (size_t)T * g.row); }
size_t ws_prefill(const Geo& g, int T, int kv_len) {
  Carver c(nullptr);
  PrefillWs w;
  carve_prefill(c, g, T, kv_len, &w);
  return c.used;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MLA_OK;
  if (!ws || ((uintptr_t)ws & (kAlign - 1)) || have < need) return MLA_ERR_WORKSPACE;
  return MLA_OK;
}

// ---------------------------------------------------------------------------
// step implementations (arguments already checked)
// ---------------------------------------------------------------------------
// job: a split plan to build during the query (in the launch of the W_DQ
// reduction on the fast path, which leaves it idle compute units)
// c^Q = W_DQ h (eq. (12)): on the MFMA path split over d and reduced to
// bf16 in the blocked layout (q.cq16), the plan of `job` built beside the GEMM
// where its tile allows, else with the reduction; on the generic path fp32
// (q.cq), the plan in a launch of its own.
int run_cq(const Geo& g, const void* W_DQ, bool wt, const void* h, int B, const QueryWs& q,
           hipStream_t s, const PlanJob* job) {
  if (is_v2_fast(g)) {
    const GemmTile tdq = tile_dq(g);
    hipError_t pe = hipErrorNotSupported;
    if (job)
      pe = wgemm_with_plan(tdq, B, g.d_cq, g.d, h, g.d, W_DQ, q.cq_part, g.d_cq,
                           (long)B * g.d_cq, wt, *job, s);
    if (pe == hipErrorNotSupported) {
      MLA_TRY(wgemm(tdq, B, g.d_cq, g.d, h, g.d, 0, 0, W_DQ, q.cq_part, g.d_cq,
                    (long)B * g.d_cq, true, 1.f, s, false, false, wt));
    } else {
      MLA_TRY(pe);
    }
    if (job && pe == hipErrorNotSupported)
      MLA_TRY(splitk_reduce_with_plan(B, g.d_cq, tdq.splits, q.cq_part, (long)B * g.d_cq, q.cq16,
                                      g.d_cq, true, *job, s));
    else
      MLA_TRY(splitk_reduce(B, g.d_cq, tdq.splits, q.cq_part, (long)B * g.d_cq, q.cq16, g.d_cq, s,
                            true));
    return MLA_OK;
  }
  if (job) {
    const PlanJob& j = *job;
    MLA_TRY(launch_plan(j.p, j.kv_lens, j.B, j.max_kv_len, j.max_pages, j.page, j.tile,
                        j.num_splits, s));
  }
  MLA_TRY(gemm_generic(st(g), st(g), G_F32, b_layout(wt, false), B, g.d_cq, g.d, h, g.d, 0, W_DQ,
                       g.d, 0, q.cq, g.d_cq, 0, 1, 1.f, s));
  return MLA_OK;
}

int run_query(const Geo& g, const mla_weights* w, const void* h, const int32_t* positions, int B,
              const float* rope, int rope_len, void* ws, void* q_abs, hipStream_t s,
              const PlanJob* job = nullptr, bool q_tiled = false) {
  Carver c(ws);
  QueryWs q;
  carve_query(c, g, B, &q);
  const bool wt = w->layout == MLA_LAYOUT_TILES;
  if (int r = run_cq(g, w->W_DQ, wt, h, B, q, s, job)) return r;
  if (is_v2_fast(g)) {
    const long nq = (long)g.n_h * g.d_h, nr = (long)g.n_h * g.d_r;
    // q^C = W_UQ c^Q (eq. (13)) in bf16; the RoPE query input W_QR c^Q in fp32
    // (one launch for both where the shape fits its tiling)
    hipError_t pe = wgemm_pair(B, g.d_cq, q.cq16, true, w->W_UQ, (int)nq, q.qc16, nq, w->W_QR, (int)nr, q.qr,
                    nr, wt, s);
    if (pe == hipErrorNotSupported) {
      MLA_TRY(wgemm(tile_uq(g), B, (int)nq, g.d_cq, q.cq16, g.d_cq, 0, 0, w->W_UQ, q.qc16, nq, 0,
                    false, 1.f, s, true, false, wt));
      MLA_TRY(wgemm(tile_qr(g), B, (int)nr, g.d_cq, q.cq16, g.d_cq, 0, 0, w->W_QR, q.qr, nr, 0,
                    true, 1.f, s, true, false, wt));
    } else {
      MLA_TRY(pe);
    }
    // absorbed query q~_i = W_UK,i^T q^C_i and RoPE(q^R_i), scaled and packed
    // (order B)
    MLA_TRY(absorb_v2(B, q.qc16, w->W_UK, wt, q_abs, q_tiled, g.scale, q.qr, positions, rope,
                      rope_len, s));
    return MLA_OK;
  }
  const GType T = st(g);
  // q^C = W_UQ c^Q (eq. (13)) and the per-head RoPE query input W_QR c^Q
  MLA_TRY(gemm_generic(G_F32, T, G_F32, b_layout(wt, false), B, g.n_h * g.d_h, g.d_cq, q.cq, g.d_cq,
                       0, w->W_UQ, g.d_cq, 0, q.qc, (long)g.n_h * g.d_h, 0, 1, 1.f, s));
  MLA_TRY(gemm_generic(G_F32, T, G_F32, b_layout(wt, false), B, g.n_h * g.d_r, g.d_cq, q.cq, g.d_cq,
                       0, w->W_QR, g.d_cq, 0, q.qr, (long)g.n_h * g.d_r, 0, 1, 1.f, s));
  // absorbed query q~_i = W_UK,i^T q^C_i, scaled (order B)
  MLA_TRY(gemm_generic(G_F32, T, T, b_layout(wt, true), B, g.d_c, g.d_h, q.qc, (long)g.n_h * g.d_h,
                       g.d_h, w->W_UK, g.d_c, (long)g.d_h * g.d_c, q_abs,
                       (long)g.n_h * g.row, g.row, g.n_h, g.scale, s));
  // RoPE(q^R_i), scaled, packed after q~_i
  MLA_TRY(pack_query_rope(g, q.qr, positions, B, rope, rope_len, q_abs, s));
  return MLA_OK;
}

// ---------------------------------------------------------------------------
// optional events around the attention kernel and its merge (measurement
// only): event 3i before the attention kernel of launch i, 3i + 1 after it,
// 3i + 2 after the merge
// ---------------------------------------------------------------------------
struct Profiler {
  static constexpr int kMax = 4096;   // launches recorded between two reads
  bool on = false;
  int used = 0;
  hipEvent_t ev[3 * kMax];
  int created = 0;
  hipError_t mark(int which, hipStream_t s) {
    if (!on) return hipSuccess;
    const int idx = 3 * used + which;
    if (idx >= 3 * kMax) return hipSuccess;
    if (idx >= created) {
      hipError_t e = hipEventCreate(&ev[idx]);
      if (e != hipSuccess) return e;
      created = idx + 1;
    }
    hipError_t e = hipEventRecord(ev[idx], s);
    if (which == 2 && e == hipSuccess) ++used;
    return e;
  }
};
Profiler g_prof;

// pre: a plan already built, ordered before s, by the caller
int run_attention(const Geo& g, const void* q_abs, const void* cache, int num_pages,
                  const int32_t* page_table, int max_pages, const int32_t* kv_lens, int B,
                  int max_kv_len, int num_splits, void* ws, void* lat, hipStream_t s,
                  const PlanPtrs* pre = nullptr, bool q_tiled = false) {
  Carver c(ws);
  AttnWs a;
  carve_attn(c, g, B, num_splits, &a, !q_tiled);
  PlanPtrs plan;
  const bool fast = is_v2_fast(g);
  if (pre) {
    plan = *pre;
  } else {
    carve_plan(a.plan, B, num_splits, &plan);
    MLA_TRY(launch_plan(plan, kv_lens, B, max_kv_len, max_pages, g.page, 64, num_splits, s));
  }
  if (fast) {
    // the MFMA kernel writes every segment as a partial; its merge follows
    // the MFMA kernel loads the query in the query-tile layout
    const void* qt = q_abs;
    if (!q_tiled) {
      MLA_TRY(pack_query_tiles(q_abs, B, a.q_tiles, s));
      qt = a.q_tiles;
    }
    MLA_TRY(g_prof.mark(0, s));
    MLA_TRY(attn_decode_v2(g, qt, q_tiled, cache, num_pages, page_table, max_pages, plan,
                           a.max_wg, a.part_o, a.part_ml, s));
    MLA_TRY(g_prof.mark(1, s));
    MLA_TRY(combine_decode_v2(plan, B, num_splits, a.part_o, a.part_ml, lat, s));
  } else {
    MLA_TRY(g_prof.mark(0, s));
    MLA_TRY(attn_decode_generic(g, q_abs, cache, num_pages, page_table, max_pages, plan,
                                a.max_segs, a.part_o, a.part_ml, lat, s));
    MLA_TRY(g_prof.mark(1, s));
    MLA_TRY(combine_partials(g, plan, B, a.part_o, a.part_ml, lat, s));
  }
  MLA_TRY(g_prof.mark(2, s));
  return MLA_OK;
}

int run_output(const Geo& g, const mla_weights* w, const void* lat, int B, void* ws, void* out,
               hipStream_t s) {
  Carver c(ws);
  OutWs o;
  carve_out(c, g, B, &o);
  const bool wt = w->layout == MLA_LAYOUT_TILES;
  if (is_v2_fast(g)) {
    const long nq = (long)g.n_h * g.d_h;
    const GemmTile to = tile_o(g);
    // o_i = W_UV,i o~_i: weight rows of head i read the latent row of head i
    MLA_TRY(wgemm(tile_uv(g), B, (int)nq, g.d_c, lat, (long)g.n_h * g.d_c, g.d_c, g.d_h, w->W_UV,
                  o.o16, nq, 0, false, 1.f, s, false, true, wt));
    // u = W_O [o_0 | ... | o_{n_h-1}], split over n_h*d_h, reduced to bf16
    MLA_TRY(wgemm(to, B, g.d, (int)nq, o.o16, nq, 0, 0, w->W_O, o.u_part, g.d, (long)B * g.d, true,
                  1.f, s, true, false, wt));
    MLA_TRY(splitk_reduce(B, g.d, to.splits, o.u_part, (long)B * g.d, out, g.d, s));
    return MLA_OK;
  }
  const GType T = st(g);
  // o_i = W_UV,i o~_i
  MLA_TRY(gemm_generic(T, T, G_F32, b_layout(wt, false), B, g.d_h, g.d_c, lat, (long)g.n_h * g.d_c,
                       g.d_c, w->W_UV, g.d_c, (long)g.d_h * g.d_c, o.o,
                       (long)g.n_h * g.d_h, g.d_h, g.n_h, 1.f, s));
  // u = W_O [o_0 | ... | o_{n_h-1}]
  MLA_TRY(gemm_generic(G_F32, T, T, b_layout(wt, false), B, g.d, g.n_h * g.d_h, o.o,
                       (long)g.n_h * g.d_h, 0, w->W_O, (long)g.n_h * g.d_h, 0, out, g.d, 0, 1,
                       1.f, s));
  return MLA_OK;
}

// Query side from the merged matrix: Q~_i = [W_UQK,i c^Q | RoPE(W_QR,i c^Q)]
// * scale ([walkthrough] §3 顺序 B with the product computed offline).
int run_query_merged(const Geo& g, const mla_merged_weights* w, const void* h,
                     const int32_t* positions, int B, const float* rope, int rope_len, void* ws,
                     void* q_abs, hipStream_t s, const PlanJob* job) {
  Carver c(ws);
  QueryWs q;
  carve_query(c, g, B, &q);
  const bool wt = w->layout == MLA_LAYOUT_TILES;
  if (int r = run_cq(g, w->W_DQ, wt, h, B, q, s, job)) return r;
  const long nk = (long)g.n_h * g.d_c, nr = (long)g.n_h * g.d_r;
  if (is_v2_fast(g)) {
    // q~ for all heads, scaled, straight into the latent part of each
    // head's row of q_abs
    MLA_TRY(wgemm(tile_uqk(g), B, (int)nk, g.d_cq, q.cq16, g.d_cq, 0, 0, w->W_UQK, q_abs,
                  (long)g.n_h * g.row, 0, false, g.scale, s, true, false, wt, g.d_c, g.row));
    MLA_TRY(wgemm(tile_qr(g), B, (int)nr, g.d_cq, q.cq16, g.d_cq, 0, 0, w->W_QR, q.qr, nr, 0,
                  true, 1.f, s, true, false, wt));
  } else {
    const GType T = st(g);
    MLA_TRY(gemm_generic(G_F32, T, T, b_layout(wt, false), B, g.d_c, g.d_cq, q.cq, g.d_cq, 0,
                         w->W_UQK, g.d_cq, (long)g.d_c * g.d_cq, q_abs, (long)g.n_h * g.row,
                         g.row, g.n_h, g.scale, s));
    MLA_TRY(gemm_generic(G_F32, T, G_F32, b_layout(wt, false), B, (int)nr, g.d_cq, q.cq, g.d_cq,
                         0, w->W_QR, g.d_cq, 0, q.qr, nr, 0, 1, 1.f, s));
  }
  MLA_TRY(pack_query_rope(g, q.qr, positions, B, rope, rope_len, q_abs, s));
  return MLA_OK;
}

// u = W_OUV [o~_0; ...; o~_{n_h-1}] ([formulas] §三: W^UV absorbed into W^O).
int run_output_merged(const Geo& g, const mla_merged_weights* w, const void* lat, int B, void* ws,
                      void* out, hipStream_t s) {
  const bool wt = w->layout == MLA_LAYOUT_TILES;
  const long nk = (long)g.n_h * g.d_c;
  if (is_v2_fast(g)) {
    const GemmTile t = tile_ouv(g);
    float* part = (float*)ws;
    MLA_TRY(wgemm(t, B, g.d, (int)nk, lat, nk, 0, 0, w->W_OUV, part, g.d, (long)B * g.d, true,
                  1.f, s, false, false, wt));
    MLA_TRY(splitk_reduce(B, g.d, t.splits, part, (long)B * g.d, out, g.d, s));
    return MLA_OK;
  }
  const GType T = st(g);
  MLA_TRY(gemm_generic(T, T, T, b_layout(wt, false), B, g.d, (int)nk, lat, nk, 0, w->W_OUV, nk, 0,
                       out, g.d, 0, 1, 1.f, s));
  return MLA_OK;
}

bool weights_ok(const mla_weights* w, bool query, bool output, bool append, bool kv) {
  if (!w) return false;
  if (w->layout != MLA_LAYOUT_ROWS && w->layout != MLA_LAYOUT_TILES) return false;
  if (query && (!w->W_DQ || !w->W_UQ || !w->W_QR || !w->W_UK)) return false;
  if (output && (!w->W_UV || !w->W_O)) return false;
  if (append && (!w->W_DKV || !w->W_KR)) return false;
  if (kv && (!w->W_UK || !w->W_UV)) return false;
  return true;
}

// weights the geometry cannot read in their layout
int layout_status(const Geo& g, const mla_weights* w) {
  return w->layout == MLA_LAYOUT_TILES && !tiles_ok(g) ? MLA_ERR_UNSUPPORTED : MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MLA_ERR_HIP: return "HIP launch or runtime error";
    case MLA_ERR_SCRATCH_LIMIT:
      return "the step needs more scratch than mla_decode_noalloc's fixed device buffer";
    default: return "unknown status";
  }
}

int mla_version(void) { return 100; }

int mla_profile_enable(int enable) {
  g_prof.on = enable != 0;
  g_prof.used = 0;
  return MLA_OK;
}

int mla_profile_read(double* attention_ms, double* attention_merge_ms, int* launches) {
  if (!attention_ms || !attention_merge_ms || !launches) return MLA_ERR_INVALID_ARG;
  double ta = 0.0, tm = 0.0;
  for (int i = 0; i < g_prof.used; ++i) {
    if (hipEventSynchronize(g_prof.ev[3 * i + 2]) != hipSuccess) return MLA_ERR_HIP;
    float a = 0.f, m = 0.f;
    if (hipEventElapsedTime(&a, g_prof.ev[3 * i], g_prof.ev[3 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&m, g_prof.ev[3 * i], g_prof.ev[3 * i + 2]) != hipSuccess)
      return MLA_ERR_HIP;
    ta += a;
    tm += m;
  }
  *attention_ms = ta;
  *attention_merge_ms = tm;
  *launches = g_prof.used;
  g_prof.used = 0;
  return MLA_OK;
}

int mla_profile_attention_ms(double* total_ms, int* launches) {
  double merge_ms = 0.0;
  return mla_profile_read(total_ms, &merge_ms, launches);
}

int mla_rope_table_init(const mla_config* cfg, int max_pos, float* d_table, void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || max_pos <= 0 || !d_table) return MLA_ERR_INVALID_ARG;
  return hip_status(rope_table_fill(d_table, max_pos, g.d_r, g.base, (hipStream_t)stream));
}

// rows and columns of the eight matrices, in the order of mla_weights
static void weight_shapes(const Geo& g, long rc[8][2]) {
  const long nq = (long)g.n_h * g.d_h, nr = (long)g.n_h * g.d_r;
  const long shapes[8][2] = {{g.d_c, g.d}, {g.d_r, g.d}, {g.d_cq, g.d}, {nq, g.d_cq},
                             {nr, g.d_cq}, {nq, g.d_c}, {nq, g.d_c}, {g.d, nq}};
  for (int i = 0; i < 8; ++i) rc[i][0] = shapes[i][0], rc[i][1] = shapes[i][1];
}

size_t mla_packed_weights_size(const mla_config* cfg) {
  Geo g;
  if (!resolve(cfg, &g) || !tiles_ok(g)) return 0;
  long rc[8][2];
  weight_shapes(g, rc);
  size_t n = 0;
  for (int i = 0; i < 8; ++i) n += al((size_t)rc[i][0] * rc[i][1] * g.esize());
  return n;
}

int mla_pack_weights(const mla_config* cfg, const mla_weights* src, void* d_dst,
                     size_t dst_bytes, mla_weights* out, void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || !src || !out || src->layout != MLA_LAYOUT_ROWS)
    return MLA_ERR_INVALID_ARG;
  if (!tiles_ok(g)) return MLA_ERR_UNSUPPORTED;
  const size_t total = mla_packed_weights_size(cfg);
  int r = check_ws(d_dst, dst_bytes, total);
  if (r) return r;
  long rc[8][2];
  weight_shapes(g, rc);
  const void* in[8] = {src->W_DKV, src->W_KR, src->W_DQ, src->W_UQ,
                       src->W_QR, src->W_UK, src->W_UV, src->W_O};
  const uintptr_t d0 = (uintptr_t)d_dst, d1 = d0 + total;
  for (int i = 0; i < 8; ++i) {
    const uintptr_t s0 = (uintptr_t)in[i], s1 = s0 + (size_t)rc[i][0] * rc[i][1] * g.esize();
    if (in[i] && s0 < d1 && d0 < s1) return MLA_ERR_INVALID_ARG;
  }
  mla_weights res{};
  const void** dst[8] = {&res.W_DKV, &res.W_KR, &res.W_DQ, &res.W_UQ,
                         &res.W_QR, &res.W_UK, &res.W_UV, &res.W_O};
  char* p = (char*)d_dst;
  for (int i = 0; i < 8; ++i) {
    if (in[i]) {
      MLA_TRY(pack_tiles(in[i], rc[i][0], rc[i][1], g.esize(), p, (hipStream_t)stream));
      *dst[i] = p;
    }
    p += al((size_t)rc[i][0] * rc[i][1] * g.esize());
  }
  res.layout = MLA_LAYOUT_TILES;
  *out = res;
  return MLA_OK;
}

size_t mla_workspace_size(const mla_config* cfg, int op, int batch, int max_kv_len,
                          int num_splits) {
  Geo g;
  if (!resolve(cfg, &g) || batch < 0 || max_kv_len < 0 || num_splits < 0) return 0;
  switch (op) {
    case MLA_OP_APPEND: return ws_append(g, batch);
    case MLA_OP_DECODE: return ws_decode(g, batch, num_splits);
    case MLA_OP_PREFILL: return ws_prefill(g, batch, max_kv_len);
    case MLA_OP_DECODE_QUERY: return ws_query(g, batch);
    case MLA_OP_DECODE_ATTENTION: return ws_attn(g, batch, num_splits);
    case MLA_OP_DECODE_OUTPUT: return ws_out(g, batch);
    case MLA_OP_DECODE_MERGED: return ws_decode_merged(g, batch, num_splits);
    case MLA_OP_MHA_DECODE: return ws_mha(g, batch, num_splits);
    case MLA_OP_ATTENTION_BACKWARD: return ws_bwd(g, batch, max_kv_len);
    default: return 0;
  }
}

int mla_append_kv(const mla_config* cfg, const mla_weights* w, const void* h,
                  const int32_t* positions, const int32_t* slot_mapping, int T,
                  const float* rope_table, int rope_len, void* kv_cache, int num_pages,
                  void* workspace, size_t ws_bytes, void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || !weights_ok(w, false, false, true, false) || T < 0 || num_pages < 0 ||
      rope_len < 0)
    return MLA_ERR_INVALID_ARG;
  if (int lr = layout_status(g, w)) return lr;
  if (T == 0) return MLA_OK;
  if (!h || !positions || !slot_mapping || !rope_table || !kv_cache || num_pages == 0 ||
      rope_len == 0)
    return MLA_ERR_INVALID_ARG;
  int r = check_ws(workspace, ws_bytes, ws_append(g, T));
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  float* y = (float*)workspace;
  const GType Ty = st(g);
  const bool wt = w->layout == MLA_LAYOUT_TILES;
  // c^KV_t = W_DKV h_t into columns [0, d_c); W_KR h_t into [d_c, d_c + d_r)
  if (is_v2_fast(g)) {
    // the weight-streaming MFMA GEMM, fp32 out (64-row activation blocks)
    MLA_TRY(wgemm(GemmTile{4, 1}, T, g.d_c, g.d, h, g.d, 0, 0, w->W_DKV, y, g.row, 0, true, 1.f,
                  s, false, false, wt));
    MLA_TRY(wgemm(GemmTile{4, 1}, T, g.d_r, g.d, h, g.d, 0, 0, w->W_KR, y + g.d_c, g.row, 0, true,
                  1.f, s, false, false, wt));
  } else {
    MLA_TRY(gemm_generic(Ty, Ty, G_F32, b_layout(wt, false), T, g.d_c, g.d, h, g.d, 0, w->W_DKV,
                         g.d, 0, y, g.row, 0, 1, 1.f, s));
    MLA_TRY(gemm_generic(Ty, Ty, G_F32, b_layout(wt, false), T, g.d_r, g.d, h, g.d, 0, w->W_KR,
                         g.d, 0, y + g.d_c, g.row, 0, 1, 1.f, s));
  }
  MLA_TRY(append_finish(g, y, positions, slot_mapping, T, rope_table, rope_len, kv_cache,
                        num_pages, s));
  return MLA_OK;
}

int mla_decode_query(const mla_config* cfg, const mla_weights* w, const void* h,
                     const int32_t* positions, int B, const float* rope_table, int rope_len,
                     void* workspace, size_t ws_bytes, void* q_abs, void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || !weights_ok(w, true, false, false, false) || B < 0 || rope_len < 0)
    return MLA_ERR_INVALID_ARG;
  if (int lr = layout_status(g, w)) return lr;
  if (B == 0) return MLA_OK;
  if (!h || !positions || !rope_table || rope_len == 0 || !q_abs) return MLA_ERR_INVALID_ARG;
  int r = check_ws(workspace, ws_bytes, ws_query(g, B));
  if (r) return r;
  return run_query(g, w, h, positions, B, rope_table, rope_len, workspace, q_abs,
                   (hipStream_t)stream);
}

static int check_attn_args(const Geo& g, const void* q_abs, const void* cache, int num_pages,
                           const int32_t* page_table, int max_pages, const int32_t* kv_lens,
                           int B, int max_kv_len, int num_splits) {
  if (B < 0 || num_pages < 0 || max_pages < 0 || max_kv_len < 0 || num_splits < 0)
    return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!q_abs || !cache || !page_table || !kv_lens || num_pages == 0 || max_pages == 0 ||
      max_kv_len == 0)
    return MLA_ERR_INVALID_ARG;
  if ((long)max_kv_len > (long)max_pages * g.page) return MLA_ERR_INVALID_ARG;
  if (num_splits > 4096) return MLA_ERR_INVALID_ARG;
  if (!is_v2_fast(g) && !generic_ok(g)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int mla_decode_attention(const mla_config* cfg, const void* q_abs, const void* kv_cache,
                         int num_pages, const int32_t* page_table, int max_pages,
                         const int32_t* kv_lens, int B, int max_kv_len, int num_splits,
                         void* workspace, size_t ws_bytes, void* latent_out, void* stream) {
  Geo g;
  if (!resolve(cfg, &g)) return MLA_ERR_INVALID_ARG;
  int r = check_attn_args(g, q_abs, kv_cache, num_pages, page_table, max_pages, kv_lens, B,
                          max_kv_len, num_splits);
  if (r || B == 0) return r;
  if (!latent_out) return MLA_ERR_INVALID_ARG;
  r = check_ws(workspace, ws_bytes, ws_attn(g, B, num_splits));
  if (r) return r;
  return run_attention(g, q_abs, kv_cache, num_pages, page_table, max_pages, kv_lens, B,
                       max_kv_len, num_splits, workspace, latent_out, (hipStream_t)stream);
}

int mla_decode_output(const mla_config* cfg, const mla_weights* w, const void* latent_out, int B,
                      void* workspace, size_t ws_bytes, void* out, void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || !weights_ok(w, false, true, false, false) || B < 0)
    return MLA_ERR_INVALID_ARG;
  if (int lr = layout_status(g, w)) return lr;
  if (B == 0) return MLA_OK;
  if (!latent_out || !out) return MLA_ERR_INVALID_ARG;
  int r = check_ws(workspace, ws_bytes, ws_out(g, B));
  if (r) return r;
  return run_output(g, w, latent_out, B, workspace, out, (hipStream_t)stream);
}

}  // extern "C"

// Host-side argument checks of mla_decode (no HIP call); MLA_OK, with *need
// the workspace bytes, when the arguments describe a launchable step.
int mla::decode_args_status(const mla_config* cfg, const mla_weights* w, const void* h,
                            const int32_t* positions, const void* kv_cache, int num_pages,
                            const int32_t* page_table, int max_pages, const int32_t* kv_lens,
                            int B, int max_kv_len, const float* rope_table, int rope_len,
                            int num_splits, const void* out, size_t* need) {
  Geo g;
  if (!resolve(cfg, &g) || !weights_ok(w, true, true, false, false) || rope_len < 0)
    return MLA_ERR_INVALID_ARG;
  if (int lr = layout_status(g, w)) return lr;
  // h stands in for the (not yet computed) absorbed query in the checks
  int r = check_attn_args(g, h, kv_cache, num_pages, page_table, max_pages, kv_lens, B, max_kv_len,
                          num_splits);
  if (r) return r;
  if (B > 0 && (!h || !positions || !rope_table || rope_len == 0 || !out))
    return MLA_ERR_INVALID_ARG;
  *need = B > 0 ? ws_decode(g, B, num_splits) : 0;
  return MLA_OK;
}

extern "C" {

int mla_decode(const mla_config* cfg, const mla_weights* w, const void* h,
               const int32_t* positions, const void* kv_cache, int num_pages,
               const int32_t* page_table, int max_pages, const int32_t* kv_lens, int B,
               int max_kv_len, const float* rope_table, int rope_len, int num_splits,
               void* workspace, size_t ws_bytes, void* out, void* stream) {
  size_t need = 0;
  int r = decode_args_status(cfg, w, h, positions, kv_cache, num_pages, page_table, max_pages,
                             kv_lens, B, max_kv_len, rope_table, rope_len, num_splits, out, &need);
  if (r || B == 0) return r;
  Geo g;
  resolve(cfg, &g);
  r = check_ws(workspace, ws_bytes, need);
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  Carver c(workspace);
  void* q_abs = c.take((size_t)B * g.n_h * g.row * g.esize());
  void* lat = c.take((size_t)B * g.n_h * g.d_c * g.esize());
  PlanPtrs plan;
  carve_plan(c.take(plan_bytes(B, num_splits)), B, num_splits, &plan);
  const PlanJob job = plan_job(plan, kv_lens, B, max_kv_len, max_pages, g.page, 64, num_splits);
  void* sub = c.base + c.used;
  // the absorbed query stays inside the step: on the V2 fast path it is
  // written in the query-tile layout the attention kernel loads contiguously
  r = run_query(g, w, h, positions, B, rope_table, rope_len, sub, q_abs, s, &job, true);
  if (r) return r;
  r = run_attention(g, q_abs, kv_cache, num_pages, page_table, max_pages, kv_lens, B, max_kv_len,
                    num_splits, sub, lat, s, &plan, true);
  if (r) return r;
  return run_output(g, w, lat, B, sub, out, s);
}

int mla_merge_weights(const mla_config* cfg, const mla_weights* src, int layout, void* d_W_UQK,
                      void* d_W_OUV, void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || !src || src->layout != MLA_LAYOUT_ROWS || !src->W_UQ || !src->W_UK ||
      !src->W_UV || !src->W_O || !d_W_UQK || !d_W_OUV ||
      (layout != MLA_LAYOUT_ROWS && layout != MLA_LAYOUT_TILES))
    return MLA_ERR_INVALID_ARG;
  const bool wt = layout == MLA_LAYOUT_TILES;
  if (wt && !tiles_ok(g)) return MLA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const GType T = st(g);
  const long nk = (long)g.n_h * g.d_c, nq = (long)g.n_h * g.d_h;
  // W_UQK,i [d_c][d_cq] = sum_d W_UK,i[d][.] (x) W_UQ,i[d][.]: A(c, d) =
  // W_UK,i[d][c] (k-major), B(k', d) = W_UQ,i[d][k'] (k-major); head i's rows
  // start at the same element in either layout
  MLA_TRY(gemm_generic(T, T, T, B_KN, g.d_c, g.d_cq, g.d_h, src->W_UK, g.d_c,
                       (long)g.d_h * g.d_c, src->W_UQ, g.d_cq, (long)g.d_h * g.d_cq, d_W_UQK,
                       g.d_cq, (long)g.d_c * g.d_cq, g.n_h, 1.f, s, true, wt));
  // W_OUV[.][i d_c + c] = sum_d W_O[.][i d_h + d] W_UV,i[d][c]: A = W_O's head
  // columns, B(c, d) = W_UV,i[d][c]; head i's column block starts i d_c
  // elements into a row-major row, 16 i d_c elements into the tiles
  MLA_TRY(gemm_generic(T, T, T, B_KN, g.d, g.d_c, g.d_h, src->W_O, nq, g.d_h, src->W_UV, g.d_c,
                       (long)g.d_h * g.d_c, d_W_OUV, nk, wt ? 16L * g.d_c : (long)g.d_c, g.n_h,
                       1.f, s, false, wt));
  return MLA_OK;
}

int mla_decode_merged(const mla_config* cfg, const mla_merged_weights* w, const void* h,
                      const int32_t* positions, const void* kv_cache, int num_pages,
                      const int32_t* page_table, int max_pages, const int32_t* kv_lens, int B,
                      int max_kv_len, const float* rope_table, int rope_len, int num_splits,
                      void* workspace, size_t ws_bytes, void* out, void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || !w || !w->W_DQ || !w->W_QR || !w->W_UQK || !w->W_OUV ||
      (w->layout != MLA_LAYOUT_ROWS && w->layout != MLA_LAYOUT_TILES) || rope_len < 0)
    return MLA_ERR_INVALID_ARG;
  if (w->layout == MLA_LAYOUT_TILES && !tiles_ok(g)) return MLA_ERR_UNSUPPORTED;
  int r = check_attn_args(g, h, kv_cache, num_pages, page_table, max_pages, kv_lens, B, max_kv_len,
                          num_splits);
  if (r || B == 0) return r;
  if (!h || !positions || !rope_table || rope_len == 0 || !out) return MLA_ERR_INVALID_ARG;
  r = check_ws(workspace, ws_bytes, ws_decode_merged(g, B, num_splits));
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  Carver c(workspace);
  void* q_abs = c.take((size_t)B * g.n_h * g.row * g.esize());
  void* lat = c.take((size_t)B * g.n_h * g.d_c * g.esize());
  PlanPtrs plan;
  carve_plan(c.take(plan_bytes(B, num_splits)), B, num_splits, &plan);
  const PlanJob job = plan_job(plan, kv_lens, B, max_kv_len, max_pages, g.page, 64, num_splits);
  void* sub = c.base + c.used;
  r = run_query_merged(g, w, h, positions, B, rope_table, rope_len, sub, q_abs, s, &job);
  if (r) return r;
  r = run_attention(g, q_abs, kv_cache, num_pages, page_table, max_pages, kv_lens, B, max_kv_len,
                    num_splits, sub, lat, s, &plan);
  if (r) return r;
  return run_output_merged(g, w, lat, B, sub, out, s);
}

int mla_mha_decode_attention(const mla_config* cfg, const void* q, const void* kv_cache,
                             int num_pages, const int32_t* page_table, int max_pages,
                             const int32_t* kv_lens, int B, int max_kv_len, float scale,
                             int num_splits, void* workspace, size_t ws_bytes, void* out,
                             void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || B < 0 || num_pages < 0 || max_pages < 0 || max_kv_len < 0 ||
      num_splits < 0 || num_splits > 4096)
    return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!q || !kv_cache || !page_table || !kv_lens || !out || num_pages == 0 || max_pages == 0 ||
      max_kv_len == 0 || (long)max_kv_len > (long)max_pages * g.page ||
      ((uintptr_t)kv_cache & 15))
    return MLA_ERR_INVALID_ARG;
  if (!mha_supported(g)) return MLA_ERR_UNSUPPORTED;
  int r = check_ws(workspace, ws_bytes, ws_mha(g, B, num_splits));
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  const PlanDims pd = plan_dims(B, num_splits);
  Carver c(workspace);
  PlanPtrs plan;
  carve_plan(c.take(plan_bytes(B, num_splits)), B, num_splits, &plan);
  float* part_o = (float*)c.take(sizeof(float) * (size_t)pd.max_segs * g.n_h * g.d_h);
  float* part_ml = (float*)c.take(sizeof(float) * 2 * (size_t)pd.max_segs * g.n_h);
  MLA_TRY(launch_plan(plan, kv_lens, B, max_kv_len, max_pages, g.page, 64, num_splits, s));
  const float sc = scale > 0.f ? scale : (float)(1.0 / sqrt((double)g.d_h));
  MLA_TRY(mha_decode(g, q, kv_cache, num_pages, page_table, max_pages, plan, pd.max_segs, sc,
                     part_o, part_ml, out, s));
  Geo gc = g;   // the merge of latent partials, with head width d_h
  gc.d_c = g.d_h;
  MLA_TRY(combine_partials(gc, plan, B, part_o, part_ml, out, s));
  return MLA_OK;
}

namespace mla {
namespace {
// Y = alpha * X . W^T over M rows: the tiled MFMA GEMM from 128 rows on, the
// weight-streaming one (tile t) below that or where no tile fits the shape.
constexpr int kTiledGemmRows = 128;
hipError_t gemm_rows(GemmTile t, int M, int N, int K, const void* X, long ldx, const void* W,
                     bool wt, void* Y, long ldy, bool out_f32, float alpha, hipStream_t s,
                     int y_grp = 0, long y_grp_stride = 0) {
  if (M >= kTiledGemmRows) {
    const hipError_t e = tgemm(M, N, K, X, ldx, W, wt, Y, ldy, out_f32, alpha, s, y_grp,
                               y_grp_stride);
    if (e != hipErrorNotSupported) return e;
  }
  return wgemm(t, M, N, K, X, ldx, 0, 0, W, Y, ldy, 0, out_f32, alpha, s, false, false, wt, y_grp,
               y_grp_stride);
}
}  // namespace
}  // namespace mla

int mla_attention_backward(const mla_config* cfg, const mla_weights* w, const float* q,
                           const int32_t* positions, const void* kv_cache, int num_pages,
                           const int32_t* page_table, int max_pages, int kv_len, int T,
                           const float* dO, void* workspace, size_t ws_bytes, float* dW_UK,
                           float* dW_UV, float* dq, float* dC, void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || !weights_ok(w, false, false, false, true) || T < 0 || kv_len < 0 ||
      num_pages < 0 || max_pages < 0)
    return MLA_ERR_INVALID_ARG;
  if (int lr = layout_status(g, w)) return lr;
  if (T == 0 || kv_len == 0) return T == 0 ? MLA_OK : MLA_ERR_INVALID_ARG;
  if (!q || !positions || !kv_cache || !page_table || !dO || !dW_UK || !dW_UV || !dq || !dC ||
      num_pages == 0 || (long)kv_len > (long)max_pages * g.page)
    return MLA_ERR_INVALID_ARG;
  if (!generic_ok(g)) return MLA_ERR_UNSUPPORTED;
  int r = check_ws(workspace, ws_bytes, ws_bwd(g, T, kv_len));
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  Carver c(workspace);
  const GType Ty = st(g);
  const bool wt = w->layout == MLA_LAYOUT_TILES;
  const int N = kv_len, dqw = g.d_h + g.d_r;
  if (use_bwd_v2(g, T, N)) {
    // DeepSeek-V2 heads: k and v per head in bf16 as the prefill makes them,
    // the attention's gradients flash style on bf16 MFMA, then the weight
    // and latent gradients as bf16 MFMA GEMMs with fp32 results
    BwdWsV2 b;
    carve_bwd_v2(c, g, T, N, &b);
    const int nq = g.n_h * g.d_h, Np = attn_bwd_v2_npad(N);
    MLA_TRY(prefill_rows_v2(g, kv_cache, num_pages, page_table, N, b.rows16, b.k16, s));
    MLA_TRY(gemm_rows(GemmTile{4, 1}, N, nq, g.d_c, b.rows16, g.row, w->W_UK, wt, b.k16,
                      (long)g.n_h * dqw, false, 1.f, s, g.d_h, dqw));
    MLA_TRY(gemm_rows(GemmTile{4, 1}, N, nq, g.d_c, b.rows16, g.row, w->W_UV, wt, b.v16, nq,
                      false, 1.f, s));
    MLA_TRY(attn_bwd_v2(g, N, T, q, dO, positions, b.k16, b.v16, b.q16, b.do16, b.rec,
                        b.qblk_far, dq, b.dkv16, b.dkT16, b.dvT16, b.dkr, s));
    // dW_UK,i = sum_j dk^C_ij c_j^T (rows [head, dim], contraction over keys)
    MLA_TRY(transpose16(b.rows16, g.row, false, g.d_c, N, Np, b.cT16, Np, 0, s));
    MLA_TRY(gemm_rows(GemmTile{4, 1}, nq, g.d_c, Np, b.dkT16, Np, b.cT16, false, dW_UK, g.d_c,
                      true, 1.f, s));
    MLA_TRY(gemm_rows(GemmTile{4, 1}, nq, g.d_c, Np, b.dvT16, Np, b.cT16, false, dW_UV, g.d_c,
                      true, 1.f, s));
    // dc_j = [dk^C_j | dv_j] . [W_UK ; W_UV] in K chunks, summed with the
    // heads' dk^R into dC
    MLA_TRY(transpose16(w->W_UK, g.d_c, wt, g.d_c, nq, nq, b.wT16, 2L * nq, 0, s));
    MLA_TRY(transpose16(w->W_UV, g.d_c, wt, g.d_c, nq, nq, b.wT16, 2L * nq, nq, s));
    const int lsp = bwd_lat_splits(N);
    MLA_TRY(tgemm(N, g.d_c, 2 * nq, b.dkv16, 2L * nq, b.wT16, false, b.lat, g.d_c, true, 1.f, s, 0,
                  0, lsp, (long)N * g.d_c));
    MLA_TRY(bwd_dc_v2(N, b.lat, lsp, b.dkr, dC, s));
    return MLA_OK;
  }
  BwdWs b;
  carve_bwd(c, g, T, kv_len, &b);
  const long hd = (long)g.n_h * g.d_h, TN = (long)T * N;
  // the forward's pieces: cached rows, K^C = W_UK,i c_j and V = W_UV,i c_j
  MLA_TRY(gather_rows_f32(g, kv_cache, num_pages, page_table, max_pages, N, b.rows, s));
  MLA_TRY(gemm_generic(G_F32, Ty, G_F32, b_layout(wt, false), N, g.d_h, g.d_c, b.rows, g.row, 0,
                       w->W_UK, g.d_c, (long)g.d_h * g.d_c, b.K, hd, g.d_h, g.n_h, 1.f, s));
  MLA_TRY(gemm_generic(G_F32, Ty, G_F32, b_layout(wt, false), N, g.d_h, g.d_c, b.rows, g.row, 0,
                       w->W_UV, g.d_c, (long)g.d_h * g.d_c, b.V, hd, g.d_h, g.n_h, 1.f, s));
  // softmax and its backward: P, dS [n_h][T][N]
  MLA_TRY(attn_bwd_ps(g, N, T, g.scale, q, positions, b.K, b.V, b.rows, dO, b.P, b.dS, s));
  // dv_ij = sum_t p_tij dO_ti;  dk^C_ij = scale sum_t ds_tij q^C_ti
  MLA_TRY(gemm_generic(G_F32, G_F32, G_F32, B_KN, N, g.d_h, T, b.P, N, TN, dO, hd, g.d_h, b.dV,
                       hd, g.d_h, g.n_h, 1.f, s, true));
  MLA_TRY(gemm_generic(G_F32, G_F32, G_F32, B_KN, N, g.d_h, T, b.dS, N, TN, q,
                       (long)g.n_h * dqw, dqw, b.dK, hd, g.d_h, g.n_h, g.scale, s, true));
  // dq^C_ti = scale sum_j ds_tij k^C_ij;  dq^R_ti = scale sum_j ds_tij k^R_j
  MLA_TRY(gemm_generic(G_F32, G_F32, G_F32, B_KN, T, g.d_h, N, b.dS, N, TN, b.K, hd, g.d_h, dq,
                       (long)g.n_h * dqw, dqw, g.n_h, g.scale, s));
  MLA_TRY(gemm_generic(G_F32, G_F32, G_F32, B_KN, T, g.d_r, N, b.dS, N, TN, b.rows + g.d_c, g.row,
                       0, dq + g.d_h, (long)g.n_h * dqw, dqw, g.n_h, g.scale, s));
  // dk^R per head: scale sum_t ds_tij q^R_ti, summed over heads below
  MLA_TRY(gemm_generic(G_F32, G_F32, G_F32, B_KN, N, g.d_r, T, b.dS, N, TN, q + g.d_h,
                       (long)g.n_h * dqw, dqw, b.dkr, g.d_r, (long)N * g.d_r, g.n_h, g.scale, s,
                       true));
  // dW_UK,i = sum_j dk^C_ij c_j^T;  dW_UV,i = sum_j dv_ij c_j^T
  MLA_TRY(gemm_generic(G_F32, G_F32, G_F32, B_KN, g.d_h, g.d_c, N, b.dK, hd, g.d_h, b.rows, g.row,
                       0, dW_UK, g.d_c, (long)g.d_h * g.d_c, g.n_h, 1.f, s, true));
  MLA_TRY(gemm_generic(G_F32, G_F32, G_F32, B_KN, g.d_h, g.d_c, N, b.dV, hd, g.d_h, b.rows, g.row,
                       0, dW_UV, g.d_c, (long)g.d_h * g.d_c, g.n_h, 1.f, s, true));
  // dc_j = sum_i W_UK,i^T dk^C_ij + W_UV,i^T dv_ij (one product over all heads each)
  MLA_TRY(gemm_generic(G_F32, Ty, G_F32, b_layout(wt, true), N, g.d_c, (int)hd, b.dK, hd, 0,
                       w->W_UK, g.d_c, 0, b.lat_k, g.d_c, 0, 1, 1.f, s));
  MLA_TRY(gemm_generic(G_F32, Ty, G_F32, b_layout(wt, true), N, g.d_c, (int)hd, b.dV, hd, 0,
                       w->W_UV, g.d_c, 0, b.lat_v, g.d_c, 0, 1, 1.f, s));
  MLA_TRY(attn_bwd_dc(g, N, b.lat_k, b.lat_v, b.dkr, dC, s));
  return MLA_OK;
}

int mla_prefill(const mla_config* cfg, const mla_weights* w, const void* h,
                const int32_t* positions, const void* kv_cache, int num_pages,
                const int32_t* page_table, int max_pages, int kv_len, int T,
                const float* rope_table, int rope_len, void* workspace, size_t ws_bytes,
                void* out, void* stream) {
  Geo g;
  if (!resolve(cfg, &g) || !weights_ok(w, true, true, false, true) || T < 0 || kv_len < 0 ||
      num_pages < 0 || max_pages < 0 || rope_len < 0)
    return MLA_ERR_INVALID_ARG;
  if (int lr = layout_status(g, w)) return lr;
  if (T == 0) return MLA_OK;
  if (!h || !positions || !kv_cache || !page_table || !rope_table || !out || kv_len == 0 ||
      num_pages == 0 || rope_len == 0)
    return MLA_ERR_INVALID_ARG;
  if ((long)kv_len > (long)max_pages * g.page) return MLA_ERR_INVALID_ARG;
  if (!generic_ok(g)) return MLA_ERR_UNSUPPORTED;
  int r = check_ws(workspace, ws_bytes, ws_prefill(g, T, kv_len));
  if (r) return r;
  hipStream_t s = (hipStream_t)stream;
  Carver c(workspace);
  PrefillWs p;
  carve_prefill(c, g, T, kv_len, &p);
  const GType Ty = st(g);
  const bool wt = w->layout == MLA_LAYOUT_TILES;
  const long wq = (long)g.n_h * (g.d_h + g.d_r);
  if (prefill_v2_supported(g)) {
    // DeepSeek-V2 heads: bf16 intermediates, every product on the
    // weight-streaming MFMA GEMM (64-row activation blocks, no K split), the
    // attention on bf16 MFMA.  The fp32 buffers of the generic path hold them.
    void* cq16 = p.cq;                                      // [T][d_cq]
    void* q16 = p.q;                                        // [T][n_h][d_h + d_r]
    float* qr = (float*)((char*)p.q + (size_t)T * wq * 2);  // [T][n_h][d_r], scaled
    void* rows16 = p.rows;                                  // [kv_len][row]
    void* k16 = p.kbuf;                                     // [kv_len][n_h][d_h + d_r]
    void* v16 = p.vbuf;                                     // [kv_len][n_h][d_h]
    void* o16 = p.o;                                        // [T][n_h d_h]
    const long nq = (long)g.n_h * g.d_h;
    // the query carries the softmax scale and log2(e): the attention kernel's
    // scores come out in log2 units
    const float qscale = g.scale * 1.4426950408889634f;
    // c^Q = W_DQ h; q^C_i = qscale W_UQ,i c^Q into columns 0..127 of head i
    MLA_TRY(gemm_rows(GemmTile{4, 1}, T, g.d_cq, g.d, h, g.d, w->W_DQ, wt, cq16, g.d_cq, false,
                      1.f, s));
    MLA_TRY(gemm_rows(GemmTile{4, 1}, T, (int)nq, g.d_cq, cq16, g.d_cq, w->W_UQ, wt, q16, wq,
                      false, qscale, s, g.d_h, g.d_h + g.d_r));
    // qscale RoPE(W_QR,i c^Q) into columns 128..191 of head i: turned and
    // packed in the tiled product's epilogue, else (fewer rows than a tile
    // takes) the product in fp32, then the rotation
    hipError_t qe = hipErrorNotSupported;
    if (T >= kTiledGemmRows)
      qe = tgemm(T, g.n_h * g.d_r, g.d_cq, cq16, g.d_cq, w->W_QR, wt, (__bf16*)q16 + g.d_h, wq,
                 false, qscale, s, g.d_r, g.d_h + g.d_r, 1, 0, positions, rope_table, rope_len);
    if (qe == hipErrorNotSupported) {
      MLA_TRY(gemm_rows(GemmTile{4, 1}, T, g.n_h * g.d_r, g.d_cq, cq16, g.d_cq, w->W_QR, wt, qr,
                        (long)g.n_h * g.d_r, true, qscale, s));
      MLA_TRY(prefill_rope_q_v2(g, qr, positions, T, rope_table, rope_len, q16, s));
    } else {
      MLA_TRY(qe);
    }
    // order A: k_ij = [W_UK,i c_j | k^R_j] and v_ij = W_UV,i c_j from the rows
    MLA_TRY(prefill_rows_v2(g, kv_cache, num_pages, page_table, kv_len, rows16, k16, s));
    MLA_TRY(gemm_rows(GemmTile{4, 1}, kv_len, (int)nq, g.d_c, rows16, g.row, w->W_UK, wt, k16,
                      wq, false, 1.f, s, g.d_h, g.d_h + g.d_r));
    MLA_TRY(gemm_rows(GemmTile{4, 1}, kv_len, (int)nq, g.d_c, rows16, g.row, w->W_UV, wt, v16, nq,
                      false, 1.f, s));
    // causal attention, then u = W_O o
    MLA_TRY(attn_prefill_v2(g, q16, k16, v16, positions, T, kv_len, o16, s));
    MLA_TRY(gemm_rows(GemmTile{5, 1}, T, g.d, (int)nq, o16, nq, w->W_O, wt, out, g.d, false, 1.f,
                      s));
    return MLA_OK;
  }
  // query: c^Q, then per head [q^C_i | q^R_i] (192-d at V2), RoPE on q^R
  MLA_TRY(gemm_generic(Ty, Ty, G_F32, b_layout(wt, false), T, g.d_cq, g.d, h, g.d, 0, w->W_DQ,
                       g.d, 0, p.cq, g.d_cq, 0, 1, 1.f, s));
  // (the softmax scale is folded into q; RoPE is linear, so rotating the
  // scaled q^R equals scaling the rotated one)
  MLA_TRY(gemm_generic(G_F32, Ty, G_F32, b_layout(wt, false), T, g.d_h, g.d_cq, p.cq, g.d_cq, 0,
                       w->W_UQ, g.d_cq, (long)g.d_h * g.d_cq, p.q, wq, g.d_h + g.d_r, g.n_h,
                       g.scale, s));
  MLA_TRY(gemm_generic(G_F32, Ty, G_F32, b_layout(wt, false), T, g.d_r, g.d_cq, p.cq, g.d_cq, 0,
                       w->W_QR, g.d_cq, (long)g.d_r * g.d_cq, p.q + g.d_h, wq, g.d_h + g.d_r,
                       g.n_h, g.scale, s));
  MLA_TRY(rope_inplace_heads(g, p.q, T, wq, g.d_h, positions, rope_table, rope_len, s));
  // order A: decompress k_j = [W_UK,i c_j | k^R_j] and v_j = W_UV,i c_j per head
  MLA_TRY(gather_rows_f32(g, kv_cache, num_pages, page_table, max_pages, kv_len, p.rows, s));
  MLA_TRY(gemm_generic(G_F32, Ty, G_F32, b_layout(wt, false), kv_len, g.d_h, g.d_c, p.rows, g.row,
                       0, w->W_UK, g.d_c, (long)g.d_h * g.d_c, p.kbuf, wq, g.d_h + g.d_r,
                       g.n_h, 1.f, s));
  MLA_TRY(broadcast_kr(g, p.rows, kv_len, p.kbuf, s));
  MLA_TRY(gemm_generic(G_F32, Ty, G_F32, b_layout(wt, false), kv_len, g.d_h, g.d_c, p.rows, g.row,
                       0, w->W_UV, g.d_c, (long)g.d_h * g.d_c, p.vbuf,
                       (long)g.n_h * g.d_h, g.d_h, g.n_h, 1.f, s));
  // causal softmax attention with 192-d scores and 128-d values, then W_O
  MLA_TRY(attn_prefill_generic(g, p.q, p.kbuf, p.vbuf, positions, T, kv_len, rope_len, p.o, s));
  MLA_TRY(gemm_generic(G_F32, Ty, Ty, b_layout(wt, false), T, g.d, g.n_h * g.d_h, p.o,
                       (long)g.n_h * g.d_h, 0, w->W_O, (long)g.n_h * g.d_h, 0, out, g.d, 0, 1,
                       1.f, s));
  return MLA_OK;
}

}  // extern "C"
