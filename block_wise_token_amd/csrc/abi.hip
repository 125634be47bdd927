// C ABI of libuniprefill: argument validation, grid planning, workspace layout and
// launches.  The operations and their page citations are documented in
// include/uniprefill.h.
#include "uniprefill.h"
#include "up_internal.h"

#include <climits>
#include <cmath>
#include <mutex>
#include <vector>

namespace {

using namespace up;

// Device error word: one copy per GPU; its device address is looked up once per
// device and passed to kernels as a plain pointer.
__device__ int g_up_error;

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int* g_err_ptr[kMaxDevices] = {};

int* error_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_err_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_up_error)) != hipSuccess) return nullptr;
    g_err_ptr[dev] = static_cast<int*>(p);
  }
  return g_err_ptr[dev];
}

__global__ void up_clear_word_kernel(int* w) { *w = 0; }

// ---- kernel timing (opt-in) ------------------------------------------------
struct Rec {
  int which;
  hipEvent_t a, b;
};
bool g_prof = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed(int which, hipStream_t st, F&& f) {
  if (!g_prof) return f();
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, st);
  if (e != hipSuccess) return e;
  e = f();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, st);
  g_recs.push_back({which, a, b});
  return e;
}

// ---- validation ----------------------------------------------------------------
bool cu_ok(const int32_t* cu_h, int B) {
  if (B < 0 || (B > 0 && !cu_h)) return false;
  if (B == 0) return cu_h == nullptr || cu_h[0] == 0;
  if (cu_h[0] != 0) return false;
  for (int i = 0; i < B; ++i)
    if (cu_h[i + 1] < cu_h[i]) return false;
  return true;
}

struct SelPlan {
  int64_t T = 0, nb_tot = 0;
  int nb_max = 0;
};

SelPlan sel_plan(const int32_t* cu_h, int B, int G) {
  SelPlan s;
  for (int i = 0; i < B; ++i) {
    const int64_t L = (int64_t)cu_h[i + 1] - cu_h[i];
    const int64_t nb = (L + G - 1) / G;
    s.nb_tot += nb;
    if (nb > s.nb_max) s.nb_max = (int)nb;
  }
  s.T = B > 0 ? cu_h[B] : 0;
  return s;
}

bool block_size_supported(int G) { return G >= 32 && G <= 1024 && G % 32 == 0; }

// Compute units of the current device (256 on MI355X; also the fallback when no
// device is visible, so host-only size queries agree with the calls).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Plan of the score pass; returns UP_OK or an error status.
int plan_scores(const int32_t* cu_h, int B, int Hq, int Hkv, int d, int n, int G, ScoreShape* s,
                Totals* t) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || n <= 0 || G <= 0 || d <= 0) return UP_EINVAL;
  if (Hq % Hkv != 0) return UP_EINVAL;
  if (!cu_ok(cu_h, B)) return UP_EINVAL;
  if (d != 64 && d != 128 && d != 256) return UP_EUNSUPPORTED;
  if (!block_size_supported(G)) return UP_EUNSUPPORTED;
  // The score kernel addresses keys as 32-bit byte offsets within a page of up to 1024
  // token rows of Hkv * d bf16 values.
  if ((int64_t)Hkv * d * 2 * 1024 >= ((int64_t)1 << 31)) return UP_EUNSUPPORTED;
  s->B = B; s->Hq = Hq; s->Hkv = Hkv; s->d = d; s->n = n; s->G = G;
  s->qt = (d == 256) ? 1 : 2;
  s->kt = (d == 256) ? 1 : (G % 64 == 0 ? 2 : 1);
  s->rows_wg = score_rows_wg(d);
  const int64_t gs = Hq / Hkv;
  // Statistics chunks per request (from the request alone, stat_chunk_blocks), then a
  // target work-item length TB for load balance: every request's items are whole runs
  // of its statistics chunks (chunks_per_item).  TB minimises the estimated time,
  // rounds of the device's CUs times the mean item cost (blocks plus a workgroup's
  // fixed cost), ties going to the longer item; it never changes a result.  For a
  // lone request on 256 CUs it picks one chunk per item.
  const int64_t cus = (int64_t)device_cus() * score_wgs_per_cu(d);
  struct Req { int64_t nb, per; int cbs; int64_t nch; };
  std::vector<Req> req(B);
  for (int i = 0; i < B; ++i) {
    const int64_t L = (int64_t)cu_h[i + 1] - cu_h[i];
    const int64_t W = L < n ? L : n;
    Req r;
    r.nb = (L + G - 1) / G;
    r.per = Hkv * ((gs * W + s->rows_wg - 1) / s->rows_wg);   // items per chunk position
    r.cbs = stat_chunk_blocks(r.nb, r.per);
    r.nch = (r.nb + r.cbs - 1) / r.cbs;
    req[i] = r;
  }
  {
    static const int kTb[] = {256, 224, 192, 160, 128, 112, 96, 80, 64, 56, 48, 40, 32,
                              28, 24, 20, 16, 14, 12, 10, 8, 6, 4, 3, 2, 1};
    double best_cost = -1.0;
    int best_tb = 1;
    for (int tb : kTb) {
      int64_t items = 0, work = 0;
      for (const Req& r : req) {
        if (r.nb == 0) continue;
        const int cps = chunks_per_item(r.cbs, r.nch, tb);
        const int64_t n_it = (r.nch + cps - 1) / cps;
        const int64_t len = std::min<int64_t>((int64_t)cps * r.cbs, r.nb);
        items += n_it * r.per;
        work += n_it * r.per * (len + kChunkOverheadBlocks);
      }
      const double cost = items ? (double)((items + cus - 1) / cus) * ((double)work / items) : 0.0;
      if (best_cost < 0 || cost < best_cost * (1.0 - 1e-9) ||
          (cost <= best_cost * (1.0 + 1e-9) && tb > best_tb)) {
        best_cost = cost;
        best_tb = tb;
      }
    }
    s->TB = best_tb;
  }
  *t = Totals{};
  for (int i = 0; i < B; ++i) {
    const int64_t L = (int64_t)cu_h[i + 1] - cu_h[i];
    const int64_t W = L < n ? L : n;
    const Req& r = req[i];
    const int64_t nb = r.nb;
    const int64_t nch = r.nch;
    const int cps = chunks_per_item(r.cbs, nch, s->TB);
    const int64_t n_it = (nch + cps - 1) / cps;
    const int64_t R = gs * W;
    const int64_t nrt = (R + s->rows_wg - 1) / s->rows_wg;
    t->win_rows += W;
    t->nb_tot += nb;
    t->items += n_it * Hkv * nrt;
    t->ml_pairs += nb * Hkv * R;
    t->cs_pairs += nch * Hkv * R;
    t->pm_parts += nb * Hkv * nrt;
    if (nb > t->nb_max) t->nb_max = (int32_t)nb;
  }
  t->T = B > 0 ? cu_h[B] : 0;
  t->rows = t->win_rows * Hq;
  if (t->items >= (int64_t)1 << 31 || t->rows >= (int64_t)1 << 31) return UP_EUNSUPPORTED;
  if ((int64_t)t->win_rows * Hq * d >= ((int64_t)1 << 40)) return UP_EUNSUPPORTED;
  return UP_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* up_status_string(int status) {
  switch (status) {
    case UP_OK: return "UP_OK";
    case UP_EINVAL: return "UP_EINVAL: invalid argument";
    case UP_EUNSUPPORTED: return "UP_EUNSUPPORTED: unsupported shape or size";
    case UP_EWORKSPACE: return "UP_EWORKSPACE: workspace missing, too small or misaligned";
    case UP_EHIP: return "UP_EHIP: HIP runtime error";
    default: return "unknown status";
  }
}

int up_abi_version(void) { return 1; }

size_t up_block_scores_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d,
                                 int n, int G) {
  ScoreShape s;
  Totals t;
  if (plan_scores(cu_seqlens_h, B, Hq, Hkv, d, n, G, &s, &t) != UP_OK) return 0;
  return score_ws_layout(B, t).total;
}

int up_block_scores_chunks(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d, int n,
                           int G, int32_t* chunk_blocks_h) {
  ScoreShape s;
  Totals t;
  const int st = plan_scores(cu_seqlens_h, B, Hq, Hkv, d, n, G, &s, &t);
  if (st != UP_OK) return st;
  if (B > 0 && !chunk_blocks_h) return UP_EINVAL;
  const int64_t gs = Hq / Hkv;
  for (int i = 0; i < B; ++i) {
    const int64_t L = (int64_t)cu_seqlens_h[i + 1] - cu_seqlens_h[i];
    const int64_t W = L < n ? L : n;
    const int64_t nrt = (gs * W + s.rows_wg - 1) / s.rows_wg;
    chunk_blocks_h[i] = stat_chunk_blocks((L + G - 1) / G, Hkv * nrt);
  }
  return UP_OK;
}

// stop_at_mass: leave the float64 block masses in the workspace and skip the
// normalisation (the fused decision normalises inside its select kernel).
static int block_scores_common(const void* qwin, const void* k, const PagedK* paged,
                               const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B,
                               int Hq, int Hkv, int d, int n, int G, float scale, float* scores,
                               float* row_lse, void* workspace, size_t workspace_bytes,
                               void* stream, bool stop_at_mass = false) {
  ScoreShape s;
  Totals t;
  const int st = plan_scores(cu_seqlens_h, B, Hq, Hkv, d, n, G, &s, &t);
  if (st != UP_OK) return st;
  if (B == 0 || t.T == 0) return UP_OK;
  if (!qwin || !k || !cu_seqlens || (!scores && !stop_at_mass)) return UP_EINVAL;
  if (!aligned(qwin, 16) || !aligned(k, 16)) return UP_EINVAL;
  const ScoreWs L = score_ws_layout(B, t);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, kWsAlign))
    return UP_EWORKSPACE;
  if (!(scale > 0.f) || std::isinf(scale)) scale = (float)(1.0 / std::sqrt((double)d));
  const float c = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
  int* err = error_word();
  if (!err) return UP_EHIP;
  hipStream_t hs = as_stream(stream);
  hipError_t e;
  e = timed(9, hs, [&] {
    return launch_score_plan(cu_seqlens, s, t, workspace, L.plan, err, hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  PagedK pk;
  if (paged) {
    pk = *paged;
    pk.err = err;
  }
  e = timed(0, hs, [&] {
    return launch_score_partial(qwin, k, s, t, workspace, L, c, paged ? &pk : nullptr, hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(1, hs, [&] { return launch_row_stats(s, t, workspace, L, row_lse, hs); });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(2, hs, [&] { return launch_block_mass(s, t, workspace, L, hs); });
  if (e != hipSuccess) return UP_EHIP;
  if (stop_at_mass) return UP_OK;
  e = timed(3, hs, [&] { return launch_normalize(s, t, workspace, L, scores, hs); });
  if (e != hipSuccess) return UP_EHIP;
  return UP_OK;
}

int up_block_scores(const void* qwin, const void* k, const int32_t* cu_seqlens,
                    const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d, int n, int G,
                    float scale, float* scores, float* row_lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return block_scores_common(qwin, k, nullptr, cu_seqlens, cu_seqlens_h, B, Hq, Hkv, d, n, G,
                             scale, scores, row_lse, workspace, workspace_bytes, stream);
}

// Host checks of a paged key cache's description; fills *pk (its error word is set later).
static int paged_args(const void* k_pages, int64_t num_pages, int page_size,
                      const int32_t* block_table, int max_pages, const int32_t* cu_seqlens_h,
                      int B, PagedK* pk) {
  if (page_size < 16 || page_size > 1024 || (page_size & (page_size - 1)) != 0)
    return UP_EUNSUPPORTED;
  if (num_pages < 0 || max_pages < 0) return UP_EINVAL;
  if (!cu_ok(cu_seqlens_h, B)) return UP_EINVAL;
  int64_t need = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t L = (int64_t)cu_seqlens_h[i + 1] - cu_seqlens_h[i];
    const int64_t p = (L + page_size - 1) / page_size;
    if (p > need) need = p;
  }
  if (need > max_pages) return UP_EINVAL;
  if (need > 0 && (!block_table || num_pages == 0)) return UP_EINVAL;
  if (k_pages && !aligned(k_pages, 16)) return UP_EINVAL;
  pk->table = block_table;
  pk->max_pages = max_pages;
  pk->num_pages = num_pages;
  int lp = 0;
  while ((1 << lp) < page_size) ++lp;
  pk->log2_page = lp;
  return UP_OK;
}

int up_block_scores_paged(const void* qwin, const void* k_pages, int64_t num_pages,
                          int page_size, const int32_t* block_table, int max_pages,
                          const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B, int Hq,
                          int Hkv, int d, int n, int G, float scale, float* scores,
                          float* row_lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  PagedK pk;
  const int st = paged_args(k_pages, num_pages, page_size, block_table, max_pages, cu_seqlens_h,
                            B, &pk);
  if (st != UP_OK) return st;
  return block_scores_common(qwin, k_pages, &pk, cu_seqlens, cu_seqlens_h, B, Hq, Hkv, d, n, G,
                             scale, scores, row_lse, workspace, workspace_bytes, stream);
}

size_t up_block_scores_lse_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d,
                                     int n, int G) {
  ScoreShape s;
  Totals t;
  if (plan_scores(cu_seqlens_h, B, Hq, Hkv, d, n, G, &s, &t) != UP_OK) return 0;
  return score_lse_ws_layout(B, t).total;
}

static int block_scores_lse_common(const void* qwin, const void* k, const PagedK* paged,
                                  const float* row_lse, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d,
                                  int n, int G, float scale, float* scores, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  ScoreShape s;
  Totals t;
  const int st = plan_scores(cu_seqlens_h, B, Hq, Hkv, d, n, G, &s, &t);
  if (st != UP_OK) return st;
  if (B == 0 || t.T == 0) return UP_OK;
  if (!qwin || !k || !row_lse || !cu_seqlens || !scores) return UP_EINVAL;
  if (!aligned(qwin, 16) || !aligned(k, 16) || !aligned(row_lse, 4)) return UP_EINVAL;
  const ScoreLseWs L = score_lse_ws_layout(B, t);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, kWsAlign))
    return UP_EWORKSPACE;
  if (!(scale > 0.f) || std::isinf(scale)) scale = (float)(1.0 / std::sqrt((double)d));
  const float c = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
  int* err = error_word();
  if (!err) return UP_EHIP;
  hipStream_t hs = as_stream(stream);
  hipError_t e;
  e = timed(9, hs, [&] {
    return launch_score_plan(cu_seqlens, s, t, workspace, L.plan, err, hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  PagedK pk;
  if (paged) {
    pk = *paged;
    pk.err = err;
  }
  e = timed(10, hs, [&] {
    return launch_score_partial_lse(qwin, k, row_lse, s, t, workspace, L, c,
                                    paged ? &pk : nullptr, hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(11, hs, [&] { return launch_lse_finalize(s, t, workspace, L, scores, hs); });
  if (e != hipSuccess) return UP_EHIP;
  return UP_OK;
}

int up_block_scores_lse(const void* qwin, const void* k, const float* row_lse,
                        const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B, int Hq,
                        int Hkv, int d, int n, int G, float scale, float* scores,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return block_scores_lse_common(qwin, k, nullptr, row_lse, cu_seqlens, cu_seqlens_h, B, Hq,
                                 Hkv, d, n, G, scale, scores, workspace, workspace_bytes, stream);
}

int up_block_scores_lse_paged(const void* qwin, const void* k_pages, int64_t num_pages,
                              int page_size, const int32_t* block_table, int max_pages,
                              const float* row_lse, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d, int n,
                              int G, float scale, float* scores, void* workspace,
                              size_t workspace_bytes, void* stream) {
  PagedK pk;
  const int st = paged_args(k_pages, num_pages, page_size, block_table, max_pages, cu_seqlens_h,
                            B, &pk);
  if (st != UP_OK) return st;
  return block_scores_lse_common(qwin, k_pages, &pk, row_lse, cu_seqlens, cu_seqlens_h, B, Hq,
                                 Hkv, d, n, G, scale, scores, workspace, workspace_bytes, stream);
}

static int select_common(const float* scores, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_h, int B, int n, int G, int mode, float p,
                         int topk, uint8_t* keep_blocks, int32_t* cu_seqlens_out, void* stream) {
  if (B < 0 || n <= 0 || G <= 0) return UP_EINVAL;
  if (!cu_ok(cu_seqlens_h, B)) return UP_EINVAL;
  if (mode == 0 && !(p > 0.f && p <= 1.f)) return UP_EINVAL;
  if (mode == 1 && topk < 0) return UP_EINVAL;
  if (!cu_seqlens_out) return UP_EINVAL;
  const SelPlan sp = sel_plan(cu_seqlens_h, B, G);
  if (sp.nb_max > kSelectMaxBlocks) return UP_EUNSUPPORTED;
  if (B > 0 && (!cu_seqlens || (sp.nb_tot > 0 && (!scores || !keep_blocks)))) return UP_EINVAL;
  int* err = error_word();
  if (!err) return UP_EHIP;
  hipStream_t hs = as_stream(stream);
  hipError_t e = timed(4, hs, [&] {
    return launch_select(scores, cu_seqlens, B, n, G, mode, p, topk, sp.nb_max, sp.T, sp.nb_tot,
                         keep_blocks, cu_seqlens_out, err, hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  if (B > 1) e = timed(5, hs, [&] { return launch_select_finalize(cu_seqlens_out, B, hs); });
  return e == hipSuccess ? UP_OK : UP_EHIP;
}

int up_topp_select(const float* scores, const int32_t* cu_seqlens, const int32_t* cu_seqlens_h,
                   int B, int n, int G, float p, uint8_t* keep_blocks, int32_t* cu_seqlens_out,
                   void* stream) {
  return select_common(scores, cu_seqlens, cu_seqlens_h, B, n, G, 0, p, 0, keep_blocks,
                       cu_seqlens_out, stream);
}

int up_topk_select(const float* scores, const int32_t* cu_seqlens, const int32_t* cu_seqlens_h,
                   int B, int n, int G, int topk, uint8_t* keep_blocks, int32_t* cu_seqlens_out,
                   void* stream) {
  return select_common(scores, cu_seqlens, cu_seqlens_h, B, n, G, 1, 1.0f, topk, keep_blocks,
                       cu_seqlens_out, stream);
}

size_t up_expand_compact_workspace(const int32_t* cu_seqlens_h, int B, int G) {
  if (G <= 0 || !cu_ok(cu_seqlens_h, B)) return 0;
  const SelPlan sp = sel_plan(cu_seqlens_h, B, G);
  return compact_ws_layout(sp.nb_tot).total;
}

int up_expand_compact(const void* hidden, int H, int elem_bytes, const int32_t* pos,
                      const uint8_t* keep_blocks, const int32_t* cu_seqlens,
                      const int32_t* cu_seqlens_out, const int32_t* cu_seqlens_h, int B, int G,
                      int32_t* idx_out, void* hidden_out, int32_t* pos_out,
                      const int32_t* prev_orig, int32_t* orig_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (B < 0 || G <= 0 || H <= 0 || elem_bytes <= 0) return UP_EINVAL;
  if (!cu_ok(cu_seqlens_h, B)) return UP_EINVAL;
  const SelPlan sp = sel_plan(cu_seqlens_h, B, G);
  if (B == 0 || sp.T == 0) return UP_OK;
  if (!hidden || !keep_blocks || !cu_seqlens || !cu_seqlens_out || !idx_out || !hidden_out)
    return UP_EINVAL;
  if (pos_out && !pos) return UP_EINVAL;
  if (orig_out && !prev_orig) return UP_EINVAL;
  const int64_t row_bytes = (int64_t)H * elem_bytes;
  if (sp.T * row_bytes / row_bytes != sp.T) return UP_EUNSUPPORTED;
  const CompactWs L = compact_ws_layout(sp.nb_tot);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, kWsAlign))
    return UP_EWORKSPACE;
  int* err = error_word();
  if (!err) return UP_EHIP;
  hipStream_t hs = as_stream(stream);
  hipError_t e = timed(6, hs, [&] {
    return launch_block_dst(keep_blocks, cu_seqlens, cu_seqlens_out, B, G, sp.T, sp.nb_tot,
                            workspace, L, err, hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(7, hs, [&] {
    return launch_gather(hidden, row_bytes, pos, workspace, L, sp.nb_tot, G, sp.T, idx_out,
                         hidden_out, pos_out, prev_orig, orig_out, err, hs);
  });
  return e == hipSuccess ? UP_OK : UP_EHIP;
}

int up_expand_compact_noalloc(const void* hidden, int H, int elem_bytes, const int32_t* pos,
                              const uint8_t* keep_blocks, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_out, const int32_t* cu_seqlens_h,
                              int B, int G, int32_t* idx_out, void* hidden_out,
                              int32_t* pos_out, const int32_t* prev_orig, int32_t* orig_out,
                              void* stream) {
  if (B < 0 || G <= 0 || H <= 0 || elem_bytes <= 0) return UP_EINVAL;
  if (!cu_ok(cu_seqlens_h, B)) return UP_EINVAL;
  const SelPlan sp = sel_plan(cu_seqlens_h, B, G);
  if (sp.nb_tot > kStaticCompactBlocks) return UP_EUNSUPPORTED;
  if (B == 0 || sp.T == 0) return UP_OK;
  if (!hidden || !keep_blocks || !cu_seqlens || !cu_seqlens_out || !idx_out || !hidden_out)
    return UP_EINVAL;
  if (pos_out && !pos) return UP_EINVAL;
  if (orig_out && !prev_orig) return UP_EINVAL;
  const int64_t row_bytes = (int64_t)H * elem_bytes;
  if (sp.T * row_bytes / row_bytes != sp.T) return UP_EUNSUPPORTED;
  const CompactWs L = compact_ws_layout(sp.nb_tot);
  size_t cap = 0;
  void* ws = static_compact_scratch(&cap);
  if (!ws) return UP_EHIP;
  if (L.total > cap) return UP_EUNSUPPORTED;
  int* err = error_word();
  if (!err) return UP_EHIP;
  // Launched directly (no per-kernel timing: its events would be allocations).
  hipStream_t hs = as_stream(stream);
  hipError_t e = launch_block_dst(keep_blocks, cu_seqlens, cu_seqlens_out, B, G, sp.T, sp.nb_tot,
                                  ws, L, err, hs);
  if (e != hipSuccess) return UP_EHIP;
  e = launch_gather(hidden, row_bytes, pos, ws, L, sp.nb_tot, G, sp.T, idx_out, hidden_out,
                    pos_out, prev_orig, orig_out, err, hs);
  return e == hipSuccess ? UP_OK : UP_EHIP;
}

int up_compose_drops(const int32_t* prev_orig, int prev_len, const int32_t* idx,
                     const int32_t* count, int capacity, int32_t* orig_out, void* stream) {
  if (capacity < 0 || prev_len < 0) return UP_EINVAL;
  if (capacity == 0) return UP_OK;
  if (!idx || !count || !orig_out || (prev_len > 0 && !prev_orig)) return UP_EINVAL;
  int* err = error_word();
  if (!err) return UP_EHIP;
  hipStream_t hs = as_stream(stream);
  hipError_t e = timed(8, hs, [&] {
    return launch_compose(prev_orig, prev_len, idx, count, capacity, orig_out, err, hs);
  });
  return e == hipSuccess ? UP_OK : UP_EHIP;
}

// ---- the whole decision in one call ---------------------------------------------

size_t up_layer_decision_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d,
                                   int n, int G) {
  ScoreShape s;
  Totals t;
  if (plan_scores(cu_seqlens_h, B, Hq, Hkv, d, n, G, &s, &t) != UP_OK) return 0;
  const SelPlan sp = sel_plan(cu_seqlens_h, B, G);
  return score_ws_layout(B, t).total + compact_ws_layout(sp.nb_tot).total +
         align_up((size_t)sp.nb_tot * sizeof(int32_t));
}

int up_layer_decision(const void* qwin, const void* k, const int32_t* cu_seqlens,
                      const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d, int n, int G,
                      float scale, float p, const void* hidden, int H, int elem_bytes,
                      const int32_t* pos, const int32_t* prev_orig, float* scores,
                      uint8_t* keep_blocks, int32_t* cu_seqlens_out, int32_t* idx_out,
                      void* hidden_out, int32_t* pos_out, int32_t* orig_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  ScoreShape s;
  Totals t;
  int st = plan_scores(cu_seqlens_h, B, Hq, Hkv, d, n, G, &s, &t);
  if (st != UP_OK) return st;
  if (!(p > 0.f && p <= 1.f) || H <= 0 || elem_bytes <= 0) return UP_EINVAL;
  const SelPlan sp = sel_plan(cu_seqlens_h, B, G);
  if (sp.nb_max > kSelectMaxBlocks) return UP_EUNSUPPORTED;
  if (B == 0) return UP_OK;
  const ScoreWs LS = score_ws_layout(B, t);
  const CompactWs LC = compact_ws_layout(sp.nb_tot);
  // After the score and compaction workspaces: the fused select's per-block request index.
  const size_t rq_bytes = align_up((size_t)sp.nb_tot * sizeof(int32_t));
  if (!workspace || workspace_bytes < LS.total + LC.total + rq_bytes ||
      !aligned(workspace, kWsAlign))
    return UP_EWORKSPACE;
  // With every request empty (T = 0) only cu_seqlens and cu_seqlens_out hold data; the
  // other buffers have no elements and may be NULL, as in the separate calls.
  if (!cu_seqlens || !cu_seqlens_out) return UP_EINVAL;
  if (t.T > 0 && (!qwin || !k || !scores || !keep_blocks || !hidden || !idx_out || !hidden_out))
    return UP_EINVAL;
  if ((pos_out && !pos) || (orig_out && !prev_orig)) return UP_EINVAL;
  const int64_t row_bytes = (int64_t)H * elem_bytes;
  if (sp.T > 0 && sp.T * row_bytes / row_bytes != sp.T) return UP_EUNSUPPORTED;
  char* cws = static_cast<char*>(workspace) + LS.total;
  // Requests of at most 4096 blocks each have their normalisation and block
  // destinations done inside the select kernel (kFusedSelect; several requests also take
  // the fused finalize): the score pass stops at the float64 masses and the normalise
  // and block-destination launches are not needed.
  if (!kFusedSelect || t.T == 0 || sp.nb_max > kFusedSelectMaxBlocks) {
    st = block_scores_common(qwin, k, nullptr, cu_seqlens, cu_seqlens_h, B, Hq, Hkv, d, n, G,
                             scale, scores, nullptr, workspace, LS.total, stream);
    if (st != UP_OK) return st;
    st = select_common(scores, cu_seqlens, cu_seqlens_h, B, n, G, 0, p, 0, keep_blocks,
                       cu_seqlens_out, stream);
    if (st != UP_OK) return st;
    return up_expand_compact(hidden, H, elem_bytes, pos, keep_blocks, cu_seqlens, cu_seqlens_out,
                             cu_seqlens_h, B, G, idx_out, hidden_out, pos_out, prev_orig,
                             orig_out, cws, LC.total, stream);
  }
  st = block_scores_common(qwin, k, nullptr, cu_seqlens, cu_seqlens_h, B, Hq, Hkv, d, n, G, scale,
                           nullptr, nullptr, workspace, LS.total, stream, /*stop_at_mass=*/true);
  if (st != UP_OK) return st;
  int* err = error_word();
  if (!err) return UP_EHIP;
  hipStream_t hs = as_stream(stream);
  FusedDecision fd;
  fd.mass = reinterpret_cast<const double*>(static_cast<char*>(workspace) + LS.mass);
  fd.splan = reinterpret_cast<const ReqPlan*>(static_cast<char*>(workspace) + LS.plan);
  fd.rq = reinterpret_cast<int32_t*>(cws + LC.total);
  fd.scores = scores;
  fd.shdr = static_cast<const WsHeader*>(workspace);
  fd.chdr = reinterpret_cast<WsHeader*>(cws + LC.hdr);
  fd.dst = reinterpret_cast<int32_t*>(cws + LC.dst);
  fd.src = reinterpret_cast<int32_t*>(cws + LC.src);
  fd.len = reinterpret_cast<int32_t*>(cws + LC.len);
  hipError_t e = timed(17, hs, [&] {
    return launch_select_fused(cu_seqlens, B, n, G, p, sp.nb_max, sp.T, sp.nb_tot, keep_blocks,
                               cu_seqlens_out, err, fd, hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(7, hs, [&] {
    return launch_gather(hidden, row_bytes, pos, cws, LC, sp.nb_tot, G, sp.T, idx_out,
                         hidden_out, pos_out, prev_orig, orig_out, err, hs);
  });
  return e == hipSuccess ? UP_OK : UP_EHIP;
}

// ---- layer on the surviving tokens --------------------------------------------

namespace {
// Shape of an attention call; returns UP_OK or an error status.
int plan_attention(const int32_t* cu_h, int B, int Hq, int Hkv, int d, AttnShape* s,
                   int n = 0) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0 || n < 0) return UP_EINVAL;
  if (!cu_ok(cu_h, B)) return UP_EINVAL;
  if (d != 64 && d != 128 && d != 256) return UP_EUNSUPPORTED;
  const int gsz = Hq / Hkv;
  s->B = B; s->Hq = Hq; s->Hkv = Hkv; s->d = d;
  s->HQ = gsz % 4 == 0 ? 4 : (gsz % 2 == 0 ? 2 : 1);
  s->TT = 4 / s->HQ;
  const int tok_tile = attn_tile_tokens(d, Hkv) * s->TT;
  int64_t Rp = 0, tiles = 0, wtiles = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t L = (int64_t)cu_h[i + 1] - cu_h[i];
    const int64_t nt = (L + tok_tile - 1) / tok_tile;
    Rp += (L + 63) / 64 * 64;
    tiles += nt;
    if (n > 0 && L > 0) wtiles += nt - (L - std::min<int64_t>(L, n)) / tok_tile;
  }
  s->n = n;
  s->wtiles = wtiles;
  s->R = B > 0 ? cu_h[B] : 0;
  s->Rp = Rp;
  s->tiles = tiles;
  if (Rp > INT32_MAX || tiles > 65535) return UP_EUNSUPPORTED;
  if ((int64_t)Hkv * (gsz / s->HQ) > 65535) return UP_EUNSUPPORTED;
  return UP_OK;
}

}  // namespace

size_t up_rope_attention_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d) {
  AttnShape s;
  if (plan_attention(cu_seqlens_h, B, Hq, Hkv, d, &s) != UP_OK) return 0;
  return attn_ws_layout(B, Hq, Hkv, d, s.Rp).total;
}

int up_rope_attention(const void* q, const void* k, const void* v, const int32_t* pos,
                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B, int Hq,
                      int Hkv, int d, float scale, float rope_theta, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  AttnShape s;
  const int st = plan_attention(cu_seqlens_h, B, Hq, Hkv, d, &s);
  if (st != UP_OK) return st;
  if (!(rope_theta > 1.f) || std::isinf(rope_theta)) return UP_EINVAL;
  if (B == 0 || s.R == 0) return UP_OK;
  if (!q || !k || !v || !pos || !cu_seqlens || !out) return UP_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return UP_EINVAL;
  const AttnWs L = attn_ws_layout(B, Hq, Hkv, d, s.Rp);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, kWsAlign))
    return UP_EWORKSPACE;
  if (!(scale > 0.f) || std::isinf(scale)) scale = (float)(1.0 / std::sqrt((double)d));
  const float c = (float)((double)scale * 1.4426950408889634);
  int* err = error_word();
  if (!err) return UP_EHIP;
  hipStream_t hs = as_stream(stream);
  hipError_t e = timed(12, hs, [&] { return launch_attn_plan(cu_seqlens, s, workspace, L, err, hs); });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(13, hs, [&] {
    return launch_rope_layout(q, k, v, pos, cu_seqlens, s, workspace, L,
                              std::log2((double)rope_theta), hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(14, hs, [&] { return launch_attention(cu_seqlens, s, workspace, L, c, out, hs); });
  return e == hipSuccess ? UP_OK : UP_EHIP;
}

// A second stream per device for the statistics launch of up_rope_attention_scores,
// forked from and joined back into the caller's stream with events; created at the
// first such call on the device and kept until the process ends.  The fork and join
// are enqueued under a lock, so calls from several host threads stay ordered.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];

SideStream* side_stream_locked() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    hipStream_t s = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess) {
      if (a) (void)hipEventDestroy(a);
      (void)hipStreamDestroy(s);
      return nullptr;
    }
    ss.s = s;
    ss.fork = a;
    ss.join = b;
  }
  return &ss;
}

size_t up_rope_attention_scores_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv,
                                          int d, int n, int G) {
  AttnShape a;
  ScoreShape s;
  Totals t;
  if (plan_attention(cu_seqlens_h, B, Hq, Hkv, d, &a, n) != UP_OK) return 0;
  if (plan_scores(cu_seqlens_h, B, Hq, Hkv, d, n, G, &s, &t) != UP_OK) return 0;
  return align_up(attn_ws_layout(B, Hq, Hkv, d, a.Rp).total) + score_ws_layout(B, t).total;
}

int up_rope_attention_scores(const void* q, const void* k, const void* v, const int32_t* pos,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B,
                             int Hq, int Hkv, int d, float scale, float rope_theta, int n, int G,
                             void* out, float* scores, float* row_lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  AttnShape a;
  int st = plan_attention(cu_seqlens_h, B, Hq, Hkv, d, &a, n);
  if (st != UP_OK) return st;
  ScoreShape s;
  Totals t;
  st = plan_scores(cu_seqlens_h, B, Hq, Hkv, d, n, G, &s, &t);
  if (st != UP_OK) return st;
  if (!(rope_theta > 1.f) || std::isinf(rope_theta)) return UP_EINVAL;
  if (B == 0 || a.R == 0) return UP_OK;
  if (!q || !k || !v || !pos || !cu_seqlens || !out || !scores) return UP_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(scores, 4) || (row_lse && !aligned(row_lse, 4)))
    return UP_EINVAL;
  const AttnWs LA = attn_ws_layout(B, Hq, Hkv, d, a.Rp);
  const size_t soff = align_up(LA.total);
  const ScoreWs LS = score_ws_layout(B, t);
  if (!workspace || workspace_bytes < soff + LS.total || !aligned(workspace, kWsAlign))
    return UP_EWORKSPACE;
  if (!(scale > 0.f) || std::isinf(scale)) scale = (float)(1.0 / std::sqrt((double)d));
  const float c = (float)((double)scale * 1.4426950408889634);
  int* err = error_word();
  if (!err) return UP_EHIP;
  hipStream_t hs = as_stream(stream);
  char* sws = static_cast<char*>(workspace) + soff;
  hipError_t e = timed(9, hs, [&] {
    return launch_score_plan(cu_seqlens, s, t, sws, LS.plan, err, hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(12, hs, [&] { return launch_attn_plan(cu_seqlens, a, workspace, LA, err, hs); });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(13, hs, [&] {
    return launch_rope_layout(q, k, v, pos, cu_seqlens, a, workspace, LA,
                              std::log2((double)rope_theta), hs);
  });
  if (e != hipSuccess) return UP_EHIP;
  const AttnScoreOut so{reinterpret_cast<WsHeader*>(sws),
                        reinterpret_cast<const ReqPlan*>(sws + LS.plan),
                        reinterpret_cast<float2*>(sws + LS.ml),
                        reinterpret_cast<float2*>(sws + LS.rs), row_lse, G};
  // The tiles that hold window rows run the attention with block statistics on a second
  // stream, beside the plain attention over the other tiles on the caller's stream.
  {
    std::lock_guard<std::mutex> lk(g_side_mu);
    SideStream* ss = side_stream_locked();
    if (!ss) return UP_EHIP;
    if (hipEventRecord(ss->fork, hs) != hipSuccess ||
        hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
      return UP_EHIP;
    // From here the second stream may hold work of this call: whatever fails below, the
    // caller's stream is joined to it before returning, so no kernel of a failed call
    // can still be reading the caller's buffers once the error is reported.
    e = timed(18, ss->s, [&] {
      return launch_attention(cu_seqlens, a, workspace, LA, c, out, ss->s, &so,
                              attn::kSlotsWindow);
    });
    if (e == hipSuccess)
      e = timed(14, hs, [&] {
        return launch_attention(cu_seqlens, a, workspace, LA, c, out, hs, nullptr,
                                attn::kSlotsRest);
      });
    if (hipEventRecord(ss->join, ss->s) != hipSuccess ||
        hipStreamWaitEvent(hs, ss->join, 0) != hipSuccess) {
      (void)hipStreamSynchronize(ss->s);   // no join could be enqueued: drain it instead
      return UP_EHIP;
    }
    if (e != hipSuccess) return UP_EHIP;
  }
  e = timed(2, hs, [&] { return launch_block_mass_pairs(s, t, sws, LS, hs); });
  if (e != hipSuccess) return UP_EHIP;
  e = timed(3, hs, [&] { return launch_normalize(s, t, sws, LS, scores, hs); });
  return e == hipSuccess ? UP_OK : UP_EHIP;
}

int up_swiglu(const void* gu, int64_t R, int F, void* a, void* stream) {
  if (R < 0 || F <= 0) return UP_EINVAL;
  if (F % 8 != 0) return UP_EUNSUPPORTED;
  if (R == 0) return UP_OK;
  if (!gu || !a || !aligned(gu, 16) || !aligned(a, 16)) return UP_EINVAL;
  hipStream_t hs = as_stream(stream);
  const hipError_t e = timed(15, hs, [&] { return launch_swiglu(gu, R, F, a, hs); });
  return e == hipSuccess ? UP_OK : UP_EHIP;
}

int up_device_error(int32_t* code_h, void* stream) {
  if (!code_h) return UP_EINVAL;
  int* err = error_word();
  if (!err) return UP_EHIP;
  hipStream_t hs = as_stream(stream);
  if (hipStreamSynchronize(hs) != hipSuccess) return UP_EHIP;
  if (hipMemcpy(code_h, err, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return UP_EHIP;
  hipLaunchKernelGGL(up_clear_word_kernel, dim3(1), dim3(1), 0, hs, err);
  if (hipGetLastError() != hipSuccess) return UP_EHIP;
  if (hipStreamSynchronize(hs) != hipSuccess) return UP_EHIP;
  return UP_OK;
}

int up_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_prof = on != 0;
  return UP_OK;
}

int up_profile_read(int which, int* launches_h, double* total_ms_h) {
  if (!launches_h || !total_ms_h) return UP_EINVAL;
  std::lock_guard<std::mutex> lk(g_mu);
  int cnt = 0;
  double tot = 0.0;
  for (const Rec& r : g_recs) {
    if (r.which != which) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return UP_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return UP_EHIP;
    tot += ms;
    ++cnt;
  }
  *launches_h = cnt;
  *total_ms_h = tot;
  return UP_OK;
}

int up_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (const Rec& r : g_recs) {
    (void)hipEventSynchronize(r.b);
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return UP_OK;
}

}  // extern "C"
