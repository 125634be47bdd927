// Internal declarations shared by the HIP translation units of libuniprefill.
// Not part of the public ABI (include/uniprefill.h is).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_geom.h"
#include <stddef.h>
#include <stdint.h>

namespace up {

constexpr size_t kWsAlign = 256;

inline size_t align_up(size_t x, size_t a = kWsAlign) { return (x + a - 1) / a * a; }

// Per-request plan of the score pass.  Built on the host from cu_seqlens_h (to size
// grids and workspaces) and rebuilt on the device from cu_seqlens by the plan
// kernel, which checks the two agree before any other kernel touches memory.
struct ReqPlan {
  int32_t tok_off;   // first token of the request in the packed batch
  int32_t L;         // length
  int32_t W;         // window rows: min(n, L)
  int32_t win_off;   // first window row of the request in qwin
  int32_t blk_off;   // first global block
  int32_t nb;        // blocks: ceil(L / G)
  int32_t nch;       // statistics chunks: ceil(nb / cbs)
  int32_t item_end;  // exclusive end of the request's work items of the score kernel
  int32_t cbs;       // blocks per statistics chunk (a function of this request alone)
  int32_t cps;       // statistics chunks per work item (load balance only)
  int64_t ml_off;    // first (m, l) pair of the request: pairs are [nb][Hkv][R], R = gs * W
  int64_t cs_off;    // first chunk-statistics pair: [nch][Hkv][R]
  int64_t pm_off;    // first block partial of the given-lse pass: [Hkv * nrt][nb]
};

// Largest work item (blocks per workgroup) of the score kernel.
constexpr int kMaxChunkBlocks = 256;

// Statistics chunks.  The score kernel restarts each query's softmax reference at
// the first key of every statistics chunk and stores one merged pair per (row,
// chunk); the row statistics merge the chunks in chunk order.  So a request's scores
// depend on how its keys are cut into chunks, and that cut is made from the request
// alone -- its block count and the call's per-chunk work (kv heads x row tiles) --
// never from the other requests of a batch or from the device: the same request gets
// bit-identical scores alone, packed with others, or on another GPU.  The cut is the
// one a lone request would take to fill kStatCus compute units in one round: with
// per = items per chunk position, floor(kStatCus / per) chunks, each ceil(nb / that)
// blocks (1 to kMaxChunkBlocks).  More rounds would only add a workgroup's fixed cost
// per round.  Work items (one workgroup each) are whole runs of statistics chunks,
// sized by the planner for load balance; that choice moves work between workgroups
// but never changes a result.
constexpr int kStatCus = 256;
constexpr int kChunkOverheadBlocks = 3;   // a workgroup's fixed cost, in blocks of work

// nb < 2^31 (the host refuses larger requests): 32-bit divisions.
__host__ __device__ inline int stat_chunk_blocks(int64_t nb, int64_t items_per_chunk) {
  const uint32_t slots = items_per_chunk >= kStatCus || items_per_chunk <= 0
                             ? 1u : (uint32_t)kStatCus / (uint32_t)items_per_chunk;
  uint32_t cb = nb > 0 ? ((uint32_t)nb - 1u) / slots + 1u : 1u;
  if (cb > (uint32_t)kMaxChunkBlocks) cb = kMaxChunkBlocks;
  return (int)cb;
}

// Statistics chunks per work item for a target item length of tb blocks: at least
// one, at most the request's chunks, and no item longer than kMaxChunkBlocks.
__host__ __device__ inline int chunks_per_item(int cbs, int64_t nch, int tb) {
  int c = tb / cbs;
  const int cmax = kMaxChunkBlocks / cbs;   // cbs <= kMaxChunkBlocks, so cmax >= 1
  if (c > cmax) c = cmax;
  if (c > nch) c = (int)nch;
  return c < 1 ? 1 : c;
}

// Launch shape of the score kernel per head dimension: query rows per workgroup
// (waves x 32-row tiles per wave x 32) and workgroups resident per CU.  One 8-wave
// workgroup per CU reads each key chunk once.  (Two 4-wave workgroups per CU, whose
// barriers are independent, measured no faster at 128K tokens and read K twice.)
constexpr int score_rows_wg(int d) { return d == 256 ? 8 * 1 * 32 : 8 * 2 * 32; }
constexpr int score_wgs_per_cu(int) { return 1; }

// Shape of the score pass, fixed by the host for one call.
struct ScoreShape {
  int B, Hq, Hkv, d, n, G;
  int TB;        // target work-item length in blocks (chunks_per_item)
  int qt;        // 32-query column tiles per wave (1 or 2)
  int kt;        // 32-key row tiles per LDS stage (1 or 2)
  int rows_wg;   // query rows per workgroup: score_rows_wg(d)
};

struct Totals {
  int64_t T;         // tokens
  int64_t win_rows;  // sum of W_i
  int64_t rows;      // window rows over all query heads: Hq * win_rows
  int64_t nb_tot;    // blocks
  int64_t items;     // score work items (workgroups)
  int64_t ml_pairs;  // (m, l) pairs
  int64_t cs_pairs;  // chunk-statistics pairs
  int64_t pm_parts;  // block partials of the given-lse pass
  int32_t nb_max;    // largest per-request block count
};

// Workspace header written by the plan kernel (first 256 bytes of a workspace).
struct WsHeader {
  int32_t valid;     // 1 when the device plan matches the host totals
  int32_t pad[63];
};

// Score-pass workspace layout (offsets in bytes from the workspace base).
// ml: per (row, block) float32 block sums, then as many float32 references (mref) of
// blocks that ended before a mid-chunk rebase -- or, for the attention's fused form,
// (reference, sum) pairs; cs: per (row, chunk) statistics; crb: per (row, chunk) the
// first block under the chunk's final reference; wt: per (row, chunk) weight of the
// chunk's block sums in the block masses; rs: per row (max, 1 / sum); mass: per block.
struct ScoreWs {
  size_t plan, ml, cs, crb, wt, rs, mass, total;
};

ScoreWs score_ws_layout(int B, const Totals& t);

// Workspace of the given-lse score pass: plan and float block partials only.
struct ScoreLseWs {
  size_t plan, pm, total;
};

ScoreLseWs score_lse_ws_layout(int B, const Totals& t);

// Launchers (score.hip).  Each returns the hipError_t of its launch.
hipError_t launch_score_plan(const int32_t* cu, const ScoreShape& s, const Totals& t,
                             void* ws, size_t plan_off, int* err, hipStream_t st);
// Paged key cache: k = [num_pages][2^log2_page][Hkv][d], table = int32 [B][max_pages].
struct PagedK {
  const int32_t* table = nullptr;
  int max_pages = 0;
  int log2_page = 0;
  int64_t num_pages = 0;
  int* err = nullptr;
};

// paged == nullptr: contiguous k = [T][Hkv][d].
hipError_t launch_score_partial(const void* qwin, const void* k, const ScoreShape& s,
                                const Totals& t, void* ws, const ScoreWs& L, float c_log2,
                                const PagedK* paged, hipStream_t st);
// Row statistics (and each (row, chunk)'s weight) from the score kernel's chunk
// statistics (row_lse: optional natural-log log-sum-exp per window row).
hipError_t launch_row_stats(const ScoreShape& s, const Totals& t, void* ws, const ScoreWs& L,
                            float* row_lse, hipStream_t st);
// The given-lse pass: row_lse [sum W_i, Hq] natural-log log-sum-exp of each window row;
// paged == nullptr: contiguous k, as for launch_score_partial.
hipError_t launch_score_partial_lse(const void* qwin, const void* k, const float* row_lse,
                                    const ScoreShape& s, const Totals& t, void* ws,
                                    const ScoreLseWs& L, float c, const PagedK* paged,
                                    hipStream_t st);
hipError_t launch_lse_finalize(const ScoreShape& s, const Totals& t, void* ws,
                               const ScoreLseWs& L, float* scores, hipStream_t st);
// Block masses of the score pass (block sums and chunk weights) ...
hipError_t launch_block_mass(const ScoreShape& s, const Totals& t, void* ws, const ScoreWs& L,
                             hipStream_t st);
// ... and of the attention's fused form ((reference, sum) pairs and row statistics).
hipError_t launch_block_mass_pairs(const ScoreShape& s, const Totals& t, void* ws,
                                   const ScoreWs& L, hipStream_t st);
hipError_t launch_normalize(const ScoreShape& s, const Totals& t, void* ws, const ScoreWs& L,
                            float* scores, hipStream_t st);

// Selection (select.hip).  mode 0: Top-p with threshold p; mode 1: Top-k with k = topk.
constexpr int kSelectMaxBlocks = 16384;
hipError_t launch_select(const float* scores, const int32_t* cu, int B, int n, int G, int mode,
                         float p, int topk, int nb_max, int64_t T_host, int64_t nb_tot_host,
                         uint8_t* keep, int32_t* cu_out, int* err, hipStream_t st);
hipError_t launch_select_finalize(int32_t* cu_out, int B, hipStream_t st);
// The fused form of select for requests of at most 4096 blocks: masses in, normalised
// scores, keep flags, cu_out and the compaction's block destinations out.  One request:
// the select kernel writes everything, absolute destinations and the compaction
// header included.  Several: each request's workgroup writes its kept count to
// cu_out[i + 1] (-1 if its checks failed), destinations relative to the request's first
// output row and the request index of each block; the fused finalize kernel then scans
// the counts, makes the destinations absolute and writes the header.
struct FusedDecision {
  const double* mass = nullptr;    // float64 block masses of the score pass
  float* scores = nullptr;         // normalised scores (output)
  const WsHeader* shdr = nullptr;  // score workspace header
  const ReqPlan* splan = nullptr;  // score pass plan (several requests)
  WsHeader* chdr = nullptr;        // compaction workspace header (written)
  int32_t* dst = nullptr;          // per block: destination row or -1
  int32_t* src = nullptr;          // per block: first source row
  int32_t* len = nullptr;          // per block: rows
  int32_t* rq = nullptr;           // per block: its request (several requests)
};
constexpr int kFusedSelectMaxBlocks = 4096;
// Whether up_layer_decision uses the fused select when no request has more than
// kFusedSelectMaxBlocks blocks.
constexpr bool kFusedSelect = true;
hipError_t launch_select_fused(const int32_t* cu, int B, int n, int G, float p, int nb_max,
                               int64_t T_host, int64_t nb_tot_host, uint8_t* keep,
                               int32_t* cu_out, int* err, const FusedDecision& fd,
                               hipStream_t st);

// Expand + compact (compact.hip).
struct CompactWs {
  size_t hdr, dst, src, len, total;
};
CompactWs compact_ws_layout(int64_t nb_tot);
// The run table of up_expand_compact_noalloc: the current device's address of the
// library's device array (looked up once per device), or null; *bytes = its size.
constexpr int64_t kStaticCompactBlocks = 65536;
void* static_compact_scratch(size_t* bytes);
hipError_t launch_block_dst(const uint8_t* keep, const int32_t* cu, const int32_t* cu_out, int B,
                            int G, int64_t T_host, int64_t nb_tot_host, void* ws,
                            const CompactWs& L, int* err, hipStream_t st);
// T: rows of hidden and the capacity of every output (a run outside is refused, error
// bit 16).
hipError_t launch_gather(const void* hidden, int64_t row_bytes, const int32_t* pos, void* ws,
                         const CompactWs& L, int64_t nb_tot, int G, int64_t T, int32_t* idx_out,
                         void* hidden_out, int32_t* pos_out, const int32_t* prev_orig,
                         int32_t* orig_out, int* err, hipStream_t st);
hipError_t launch_compose(const int32_t* prev, int prev_len, const int32_t* idx,
                          const int32_t* count, int capacity, int32_t* out, int* err,
                          hipStream_t st);

// Layer on the surviving tokens (consumer.hip).
// The 8-wave attention kernel (64-token tiles per query-head pair) serves d = 64 and
// 128 up to attn::kMaxKvHeads kv heads; the 4-wave kernel (32-token tiles) the rest.
constexpr int kMaxAttnKvHeads = attn::kMaxKvHeads;
constexpr bool attn_w8(int d, int Hkv) { return attn::w8_serves(d, Hkv); }
constexpr int attn_tile_tokens(int d, int Hkv) { return attn_w8(d, Hkv) ? 64 : 32; }
struct AttnShape {
  int B, Hq, Hkv, d;
  int HQ, TT;       // query heads and per-head token tiles per attention workgroup (HQ * TT = 4)
  int64_t R, Rp;    // rows; padded rows (every request rounded up to 64)
  int64_t tiles;    // attention workgroup tiles of attn_tile_tokens(d, Hkv) * TT tokens
  int n;            // window rows whose block statistics are kept (0: none)
  int64_t wtiles;   // workgroup tiles holding window rows (0 when n = 0)
};
struct AttnWs {
  size_t hdr, po, tp, wp, qr, kr, vt, kn, total;   // kn: 8-wave kernel only (else empty)
};
AttnWs attn_ws_layout(int B, int Hq, int Hkv, int d, int64_t Rp);
hipError_t launch_attn_plan(const int32_t* cu, const AttnShape& s, void* ws, const AttnWs& L,
                            int* err, hipStream_t st);
hipError_t launch_rope_layout(const void* q, const void* k, const void* v, const int32_t* pos,
                              const int32_t* cu, const AttnShape& s, void* ws, const AttnWs& L,
                              double log2_theta, hipStream_t st);
// Block statistics of the window rows, written by the attention kernel when given
// (the fused form of the block scores): per request the same (reference, block sum)
// pairs [nb][Hkv][gs * W] and row statistics (row max, 1 / row sum) [W][Hq] that the
// score pass leaves in its workspace, so the block masses and the normalisation run
// on them unchanged.  hdr and plan are the score pass's plan.
struct AttnScoreOut {
  WsHeader* hdr;
  const ReqPlan* plan;
  float2* ml;
  float2* rs;
  float* row_lse;   // optional: natural-log log-sum-exp per window row, [sum W][Hq]
  int G;
};
// mode: attn::kSlotsAll, or kSlotsWindow (with so: the statistics kernel over the
// window tiles) and kSlotsRest (the plain kernel over the others).
hipError_t launch_attention(const int32_t* cu, const AttnShape& s, void* ws, const AttnWs& L,
                            float c, void* out, hipStream_t st,
                            const AttnScoreOut* so = nullptr, int mode = attn::kSlotsAll);
hipError_t launch_swiglu(const void* gu, int64_t R, int F, void* a, hipStream_t st);

}  // namespace up
