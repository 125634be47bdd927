/*
 * uniprefill.h -- C ABI of the block-wise token-dropping hot path (MI355X / gfx950).
 *
 * One full-attention layer decision, as described by the UniPrefill pages:
 *   1. up_block_scores   : per-block importance from the last n window queries
 *   2. up_topp_select    : Top-p cut over the sorted block scores
 *   3. up_expand_compact : kept blocks -> token indices; gather hidden rows and positions
 *   4. up_compose_drops  : map survivors back to original indices across layers
 * and the layer that then runs on the survivors (5: up_rope_attention, up_swiglu;
 * its GEMMs up_linear and up_swiglu_ffn are in libuniprefill_layer.so).
 *
 * Pages cited (by title and paragraph / section):
 *   [UP]  "UniPrefill: 블록 단위 동적 희소화를 통한 범용적 롱 컨텍스트 프리필 가속화"
 *         (AI Trends article on UniPrefill)
 *   [UPA] "UniPrefill: Universal Long-Context Prefill Acceleration via Block-wise
 *         Dynamic Sparsification" (ChatPaper abstract page)
 *   [CP]  "Chunked Prefill" (Ultralytics glossary)
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless their name ends in _h (host memory).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream), never synchronises, never allocates device memory, and returns an
 *    up_status (0 = UP_OK, negative = error).  Arguments are validated on the
 *    host before anything is launched; on error nothing is launched.
 *  - The caller owns every buffer.  Outputs are sized for the worst case
 *    (everything kept); the number of valid rows lives on the device, in
 *    cu_seqlens_out[B].
 *  - Batches are packed ("varlen", [UPA]: the operator serves continuous
 *    batching): request i owns tokens [cu_seqlens[i], cu_seqlens[i+1]) and its
 *    length is L_i.  cu_seqlens_h must hold the same values as the device
 *    cu_seqlens; it is used to size grids and workspaces.  A kernel that finds
 *    the device copy inconsistent with the host-derived totals does nothing and
 *    raises the device error word (up_device_error).
 *  - Request i has W_i = min(n, L_i) window queries and nb_i = ceil(L_i / G)
 *    blocks of G tokens counted from its token 0 (the last may be partial).
 *    Blocks are numbered globally: request i's blocks start at sum_{i'<i} nb_i'.
 *  - Results are bitwise reproducible run to run: no floating-point atomics,
 *    every reduction has a fixed order.
 *  - Thread safety: calls on different streams may overlap as long as their
 *    buffers and workspaces are distinct.
 */
#ifndef UNIPREFILL_H
#define UNIPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  UP_OK = 0,
  UP_EINVAL = -1,        /* bad argument (null pointer, bad size, bad cu_seqlens_h, p out of range) */
  UP_EUNSUPPORTED = -2,  /* valid but not implemented (head dim, block size, too many blocks) */
  UP_EWORKSPACE = -3,    /* workspace missing, too small or misaligned (needs 256-byte alignment) */
  UP_EHIP = -4           /* a HIP runtime call failed */
} up_status;

/* Human-readable name of a status code (static string). */
const char* up_status_string(int status);

/* ABI version, currently 1. */
int up_abi_version(void);

/* ---------------------------------------------------------------------------
 * 1. Block scores  ([UP] "drop" paragraph: softmax probabilities near zero mark
 *    droppable tokens; [UP] "block-wise estimation" paragraph: blocks of G tokens,
 *    the last n queries, per-block average attention normalised into per-block
 *    importance scores; [UP] "Triton kernels" paragraph: online softmax and block
 *    reduction on the GPU; [CP] causal mask over absolute positions)
 *
 * For request i, window row j (absolute position t = L_i - W_i + j) and query head
 * h, with kv head g = floor(h / (Hq/Hkv)):
 *   P[h, j, k] = softmax over keys k <= t of  scale * <q[j, h], K[k, g]>
 *   mass[b]    = sum_h sum_j sum_{k in block b} P[h, j, k]
 *   scores[b]  = mass[b] / sum_{b'} mass[b']          (scores of a request sum to 1)
 *
 * qwin  : bf16 [sum_i W_i, Hq, d]; request i's last W_i query tokens, in order,
 *         requests in batch order.  Row (w, h) at ((w * Hq) + h) * d.
 * k     : bf16 [T, Hkv, d]; T = cu_seqlens[B].  Key (t, g) at ((t * Hkv) + g) * d.
 * cu_seqlens / cu_seqlens_h : int32 [B+1], cu[0] = 0, non-decreasing.
 * Hq % Hkv == 0.  d in {64, 128, 256}.  G a multiple of 32 in [32, 1024].  n >= 1.
 * Hkv * d < 2^20 (1024 key rows stay below 2 GiB; UP_EUNSUPPORTED otherwise).
 * scale : softmax scale; <= 0 or NaN selects 1/sqrt(d) (as float32).
 * scores: float32 [NB_tot] output, NB_tot = sum_i nb_i.
 * row_lse: float32 [sum_i W_i, Hq] output, or NULL: each window row's natural-log
 *         log-sum-exp of scale * q.k over its causal keys, rows laid out like qwin
 *         (the statistics up_block_scores_lse takes).
 * workspace: device buffer of at least up_block_scores_workspace(...) bytes,
 *         256-byte aligned; its contents on entry are ignored.
 * Precision: bf16 products accumulated in float32 on the matrix cores; softmax and
 * probabilities in float32 (never rounded to bf16); cross-row sums in float64.
 * ------------------------------------------------------------------------- */
size_t up_block_scores_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv,
                                 int d, int n, int G);

int up_block_scores(const void* qwin, const void* k,
                    const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B,
                    int Hq, int Hkv, int d, int n, int G, float scale,
                    float* scores, float* row_lse, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Statistics chunks of the score pass (host only; launches nothing).  The pass
 * restarts each query's softmax reference at the first key of every statistics
 * chunk, so its float32 results depend on where the chunks start.  Request i's chunks
 * are chunk_blocks_h[i] blocks long (its first chunk starts at its block 0), chosen
 * from that request's block count and the call's shape (Hq, Hkv, d, n) alone: a request
 * gets bit-identical scores and row statistics whatever other requests share the
 * batch and whatever GPU runs it ([UPA]: the operator serves continuous batching,
 * where requests are independent).  chunk_blocks_h: host int32 [B], written.
 * Returns UP_OK or the argument error up_block_scores would return. */
int up_block_scores_chunks(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d, int n,
                           int G, int32_t* chunk_blocks_h);

/* Same computation with the keys in a paged cache (the layout of a KV cache that
 * serves continuous batching, [UPA]; chunked prefill reads earlier chunks' keys from
 * it, [CP]):
 * k_pages     : bf16 [num_pages, page_size, Hkv, d]; token t of request i is
 *               k_pages[block_table[i * max_pages + t / page_size], t % page_size].
 * page_size   : a power of two in [16, 1024] (UP_EUNSUPPORTED otherwise).
 * block_table : int32 [B, max_pages]; max_pages >= ceil(L_i / page_size) for every
 *               request (UP_EINVAL otherwise).
 * A page index outside [0, num_pages) reads page 0 instead and raises device error
 * bit 8.  Workspace: up_block_scores_workspace(...).  Other arguments as above. */
int up_block_scores_paged(const void* qwin, const void* k_pages, int64_t num_pages,
                          int page_size, const int32_t* block_table, int max_pages,
                          const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B,
                          int Hq, int Hkv, int d, int n, int G, float scale, float* scores,
                          float* row_lse, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---------------------------------------------------------------------------
 * 1b. Block scores from the layer's own softmax statistics  ([UP] "Triton kernels"
 *     paragraph: the full-attention layer runs an online softmax over these rows,
 *     so each window row's log-sum-exp already exists when the decision is made)
 *
 * Same result as up_block_scores, given each window row's log-sum-exp instead of
 * computing it: the weights exp(scale * q.k - row_lse) are the softmax probabilities
 * directly, so one pass sums them per block (no per-row statistics, no second
 * reduction over rows):
 *   mass[b]   = sum_h sum_j sum_{k in block b, k <= t} exp(scale * q.k - row_lse[j, h])
 *   scores[b] = mass[b] / sum_{b'} mass[b']
 * row_lse : float32 [sum_i W_i, Hq], natural log, window rows laid out like qwin (as
 *           produced by up_block_scores, or kept by the layer's attention forward).
 *           A row_lse far below the true value makes exp overflow; the result is then
 *           meaningless (no fault).
 * Other arguments as up_block_scores; workspace: up_block_scores_lse_workspace(...).
 * ------------------------------------------------------------------------- */
size_t up_block_scores_lse_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv,
                                     int d, int n, int G);

int up_block_scores_lse(const void* qwin, const void* k, const float* row_lse,
                        const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B,
                        int Hq, int Hkv, int d, int n, int G, float scale, float* scores,
                        void* workspace, size_t workspace_bytes, void* stream);

/* The given-lse pass over keys in a paged cache: the last chunk of a chunked prefill
 * scores its window rows against every earlier chunk's keys where the cache holds
 * them, with the log-sum-exp its own attention forward produced ([CP]; [UP] "Triton
 * kernels" paragraph).  k_pages, page_size, block_table, max_pages and num_pages as
 * for up_block_scores_paged (same checks, same device error bit 8); everything else as
 * for up_block_scores_lse, whose workspace size applies. */
int up_block_scores_lse_paged(const void* qwin, const void* k_pages, int64_t num_pages,
                              int page_size, const int32_t* block_table, int max_pages,
                              const float* row_lse, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d,
                              int n, int G, float scale, float* scores, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * 2. Top-p selection  ([UP] "Top-p selection" paragraph: sort blocks by descending
 *    importance and keep them until the cumulative sum reaches p, e.g. 0.99;
 *    [UP] "ablation" paragraph: G = 64, n = 128 are the chosen defaults)
 *
 * Per request: order its blocks by (score descending, block index ascending);
 * keep the shortest prefix whose running sum reaches p (>=).  The running sum of
 * the float32 scores is exact (no rounding; compared with p as float32), so the cut
 * does not depend on summation order.  p == 1 keeps every block; so does a running
 * sum that never reaches p.  The blocks holding window tokens ((b+1)*G > L_i - W_i)
 * are always kept as well.
 *
 * scores        : float32 [NB_tot], each request's scores >= 0 (as produced by 1.).
 * p             : in (0, 1].
 * keep_blocks   : uint8 [NB_tot] output, 1 = kept, 0 = dropped.
 * cu_seqlens_out: int32 [B+1] output, packed offsets of the kept tokens.
 * Limit: nb_i <= 16384 blocks per request (UP_EUNSUPPORTED otherwise).
 * ------------------------------------------------------------------------- */
int up_topp_select(const float* scores, const int32_t* cu_seqlens,
                   const int32_t* cu_seqlens_h, int B, int n, int G, float p,
                   uint8_t* keep_blocks, int32_t* cu_seqlens_out, void* stream);

/* Same cut with a fixed number of blocks per request instead of a mass threshold:
 * keep the top `topk` blocks (all if nb_i <= topk) plus the window blocks.
 * ([UP] "ablation" paragraph compares Top-p against this fixed-count Top-k.) */
int up_topk_select(const float* scores, const int32_t* cu_seqlens,
                   const int32_t* cu_seqlens_h, int B, int n, int G, int topk,
                   uint8_t* keep_blocks, int32_t* cu_seqlens_out, void* stream);

/* ---------------------------------------------------------------------------
 * 3. Expand + compact  ([UP] "Top-p selection" paragraph: the output is the set of
 *    token indices to keep; [UP] "propagation" and "Sparsity Propagation"
 *    paragraphs: later layers receive only the surviving tokens; [UP] "scheduler"
 *    paragraph: positions of the survivors are carried along)
 *
 * For each request, kept blocks in ascending order, tokens in ascending order:
 *   idx_out[r]    = packed input row of the r-th surviving token
 *   hidden_out[r] = hidden[idx_out[r]]   (a bit copy of row_bytes = H * elem_bytes)
 *   pos_out[r]    = pos[idx_out[r]]      (original positions, never renumbered)
 *   orig_out[r]   = prev_orig[idx_out[r]] (drop composition, as up_compose_drops)
 * Rows r in [cu_seqlens_out[i], cu_seqlens_out[i+1]) belong to request i.
 *
 * hidden     : [T, H] rows of elem_bytes each (bf16: elem_bytes = 2).
 * pos        : int32 [T], or NULL (then pos_out is not written and may be NULL).
 * keep_blocks, cu_seqlens_out : as produced by up_topp_select.
 * idx_out    : int32 [T] capacity;  hidden_out: [T, H] capacity;  pos_out: int32 [T].
 * prev_orig, orig_out : int32 [T] each, or both NULL.  When given, the composition
 *              of up_compose_drops is written in the same pass (no extra launch);
 *              orig_out without prev_orig is UP_EINVAL.
 * workspace  : at least up_expand_compact_workspace(...) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------- */
size_t up_expand_compact_workspace(const int32_t* cu_seqlens_h, int B, int G);

int up_expand_compact(const void* hidden, int H, int elem_bytes, const int32_t* pos,
                      const uint8_t* keep_blocks, const int32_t* cu_seqlens,
                      const int32_t* cu_seqlens_out, const int32_t* cu_seqlens_h, int B,
                      int G, int32_t* idx_out, void* hidden_out, int32_t* pos_out,
                      const int32_t* prev_orig, int32_t* orig_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The same operation with no workspace argument, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the per-block run table lives in a device array of the library
 * (786,688 bytes per GPU, held until the process ends), so the call allocates
 * nothing.  At most 65,536 blocks in the batch (nb_tot = sum_i ceil(L_i / G));
 * more is UP_EUNSUPPORTED, with nothing launched.  Every call on one GPU uses that
 * GPU's one array: calls that overlap on the same GPU (different streams without
 * ordering, or host threads) race and must be ordered by the caller; calls on
 * different GPUs do not interact.  No state is carried from one call to the next
 * (each call rewrites the whole table before the copy reads it).  Other arguments,
 * outputs and results are those of up_expand_compact. */
int up_expand_compact_noalloc(const void* hidden, int H, int elem_bytes, const int32_t* pos,
                              const uint8_t* keep_blocks, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_out, const int32_t* cu_seqlens_h,
                              int B, int G, int32_t* idx_out, void* hidden_out,
                              int32_t* pos_out, const int32_t* prev_orig, int32_t* orig_out,
                              void* stream);

/* ---------------------------------------------------------------------------
 * 4. Drop composition  ([UP] "propagation" paragraph: a drop carries into every
 *    later layer; [UP] "scheduler" paragraph: the drop history maps survivors to
 *    their original positions)
 *
 *   orig_out[r] = prev_orig[idx[r]]   for r < *count
 * prev_orig : int32 [prev_len], the original index of every row of the previous
 *             layer's input (the identity at the first decision).
 * idx       : int32 [capacity], e.g. idx_out of up_expand_compact.
 * count     : device int32 scalar, e.g. &cu_seqlens_out[B]; must be <= capacity.
 * Rows with idx outside [0, prev_len), or a count above capacity, raise the device
 * error word; such rows get -1.
 * ------------------------------------------------------------------------- */
int up_compose_drops(const int32_t* prev_orig, int prev_len, const int32_t* idx,
                     const int32_t* count, int capacity, int32_t* orig_out, void* stream);

/* ---------------------------------------------------------------------------
 * 1-4 in one call  ([UP] "Triton kernels" paragraph: the method's steps run as a
 *    GPU pipeline with no host round trip)
 *
 * The decision of up_block_scores + up_topp_select + up_expand_compact (with the
 * drop composition when prev_orig / orig_out are given), with the same arguments,
 * outputs and results, bit for bit.  When no request has more than 4096 blocks the
 * select kernel also normalises the block masses and assigns the compaction's block
 * destinations (two launches fewer); otherwise the three calls run in sequence.
 * When every request is empty (T = 0) only cu_seqlens_out is written (all zeros); the
 * buffers sized by T or by the block count may then be NULL.
 * workspace : at least up_layer_decision_workspace(...) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------- */
size_t up_layer_decision_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d,
                                   int n, int G);

int up_layer_decision(const void* qwin, const void* k, const int32_t* cu_seqlens,
                      const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d, int n, int G,
                      float scale, float p, const void* hidden, int H, int elem_bytes,
                      const int32_t* pos, const int32_t* prev_orig, float* scores,
                      uint8_t* keep_blocks, int32_t* cu_seqlens_out, int32_t* idx_out,
                      void* hidden_out, int32_t* pos_out, int32_t* orig_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * 5. The layer on the surviving tokens  ([UP] "propagation" paragraph: after a
 *    drop every later layer computes on the survivors only, so its GEMMs shrink
 *    as well as its attention; [UP] "Sparsity Propagation" paragraph: FFN work
 *    falls from O(N) to O(rho N) and attention shrinks with the kept fraction;
 *    [UP] "scheduler" paragraph: survivors keep their original positions)
 *
 * These calls take the compacted rows of up_expand_compact (R = cu_seqlens_out[B]
 * rows, request i owning [cu_seqlens_out[i], cu_seqlens_out[i+1])) and pos_out.
 * ------------------------------------------------------------------------- */

/* Rotary embedding at the carried positions, then causal GQA attention per request:
 *   q' = rope(q, pos), k' = rope(k, pos)   element j pairs with element j + d/2 and
 *        turns by pos * rope_theta^(-2j/d); computed in float64, rounded once to bf16
 *   out[r, h] = sum_{r' <= r, same request} softmax_r'(scale q'[r, h] . k'[r', h / g]) v[r', h / g]
 *   with g = Hq / Hkv.  Survivors are in ascending original order, so "r' <= r" is
 *   causality over the original positions.
 * q   : bf16 [R, Hq, d];  k, v : bf16 [R, Hkv, d];  out : bf16 [R, Hq, d] (16-byte aligned).
 * pos : int32 [R] (pos_out: original positions).
 * cu_seqlens / cu_seqlens_h : int32 [B+1] row offsets (cu_seqlens_out and its host copy).
 * d in {64, 128, 256} (UP_EUNSUPPORTED otherwise); scale <= 0 means 1/sqrt(d);
 * rope_theta > 1 (e.g. 500000 for the Llama-3.1 shape).
 * Probabilities enter the P.V product as bf16; softmax statistics and accumulation
 * are float32.  Limits: sum of ceil(L_i / 64) padded rows < 2^31 and at most 65535
 * workgroup tiles, a tile spanning t * 4 / m query tokens, m = the largest of 4, 2, 1
 * dividing Hq / Hkv, t = 64 for d = 64 and 128 with Hkv <= 256, else 32 (about 4M
 * rows at d = 128 and Hq / Hkv = 4).
 * workspace : at least up_rope_attention_workspace(...) bytes, 256-byte aligned
 *             (rotated q and k, transposed v, plan; for d = 64 and 128 with
 *             Hkv <= 256 also the largest key norm of each 64-row tile per kv head).
 * A device cu_seqlens whose totals (rows, padded rows, workgroup tiles) differ from
 * those of cu_seqlens_h raises error bit 1 and nothing is written. */
size_t up_rope_attention_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv, int d);

int up_rope_attention(const void* q, const void* k, const void* v, const int32_t* pos,
                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B, int Hq,
                      int Hkv, int d, float scale, float rope_theta, void* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The same attention, and the block scores of its window rows from the probabilities
 * it computes anyway ([UP] "Triton kernels" paragraph: online softmax and block
 * reduction in the GPU pipeline; "drop" paragraph: the scoring happens at the
 * full-attention layer, whose attention already runs that softmax).  Per request the
 * window is its last W = min(n, L) rows; for every window row and query head the
 * attention kernel keeps, beside its softmax, the sum of the probabilities of each
 * block of G keys and stores it with the softmax reference it was taken against,
 * then the row's own maximum and sum; the block masses and the normalisation follow
 * as in up_block_scores.  So
 *   scores[blk_off(i) + b] = (sum over window rows w and query heads h of
 *       P_{w,h}(block b)) / (the same sum over all blocks of request i),
 * P_{w,h}(block b) the softmax probability mass that window row w of head h puts on
 * the keys of block b, computed from the rotated bf16 operands q', k' of the
 * attention (the scores up_block_scores gives for window queries q'[last W rows]
 * and keys k').  out is exactly up_rope_attention's output.  The workgroup tiles that
 * hold window rows run a statistics-keeping instance of the attention kernel on a
 * second stream of the library's (one per device, created at the first call and kept;
 * it joins back into `stream` with events before the block masses), beside the plain
 * kernel over the other tiles on `stream`.
 * q, k, v, pos, cu_seqlens, cu_seqlens_h, d, scale, rope_theta, out: as up_rope_attention
 * (scale also scales the scores' logits).
 * n >= 1 window rows, G block size (a multiple of 32 in [32, 1024], else UP_EUNSUPPORTED).
 * scores  : float32 [sum_i ceil(L_i / G)], blocks of request i from blk_off(i) = sum of
 *           the earlier requests' block counts (as up_block_scores).
 * row_lse : optional float32 [sum_i W_i, Hq] natural-log log-sum-exp of each window
 *           row's scaled logits (NULL to skip).
 * workspace : at least up_rope_attention_scores_workspace(...) bytes, 256-byte aligned.
 * Errors: as up_rope_attention and up_block_scores; when either plan finds the device
 * cu_seqlens inconsistent, error bit 1 is raised and the scores are not written.  A
 * launch error after the fork still joins `stream` to the second stream before
 * UP_EHIP is returned (if even the join cannot be enqueued, the second stream is
 * synchronised), so no kernel of the failed call outlives the report. */
size_t up_rope_attention_scores_workspace(const int32_t* cu_seqlens_h, int B, int Hq, int Hkv,
                                          int d, int n, int G);

int up_rope_attention_scores(const void* q, const void* k, const void* v, const int32_t* pos,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_h, int B,
                             int Hq, int Hkv, int d, float scale, float rope_theta, int n, int G,
                             void* out, float* scores, float* row_lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* SwiGLU gate: a[r, j] = silu(gu[r, j]) * gu[r, F + j], float32 math, bf16 result.
 * gu : bf16 [R, 2F] (gate columns first);  a : bf16 [R, F];  F % 8 == 0. */
int up_swiglu(const void* gu, int64_t R, int F, void* a, void* stream);

/* The layer's GEMMs (up_linear, up_swiglu_ffn) are plain bf16 GEMMs served by
 * hipBLASLt; they live in a separate library, libuniprefill_layer.so, declared in
 * include/uniprefill_layer.h, so that this library links no vendor GEMM library. */

/* ---------------------------------------------------------------------------
 * Diagnostics (not on the hot path)
 * ------------------------------------------------------------------------- */

/* Device error word: bit 1 = cu_seqlens inconsistent with the host copy (or a
 * selection whose kept counts disagree with its flags), bit 2 = index out of range in
 * up_compose_drops, bit 4 = count above capacity, bit 8 = page index outside the paged
 * key cache (up_block_scores_paged), bit 16 = a compaction run whose destination or
 * source rows fall outside the buffers (the run is not copied).
 * Synchronises `stream`, copies the word to *code_h and clears it. */
int up_device_error(int32_t* code_h, void* stream);

/* Kernel timing with HIP events recorded by the library on the launch stream.
 * up_profile_enable(1) starts recording an event pair around every kernel the
 * library launches; up_profile_read() synchronises the recorded events and
 * returns, for kernel family `which` (0 score partials, 1 row statistics,
 * 2 block masses, 3 normalise, 4 select, 5 select finalise, 6 block
 * destinations, 7 gather, 8 compose, 9 plan, 10 given-lse score partials,
 * 11 given-lse finalise, 12 attention plan, 13 rotary layout, 14 attention,
 * 15 SwiGLU gate, 16 hipBLASLt GEMM, 17 select with normalisation and block
 * destinations inside up_layer_decision, 18 the attention over the window tiles with
 * block statistics inside up_rope_attention_scores, timed on its second stream), the
 * number of launches and their
 * summed duration in milliseconds; up_profile_reset() forgets them.
 * up_profile_enable(0) stops recording.  Not thread safe. */
int up_profile_enable(int on);
int up_profile_read(int which, int* launches_h, double* total_ms_h);
int up_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* UNIPREFILL_H */
