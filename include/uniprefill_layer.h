/* libuniprefill_layer: the plain GEMMs of the layer that runs on the surviving tokens.
 *
 * [UP] "propagation" and "Sparsity Propagation" paragraphs: after a drop every later
 * sub-layer, attention and FFN alike, computes on the kept tokens only.  The
 * attention of that layer (up_rope_attention) and the SwiGLU gate (up_swiglu) are
 * hand-written kernels of libuniprefill.so (include/uniprefill.h); the projection and
 * FFN GEMMs are plain bf16 GEMMs, served here by hipBLASLt, in a library of their own
 * so that the decision library links no vendor GEMM library.
 *
 * Conventions are those of include/uniprefill.h (device pointers, asynchronous calls
 * on `stream`, up_status return codes, caller-owned buffers), with one exception:
 * the first call for a shape on a device creates that device's hipBLASLt handle and
 * picks the algorithm (host work and a library-internal allocation, cached); later
 * calls only launch.  This library loads libuniprefill.so (same directory).
 */
#ifndef UNIPREFILL_LAYER_H
#define UNIPREFILL_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* y[R, N] = x[R, K] . w[N, K]^T (+ residual[R, N] when not NULL); bf16 in and out,
 * float32 accumulation.  residual may alias y.  workspace may be NULL with
 * workspace_bytes = 0; otherwise 256-byte aligned and offered to hipBLASLt.
 * UP_EUNSUPPORTED if hipBLASLt has no algorithm for the shape, or if x, w or y has
 * 2^32 elements or more (such GEMMs have not been shown to run safely here: the largest
 * that ran had 4.03e9 elements per operand, and a run with a 6.3e9-element FFN output
 * faulted the GPU). */
int up_linear(const void* x, const void* w, const void* residual, int64_t R, int K, int N,
              void* y, void* workspace, size_t workspace_bytes, void* stream);

/* SwiGLU FFN on R rows: y = swiglu(x . w_gu^T) . w_down^T (+ residual).
 * x : bf16 [R, H];  w_gu : bf16 [2F, H] (gate rows first);  w_down : bf16 [H, F];
 * residual : bf16 [R, H] or NULL (may alias y);  y : bf16 [R, H];  F % 8 == 0.
 * The intermediate x . w_gu^T and the gated activation (up_swiglu of
 * libuniprefill.so) are stored as bf16 in the workspace: at least
 * up_swiglu_ffn_workspace(R, H, F) bytes, 256-byte aligned.  UP_EUNSUPPORTED when
 * either GEMM would have an operand of 2^32 elements or more (R * 2F below 2^32, as for
 * up_linear). */
size_t up_swiglu_ffn_workspace(int64_t R, int H, int F);

int up_swiglu_ffn(const void* x, const void* w_gu, const void* w_down, const void* residual,
                  int64_t R, int H, int F, void* y, void* workspace, size_t workspace_bytes,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UNIPREFILL_LAYER_H */
