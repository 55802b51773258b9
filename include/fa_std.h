/*
 * fa_std.h: C ABI of the standard (materializing) attention forward
 * (libfa_std.so, gfx950): the comparison baseline for fa_fwd.
 *
 * Standard attention writes the N x N score matrix to HBM, reads it back for
 * the row softmax, writes the probabilities, and reads them back for the
 * product with V; these round trips, not the arithmetic, dominate its time.
 * [FlashAttention: The GPU Memory Hack That Changed Everything
 *  (ai.branddocks.com, episode 75), "Standard Attention" and "The Problem:
 *  GPU Memory Hierarchy"]
 * [Flash Attention Optimization (aicomputerinstitute.com), "Attention is not
 *  slow because of arithmetic"]
 *
 * Same operation, layout and outputs as fa_fwd (include/fa.h): bf16 q, k, v,
 * o [B][H][N][d], fp32 lse [B][H][N] (natural log), causal: key j visible to
 * query i iff j <= i. It runs as three steps through a caller workspace:
 *
 *   1. fa_std_scores:  S = scale * Q K^T, fp32 [B][H][N][N]   (rocBLAS GEMM)
 *   2. fa_std_softmax: P = softmax(S) per row (masked entries 0), bf16
 *                      [B][H][N][N], and lse                   (HIP kernel)
 *   3. fa_std_output:  O = P V, bf16                           (rocBLAS GEMM)
 *
 * The GEMMs compute the full N x N product also when causal (the mask is
 * applied in step 2, as standard attention does); step 2 reads only the
 * visible scores of a row and writes zeros for the rest.
 *
 * Pointers are device pointers; the caller allocates every buffer. Status
 * codes are fa_status (include/fa.h); every check runs before anything is
 * enqueued. Work is enqueued on `stream` (hipStream_t, NULL = default). The
 * GEMMs go through one rocBLAS handle per device, created on first use and
 * kept until the process ends, and use the caller's workspace as rocBLAS
 * workspace; calls that use the same device are serialized by a lock while
 * they enqueue.
 */
#ifndef IO_AWARE_TILED_09_FA_STD_H
#define IO_AWARE_TILED_09_FA_STD_H

#include <stddef.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of workspace fa_std_fwd needs: S (fp32) + P (bf16) + 32 MiB of GEMM
 * workspace, each part 256-byte aligned. 0 for an empty or invalid shape. */
size_t fa_std_workspace_bytes(int B, int H, int N);

/*
 * All three steps. q, k, v, o: bf16 [B][H][N][d] (16-byte aligned); lse:
 * fp32 [B][H][N]; ws: ws_bytes >= fa_std_workspace_bytes(B, H, N), 256-byte
 * aligned, contents ignored and overwritten. d in {64, 128}; scale finite and
 * >= 0. Errors as fa_fwd, plus FA_ERR_WORKSPACE and FA_ERR_LIBRARY.
 */
int fa_std_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
               void *ws, size_t ws_bytes, int B, int H, int N, int d,
               float scale, int causal, void *stream);

/* Step 1: s (fp32 [B][H][N][N], 16-byte aligned) = scale * Q K^T, full.
 * gemm_ws: 32 MiB of device memory (256-byte aligned) rocBLAS may use. */
int fa_std_scores(const void *q, const void *k, float *s, void *gemm_ws, int B,
                  int H, int N, int d, float scale, void *stream);

/* Step 2: p (bf16 [B][H][N][N]) = row softmax of s over the visible keys
 * (0 elsewhere); lse (fp32 [B][H][N]) = ln sum_j exp(s_ij) over them. */
int fa_std_softmax(const float *s, void *p, float *lse, int B, int H, int N,
                   int causal, void *stream);

/* Step 3: o (bf16 [B][H][N][d]) = P V with fp32 accumulation. */
int fa_std_output(const void *p, const void *v, void *o, void *gemm_ws, int B,
                  int H, int N, int d, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_TILED_09_FA_STD_H */
