/*
 * fa.h: C ABI of the FlashAttention library (libfa.so, gfx950): the forward
 * pass (bf16 storage, fp32 storage, FP8 inputs), the backward pass, and
 * decode-step attention over a paged KV cache. The standard, materializing
 * baseline has its own library and header (fa_std.h).
 *
 * The forward operation is exact softmax attention for every (batch, head):
 *
 *     S = scale * Q K^T          (N x N, never stored)
 *     P = softmax(S) row-wise    (causal: key j visible to query i iff j <= i)
 *     O = P V
 *     lse_i = ln sum_j exp(S_ij)  over the visible keys j
 *
 * [FlashAttention: The GPU Memory Hack That Changed Everything
 *  (ai.branddocks.com, episode 75), "Standard Attention" for S, P, O and
 *  "FlashAttention: IO-Aware Tiling" for the tiled evaluation]
 * [Flash Attention Optimization (aicomputerinstitute.com), "Attention is not
 *  slow because of arithmetic" for S = QK^T / sqrt(d); "Sizing a tile, and
 *  why the backward pass recomputes" for keeping per-row statistics (lse)]
 * [same first page, "Integration": is_causal]
 *
 * Layout: q, k, v and o are contiguous row-major [B][H][N][d]; lse is
 * contiguous [B][H][N] fp32 (the decode entry point documents its own
 * layout). Every pointer is a DEVICE pointer on the current HIP device. The
 * caller allocates and frees every buffer, workspaces included; the library
 * allocates nothing, frees nothing and does not synchronize. It keeps no
 * state between calls, except the static scratch array of fa_bwd_noalloc
 * (see there).
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL means the
 * default stream) and the call returns once it is launched. Results are
 * valid after the caller synchronizes that stream. Faults during execution
 * surface at that synchronization, not as a return code.
 *
 * Errors: every argument check runs before anything is launched; a non-zero
 * status means nothing was enqueued (FA_ERR_LAUNCH: the launch itself was
 * rejected by the runtime). B*H*N == 0 is a valid empty call: it returns
 * FA_OK at once and the pointers are not looked at.
 */
#ifndef IO_AWARE_TILED_09_FA_H
#define IO_AWARE_TILED_09_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL_PTR = 1,            /* a pointer is NULL in a non-empty call      */
    FA_ERR_BAD_SHAPE = 2,           /* B, H or N negative                          */
    FA_ERR_UNSUPPORTED_HEAD_DIM = 3,/* d is not 64 or 128                          */
    FA_ERR_BAD_SCALE = 4,           /* scale negative, NaN or infinite             */
    FA_ERR_MISALIGNED = 5,          /* q/k/v/o not 16-byte aligned, lse not 4-byte */
    FA_ERR_ALIASING = 6,            /* an output overlaps an input or an output    */
    FA_ERR_LAUNCH = 7,              /* the HIP runtime rejected the launch         */
    FA_ERR_TOO_LARGE = 8,           /* B*H*ceil(N/128) workgroups exceed 2^31 - 1  */
    FA_ERR_WORKSPACE = 9,           /* workspace NULL, misaligned or too small     */
    FA_ERR_LIBRARY = 10,            /* a library call (rocBLAS) failed             */
    FA_ERR_SCRATCH_LIMIT = 11       /* B*H*N above fa_bwd_noalloc's static scratch */
} fa_status;

/*
 * bf16 attention forward.
 * q, k, v: const bf16 (raw 16-bit bfloat16 bits) [B][H][N][d];
 * o: bf16 [B][H][N][d], written with round-to-nearest-even;
 * lse: fp32 [B][H][N], natural log;
 * B, H, N >= 0; d in {64, 128}; scale >= 0 and finite (1/sqrt(d) is usual);
 * causal: 0 or non-zero; stream: hipStream_t or NULL.
 * Scores are accumulated in fp32 from exact bf16 products; softmax runs in
 * fp32; P is rounded to bf16 before the P V product, which accumulates in fp32.
 * Returns an fa_status.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N, int d, float scale, int causal, void *stream);

/*
 * fp32-storage attention forward: q, k, v and o are fp32 [B][H][N][d]; every
 * other argument as in fa_fwd. Each fp32 operand x is split into two bf16
 * terms, hi = rn(x) and lo = rn(x - hi), and every product is taken as
 * hi*hi + lo*hi + hi*lo on the bf16 matrix cores with fp32 accumulation, so
 * scores and P V keep close to fp32 accuracy; o is stored in fp32.
 */
int fa_fwd_f32(const float *q, const float *k, const float *v, float *o,
               float *lse, int B, int H, int N, int d, float scale, int causal,
               void *stream);

/*
 * bf16 attention backward pass: dq, dk, dv from dout for the forward pass
 * fa_fwd computed with the same q, k, v, scale and causal flag.
 * [Flash Attention Optimization (aicomputerinstitute.com), "Sizing a tile,
 *  and why the backward pass recomputes instead of storing": P is
 *  recomputed block by block from q, k and the forward's per-row lse]
 *
 * With S = scale * q k^T (+ mask) and P = softmax(S) row-wise:
 *     dv = P^T dout,  dS = P * (dout v^T - D),  D_i = sum_t dout_it o_it,
 *     dq = scale * dS k,  dk = scale * dS^T q.
 * q, k, v, o, dout: const bf16 [B][H][N][d] (o = fa_fwd's output);
 * lse: const fp32 [B][H][N] (fa_fwd's lse, natural log);
 * dq, dk, dv: bf16 [B][H][N][d] outputs (round-to-nearest-even);
 * ws: fp32 workspace of B*H*N elements, overwritten (holds D);
 * every other argument as in fa_fwd. All pointers are DEVICE pointers; the
 * outputs and ws must not overlap any input or each other
 * (FA_ERR_ALIASING). Products take bf16 operands (P and dS rounded to bf16)
 * and accumulate in fp32. Launches three kernels on `stream` and returns.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const float *lse, const void *dout, void *dq, void *dk, void *dv,
           float *ws, int B, int H, int N, int d, float scale, int causal,
           void *stream);

/*
 * The backward pass of fa_bwd for callers that cannot allocate: code being
 * captured into a HIP graph, tight serving loops, and harnesses that forbid
 * hipMalloc. Same arguments, results and checks as fa_bwd, without ws: the
 * per-row D values live in a static device array of the library (16 MiB per
 * GPU, held from the first call on that GPU until the process ends), so the
 * call allocates and frees nothing. B*H*N must not exceed
 * fa_bwd_noalloc_max_rows() (4,194,304; FA_ERR_SCRATCH_LIMIT otherwise).
 * Every call on one GPU shares that array: calls that overlap on one GPU
 * (other streams, other threads) race and must be serialized by the caller.
 * The first call on each GPU looks the array's device address up on the
 * current device (no allocation).
 */
int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                   const float *lse, const void *dout, void *dq, void *dk,
                   void *dv, int B, int H, int N, int d, float scale,
                   int causal, void *stream);
long long fa_bwd_noalloc_max_rows(void);

/*
 * FP8 attention forward: Q, K and V as 8-bit E4M3 codes (OCP FP8 E4M3: 4
 * exponent bits, bias 7, 3 mantissa bits, no infinities) with one positive
 * scale per tensor, so that the attended values are q_scale * Q, k_scale * K
 * and v_scale * V; everything else as fa_fwd.
 * [FlashAttention: The GPU Memory Hack That Changed Everything
 *  (ai.branddocks.com, episode 75), "FlashAttention-3: Hopper Architecture":
 *  attention in FP8 on the matrix units]
 * q, k, v: const uint8 [B][H][N][d] codes (16-byte aligned); o: bf16
 * [B][H][N][d]; lse: fp32 [B][H][N], natural log of the scaled scores;
 * d == 128 only (FA_ERR_UNSUPPORTED_HEAD_DIM otherwise); scale >= 0 and
 * finite; q_scale, k_scale, v_scale > 0 and finite (FA_ERR_BAD_SCALE).
 * Both products run on the FP8 matrix instructions with fp32 accumulation;
 * the softmax weights are rounded to E4M3 (as 48 p, p <= 8) for the second
 * product.
 * Codes 0x7F and 0xFF (NaN) propagate as NaN.
 */
int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int H, int N, int d, float scale, float q_scale,
               float k_scale, float v_scale, int causal, void *stream);

/*
 * Decode-step attention over a paged KV cache: for each sequence b one new
 * query token (q[b][h]) attends to the sequence's seq_lens[b] cached tokens.
 * Token t of sequence b is row t % page_size of physical page
 * page_table[b][t / page_size]; query head h reads KV head h / (H / H_kv).
 * o[b][h] = sum_t softmax_t(scale * q . k_t) v_t and lse[b][h] = ln sum_t
 * exp(scale * q . k_t) (natural log); the new token's own K and V are
 * expected in the cache already (no mask).
 * [FlashAttention: The GPU Memory Hack That Changed Everything
 *  (ai.branddocks.com, episode 75), "What's Next?": PagedAttention's pages
 *  and page tables for the KV cache]
 * q, o: bf16 [B][H][d]; k_cache, v_cache: bf16 [num_pages][H_kv][page_size]
 * [d] (16-byte aligned); page_table: int32 [B][max_pages]; seq_lens: int32
 * [B]; lse: fp32 [B][H]; ws: fp32 workspace of at least
 * fa_decode_workspace_bytes(B, H, d, page_size, max_pages) bytes, 16-byte
 * aligned, contents overwritten. d in {64, 128}; H / H_kv in {1, 2, 4, 8};
 * page_size a positive multiple of 16; scale >= 0 and finite.
 * Device-side values are not checked on the host; the kernels clamp
 * seq_lens[b] to max_pages * page_size, treat tokens whose page entry is
 * outside [0, num_pages) as absent (weight 0, never read), and a sequence
 * with no token gets o = 0 and lse = -inf. Rows of the cache that no
 * sequence owns are never used, whatever they hold.
 */
size_t fa_decode_workspace_bytes(int B, int H, int d, int page_size, int max_pages);
int fa_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                    const int *page_table, const int *seq_lens, void *o, float *lse,
                    void *ws, size_t ws_bytes, int B, int H, int H_kv, int d,
                    int num_pages, int page_size, int max_pages, float scale,
                    void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *fa_status_string(int status);

/* Queries per workgroup tile (Br) of the bf16 kernel on grids that fill the
 * CUs (fa_fwd; smaller grids use 128-row blocks, see fa_fwd_grid; fa_fwd_f32
 * uses 128) and keys per K/V tile (Bc) of both kernels; informational, for
 * grid-size arithmetic in callers and tests. */
int fa_tile_rows(void);
int fa_tile_cols(void);

/* Launch shape of fa_fwd for (B, H, N, causal): host arithmetic only, no GPU
 * work, the same rule fa_fwd applies. The split over (batch*head x query
 * block) follows [FlashAttention: The GPU Memory Hack That Changed
 * Everything, "FlashAttention-2"] (parallelism over the sequence). Returns
 * the number of workgroups fa_fwd launches: 0 for an empty shape,
 * -FA_ERR_BAD_SHAPE for a negative size, -FA_ERR_TOO_LARGE past the grid
 * limit. Where non-NULL, *rows_per_block receives the query rows of one
 * block (256; 128 when a grid of 256-row blocks would leave CUs idle and the
 * 128-row grid fits one workgroup per CU: the workgroup's two wave groups
 * then take alternate key tiles of the block and merge their partial
 * (max, sum, output) states with the two correction factors of [Flash
 * Attention Optimization, "The fix: tile the computation..."]) and *paired
 * whether causal blocks run two per workgroup (on small causal grids grouped
 * so that every workgroup carries the heaviest block's work: {nqb-1},
 * {nqb-2-p, p} and the middle blocks of two heads). For callers that size
 * work around the forward's grid, and for tests. */
long long fa_fwd_grid(int B, int H, int N, int causal, int *rows_per_block, int *paired);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_TILED_09_FA_H */
