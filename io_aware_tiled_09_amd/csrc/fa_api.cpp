// C ABI of the attention-forward library: argument checks, then one kernel
// launch on the caller's stream. See include/fa.h for the contract.
#include <hip/hip_runtime_api.h>
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_kernels.h"

namespace {

constexpr double kLog2e = 1.4426950408889634;  // log2(e)

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Checks shared by both entry points. Returns FA_OK when a launch may follow;
// *empty is set when the call has nothing to do.
int validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
             int B, int H, int N, int d, float scale, size_t elem, bool* empty)
{
    *empty = false;
    if (B < 0 || H < 0 || N < 0)
        return FA_ERR_BAD_SHAPE;
    if (B == 0 || H == 0 || N == 0) {
        *empty = true;
        return FA_OK;
    }
    if (!q || !k || !v || !o || !lse)
        return FA_ERR_NULL_PTR;
    if (d != 64 && d != 128)
        return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (!isfinite(scale) || scale < 0.0f)
        return FA_ERR_BAD_SCALE;
    const long long nqb = ((long long)N + fa::kBr - 1) / fa::kBr;
    if ((long long)B * H * nqb > 0x7fffffffLL)
        return FA_ERR_TOO_LARGE;
    auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    if ((addr(q) | addr(k) | addr(v) | addr(o)) & 15u)
        return FA_ERR_MISALIGNED;
    if (addr(lse) & 3u)
        return FA_ERR_MISALIGNED;
    const uintptr_t tensor_bytes = (uintptr_t)B * (uintptr_t)H * (uintptr_t)N * (uintptr_t)d * elem;
    const uintptr_t lse_bytes = (uintptr_t)B * (uintptr_t)H * (uintptr_t)N * sizeof(float);
    const Range rq{addr(q), addr(q) + tensor_bytes}, rk{addr(k), addr(k) + tensor_bytes},
        rv{addr(v), addr(v) + tensor_bytes}, ro{addr(o), addr(o) + tensor_bytes},
        rl{addr(lse), addr(lse) + lse_bytes};
    if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv) || overlaps(ro, rl) ||
        overlaps(rl, rq) || overlaps(rl, rk) || overlaps(rl, rv))
        return FA_ERR_ALIASING;
    return FA_OK;
}

// The kernels take scale*log2(e) and need it > 0, so that a masked score
// (-inf) always gives exp2(-inf) = 0. Raising a smaller value to FLT_MIN
// changes nothing: with scale*log2(e) <= FLT_MIN every exponent of a visible
// key rounds to 0 in fp32, exactly as with scale 0 (all weights 1).
float kernel_scale(float scale)
{
    const float c = (float)((double)scale * kLog2e);
    return c < FLT_MIN ? FLT_MIN : c;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int N, int d, float scale, int causal, void* stream)
{
    bool empty;
    const int st = validate(q, k, v, o, lse, B, H, N, d, scale, 2, &empty);
    if (st != FA_OK || empty)
        return st;
    const float scale_log2 = kernel_scale(scale);
    const hipError_t e = fa::launch_bf16(q, k, v, o, lse, B * H, N, d, scale_log2, causal != 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
               int H, int N, int d, float scale, int causal, void* stream)
{
    bool empty;
    const int st = validate(q, k, v, o, lse, B, H, N, d, scale, 4, &empty);
    if (st != FA_OK || empty)
        return st;
    const float scale_log2 = kernel_scale(scale);
    const hipError_t e = fa::launch_f32(q, k, v, o, lse, B * H, N, d, scale_log2, causal != 0,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, float q_scale, float k_scale, float v_scale, int causal,
               void* stream)
{
    if (B < 0 || H < 0 || N < 0)
        return FA_ERR_BAD_SHAPE;
    if (B == 0 || H == 0 || N == 0)
        return FA_OK;
    if (!q || !k || !v || !o || !lse)
        return FA_ERR_NULL_PTR;
    if (d != 128)
        return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (!isfinite(scale) || scale < 0.0f)
        return FA_ERR_BAD_SCALE;
    for (float t : {q_scale, k_scale, v_scale})
        if (!isfinite(t) || t <= 0.0f)
            return FA_ERR_BAD_SCALE;
    const long long nqb = ((long long)N + fa::kBr - 1) / fa::kBr;
    if ((long long)B * H * nqb > 0x7fffffffLL)
        return FA_ERR_TOO_LARGE;
    auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    if ((addr(q) | addr(k) | addr(v) | addr(o)) & 15u || (addr(lse) & 3u))
        return FA_ERR_MISALIGNED;
    const uintptr_t in_bytes = (uintptr_t)B * (uintptr_t)H * (uintptr_t)N * (uintptr_t)d;
    const uintptr_t rows = (uintptr_t)B * (uintptr_t)H * (uintptr_t)N;
    const Range rq{addr(q), addr(q) + in_bytes}, rk{addr(k), addr(k) + in_bytes},
        rv{addr(v), addr(v) + in_bytes}, ro{addr(o), addr(o) + 2 * in_bytes},
        rl{addr(lse), addr(lse) + rows * sizeof(float)};
    if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv) || overlaps(ro, rl) ||
        overlaps(rl, rq) || overlaps(rl, rk) || overlaps(rl, rv))
        return FA_ERR_ALIASING;
    // The scores' constant folds the two input scales in; kept > 0 as in fa_fwd.
    const double c = (double)scale * (double)q_scale * (double)k_scale * kLog2e;
    const float c_log2 = c < FLT_MIN ? FLT_MIN : (float)c;
    const hipError_t e = fa::launch_fp8(q, k, v, o, lse, B * H, N, c_log2, v_scale, causal != 0,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int page_size, int max_pages)
{
    if (B < 1 || H < 1 || d < 1 || page_size < 1 || max_pages < 1)
        return 0;
    return (size_t)B * (size_t)H * (size_t)fa::decode_max_splits(max_pages, page_size) *
           (size_t)(d + 2) * sizeof(float);
}

int fa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                    const int* page_table, const int* seq_lens, void* o, float* lse, void* ws,
                    size_t ws_bytes, int B, int H, int H_kv, int d, int num_pages, int page_size,
                    int max_pages, float scale, void* stream)
{
    if (B < 0 || H < 1 || H_kv < 1 || num_pages < 1 || page_size < 1 || max_pages < 1 ||
        H % H_kv != 0 || page_size % 16 != 0)
        return FA_ERR_BAD_SHAPE;
    const int G = H / H_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return FA_ERR_BAD_SHAPE;
    if (B == 0)
        return FA_OK;
    if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !o || !lse)
        return FA_ERR_NULL_PTR;
    if (d != 64 && d != 128)
        return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (!isfinite(scale) || scale < 0.0f)
        return FA_ERR_BAD_SCALE;
    if (B > 65535 || H_kv > 65535 || H > 65535 ||
        (long long)max_pages * page_size > 0x7fffffffLL)
        return FA_ERR_TOO_LARGE;
    const size_t need = fa_decode_workspace_bytes(B, H, d, page_size, max_pages);
    auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    if (!ws || (addr(ws) & 15u) || ws_bytes < need)
        return FA_ERR_WORKSPACE;
    if ((addr(q) | addr(k_cache) | addr(v_cache) | addr(o)) & 15u ||
        (addr(page_table) | addr(seq_lens) | addr(lse)) & 3u)
        return FA_ERR_MISALIGNED;
    const uintptr_t qb = (uintptr_t)B * H * d * 2, cb = (uintptr_t)num_pages * H_kv * page_size * d * 2;
    const Range in[5] = {{addr(q), addr(q) + qb}, {addr(k_cache), addr(k_cache) + cb},
                         {addr(v_cache), addr(v_cache) + cb},
                         {addr(page_table), addr(page_table) + (uintptr_t)B * max_pages * 4},
                         {addr(seq_lens), addr(seq_lens) + (uintptr_t)B * 4}};
    const Range out[3] = {{addr(o), addr(o) + qb}, {addr(lse), addr(lse) + (uintptr_t)B * H * 4},
                          {addr(ws), addr(ws) + need}};
    for (int x = 0; x < 3; ++x) {
        for (int y = 0; y < 5; ++y)
            if (overlaps(out[x], in[y]))
                return FA_ERR_ALIASING;
        for (int y = x + 1; y < 3; ++y)
            if (overlaps(out[x], out[y]))
                return FA_ERR_ALIASING;
    }
    const hipError_t e = fa::launch_decode(q, k_cache, v_cache, page_table, seq_lens, o, lse,
                                           static_cast<float*>(ws), B, H, H_kv, d, num_pages,
                                           page_size, max_pages, kernel_scale(scale),
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Checks shared by the two backward entry points. ws == NULL: the workspace
// is the library's static scratch (fa_bwd_noalloc), which no caller buffer
// can overlap.
int validate_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, const void* dq, const void* dk, const void* dv,
                 const float* ws, bool need_ws, int B, int H, int N, int d, float scale,
                 bool* empty)
{
    *empty = false;
    if (B < 0 || H < 0 || N < 0)
        return FA_ERR_BAD_SHAPE;
    if (B == 0 || H == 0 || N == 0) {
        *empty = true;
        return FA_OK;
    }
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || (need_ws && !ws))
        return FA_ERR_NULL_PTR;
    if (d != 64 && d != 128)
        return FA_ERR_UNSUPPORTED_HEAD_DIM;
    if (!isfinite(scale) || scale < 0.0f)
        return FA_ERR_BAD_SCALE;
    const long long nqb = ((long long)N + fa::kBr - 1) / fa::kBr;
    if ((long long)B * H * nqb > 0x7fffffffLL)
        return FA_ERR_TOO_LARGE;
    auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    if ((addr(q) | addr(k) | addr(v) | addr(o) | addr(dout) | addr(dq) | addr(dk) | addr(dv)) & 15u)
        return FA_ERR_MISALIGNED;
    if ((addr(lse) | addr(ws)) & 3u)
        return FA_ERR_MISALIGNED;
    const uintptr_t tb = (uintptr_t)B * (uintptr_t)H * (uintptr_t)N * (uintptr_t)d * 2;
    const uintptr_t rb = (uintptr_t)B * (uintptr_t)H * (uintptr_t)N * sizeof(float);
    const Range in[6] = {{addr(q), addr(q) + tb},     {addr(k), addr(k) + tb},
                         {addr(v), addr(v) + tb},     {addr(o), addr(o) + tb},
                         {addr(lse), addr(lse) + rb}, {addr(dout), addr(dout) + tb}};
    const Range out[4] = {{addr(dq), addr(dq) + tb}, {addr(dk), addr(dk) + tb},
                          {addr(dv), addr(dv) + tb}, {addr(ws), addr(ws) + (need_ws ? rb : 0)}};
    for (int a = 0; a < 4; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlaps(out[a], in[b]))
                return FA_ERR_ALIASING;
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(out[a], out[b]))
                return FA_ERR_ALIASING;
    }
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* ws, int B, int H, int N, int d,
           float scale, int causal, void* stream)
{
    bool empty;
    const int st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, true, B, H, N, d, scale,
                                &empty);
    if (st != FA_OK || empty)
        return st;
    const hipError_t e = fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, ws, B * H, N, d,
                                             kernel_scale(scale), scale, causal != 0,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float scale, int causal, void* stream)
{
    bool empty;
    const int st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, false, B, H, N, d,
                                scale, &empty);
    if (st != FA_OK || empty)
        return st;
    if ((long long)B * H * N > fa::kBwdScratchRows)
        return FA_ERR_SCRATCH_LIMIT;
    float* ws = nullptr;
    if (fa::bwd_scratch(&ws) != hipSuccess)
        return FA_ERR_LAUNCH;
    const hipError_t e = fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, ws, B * H, N, d,
                                             kernel_scale(scale), scale, causal != 0,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

long long fa_bwd_noalloc_max_rows(void) { return fa::kBwdScratchRows; }

const char* fa_status_string(int status)
{
    switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_PTR: return "a tensor pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "B, H and N must be >= 0";
    case FA_ERR_UNSUPPORTED_HEAD_DIM: return "head dimension d must be 64 or 128";
    case FA_ERR_BAD_SCALE: return "scale must be finite and >= 0";
    case FA_ERR_MISALIGNED: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIASING: return "an output overlaps an input or another output";
    case FA_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    case FA_ERR_TOO_LARGE: return "too many workgroups (B*H*ceil(N/128) >= 2^31)";
    case FA_ERR_WORKSPACE:
        return "workspace NULL, misaligned (fa_decode_paged: 16 bytes; fa_std_*: 256 bytes) "
               "or smaller than its *_workspace_bytes()";
    case FA_ERR_LIBRARY: return "a rocBLAS call failed";
    case FA_ERR_SCRATCH_LIMIT:
        return "B*H*N exceeds the static scratch of fa_bwd_noalloc (fa_bwd_noalloc_max_rows())";
    default: return "unknown status";
    }
}

int fa_tile_rows(void) { return fa::kBrBf16; }
int fa_tile_cols(void) { return fa::kBc; }

long long fa_fwd_grid(int B, int H, int N, int causal, int* rows_per_block, int* paired)
{
    if (B < 0 || H < 0 || N < 0)
        return -FA_ERR_BAD_SHAPE;
    if (B == 0 || H == 0 || N == 0) {
        if (rows_per_block) *rows_per_block = fa::kBrBf16;
        if (paired) *paired = 0;
        return 0;
    }
    const long long nqb = ((long long)N + fa::kBr - 1) / fa::kBr;
    if ((long long)B * H * nqb > 0x7fffffffLL)
        return -FA_ERR_TOO_LARGE;
    const fa::FwdPlan pl = fa::fwd_plan((long long)B * H, N, causal != 0);
    if (rows_per_block) *rows_per_block = pl.rows;
    if (paired) *paired = pl.paired ? 1 : 0;
    return pl.grid;
}

}  // extern "C"
