// Standard (materializing) attention forward on gfx950: the baseline that
// FlashAttention is compared against.
//
// [FlashAttention: The GPU Memory Hack That Changed Everything
//  (ai.branddocks.com, episode 75), "Standard Attention": S = QK^T is written
//  to HBM, read back for softmax, P is written and read back for PV; "The
//  Problem: GPU Memory Hierarchy": those N x N round trips dominate.]
//
// Steps 1 and 3 are plain batched GEMMs and go to rocBLAS (bf16 inputs, fp32
// accumulation). Step 2, the row softmax over the stored scores, is this
// file's kernel: one workgroup of 256 threads per query row. Rows of up to
// 8192 scores (N % 4 == 0) are read once into registers with 16-byte loads;
// longer or odd rows use an online (max, sum) per thread merged across the
// workgroup and a second pass over the row (then in L2). Either way it is
// HBM-bound: 4 bytes read per visible score and 2 bytes written per entry of P.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa_std.h"
#include "fa_common.h"

namespace fa {
namespace {

constexpr int kSmThreads = 256;
constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;
constexpr size_t kGemmWsBytes = size_t(32) << 20;

// Merge two online-softmax states (m, l): l relative to exp2(m * log2e).
__device__ inline void merge(float& m, float& l, float m2, float l2)
{
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;  // both empty
    l = l * __builtin_amdgcn_exp2f((m - mn) * kLog2eF) +
        l2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2eF);
    m = mn;
}

__device__ inline void push(float& m, float& l, float x)
{
    if (x > m) {
        l = l * __builtin_amdgcn_exp2f((m - x) * kLog2eF) + 1.0f;
        m = x;
    } else {
        l += __builtin_amdgcn_exp2f((x - m) * kLog2eF);
    }
}

template <bool CAUSAL, bool VEC4>
__global__ __launch_bounds__(kSmThreads) void fa_std_softmax_kernel(const float* __restrict__ s,
                                                                    __bf16* __restrict__ p,
                                                                    float* __restrict__ lse,
                                                                    int N)
{
    __shared__ float red_m[kSmThreads / 64], red_l[kSmThreads / 64];
    const long long row = blockIdx.x;
    const int i = (int)(row % N);
    const int nvis = CAUSAL ? i + 1 : N;
    const float* srow = s + row * (long long)N;
    __bf16* prow = p + row * (long long)N;
    const int tid = threadIdx.x;

    // Pass 1: per-thread online max and sum over the visible scores.
    float m = -INFINITY, l = 0.f;
    if constexpr (VEC4) {
        const int nv4 = nvis / 4;
        for (int x = tid; x < nv4; x += kSmThreads) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(srow + 4 * x);
            push(m, l, v[0]);
            push(m, l, v[1]);
            push(m, l, v[2]);
            push(m, l, v[3]);
        }
        for (int j = 4 * nv4 + tid; j < nvis; j += kSmThreads) push(m, l, srow[j]);
    } else {
        for (int j = tid; j < nvis; j += kSmThreads) push(m, l, srow[j]);
    }
    // Workgroup merge: within each wave by shuffles, then across waves.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        merge(m, l, __shfl_xor(m, off, 64), __shfl_xor(l, off, 64));
    if ((tid & 63) == 0) {
        red_m[tid >> 6] = m;
        red_l[tid >> 6] = l;
    }
    __syncthreads();
    m = red_m[0];
    l = red_l[0];
#pragma unroll
    for (int w = 1; w < kSmThreads / 64; ++w) merge(m, l, red_m[w], red_l[w]);
    // Every row sees key 0, so m is finite and l >= 1.
    const float inv_l = 1.0f / l;
    const float mc = m * kLog2eF;

    // Pass 2: P = exp(s - m) / l over the visible scores, 0 after them.
    if constexpr (VEC4) {
        const int n4 = N / 4;
        for (int x = tid; x < n4; x += kSmThreads) {
            const int j = 4 * x;
            float e[4] = {0.f, 0.f, 0.f, 0.f};
            if (j < nvis) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(srow + j);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    e[c] = j + c < nvis
                               ? __builtin_amdgcn_exp2f(__builtin_fmaf(v[c], kLog2eF, -mc)) * inv_l
                               : 0.f;
            }
            bf16x4 out;
#pragma unroll
            for (int c = 0; c < 4; ++c) out[c] = (__bf16)e[c];
            *reinterpret_cast<bf16x4*>(prow + j) = out;
        }
    } else {
        for (int j = tid; j < N; j += kSmThreads)
            prow[j] = (__bf16)(j < nvis ? __builtin_amdgcn_exp2f(__builtin_fmaf(srow[j], kLog2eF, -mc)) * inv_l
                                        : 0.f);
    }
    if (tid == 0) lse[row] = m + __builtin_amdgcn_logf(l) * kLn2F;
}

// Rows of up to kSmThreads * 4 * NV scores (N % 4 == 0): the visible part of
// the row is read once into registers (NV 16-byte loads per thread, all in
// flight together), then max, sum and the bf16 row of P come from there.
template <bool CAUSAL, int NV>
__global__ __launch_bounds__(kSmThreads) void fa_std_softmax_reg_kernel(const float* __restrict__ s,
                                                                        __bf16* __restrict__ p,
                                                                        float* __restrict__ lse,
                                                                        int N)
{
    __shared__ float red[kSmThreads / 64];
    const long long row = blockIdx.x;
    const int i = (int)(row % N);
    const int nvis = CAUSAL ? i + 1 : N;
    const float* srow = s + row * (long long)N;
    __bf16* prow = p + row * (long long)N;
    const int tid = threadIdx.x;
    const int n4 = N / 4;

    f32x4 r[NV];
#pragma unroll
    for (int c = 0; c < NV; ++c) {
        const int j = 4 * (tid + c * kSmThreads);
        r[c] = j < nvis ? *reinterpret_cast<const f32x4*>(srow + j)
                        : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (j < nvis && j + 4 > nvis)  // the row's last visible float4
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e >= nvis) r[c][e] = -INFINITY;
    }
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < NV; ++c)
        m = fmaxf(m, fmaxf(fmaxf(r[c][0], r[c][1]), fmaxf(r[c][2], r[c][3])));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();  // red is reused for the sums
    const float mc = m * kLog2eF;  // every row sees key 0: m is finite
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[c][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(r[c][e], kLog2eF, -mc));  // -inf -> 0
            l += r[c][e];
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
    if ((tid & 63) == 0) red[tid >> 6] = l;
    __syncthreads();
    l = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv_l = 1.0f / l;
#pragma unroll
    for (int c = 0; c < NV; ++c) {
        const int x = tid + c * kSmThreads;
        if (x < n4) {
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (__bf16)(r[c][e] * inv_l);
            *reinterpret_cast<bf16x4*>(prow + 4 * x) = out;
        }
    }
    if (tid == 0) lse[row] = m + __builtin_amdgcn_logf(l) * kLn2F;
}
static_assert(kSmThreads == 256, "the reductions above assume four waves");

struct Range {
    uintptr_t lo, hi;
};
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
uintptr_t addr(const void* p) { return reinterpret_cast<uintptr_t>(p); }
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

int check_shape(int B, int H, int N, int d, bool* empty)
{
    *empty = false;
    if (B < 0 || H < 0 || N < 0) return FA_ERR_BAD_SHAPE;
    if (B == 0 || H == 0 || N == 0) {
        *empty = true;
        return FA_OK;
    }
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEAD_DIM;
    // One softmax workgroup per row, and rocBLAS takes 32-bit sizes.
    if ((long long)B * H * N > 0x7fffffffLL || (long long)B * H > 0x7fffffffLL)
        return FA_ERR_TOO_LARGE;
    return FA_OK;
}

// One rocBLAS handle per device, created on first use, never destroyed (the
// process owns it until exit). The lock covers set_stream / set_workspace /
// GEMM enqueue, so concurrent callers on one device do not race on the
// handle's stream.
constexpr int kMaxDevices = 64;
std::mutex g_lock;
rocblas_handle g_handle[kMaxDevices];

rocblas_handle handle_for_current_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    if (!g_handle[dev] && rocblas_create_handle(&g_handle[dev]) != rocblas_status_success)
        g_handle[dev] = nullptr;
    return g_handle[dev];
}

// Column-major views of the row-major [N][d] head matrices (a row-major
// [N][d] matrix is a column-major d x N matrix with leading dimension d):
// S^T(j, i) = sum_t K(j, t) Q(i, t): C = A^T B with A = K (d x N), B = Q
// (d x N), C = S as column-major N x N (S row-major [i][j]).
int gemm_scores(const void* q, const void* k, float* s, void* ws, int BH, int N, int d,
                float scale, hipStream_t stream)
{
    std::lock_guard<std::mutex> guard(g_lock);
    rocblas_handle h = handle_for_current_device();
    if (!h) return FA_ERR_LIBRARY;
    if (rocblas_set_stream(h, stream) != rocblas_status_success) return FA_ERR_LIBRARY;
    if (rocblas_set_workspace(h, ws, kGemmWsBytes) != rocblas_status_success)
        return FA_ERR_LIBRARY;
    const float alpha = scale, beta = 0.f;
    const rocblas_stride sqk = (rocblas_stride)N * d, ss = (rocblas_stride)N * N;
    const rocblas_status st = rocblas_gemm_strided_batched_ex(
        h, rocblas_operation_transpose, rocblas_operation_none, N, N, d, &alpha, k,
        rocblas_datatype_bf16_r, d, sqk, q, rocblas_datatype_bf16_r, d, sqk, &beta, s,
        rocblas_datatype_f32_r, N, ss, s, rocblas_datatype_f32_r, N, ss, BH,
        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    return st == rocblas_status_success ? FA_OK : FA_ERR_LIBRARY;
}

// O^T(t, i) = sum_j V(j, t) P(i, j): C = A B with A = V (column-major d x N),
// B = P (column-major N x N holding P^T), C = O (column-major d x N).
int gemm_output(const void* p, const void* v, void* o, void* ws, int BH, int N, int d,
                hipStream_t stream)
{
    std::lock_guard<std::mutex> guard(g_lock);
    rocblas_handle h = handle_for_current_device();
    if (!h) return FA_ERR_LIBRARY;
    if (rocblas_set_stream(h, stream) != rocblas_status_success) return FA_ERR_LIBRARY;
    if (rocblas_set_workspace(h, ws, kGemmWsBytes) != rocblas_status_success)
        return FA_ERR_LIBRARY;
    const float alpha = 1.f, beta = 0.f;
    const rocblas_stride sv = (rocblas_stride)N * d, sp = (rocblas_stride)N * N;
    const rocblas_status st = rocblas_gemm_strided_batched_ex(
        h, rocblas_operation_none, rocblas_operation_none, d, N, N, &alpha, v,
        rocblas_datatype_bf16_r, d, sv, p, rocblas_datatype_bf16_r, N, sp, &beta, o,
        rocblas_datatype_bf16_r, d, sv, o, rocblas_datatype_bf16_r, d, sv, BH,
        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    return st == rocblas_status_success ? FA_OK : FA_ERR_LIBRARY;
}

int launch_softmax(const float* s, void* p, float* lse, int BH, int N, bool causal,
                   hipStream_t stream)
{
    const dim3 grid((unsigned)((long long)BH * N));
    const bool vec = N % 4 == 0;
    __bf16* pb = static_cast<__bf16*>(p);
    if (vec && N <= kSmThreads * 4 * 8) {
        const int nv = (N + kSmThreads * 4 - 1) / (kSmThreads * 4);  // 1..8
#define FA_STD_REG(NV)                                                                          \
    if (causal)                                                                                \
        hipLaunchKernelGGL((fa_std_softmax_reg_kernel<true, NV>), grid, dim3(kSmThreads), 0,  \
                           stream, s, pb, lse, N);                                             \
    else                                                                                       \
        hipLaunchKernelGGL((fa_std_softmax_reg_kernel<false, NV>), grid, dim3(kSmThreads), 0, \
                           stream, s, pb, lse, N);
        if (nv == 1) { FA_STD_REG(1) }
        else if (nv == 2) { FA_STD_REG(2) }
        else if (nv <= 4) { FA_STD_REG(4) }
        else { FA_STD_REG(8) }
#undef FA_STD_REG
    } else if (causal && vec)
        hipLaunchKernelGGL((fa_std_softmax_kernel<true, true>), grid, dim3(kSmThreads), 0, stream, s, pb, lse, N);
    else if (causal)
        hipLaunchKernelGGL((fa_std_softmax_kernel<true, false>), grid, dim3(kSmThreads), 0, stream, s, pb, lse, N);
    else if (vec)
        hipLaunchKernelGGL((fa_std_softmax_kernel<false, true>), grid, dim3(kSmThreads), 0, stream, s, pb, lse, N);
    else
        hipLaunchKernelGGL((fa_std_softmax_kernel<false, false>), grid, dim3(kSmThreads), 0, stream, s, pb, lse, N);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace
}  // namespace fa

extern "C" {

size_t fa_std_workspace_bytes(int B, int H, int N)
{
    bool empty;
    if (fa::check_shape(B, H, N, 64, &empty) != FA_OK || empty) return 0;
    const size_t nn = (size_t)B * H * (size_t)N * (size_t)N;
    return fa::round256(nn * 4) + fa::round256(nn * 2) + fa::kGemmWsBytes;
}

int fa_std_scores(const void* q, const void* k, float* s, void* gemm_ws, int B, int H, int N,
                  int d, float scale, void* stream)
{
    using namespace fa;
    bool empty;
    int st = check_shape(B, H, N, d, &empty);
    if (st != FA_OK || empty) return st;
    if (!q || !k || !s) return FA_ERR_NULL_PTR;
    if (!gemm_ws || (addr(gemm_ws) & 255u)) return FA_ERR_WORKSPACE;
    if (!isfinite(scale) || scale < 0.0f) return FA_ERR_BAD_SCALE;
    if ((addr(q) | addr(k) | addr(s)) & 15u) return FA_ERR_MISALIGNED;
    const size_t tb = (size_t)B * H * (size_t)N * d * 2;
    const size_t sb = (size_t)B * H * (size_t)N * (size_t)N * 4;
    const Range rs{addr(s), addr(s) + sb}, rw{addr(gemm_ws), addr(gemm_ws) + kGemmWsBytes};
    if (overlaps(rs, {addr(q), addr(q) + tb}) || overlaps(rs, {addr(k), addr(k) + tb}) ||
        overlaps(rs, rw) || overlaps(rw, {addr(q), addr(q) + tb}) ||
        overlaps(rw, {addr(k), addr(k) + tb}))
        return FA_ERR_ALIASING;
    return gemm_scores(q, k, s, gemm_ws, B * H, N, d, scale, static_cast<hipStream_t>(stream));
}

int fa_std_softmax(const float* s, void* p, float* lse, int B, int H, int N, int causal,
                   void* stream)
{
    using namespace fa;
    bool empty;
    int st = check_shape(B, H, N, 64, &empty);
    if (st != FA_OK || empty) return st;
    if (!s || !p || !lse) return FA_ERR_NULL_PTR;
    if ((addr(s) | addr(p)) & 15u || (addr(lse) & 3u)) return FA_ERR_MISALIGNED;
    const size_t nn = (size_t)B * H * (size_t)N * (size_t)N;
    const Range rs{addr(s), addr(s) + nn * 4}, rp{addr(p), addr(p) + nn * 2},
        rl{addr(lse), addr(lse) + (size_t)B * H * N * 4};
    if (overlaps(rp, rs) || overlaps(rl, rs) || overlaps(rl, rp)) return FA_ERR_ALIASING;
    return launch_softmax(s, p, lse, B * H, N, causal != 0, static_cast<hipStream_t>(stream));
}

int fa_std_output(const void* p, const void* v, void* o, void* gemm_ws, int B, int H, int N,
                  int d, void* stream)
{
    using namespace fa;
    bool empty;
    int st = check_shape(B, H, N, d, &empty);
    if (st != FA_OK || empty) return st;
    if (!p || !v || !o) return FA_ERR_NULL_PTR;
    if (!gemm_ws || (addr(gemm_ws) & 255u)) return FA_ERR_WORKSPACE;
    if ((addr(p) | addr(v) | addr(o)) & 15u) return FA_ERR_MISALIGNED;
    const size_t tb = (size_t)B * H * (size_t)N * d * 2;
    const size_t pb = (size_t)B * H * (size_t)N * (size_t)N * 2;
    const Range ro{addr(o), addr(o) + tb}, rw{addr(gemm_ws), addr(gemm_ws) + kGemmWsBytes};
    if (overlaps(ro, {addr(p), addr(p) + pb}) || overlaps(ro, {addr(v), addr(v) + tb}) ||
        overlaps(ro, rw) || overlaps(rw, {addr(p), addr(p) + pb}) ||
        overlaps(rw, {addr(v), addr(v) + tb}))
        return FA_ERR_ALIASING;
    return gemm_output(p, v, o, gemm_ws, B * H, N, d, static_cast<hipStream_t>(stream));
}

int fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
               size_t ws_bytes, int B, int H, int N, int d, float scale, int causal, void* stream)
{
    using namespace fa;
    bool empty;
    int st = check_shape(B, H, N, d, &empty);
    if (st != FA_OK || empty) return st;
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
    if (!isfinite(scale) || scale < 0.0f) return FA_ERR_BAD_SCALE;
    if ((addr(q) | addr(k) | addr(v) | addr(o)) & 15u || (addr(lse) & 3u))
        return FA_ERR_MISALIGNED;
    const size_t need = fa_std_workspace_bytes(B, H, N);
    if (!ws || (addr(ws) & 255u) || ws_bytes < need) return FA_ERR_WORKSPACE;
    const size_t tb = (size_t)B * H * (size_t)N * d * 2;
    const size_t lb = (size_t)B * H * (size_t)N * 4;
    const Range in[3] = {{addr(q), addr(q) + tb}, {addr(k), addr(k) + tb}, {addr(v), addr(v) + tb}};
    const Range out[3] = {{addr(o), addr(o) + tb}, {addr(lse), addr(lse) + lb},
                          {addr(ws), addr(ws) + need}};
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 3; ++b)
            if (overlaps(out[a], in[b])) return FA_ERR_ALIASING;
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(out[a], out[b])) return FA_ERR_ALIASING;
    }
    const size_t nn = (size_t)B * H * (size_t)N * (size_t)N;
    unsigned char* base = static_cast<unsigned char*>(ws);
    float* s = reinterpret_cast<float*>(base);
    void* p = base + round256(nn * 4);
    void* gws = base + round256(nn * 4) + round256(nn * 2);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    st = gemm_scores(q, k, s, gws, B * H, N, d, scale, hs);
    if (st != FA_OK) return st;
    st = launch_softmax(s, p, lse, B * H, N, causal != 0, hs);
    if (st != FA_OK) return st;
    return gemm_output(p, v, o, gws, B * H, N, d, hs);
}

}  // extern "C"
