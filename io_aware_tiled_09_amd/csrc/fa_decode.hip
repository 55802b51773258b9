// Decode-step attention over a paged KV cache on gfx950.
//
// One new query token per sequence attends to the sequence's L_b cached
// tokens, whose K and V rows live in fixed-size pages found through a
// per-sequence page table. [FlashAttention: The GPU Memory Hack That Changed
// Everything (ai.branddocks.com, episode 75), "What's Next?": PagedAttention
// stores the KV cache in pages with page tables.] With a single query row
// there is no matrix product to speak of: the step reads every cached row
// once and is bound by HBM bandwidth, so the design is about streaming.
//
// Two kernels, no atomics:
//  * split: kRunGroups * G workgroups of 256 threads per (sequence, KV
//    head), each taking every (kRunGroups * G)-th run of kSplit keys. With G
//    query heads per KV head there are G times fewer (sequence, KV head)
//    pairs and G times the arithmetic per row, so G times the workgroups keep
//    as many rows in flight (measured on 50 sequences, H = 32, H_kv = 8:
//    3.6 TB/s against 3.1 with 3; 4 * G or one per run: 2.0). The run's
//    page-table entries are looked up once into LDS.
//    The 16 lane-groups of 16 lanes each take one key of every 16-key row
//    block of a page (16 consecutive rows: coalesced 16-byte loads), kUnroll
//    blocks at a time with all loads issued first. A group keeps, for each of the G
//    query heads that share the KV head, the online-softmax state of its keys
//    (running max m, sum l, and its d/16 slice of the weighted V sum). The
//    16 group states are merged (within a wave by lane shuffles, across the
//    four waves through LDS) with the two-correction-factor merge
//    [Flash Attention Optimization (aicomputerinstitute.com), "The fix: tile
//    the computation..."], and the run's (m, l, acc) go to the workspace.
//  * merge: one wave per (sequence, query head) combines the runs the same
//    way and writes O (bf16) and lse.
// Keys past L_b, and page-table entries outside [0, num_pages), are masked:
// their weight is 0 and their V is never used (rows the sequence does not own
// may hold anything, NaN included).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_common.h"

namespace fa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kBlocks = kSplit / 16;        // 16-row blocks per run
constexpr int kRunGroups = 3;               // workgroups per (sequence, KV head) and query head of it

struct DecodeArgs {
    const __bf16* q;
    const __bf16* k_cache;
    const __bf16* v_cache;
    const int* page_table;
    const int* seq_lens;
    float* ws_acc;  // [B][H][max_splits][D]
    float* ws_ml;   // [B][H][max_splits][2]
    __bf16* o;
    float* lse;
    int H, H_kv, num_pages, page_size, max_pages, max_splits;
    float c_log2;   // scale * log2(e)
};

__device__ inline void merge_state(float& m, float& l, float* acc, int n, float m2, float l2,
                                   const float* acc2)
{
    const float mn = fmaxf(m, m2);
    if (mn == neg_inf()) return;  // both empty
    const float a = __builtin_amdgcn_exp2f(m - mn), b = __builtin_amdgcn_exp2f(m2 - mn);
    l = l * a + l2 * b;
    for (int e = 0; e < n; ++e) acc[e] = acc[e] * a + acc2[e] * b;
    m = mn;
}

template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void fa_decode_split_kernel(DecodeArgs a)
{
    constexpr int E = D / 16;                    // d-elements per lane
    constexpr int kUnroll = G <= 2 ? 8 : 4;      // row blocks in flight per group
    const int hk = blockIdx.y, b = blockIdx.z;
    const int L = min(a.seq_lens[b], a.max_pages * a.page_size);
    // Workgroup x takes runs x, x + gridDim.x, ... of its (sequence, KV head):
    // a short sequence leaves few workgroups idle, a long one is still spread.
    for (int split = blockIdx.x; split * kSplit < L; split += gridDim.x) {
    const int j_begin = split * kSplit;
    const int j_end = min(L, j_begin + kSplit);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = tid >> 4;    // 0..15: the key of each 16-row block
    const int e0 = (tid & 15) * E;

    // The run's first row of every 16-row block, as an element offset into
    // the caches (or -1: past the end or an unmapped page), looked up once.
    __shared__ long long blk_row[kBlocks];
    if (tid < kBlocks) {
        const int blk = j_begin + tid * 16;
        long long r = -1;
        if (blk < j_end) {
            const int pg = a.page_table[(size_t)b * a.max_pages + blk / a.page_size];
            if (pg >= 0 && pg < a.num_pages)
                r = (((long long)pg * a.H_kv + hk) * a.page_size + blk % a.page_size) * D;
        }
        blk_row[tid] = r;
    }

    // This lane's slice of each of the G query rows, fp32.
    float qv[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const __bf16* qrow = a.q + ((size_t)b * a.H + (size_t)hk * G + g) * D + e0;
#pragma unroll
        for (int e = 0; e < E; ++e) qv[g][e] = (float)qrow[e];
    }
    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = neg_inf();
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
    }
    __syncthreads();  // blk_row is ready

    const int nblk = (j_end - j_begin + 15) / 16;
    for (int bb = 0; bb < nblk; bb += kUnroll) {
        // Issue every load of kUnroll row blocks first.
        typedef __bf16 bfE __attribute__((ext_vector_type(E)));
        bfE kr[kUnroll], vr[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int blk = bb + u;
            const long long r0 = blk < nblk ? blk_row[blk] : -1;
            ok[u] = r0 >= 0 && j_begin + blk * 16 + grp < j_end;
            const size_t off = ok[u] ? (size_t)r0 + (size_t)grp * D + e0 : 0;
            kr[u] = ok[u] ? *reinterpret_cast<const bfE*>(a.k_cache + off) : bfE{};
            vr[u] = ok[u] ? *reinterpret_cast<const bfE*>(a.v_cache + off) : bfE{};
        }
        // Scores of the group's kUnroll keys for each query head.
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float s[kUnroll];
            float mx = neg_inf();
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) dot = __builtin_fmaf(qv[g][e], (float)kr[u][e], dot);
#pragma unroll
                for (int off = 8; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 16);
                s[u] = ok[u] ? dot * a.c_log2 : neg_inf();
                mx = fmaxf(mx, s[u]);
            }
            const float mn = fmaxf(m[g], mx);
            if (mn == neg_inf()) continue;  // no valid key yet (the whole group)
            const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
            m[g] = mn;
            l[g] *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float p = __builtin_amdgcn_exp2f(s[u] - mn);  // 0 when masked
                l[g] += p;
                if (ok[u]) {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[g][e] = __builtin_fmaf(p, (float)vr[u][e], acc[g][e]);
                }
            }
        }
    }

    // Merge the 4 groups of each wave (lanes l, l^16, l^32, l^48 hold the same
    // d slice), then the 4 waves through LDS.
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float m2 = __shfl_xor(m[g], off, 64), l2 = __shfl_xor(l[g], off, 64);
            float a2[E];
#pragma unroll
            for (int e = 0; e < E; ++e) a2[e] = __shfl_xor(acc[g][e], off, 64);
            merge_state(m[g], l[g], acc[g], E, m2, l2, a2);
        }
    __shared__ float red_acc[4][G][D];
    __shared__ float red_ml[4][G][2];
    if (lane < 16) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int e = 0; e < E; ++e) red_acc[wave][g][e0 + e] = acc[g][e];
            if (lane == 0) {
                red_ml[wave][g][0] = m[g];
                red_ml[wave][g][1] = l[g];
            }
        }
    }
    __syncthreads();
    // Thread t < G * D combines element t % D of head t / D over the 4 waves.
    for (int t = tid; t < G * D; t += kDecThreads) {
        const int g = t / D, e = t % D;
        float mm = red_ml[0][g][0], ll = red_ml[0][g][1], aa = red_acc[0][g][e];
#pragma unroll
        for (int w = 1; w < 4; ++w) merge_state(mm, ll, &aa, 1, red_ml[w][g][0], red_ml[w][g][1], &red_acc[w][g][e]);
        const size_t slot = ((size_t)b * a.H + (size_t)hk * G + g) * a.max_splits + split;
        a.ws_acc[slot * D + e] = aa;
        if (e == 0) {
            a.ws_ml[slot * 2] = mm;
            a.ws_ml[slot * 2 + 1] = ll;
        }
    }
    __syncthreads();  // the LDS arrays are reused by the next run
    }
}

template <int D>
__global__ __launch_bounds__(64) void fa_decode_merge_kernel(DecodeArgs a)
{
    constexpr int E = D / 64;
    const int h = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x;
    const int L = min(a.seq_lens[b], a.max_pages * a.page_size);
    const size_t row = (size_t)b * a.H + h;
    __bf16* orow = a.o + row * D;
    if (L <= 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) orow[lane * E + e] = (__bf16)0.f;
        if (lane == 0) a.lse[row] = neg_inf();
        return;
    }
    const int ns = (L + kSplit - 1) / kSplit;
    float m = neg_inf(), l = 0.f, acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int s = 0; s < ns; ++s) {
        const size_t slot = row * a.max_splits + s;
        float a2[E];
#pragma unroll
        for (int e = 0; e < E; ++e) a2[e] = a.ws_acc[slot * D + lane * E + e];
        merge_state(m, l, acc, E, a.ws_ml[slot * 2], a.ws_ml[slot * 2 + 1], a2);
    }
    // Every key of the sequence masked (invalid page entries): O = 0, lse = -inf.
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) orow[lane * E + e] = (__bf16)(acc[e] * inv);
    if (lane == 0) a.lse[row] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : neg_inf();
}

template <int D, int G>
hipError_t launch_decode_dg(const DecodeArgs& a, int B, hipStream_t stream)
{
    hipLaunchKernelGGL((fa_decode_split_kernel<D, G>), dim3(min(a.max_splits, kRunGroups * G), a.H_kv, B),
                       dim3(kDecThreads), 0, stream, a);
    hipLaunchKernelGGL((fa_decode_merge_kernel<D>), dim3(a.H, B), dim3(64), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, int B, int G, hipStream_t stream)
{
    switch (G) {
    case 1: return launch_decode_dg<D, 1>(a, B, stream);
    case 2: return launch_decode_dg<D, 2>(a, B, stream);
    case 4: return launch_decode_dg<D, 4>(a, B, stream);
    default: return launch_decode_dg<D, 8>(a, B, stream);
    }
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int* page_table, const int* seq_lens, void* o, float* lse,
                         float* ws, int B, int H, int H_kv, int d, int num_pages, int page_size,
                         int max_pages, float c_log2, hipStream_t stream)
{
    DecodeArgs a;
    a.q = static_cast<const __bf16*>(q);
    a.k_cache = static_cast<const __bf16*>(k_cache);
    a.v_cache = static_cast<const __bf16*>(v_cache);
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.max_splits = decode_max_splits(max_pages, page_size);
    a.ws_acc = ws;
    a.ws_ml = ws + (size_t)B * H * a.max_splits * d;
    a.o = static_cast<__bf16*>(o);
    a.lse = lse;
    a.H = H;
    a.H_kv = H_kv;
    a.num_pages = num_pages;
    a.page_size = page_size;
    a.max_pages = max_pages;
    a.c_log2 = c_log2;
    const int G = H / H_kv;
    return d == 64 ? launch_decode_d<64>(a, B, G, stream) : launch_decode_d<128>(a, B, G, stream);
}

}  // namespace fa
