// Attention forward for fp32 storage (gfx950): the same tiled online-softmax
// method as the bf16 kernel, for q, k, v, o held in fp32.
//
// Method: [FlashAttention: The GPU Memory Hack That Changed Everything
// (ai.branddocks.com, episode 75), "FlashAttention: IO-Aware Tiling" / "The
// Tiling Strategy" and "The Online Softmax Trick"].
//
// The matrix cores have no fp32 inputs of this shape, so every operand x is
// split into bf16 hi = rn(x) and lo = rn(x - hi), and each product uses
// hi*hi + lo*hi + hi*lo (3 MFMAs): scores and P V keep close to fp32
// accuracy. The split happens while a K/V tile goes from registers to LDS,
// so tiles are staged through VGPRs (not loaded straight into LDS) and V is
// written transposed, [d][keys], keys permuted so a lane's 8 keys of a
// 16-key chunk are one 16-byte read. Layout of work and scores is the one
// described in fa_fwd_bf16.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.h"

namespace fa {
namespace {

constexpr int kPad = 8;  // bf16 elements of padding per LDS row (16 bytes)

template <int D>
struct alignas(16) SmemF32 {
    __bf16 k[2][2][kBc][D + kPad];    // [buffer][hi/lo] K tile, row-major [key][d]
    __bf16 vt[2][2][D][kBc + kPad];   // [buffer][hi/lo] V tile transposed [d][permuted key]
};

// 8 consecutive fp32 elements of a row and their two bf16 terms.
struct Chunk8 {
    f32x4 a, b;
    __device__ static Chunk8 load(const float* p) {
        const f32x4* v = reinterpret_cast<const f32x4*>(p);
        return Chunk8{v[0], v[1]};
    }
    __device__ static Chunk8 zero() { return Chunk8{f32x4{}, f32x4{}}; }
    // term 0: round-to-nearest bf16 of x; term 1: bf16 of the remainder.
    __device__ bf16x8 term(int t) const {
        bf16x8 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const __bf16 ha = (__bf16)a[i], hb = (__bf16)b[i];
            r[i] = t == 0 ? ha : (__bf16)(a[i] - (float)ha);
            r[i + 4] = t == 0 ? hb : (__bf16)(b[i] - (float)hb);
        }
        return r;
    }
};

// Position of key offset `jo` (multiple of 4, within a 64-key tile) in a
// transposed V row. Inside each 16-key chunk, key 4*a+b (a, b in 0..3) goes
// to 8*(a&1) + 4*(a>>1) + b: lane half h of the score layout holds keys
// {4h..4h+3, 8+4h..8+4h+3} of the chunk, now positions 8h..8h+7.
__device__ inline int vt_pos(int jo) {
    const int a = (jo >> 2) & 3;
    return (jo & ~15) + ((a & 1) << 3) + ((a >> 1) << 2);
}

// Global -> registers staging of one K/V tile, and registers -> LDS.
template <int D>
struct TileLoaderF32 {
    static constexpr int kKChunks = kBc * D / 8;            // 8-element K chunks
    static constexpr int kKPer = kKChunks / kThreads;       // per thread
    static constexpr int kVGroups = (kBc / 4) * (D / 8);    // 4 keys x 8 d
    static constexpr int kVPer = (kVGroups + kThreads - 1) / kThreads;
    static_assert(kKChunks % kThreads == 0, "K tile must split evenly");

    Chunk8 kr[kKPer];
    Chunk8 vr[kVPer][4];

    __device__ void load(const float* __restrict__ kh, const float* __restrict__ vh, int j0,
                         int N, int tid) {
#pragma unroll
        for (int it = 0; it < kKPer; ++it) {
            const int c = tid + it * kThreads;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            const int j = j0 + row;
            kr[it] = j < N ? Chunk8::load(kh + (size_t)j * D + col) : Chunk8::zero();
        }
#pragma unroll
        for (int it = 0; it < kVPer; ++it) {
            const int g = tid + it * kThreads;
            if (kVGroups % kThreads == 0 || g < kVGroups) {
                const int kg = g / (D / 8), col = (g % (D / 8)) * 8;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int j = j0 + kg * 4 + a;
                    vr[it][a] = j < N ? Chunk8::load(vh + (size_t)j * D + col) : Chunk8::zero();
                }
            }
        }
    }

    __device__ void store(SmemF32<D>& sm, int buf, int tid) const {
#pragma unroll
        for (int it = 0; it < kKPer; ++it) {
            const int c = tid + it * kThreads;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
#pragma unroll
            for (int t = 0; t < 2; ++t)
                *reinterpret_cast<bf16x8*>(&sm.k[buf][t][row][col]) = kr[it].term(t);
        }
#pragma unroll
        for (int it = 0; it < kVPer; ++it) {
            const int g = tid + it * kThreads;
            if (kVGroups % kThreads == 0 || g < kVGroups) {
                const int kg = g / (D / 8), col = (g % (D / 8)) * 8;
                const int pos = vt_pos(kg * 4);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const bf16x8 r0 = vr[it][0].term(t), r1 = vr[it][1].term(t);
                    const bf16x8 r2 = vr[it][2].term(t), r3 = vr[it][3].term(t);
#pragma unroll
                    for (int b = 0; b < 8; ++b) {
                        bf16x4 x;
                        x[0] = r0[b]; x[1] = r1[b]; x[2] = r2[b]; x[3] = r3[b];
                        *reinterpret_cast<bf16x4*>(&sm.vt[buf][t][col + b][pos]) = x;
                    }
                }
            }
        }
    }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                       const float* __restrict__ v, float* __restrict__ o,
                       float* __restrict__ lse, int BH, int N, int nqb, float scale_log2)
{
    __shared__ SmemF32<D> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 31;   // query column of this lane in the wave's 32
    const int lh = lane >> 5;   // which 8-element half of each 16-wide k slice

    int qb, bh;
    block_coords<CAUSAL>(blockIdx.x, BH, nqb, qb, bh);
    const size_t head_off = (size_t)bh * (size_t)N * D;
    const float* qh = q + head_off;
    const float* kh = k + head_off;
    const float* vh = v + head_off;

    const int q0 = qb * kBr;
    const int qw0 = q0 + wave * 32;   // first query of this wave
    const int qi = qw0 + li;          // this lane's query row

    // Q fragment (B operand of S^T = K Q^T): row qi, d slice c*16 + lh*8 + 0..7.
    bf16x8 qf[2][D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        const Chunk8 ch = qi < N ? Chunk8::load(qh + (size_t)qi * D + c * 16 + lh * 8)
                                 : Chunk8::zero();
        qf[0][c] = ch.term(0);
        qf[1][c] = ch.term(1);
    }

    const int nkb_all = (N + kBc - 1) / kBc;
    const int kb_end = CAUSAL ? min(nkb_all, (q0 + kBr - 1) / kBc + 1) : nkb_all;

    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    float m_run = neg_inf();  // running max, base-2 scaled domain
    float l_run = 0.f;        // this lane's share of the running sum

    TileLoaderF32<D> ld;
    ld.load(kh, vh, 0, N, tid);
    ld.store(sm, 0, tid);
    __syncthreads();

    for (int kb = 0; kb < kb_end; ++kb) {
        const int buf = kb & 1;
        const int j0 = kb * kBc;
        const bool has_next = kb + 1 < kb_end;
        if (has_next) ld.load(kh, vh, j0 + kBc, N, tid);

        if (!CAUSAL || j0 <= qw0 + 31) {
            f32x16 s[kBc / 32];
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st) {
                s[st] = f32x16{};
#pragma unroll
                for (int c = 0; c < D / 16; ++c) {
                    const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(&sm.k[buf][0][st * 32 + li][c * 16 + lh * 8]);
                    const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(&sm.k[buf][1][st * 32 + li][c * 16 + lh * 8]);
                    s[st] = mfma(k0, qf[0][c], s[st]);
                    s[st] = mfma(k1, qf[0][c], s[st]);
                    s[st] = mfma(k0, qf[1][c], s[st]);
                }
            }
            const bool need_mask = (j0 + kBc > N) || (CAUSAL && j0 + kBc - 1 > qw0);
            if (need_mask) {
#pragma unroll
                for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = j0 + score_key(st, r, lh);
                        const bool ok = j < N && (!CAUSAL || j <= qi);
                        s[st][r] = ok ? s[st][r] : neg_inf();
                    }
            }
            float mraw = neg_inf();
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, s[st][r]);
            mraw = max_with_partner(mraw);
            const float mtile = mraw > neg_inf() ? mraw * scale_log2 : neg_inf();
            const bool grow = mtile > m_run;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float m_new = grow ? mtile : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < D / 32; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
            }
            bf16x8 pf[2][kBc / 32][2];
            l_run += need_mask ? probs<true, 2>(s, scale_log2, m_run, pf)
                               : probs<false, 2>(s, scale_log2, m_run, pf);
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
#pragma unroll
                for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int kc = st * 32 + h2 * 16 + lh * 8;
                        const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(&sm.vt[buf][0][t * 32 + li][kc]);
                        const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(&sm.vt[buf][1][t * 32 + li][kc]);
                        acc[t] = mfma(v0, pf[0][st][h2], acc[t]);
                        acc[t] = mfma(v1, pf[0][st][h2], acc[t]);
                        acc[t] = mfma(v0, pf[1][st][h2], acc[t]);
                    }
        }

        if (has_next) ld.store(sm, buf ^ 1, tid);
        __syncthreads();
    }

    const float l_tot = sum_with_partner(l_run);
    if (qi < N) {
        const float inv = 1.0f / l_tot;
        float* orow = o + head_off + (size_t)qi * D;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store4(orow + t * 32 + g * 8 + lh * 4, acc[t][g * 4 + 0] * inv,
                       acc[t][g * 4 + 1] * inv, acc[t][g * 4 + 2] * inv, acc[t][g * 4 + 3] * inv);
        if (lh == 0)
            lse[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const float* q, const float* k, const float* v, float* o, float* lse,
                      int BH, int N, float scale_log2, hipStream_t stream)
{
    const int nqb = (N + kBr - 1) / kBr;
    const dim3 grid((unsigned)((long long)BH * nqb));
    hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, stream, q, k, v,
                       o, lse, BH, N, nqb, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                      int BH, int N, int d, float scale_log2, bool causal, hipStream_t stream)
{
    if (d == 64)
        return causal ? launch_one<64, true>(q, k, v, o, lse, BH, N, scale_log2, stream)
                      : launch_one<64, false>(q, k, v, o, lse, BH, N, scale_log2, stream);
    return causal ? launch_one<128, true>(q, k, v, o, lse, BH, N, scale_log2, stream)
                  : launch_one<128, false>(q, k, v, o, lse, BH, N, scale_log2, stream);
}

}  // namespace fa
