// FlashAttention forward kernel for CDNA4 (gfx950, MI355X).
//
// Method: [FlashAttention: The GPU Memory Hack That Changed Everything
// (ai.branddocks.com, episode 75), "FlashAttention: IO-Aware Tiling" / "The
// Tiling Strategy" and "The Online Softmax Trick"]: an outer loop over query
// blocks, an inner loop over key/value blocks staged in on-chip memory, and a
// running (max, sum, unnormalized output) per query row that is rescaled
// when the running max grows; the output is divided by the sum once, at the
// end. The work split over (batch*head x query block) follows the same
// page's "FlashAttention-2" section (parallelism over the sequence).
//
// gfx950 mapping (this file's own design):
//  * One workgroup = 4 wave64s = 128 query rows; each wave owns 32 rows.
//  * Scores are produced transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    A = K tile from LDS (32 keys x 16 of d), B = the wave's Q fragment held
//    in VGPRs for the whole loop. In the 32x32 accumulator layout a lane
//    holds ONE query (column) and 16 keys, so the row max and row sum are
//    almost entirely lane-local (one exchange with lane^32).
//  * O^T = V^T P^T on the same MFMA: the lane's 16 probabilities of a 32-key
//    sub-tile are directly the B operand of two MFMAs (8 keys per lane each),
//    so P never leaves registers. V is stored in LDS transposed, [d][keys],
//    with the keys of every 16-key chunk permuted so that each lane's 8 keys
//    are one contiguous 16-byte LDS read.
//  * K/V tiles (64 keys) are double-buffered in LDS: the next tile's global
//    loads are issued before the current tile's MFMAs and written to the
//    other LDS buffer afterwards; one barrier per tile.
//  * Softmax in base 2: p = exp2(s * scale*log2(e) - m) is one FMA and one
//    v_exp_f32 per score; the row max is taken on the raw scores.
//  * The running max is exact (the top probability of a row is exactly 1.0,
//    which bf16 P represents exactly), but a wave in which no row's max grew
//    in this tile skips the acc *= alpha pass: alpha would be exactly 1.
//  * Causal: key tiles past the workgroup's last query are never loaded, a
//    wave skips tiles that lie wholly above its 32 rows, and the mask is
//    applied only on tiles that cross a wave's diagonal or the sequence end.
//  * fp32 storage: every operand x is split into bf16 hi = rn(x) and
//    lo = rn(x - hi); products use hi*hi + lo*hi + hi*lo (3 MFMAs), which
//    keeps scores and P V near fp32 accuracy on the bf16 matrix cores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_kernel.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = kWaves * 64;
constexpr int kPad = 8;                // bf16 elements of padding per LDS row (16 bytes)

template <typename T> struct Terms { static constexpr int n = 1; };  // bf16: exact operands
template <> struct Terms<float> { static constexpr int n = 2; };     // fp32: hi + lo

template <int D, int NT>
struct alignas(16) Smem {
    __bf16 k[2][NT][kBc][D + kPad];    // K tile, row-major [key][d]
    __bf16 vt[2][NT][D][kBc + kPad];   // V tile transposed [d][permuted key]
};

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- global I/O

// 8 consecutive elements of a row, as raw storage, and their bf16 terms.
template <typename T> struct Chunk;
template <> struct Chunk<__bf16> {
    bf16x8 x;
    __device__ static Chunk load(const __bf16* p) { return Chunk{*reinterpret_cast<const bf16x8*>(p)}; }
    __device__ static Chunk zero() { return Chunk{bf16x8{}}; }
    __device__ bf16x8 term(int) const { return x; }
};
template <> struct Chunk<float> {
    f32x4 a, b;
    __device__ static Chunk load(const float* p) {
        const f32x4* v = reinterpret_cast<const f32x4*>(p);
        return Chunk{v[0], v[1]};
    }
    __device__ static Chunk zero() { return Chunk{f32x4{}, f32x4{}}; }
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

__device__ inline void store4(__bf16* p, float a, float b, float c, float d) {
    bf16x4 r;
    r[0] = (__bf16)a; r[1] = (__bf16)b; r[2] = (__bf16)c; r[3] = (__bf16)d;
    *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ inline void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Position of key offset `jo` (multiple of 4, within a 64-key tile) in a
// transposed V row. Inside each 16-key chunk, key 4*a+b (a, b in 0..3) goes
// to 8*(a&1) + 4*(a>>1) + b: lane half h of the score layout holds keys
// {4h..4h+3, 8+4h..8+4h+3} of the chunk, now positions 8h..8h+7.
__device__ inline int vt_pos(int jo) {
    const int a = (jo >> 2) & 3;
    return (jo & ~15) + ((a & 1) << 3) + ((a >> 1) << 2);
}

// Global -> registers staging of one K/V tile, and registers -> LDS.
template <int D, typename T>
struct TileLoader {
    static constexpr int NT = Terms<T>::n;
    static constexpr int kKChunks = kBc * D / 8;            // 8-element K chunks
    static constexpr int kKPer = kKChunks / kThreads;       // per thread
    static constexpr int kVGroups = (kBc / 4) * (D / 8);    // 4 keys x 8 d
    static constexpr int kVPer = (kVGroups + kThreads - 1) / kThreads;
    static_assert(kKChunks % kThreads == 0, "K tile must split evenly");

    Chunk<T> kr[kKPer];
    Chunk<T> vr[kVPer][4];

    __device__ void load(const T* __restrict__ kh, const T* __restrict__ vh, int j0, int N, int tid) {
#pragma unroll
        for (int it = 0; it < kKPer; ++it) {
            const int c = tid + it * kThreads;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
            const int j = j0 + row;
            kr[it] = j < N ? Chunk<T>::load(kh + (size_t)j * D + col) : Chunk<T>::zero();
        }
#pragma unroll
        for (int it = 0; it < kVPer; ++it) {
            const int g = tid + it * kThreads;
            if (kVGroups % kThreads == 0 || g < kVGroups) {
                const int kg = g / (D / 8), col = (g % (D / 8)) * 8;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int j = j0 + kg * 4 + a;
                    vr[it][a] = j < N ? Chunk<T>::load(vh + (size_t)j * D + col) : Chunk<T>::zero();
                }
            }
        }
    }

    __device__ void store(Smem<D, NT>& sm, int buf, int tid) const {
#pragma unroll
        for (int it = 0; it < kKPer; ++it) {
            const int c = tid + it * kThreads;
            const int row = c / (D / 8), col = (c % (D / 8)) * 8;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *reinterpret_cast<bf16x8*>(&sm.k[buf][t][row][col]) = kr[it].term(t);
        }
#pragma unroll
        for (int it = 0; it < kVPer; ++it) {
            const int g = tid + it * kThreads;
            if (kVGroups % kThreads == 0 || g < kVGroups) {
                const int kg = g / (D / 8), col = (g % (D / 8)) * 8;
                const int pos = vt_pos(kg * 4);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
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

// ---------------------------------------------------------------- softmax step

// p = exp2(s * c - m) for the lane's kBc/2 scores, packed to bf16 as the B
// operand of the P V product; returns the lane's sum of p. MASKED: masked
// scores hold -inf and must give p = 0 even when c = 0.
template <bool MASKED, int NT>
__device__ inline float probs(const f32x16 (&s)[kBc / 32], float c, float m,
                              bf16x8 (&pf)[NT][kBc / 32][2])
{
    float lsum = 0.f;
#pragma unroll
    for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float x = s[st][h2 * 8 + r];
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -m));
                if (MASKED) p = x > -__builtin_inff() ? p : 0.f;
                lsum += p;
                const __bf16 ph = (__bf16)p;
                pf[0][st][h2][r] = ph;
                if constexpr (NT == 2) pf[1][st][h2][r] = (__bf16)(p - (float)ph);
            }
    return lsum;
}

// ---------------------------------------------------------------- the kernel

template <int D, bool CAUSAL, typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   T* __restrict__ o, float* __restrict__ lse, int BH, int N, int nqb,
                   float scale_log2)
{
    constexpr int NT = Terms<T>::n;
    __shared__ Smem<D, NT> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 31;   // query column of this lane in the wave's 32
    const int lh = lane >> 5;   // which 8-element half of each 16-wide k slice

    // Work split: causal blocks heaviest-first (largest query block index),
    // heads fastest so concurrently running blocks spread over heads.
    const int L = blockIdx.x;
    int qb, bh;
    if (CAUSAL) {
        qb = nqb - 1 - L / BH;
        bh = L % BH;
    } else {
        qb = L % nqb;
        bh = L / nqb;
    }
    const size_t head_off = (size_t)bh * (size_t)N * D;
    const T* qh = q + head_off;
    const T* kh = k + head_off;
    const T* vh = v + head_off;

    const int q0 = qb * kBr;
    const int qw0 = q0 + wave * 32;           // first query of this wave
    const int qi = qw0 + li;                  // this lane's query row

    // Q fragment (B operand of S^T = K Q^T): row qi, d slice c*16 + lh*8 + 0..7.
    bf16x8 qf[NT][D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        const Chunk<T> ch = qi < N ? Chunk<T>::load(qh + (size_t)qi * D + c * 16 + lh * 8)
                                   : Chunk<T>::zero();
#pragma unroll
        for (int t = 0; t < NT; ++t) qf[t][c] = ch.term(t);
    }

    const int nkb_all = (N + kBc - 1) / kBc;
    const int kb_end = CAUSAL ? min(nkb_all, (q0 + kBr - 1) / kBc + 1) : nkb_all;

    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    float m_run = -__builtin_inff();  // reference max, base-2 scaled domain
    float l_run = 0.f;                // this lane's share of the running sum

    TileLoader<D, T> ld;
    ld.load(kh, vh, 0, N, tid);
    ld.store(sm, 0, tid);
    __syncthreads();

    for (int kb = 0; kb < kb_end; ++kb) {
        const int buf = kb & 1;
        const int j0 = kb * kBc;
        const bool has_next = kb + 1 < kb_end;
        if (has_next) ld.load(kh, vh, j0 + kBc, N, tid);

        // A wave whose 32 rows all precede this tile's first key has nothing to do.
        const bool active = !CAUSAL || j0 <= qw0 + 31;
        if (active) {
            // ---- S^T = K Q^T: two 32-key sub-tiles
            f32x16 s[kBc / 32];
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st) {
                s[st] = f32x16{};
#pragma unroll
                for (int c = 0; c < D / 16; ++c) {
                    const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(&sm.k[buf][0][st * 32 + li][c * 16 + lh * 8]);
                    s[st] = mfma(k0, qf[0][c], s[st]);
                    if constexpr (NT == 2) {
                        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(&sm.k[buf][1][st * 32 + li][c * 16 + lh * 8]);
                        s[st] = mfma(k1, qf[0][c], s[st]);
                        s[st] = mfma(k0, qf[1][c], s[st]);
                    }
                }
            }
            // ---- mask where needed; tile row max on the raw scores
            const bool need_mask = (j0 + kBc > N) || (CAUSAL && j0 + kBc - 1 > qw0);
            if (need_mask) {
#pragma unroll
                for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = j0 + st * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
                        const bool ok = j < N && (!CAUSAL || j <= qi);
                        s[st][r] = ok ? s[st][r] : -__builtin_inff();
                    }
            }
            float mraw = -__builtin_inff();
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, s[st][r]);
            mraw = fmaxf(mraw, __shfl_xor(mraw, 32));
            // scale >= 0, so the scaled max is scale_log2 * raw max
            const float mtile = mraw > -__builtin_inff() ? mraw * scale_log2 : -__builtin_inff();

            // ---- new running max; rescale only if some row's max grew
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

            // ---- probabilities p = exp2(s * c - m), row sum, bf16 P fragments
            bf16x8 pf[NT][kBc / 32][2];
            const float lsum = need_mask ? probs<true, NT>(s, scale_log2, m_run, pf)
                                         : probs<false, NT>(s, scale_log2, m_run, pf);
            l_run += lsum;

            // ---- O^T += V^T P^T
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
#pragma unroll
                for (int st = 0; st < kBc / 32; ++st) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int kc = st * 32 + h2 * 16 + lh * 8;
                        const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(&sm.vt[buf][0][t * 32 + li][kc]);
                        acc[t] = mfma(v0, pf[0][st][h2], acc[t]);
                        if constexpr (NT == 2) {
                            const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(&sm.vt[buf][1][t * 32 + li][kc]);
                            acc[t] = mfma(v1, pf[0][st][h2], acc[t]);
                            acc[t] = mfma(v0, pf[1][st][h2], acc[t]);
                        }
                    }
                }
            }
        }

        if (has_next) ld.store(sm, buf ^ 1, tid);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, lse = (m2 + log2 l) * ln 2
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qi < N) {
        const float inv = 1.0f / l_tot;
        T* orow = o + head_off + (size_t)qi * D;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = t * 32 + g * 8 + lh * 4;
                store4(orow + d0, acc[t][g * 4 + 0] * inv, acc[t][g * 4 + 1] * inv,
                       acc[t][g * 4 + 2] * inv, acc[t][g * 4 + 3] * inv);
            }
        if (lh == 0)
            lse[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
    }
}

// ---------------------------------------------------------------- launchers

template <int D, bool CAUSAL, typename T>
static hipError_t launch_one(const T* q, const T* k, const T* v, T* o, float* lse,
                             int BH, int N, float scale_log2, hipStream_t stream)
{
    const int nqb = (N + kBr - 1) / kBr;
    const dim3 grid((unsigned)((long long)BH * nqb));
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, T>), grid, dim3(kThreads), 0, stream,
                       q, k, v, o, lse, BH, N, nqb, scale_log2);
    return hipGetLastError();
}

template <typename T>
static hipError_t dispatch(const T* q, const T* k, const T* v, T* o, float* lse, int BH,
                           int N, int d, float scale_log2, bool causal, hipStream_t stream)
{
    if (d == 64)
        return causal ? launch_one<64, true>(q, k, v, o, lse, BH, N, scale_log2, stream)
                      : launch_one<64, false>(q, k, v, o, lse, BH, N, scale_log2, stream);
    return causal ? launch_one<128, true>(q, k, v, o, lse, BH, N, scale_log2, stream)
                  : launch_one<128, false>(q, k, v, o, lse, BH, N, scale_log2, stream);
}

hipError_t launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                       int BH, int N, int d, float scale_log2, bool causal, hipStream_t stream)
{
    return dispatch(static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                    static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, BH, N, d,
                    scale_log2, causal, stream);
}

hipError_t launch_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                      int BH, int N, int d, float scale_log2, bool causal, hipStream_t stream)
{
    return dispatch(q, k, v, o, lse, BH, N, d, scale_log2, causal, stream);
}

}  // namespace fa
