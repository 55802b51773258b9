// Device helpers shared by the attention-forward kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>

#include "fa_kernels.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = kWaves * 64;

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float neg_inf() { return -__builtin_inff(); }

// max(x[l], x[l ^ 32]) in every lane: v_permlane32_swap(x, x) hands lane l
// the pair (x[l % 32], x[l % 32 + 32]).
__device__ inline float max_with_partner(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_with_partner(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline void store4(__bf16* p, float a, float b, float c, float d) {
    bf16x4 r;
    r[0] = (__bf16)a; r[1] = (__bf16)b; r[2] = (__bf16)c; r[3] = (__bf16)d;
    *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ inline void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Score layout of one wave (S^T = K Q^T on 32x32x16 MFMAs): lane l holds
// query column l % 32 of the wave's 32 rows and, for each 32-key sub-tile,
// the 16 keys (r >> 2) * 8 + (l >> 5) * 4 + (r & 3), r = 0..15.
__device__ inline int score_key(int st, int r, int lh) {
    return st * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
}

// p = exp2(s * c - m) for the lane's kBc/2 scores, rounded to bf16 as the B
// operand of the P V product (pf[0]; pf[1] = bf16 remainder when NT == 2);
// returns the lane's sum of the unrounded p. MASKED: masked scores hold -inf
// and give p = 0 even when c = 0.
// [FlashAttention: The GPU Memory Hack That Changed Everything, "The Tiling
//  Strategy": exp(S_ij - m_new) and its row sum, in base 2 with the scale
//  folded into one FMA]
template <bool MASKED, int NT>
__device__ inline float probs(const f32x16 (&s)[kBc / 32], float c, float m,
                              bf16x8 (&pf)[NT][kBc / 32][2])
{
    float ls[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short dependency chains
#pragma unroll
    for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float x = s[st][h2 * 8 + r];
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -m));
                if (MASKED) p = x > neg_inf() ? p : 0.f;
                ls[r & 3] += p;
                const __bf16 ph = (__bf16)p;
                pf[0][st][h2][r] = ph;
                if constexpr (NT == 2) pf[1][st][h2][r] = (__bf16)(p - (float)ph);
            }
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
}

// Work split over (batch*head, query block).
// [FlashAttention: The GPU Memory Hack That Changed Everything,
//  "FlashAttention-2": parallelism over the sequence dimension]
// Consecutive workgroup ids go round-robin to the 8 XCDs, each with its own
// L2. When the grid divides evenly, XCD x gets one contiguous run of the
// (head, query block) sequence, so the query blocks of a head run side by
// side on one XCD and read the same K/V tiles through the same L2. Within a
// head, causal blocks go heaviest first (largest query-block index), so each
// XCD's stream ends with short blocks.
constexpr int kXcds = 8;

template <bool CAUSAL>
__device__ inline void block_coords(int L, int BH, int nqb, int& qb, int& bh) {
    const int total = BH * nqb;
    const int idx = total % kXcds == 0 ? (L % kXcds) * (total / kXcds) + L / kXcds : L;
    bh = idx / nqb;
    const int r = idx - bh * nqb;
    qb = CAUSAL ? nqb - 1 - r : r;
}

}  // namespace fa
