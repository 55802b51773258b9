// FlashAttention forward kernel for bf16 storage on CDNA4 (gfx950, MI355X).
//
// Method: [FlashAttention: The GPU Memory Hack That Changed Everything
// (ai.branddocks.com, episode 75), "FlashAttention: IO-Aware Tiling" / "The
// Tiling Strategy" and "The Online Softmax Trick"]: an outer loop over query
// blocks, an inner loop over key/value blocks staged in on-chip memory, and a
// running (max, sum, unnormalized output) per query row that is rescaled
// when the running max grows; the output is divided by the sum once, at the
// end. The split over (batch*head x query block) follows the same page's
// "FlashAttention-2" section (parallelism over the sequence).
//
// gfx950 mapping (this file's own design):
//  * One workgroup = 4 wave64s = 128 query rows; each wave owns 32 rows.
//  * Scores are produced transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    A = K tile from LDS (32 keys x 16 of d), B = the wave's Q fragment held
//    in VGPRs for the whole loop. In the 32x32 accumulator layout a lane
//    holds ONE query (column) and 16 keys, so the row max and row sum are
//    lane-local up to one v_permlane32_swap with the partner lane l ^ 32.
//  * O^T = V^T P^T on the same MFMA: the lane's probabilities of a 32-key
//    sub-tile are directly the B operand of two MFMAs, so P never leaves
//    registers. V stays row-major in LDS; its A operand (8 keys of one d
//    column per lane) comes from two ds_read_b64_tr_b16 transpose reads: in
//    each 16-lane group, lanes 4k..4k+3 point at 16 consecutive d values of
//    key k and lane i receives d column i of the 4 keys.
//  * K/V tiles (64 keys) go from HBM straight into LDS with
//    buffer_load_dwordx4 ... lds (no VGPR staging), double-buffered: the next
//    tile is in flight while the current one is consumed; one barrier per
//    tile. Buffer-resource bounds make rows past the sequence end read as 0.
//  * LDS rows hold 16-byte chunks XOR-swizzled by row, so that the K reads
//    (16 rows, same chunk) and the V transpose reads (4 rows x 4 chunks per
//    32 lanes) hit distinct banks.
//  * Softmax in base 2: p = exp2(s * scale*log2(e) - m) is one FMA and one
//    v_exp_f32 per score; the row max is taken on the raw scores. The running
//    max is exact, but a wave in which no row's max grew skips the
//    acc *= alpha pass (alpha would be exactly 1).
//  * Causal: key tiles past the workgroup's last query are never loaded, a
//    wave skips tiles that lie wholly above its 32 rows, and the mask is
//    applied only on tiles that cross a wave's diagonal or the sequence end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_common.h"

namespace fa {
namespace {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct Tile {
    static constexpr int kRowBytes = D * 2;                 // one key row, bf16
    static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
    static constexpr int kBytes = kBc * kRowBytes;          // one K or V tile
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;   // rows per wave-wide load
    static constexpr int kLoadsPerWave = kBytes / 1024 / kWaves;
    static_assert(kLoadsPerWave * 1024 * kWaves == kBytes, "tile must split over waves");

    // Physical 16-byte chunk slot of logical chunk c in tile row r is c ^ swz(r).
    // D = 128 (16 chunks/row, rows 256 B apart): a bijection of r mod 16 whose
    //   value over 4 consecutive rows differs in bits 2-3.
    // D = 64 (8 chunks/row, rows 128 B apart, so row parity picks the bank
    //   half): a bijection of (r >> 1) mod 8 whose value over rows r, r+2
    //   differs in bit 2.
    __device__ static int swz(int r) {
        if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
        else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    }
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate (gfx9 encoding): vmcnt(0), expcnt and lgkmcnt unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;

// Raw buffer resource over [base, base + bytes): offsets past `bytes` read 0.
__device__ inline i32x4 buffer_rsrc(const void* base, unsigned bytes) {
    const unsigned long long a = reinterpret_cast<unsigned long long>(base);
    return i32x4{(int)(unsigned)a, (int)(unsigned)(a >> 32), (int)bytes, 0x00020000};
}

__device__ inline unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// One wave-wide load straight into LDS: lane i's 16 bytes at byte offset
// `voff` of the buffer land at LDS address base + 16*i. Issued as inline asm
// so that the compiler's wait-count pass does not treat later LDS reads of
// the other buffer as dependent on it; the kernel waits for these loads
// explicitly (vmcnt) before the barrier that publishes the tile. M0 carries
// the LDS base; the kernel uses M0 for nothing else.
__device__ inline void lds_dma16(i32x4 rsrc, unsigned voff, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :: "v"(voff), "s"(lds_base), "s"(rsrc) : "memory");
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                        const __bf16* __restrict__ v, __bf16* __restrict__ o,
                        float* __restrict__ lse, int BH, int N, int nqb, float scale_log2)
{
    using TL = Tile<D>;
    // K and V tiles, double-buffered each, rows swizzled. K runs one tile
    // ahead of V: while the softmax of tile j runs, the scores of tile j+1
    // are produced from K_{j+1}, and P_j meets V_j afterwards.
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf[2][TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf[2][TL::kBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases in SGPRs
    const int lane = tid & 63;
    const int li = lane & 31;   // query column of this lane in the wave's 32
    const int lh = lane >> 5;   // which 8-element half of each 16-wide k slice

    int qb, bh;
    block_coords<CAUSAL>(blockIdx.x, BH, nqb, qb, bh);
    const size_t head_off = (size_t)bh * (size_t)N * D;
    const __bf16* qh = q + head_off;
    const __bf16* kh = k + head_off;
    const __bf16* vh = v + head_off;

    const int q0 = qb * kBr;
    const int qw0 = q0 + wave * 32;   // first query of this wave
    const int qi = qw0 + li;          // this lane's query row

    // Q fragment (B operand of S^T = K Q^T): row qi, d slice c*16 + lh*8 + 0..7.
    bf16x8 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qf[c] = qi < N ? *reinterpret_cast<const bf16x8*>(qh + (size_t)qi * D + c * 16 + lh * 8)
                       : bf16x8{};
    // Retire the Q loads here, visibly to the compiler's wait-count pass
    // (s_waitcnt vmcnt(0)); otherwise it keeps a vmcnt(0) inside the loop,
    // which would also wait for the next tiles' loads in flight.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // Direct loads: this wave's load `it` of a tile fills LDS bytes
    // [n*1024, n*1024 + 1024), n = wave*kLoadsPerWave + it; lane i fills the
    // 16-byte slot i there, i.e. row n*kRowsPerLoad + i / kChunks, physical
    // chunk i % kChunks, which holds logical chunk (i % kChunks) ^ swz(row).
    int ld_off[TL::kLoadsPerWave];
#pragma unroll
    for (int it = 0; it < TL::kLoadsPerWave; ++it) {
        const int n = wave * TL::kLoadsPerWave + it;
        const int row = n * TL::kRowsPerLoad + lane / TL::kChunks;
        const int lchunk = (lane % TL::kChunks) ^ TL::swz(row);
        ld_off[it] = row * TL::kRowBytes + lchunk * 16;
    }
    auto issue = [&](const __bf16* src, int kb, unsigned char* dst) {
        const int j0 = kb * kBc;
        const unsigned bytes = (unsigned)min(kBc, N - j0) * TL::kRowBytes;
        const i32x4 rs = buffer_rsrc(src + (size_t)j0 * D, bytes);
#pragma unroll
        for (int it = 0; it < TL::kLoadsPerWave; ++it)
            lds_dma16(rs, ld_off[it], lds_addr(dst + (wave * TL::kLoadsPerWave + it) * 1024));
    };
    // Rows of a partial last V tile past the sequence end must hold finite
    // values (their probabilities are 0, and 0 * NaN would leak), so they are
    // cleared once the tile's loads have landed. Partial K rows need nothing:
    // their scores are replaced by -inf.
    auto clear_tail = [&](int kb, unsigned char* dst) {
        const int rows = N - kb * kBc;
        if (rows >= kBc) return;
        for (int x = tid; x < (kBc - rows) * TL::kChunks; x += kThreads) {
            const int row = rows + x / TL::kChunks;
            *reinterpret_cast<bf16x8*>(dst + row * TL::kRowBytes + (x % TL::kChunks) * 16) = bf16x8{};
        }
    };

    // K fragment (A operand of S^T): key row st*32 + li, logical chunk 2c + lh.
    int k_off[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        k_off[c] = li * TL::kRowBytes + (((2 * c + lh) ^ TL::swz(li)) * 16);

    // V^T fragment (A operand of O^T += V^T P^T) by two transpose reads: for
    // read s (slots 4s..4s+3) lane l points at key 4*lh + (l % 16) / 4 + 8s of
    // the 16-key chunk and d = tt*32 + ((l / 16) % 2) * 16 + 4 * (l % 4).
    int v_off[D / 32][2];
#pragma unroll
    for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int key = 4 * lh + (lane % 16) / 4 + 8 * s;
            const int d0 = tt * 32 + ((lane / 16) % 2) * 16 + 4 * (lane % 4);
            v_off[tt][s] = key * TL::kRowBytes + (((d0 / 8) ^ TL::swz(key)) * 16) + (d0 % 8) * 2;
        }

    // S^T tile of 64 keys from the K tile at kt.
    auto scores = [&](const unsigned char* kt, f32x16 (&s)[kBc / 32]) {
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) {
            s[st] = f32x16{};
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + st * 32 * TL::kRowBytes + k_off[c]);
                s[st] = mfma(kf, qf[c], s[st]);
            }
        }
    };
    // Replace the scores of invisible keys (past N, or after the query when
    // causal) by -inf.
    auto mask = [&](int kb, f32x16 (&s)[kBc / 32]) {
        const int j0 = kb * kBc;
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = j0 + score_key(st, r, lh);
                const bool ok = j < N && (!CAUSAL || j <= qi);
                s[st][r] = ok ? s[st][r] : neg_inf();
            }
    };
    // A wave whose 32 rows all precede a tile's first key skips that tile.
    auto active = [&](int kb) { return !CAUSAL || kb * kBc <= qw0 + 31; };

    const int nkb_all = (N + kBc - 1) / kBc;
    const int nkb = CAUSAL ? min(nkb_all, (q0 + kBr - 1) / kBc + 1) : nkb_all;
    // Tiles [0, nfull) need no mask for any wave of the workgroup: all their
    // keys are < N and (causal) <= the workgroup's first query q0.
    const int nfull = min(CAUSAL ? (q0 + 1) / kBc : nkb_all, N / kBc);

    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    float m_run = neg_inf();  // running max, base-2 scaled domain
    float l_run = 0.f;        // this lane's share of the running sum

    // ---- prologue: K_0, V_0 (and K_1) in LDS; scores of tile 0
    issue(kh, 0, kbuf[0]);
    issue(vh, 0, vbuf[0]);
    if (nkb > 1) issue(kh, 1, kbuf[1]);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    clear_tail(0, vbuf[0]);
    __syncthreads();
    f32x16 s_cur[kBc / 32];
    scores(kbuf[0], s_cur);
    __syncthreads();  // kbuf[0] is free for K_2

    // One key tile: softmax of tile kb (its scores are in s_cur) and, in the
    // same block so that they overlap, the scores of tile kb+1; then
    // O^T = alpha * O^T + V^T P^T. MASKED tiles first replace invisible
    // scores by -inf (a compile-time choice: the interior loop carries no
    // mask code at all).
    auto tile = [&](auto masked, int kb) {
        constexpr bool MASKED = decltype(masked)::value;
        // In LDS now: K_{kb+1} in kbuf[(kb+1)&1], V_kb in vbuf[kb&1].
        if (kb + 2 < nkb) issue(kh, kb + 2, kbuf[kb & 1]);
        if (kb + 1 < nkb) issue(vh, kb + 1, vbuf[(kb + 1) & 1]);
        const bool has_next = kb + 1 < nkb && active(kb + 1);
        f32x16 s_next[kBc / 32];

        if (active(kb)) {
            if constexpr (MASKED) mask(kb, s_cur);
            bool grow;
            float alpha;
            bf16x8 pf[1][kBc / 32][2];
            auto softmax = [&]() {
                float mraw = neg_inf();
#pragma unroll
                for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, s_cur[st][r]);
                mraw = max_with_partner(mraw);
                // scale >= 0, so the scaled max is scale_log2 * raw max
                const float mtile = mraw > neg_inf() ? mraw * scale_log2 : neg_inf();
                grow = mtile > m_run;
                const float m_new = grow ? mtile : m_run;
                alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                const float lsum = probs<false, 1>(s_cur, scale_log2, m_run, pf);
                l_run = l_run * alpha + lsum;
            };
            if (has_next) {
                softmax();
                scores(kbuf[(kb + 1) & 1], s_next);
            } else {
                softmax();
            }

            // alpha == 1 unless some row's max grew
            if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
                for (int t = 0; t < D / 32; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
            }
            const unsigned char* vt = vbuf[kb & 1];
#pragma unroll
            for (int tt = 0; tt < D / 32; ++tt) {
#pragma unroll
                for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const unsigned char* base = vt + (st * 32 + h2 * 16) * TL::kRowBytes;
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s16x4*)(base + v_off[tt][0]));
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s16x4*)(base + v_off[tt][1]));
                        const s16x4 lohi[2] = {lo, hi};
                        bf16x8 vf;
                        __builtin_memcpy(&vf, lohi, sizeof(vf));
                        acc[tt] = mfma(vf, pf[0][st][h2], acc[tt]);
                    }
            }
        }

        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's loads of the next tiles
        if (kb + 1 < nkb) clear_tail(kb + 1, vbuf[(kb + 1) & 1]);
        __syncthreads();
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) s_cur[st] = s_next[st];
    };

    int kb = 0;
    for (; kb < nfull; ++kb) tile(std::false_type{}, kb);
    for (; kb < nkb; ++kb) tile(std::true_type{}, kb);

    // ---- epilogue: O = acc / l, lse = (m2 + log2 l) * ln 2
    const float l_tot = sum_with_partner(l_run);
    if (qi < N) {
        const float inv = 1.0f / l_tot;
        __bf16* orow = o + head_off + (size_t)qi * D;
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
hipError_t launch_one(const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o, float* lse,
                      int BH, int N, float scale_log2, hipStream_t stream)
{
    const int nqb = (N + kBr - 1) / kBr;
    const dim3 grid((unsigned)((long long)BH * nqb));
    hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, stream, q, k, v,
                       o, lse, BH, N, nqb, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                       int BH, int N, int d, float scale_log2, bool causal, hipStream_t stream)
{
    const __bf16* q_ = static_cast<const __bf16*>(q);
    const __bf16* k_ = static_cast<const __bf16*>(k);
    const __bf16* v_ = static_cast<const __bf16*>(v);
    __bf16* o_ = static_cast<__bf16*>(o);
    if (d == 64)
        return causal ? launch_one<64, true>(q_, k_, v_, o_, lse, BH, N, scale_log2, stream)
                      : launch_one<64, false>(q_, k_, v_, o_, lse, BH, N, scale_log2, stream);
    return causal ? launch_one<128, true>(q_, k_, v_, o_, lse, BH, N, scale_log2, stream)
                  : launch_one<128, false>(q_, k_, v_, o_, lse, BH, N, scale_log2, stream);
}

}  // namespace fa
