// Attention backward pass for bf16 storage on CDNA4 (gfx950, MI355X).
//
// Method: [Flash Attention Optimization (aicomputerinstitute.com), "Sizing a
// tile, and why the backward pass recomputes instead of storing"]: the
// forward pass keeps only per-row statistics (here the log-sum-exp), and the
// backward pass recomputes each block of P from Q, K and that statistic
// instead of reading a stored N x N matrix. The gradients are the plain
// derivatives of O = softmax(scale * Q K^T + mask) V:
//     dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij = sum_t dO_it O_it,
//     dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// gfx950 mapping (this file's own design): three kernels, no atomics.
//  * delta: D_i = sum_t dO_it O_it per row into a workspace (HBM-bound).
//  * dkdv: one workgroup per 128 keys of a head, 8 waves: 4 key groups of
//    32, each served by a pair of waves (one keeps the group's K rows, the
//    other its V rows, as MFMA B operands in VGPRs); 64-query tiles of Q and
//    dO stream through LDS. S = Q K^T and dP = dO V^T come out of
//    v_mfma_f32_32x32x16_bf16 with one key per lane column, so P and dS
//    (bf16) are directly the B operands of dV^T += dO^T P and
//    dK^T += Q^T dS, whose A operands are transpose reads of the dO and Q
//    tiles (ds_read_b64_tr_b16) -- the forward kernel's layout with the
//    roles of queries and keys exchanged.
//  * dq: one workgroup per 128 queries (4 waves x 32 rows, two workgroups
//    per CU), streaming K and V tiles like the forward kernel:
//    S^T = K Q^T and dP^T = V dO^T, then dQ^T += K^T dS^T with K^T from
//    transpose reads of the K tile. Grids of at least four rounds of
//    workgroups run the phased form instead: 256 queries per workgroup in
//    two phase-offset wave groups (the forward kernel's structure), one
//    forming dS while the other runs the dQ and score MFMAs. Both forms
//    accumulate in the same order, so their gradients are bitwise equal.
//  * P is recomputed as exp2(s * scale*log2(e) - lse*log2(e)); masked and
//    out-of-range entries are 0. dS is formed in fp32 and rounded to bf16 for
//    its products; all products accumulate in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_common.h"
#include "fa_lds.h"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kBwdRows = kBwdWaves * 32;     // queries (dq) or keys (dkdv) per workgroup
// __builtin_amdgcn_sched_group_barrier instruction classes, and how many MFMAs
// ahead of their use the dq kernel's LDS fragment reads are issued (2, 4 and 6
// measured within 0.3%; more would not fit the VGPR budget).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kDqReadAhead = 4;
constexpr int kDkdvReadAhead = 4;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- delta
// D_i = sum_t dO_it O_it: 16 lanes per row, D/16 elements per lane.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_delta_kernel(const __bf16* __restrict__ o,
                                                           const __bf16* __restrict__ dout,
                                                           float* __restrict__ delta,
                                                           long long rows)
{
    constexpr int kPer = D / 16;
    const long long row = (long long)blockIdx.x * 16 + threadIdx.x / 16;
    const int j = threadIdx.x % 16;
    float s = 0.f;
    if (row < rows) {
        const __bf16* orow = o + row * D + j * kPer;
        const __bf16* drow = dout + row * D + j * kPer;
#pragma unroll
        for (int t = 0; t < kPer; ++t) s += (float)orow[t] * (float)drow[t];
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 16);
    if (row < rows && j == 0) delta[row] = s;
}

// Store 32 columns x 4 of a 32x32 accumulator tile for this lane's row:
// acc[t][g*4+i] is column t*32 + g*8 + lh*4 + i.
template <int D>
__device__ inline void store_row(__bf16* row, const f32x16 (&acc)[D / 32], float mul, int lh)
{
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            store4(row + t * 32 + g * 8 + lh * 4, acc[t][g * 4 + 0] * mul, acc[t][g * 4 + 1] * mul,
                   acc[t][g * 4 + 2] * mul, acc[t][g * 4 + 3] * mul);
}

// Direct loads of one 64-row tile of `src` (rows >= N read as 0 / are not
// written) into LDS, this wave's share.
template <typename TL>
__device__ inline void issue_tile(const __bf16* src, int t, int N, unsigned char* dst,
                                  const int* ld_off, int wave)
{
    constexpr int D = TL::kRowBytes / 2;
    const int j0 = t * kBc;
    const unsigned bytes = (unsigned)min(kBc, N - j0) * TL::kRowBytes;
    const i32x4 rs = buffer_rsrc(src + (size_t)j0 * D, bytes);
#pragma unroll
    for (int it = 0; it < TL::kLoadsPerWave; ++it)
        lds_dma16(rs, ld_off[it], lds_addr(dst + (wave * TL::kLoadsPerWave + it) * 1024));
}

// Rows of a partial last tile past the sequence end are cleared once the
// tile has landed: their weights are 0, and 0 * NaN would leak.
template <typename TL, int THREADS = kBwdThreads>
__device__ inline void clear_tile_tail(int t, int N, unsigned char* dst, int tid)
{
    const int rows = N - t * kBc;
    if (rows >= kBc) return;
    for (int x = tid; x < (kBc - rows) * TL::kChunks; x += THREADS) {
        const int row = rows + x / TL::kChunks;
        *reinterpret_cast<bf16x8*>(dst + row * TL::kRowBytes + (x % TL::kChunks) * 16) = bf16x8{};
    }
}

// ---------------------------------------------------------------- dk, dv
// One workgroup per 128 keys of a head: 4 key groups of 32, each served by a
// pair of waves that share the work of every 64-query tile:
//  * the P-wave keeps its keys' K rows as B operands, forms S = Q K^T and
//    P = exp2(S c - lse2), hands P (bf16) to its partner through LDS, and
//    accumulates dV^T += dO^T P;
//  * the dS-wave keeps the V rows, forms dP = dO V^T, takes P, forms
//    dS = P (dP - D) and accumulates dK^T += Q^T dS.
// Each wave holds one 32x128 accumulator and one operand set (about half the
// registers of a wave doing both), so two waves fit per SIMD; waves w and
// w + 4 share a SIMD and serve different key groups.
// The pair is software-pipelined by one tile and each step has two phases:
// in phase 1 the P-wave runs dV(t) and S(t+1) on the matrix core while the
// dS-wave forms dS(t); in phase 2 the dS-wave runs dK(t) and dP(t+1) while the
// P-wave forms P(t+1). On every SIMD (a P-wave and the dS-wave of another
// group) one wave feeds the matrix core while the other works on the VALU,
// and the barrier between the phases
// also orders the reads of P(t) before the writes of P(t+1), so P needs one
// LDS buffer. Q and dO tiles use three (t, t+1 in use, t+2 loading).
constexpr int kDkdvWaves = 8;
constexpr int kDkdvThreads = kDkdvWaves * 64;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDkdvThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                        const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                        const float* __restrict__ lse, const float* __restrict__ delta,
                        __bf16* __restrict__ dk, __bf16* __restrict__ dv, int BH, int N,
                        int nkblk, float scale_log2, float scale)
{
    using TL = Tile<D, kDkdvWaves>;
    constexpr int L = TL::kLoadsPerWave;
    __shared__ __attribute__((aligned(1024))) unsigned char qbuf[3][TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char dobuf[3][TL::kBytes];
    __shared__ __attribute__((aligned(16))) float lse_s[3][kBc];  // lse * log2(e) per query
    __shared__ __attribute__((aligned(16))) float dl_s[3][kBc];   // D per query
    // P of a tile per key group: [tile & 1][group][sub-tile][half][lane] x 8
    // bf16 (lane-major 16-byte slots, conflict-free).
    __shared__ __attribute__((aligned(16))) bf16x8 p_x[kBwdWaves][kBc / 32][2][64];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int li = lane & 31;
    const int lh = lane >> 5;
    const bool pwave = wave < kBwdWaves;                     // forms P, accumulates dV
    const int grp = pwave ? wave : (wave + kBwdWaves - 1) % kBwdWaves;

    // Key blocks in ascending order: for causal attention the first key
    // blocks see the most queries, so the heaviest work starts first.
    int kblk, bh;
    block_coords<false>(blockIdx.x, BH, nkblk, kblk, bh);
    const size_t head_off = (size_t)bh * (size_t)N * D;
    const __bf16* qh = q + head_off;
    const __bf16* doh = dout + head_off;
    const float* lseh = lse + (size_t)bh * N;
    const float* dlh = delta + (size_t)bh * N;

    const int k0 = kblk * kBwdRows;
    const int kw0 = k0 + grp * 32;    // first key of this wave's group
    const int kj = kw0 + li;          // this lane's key

    // K rows (P-wave) or V rows (dS-wave) of this lane's key as B operands.
    bf16x8 bf[D / 16];
    {
        const __bf16* row = (pwave ? k : v) + head_off + (size_t)kj * D;
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            bf[c] = kj < N ? *reinterpret_cast<const bf16x8*>(row + c * 16 + lh * 8) : bf16x8{};
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    int ld_off[L];
#pragma unroll
    for (int it = 0; it < L; ++it) ld_off[it] = TL::load_offset(wave, it, lane);
    // Fragment and transpose-read offsets from two bases: chunk 2c + lh of a
    // row sits at base ^ (c << 5), and the transpose reads of column block tt
    // at base ^ (tt << 6) (the swizzle XORs only chunk bits).
    const int f_base = TL::frag_offset(li, lh);
    const int t_base[2] = {TL::tr_offset(0, 0, lane), TL::tr_offset(0, 1, lane)};

    const int nqt = (N + kBc - 1) / kBc;
    // Causal: query tiles before the block's first key see none of its keys.
    const int t0 = CAUSAL ? k0 / kBc : 0;
    if (t0 >= nqt) return;  // uniform over the workgroup: no barrier is skipped
    // Tiles where some (query, key) pair of the group is invalid: the causal
    // diagonal (including the first tile, whose queries may all precede a
    // group's keys; there every P is 0) and the sequence tail.
    auto need_mask = [&](int u) __attribute__((always_inline)) {
        return (CAUSAL && u * kBc < kw0 + 31) || u * kBc + kBc > N;
    };

    // Tile u of the block's range lives in slot (u - t0) % 3 of the Q, dO
    // and statistics buffers; the straight-line steps below take their slots
    // as compile-time constants.
    // Per-query statistics of tile u: threads 0..63 fetch lse, 64..127 D.
    auto fetch_stats = [&](int u) __attribute__((always_inline)) {
        const int qq = u * kBc + (tid & 63);
        float x = 0.f;
        if (tid < 2 * kBc && qq < N) x = tid < kBc ? lseh[qq] * kLog2e : dlh[qq];
        return x;
    };
    auto put_stats = [&](int sl, float x) __attribute__((always_inline)) {
        if (tid < kBc) lse_s[sl][tid] = x;
        else if (tid < 2 * kBc) dl_s[sl][tid - kBc] = x;
    };
    auto load_tile = [&](int u, int sl) __attribute__((always_inline)) {
        issue_tile<TL>(qh, u, N, qbuf[sl], ld_off, wave);
        issue_tile<TL>(doh, u, N, dobuf[sl], ld_off, wave);
    };
    auto clear_tails = [&](int u, int sl) __attribute__((always_inline)) {
        clear_tile_tail<TL, kDkdvThreads>(u, N, qbuf[sl], tid);
        clear_tile_tail<TL, kDkdvThreads>(u, N, dobuf[sl], tid);
    };

    // S (P-wave, from Q) or dP (dS-wave, from dO) of the tile in slot sl:
    // lane = key, 16 queries per 32-query sub-tile. The A fragments are read
    // kDkdvReadAhead MFMAs ahead of their use.
    f32x16 x[kBc / 32];
    auto scores = [&](auto role, int sl) __attribute__((always_inline)) {
        const unsigned char* at = decltype(role)::value ? qbuf[sl] : dobuf[sl];
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) {
            x[st] = f32x16{};
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                x[st] = mfma(*reinterpret_cast<const bf16x8*>(at + st * 32 * TL::kRowBytes +
                                                              (f_base ^ (c << 5))),
                             bf[c], x[st]);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kDkdvReadAhead, 0);
#pragma unroll
        for (int i = 0; i < kBc / 32 * D / 16 - kDkdvReadAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kDkdvReadAhead, 0);
    };
    // P-wave: P = exp2(s c - lse2) of tile u (slot sl), 0 where masked, into
    // pf and p_x. Query qloc + i of the tile is valid for this lane's key iff
    // lo <= qloc + i < hi (one unsigned compare); tiles that need no mask
    // take a separate path without it.
    bf16x8 pf[kBc / 32][2];
    auto probs = [&](int u, int sl, auto nomask) __attribute__((always_inline)) {
        const int lo = CAUSAL ? kj - u * kBc : 0;
        const int hi = N - u * kBc;
        const float* ls = lse_s[sl];
        auto run = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int qloc = st * 32 + g * 8 + lh * 4;  // queries qloc .. qloc+3
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(&ls[qloc]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = g * 4 + i;
                        float p = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(x[st][r], scale_log2, -l4[i]));
                        if constexpr (decltype(masked)::value)
                            p = (unsigned)(qloc + i - lo) < (unsigned)(hi - lo) ? p : 0.f;
                        pf[st][r >> 3][r & 7] = (__bf16)p;
                    }
                }
                p_x[grp][st][0][lane] = pf[st][0];
                p_x[grp][st][1][lane] = pf[st][1];
            }
        };
        if (!decltype(nomask)::value && need_mask(u)) run(std::true_type{});
        else run(std::false_type{});
    };
    // dS-wave: dS = P (dP - D) of the tile in slot sl into pf, P from the partner.
    auto dscores = [&](int sl) __attribute__((always_inline)) {
        const float* ds_ = dl_s[sl];
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) {
            const bf16x8 p0 = p_x[grp][st][0][lane];
            const bf16x8 p1 = p_x[grp][st][1][lane];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int qloc = st * 32 + g * 8 + lh * 4;
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&ds_[qloc]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = g * 4 + i;
                    const float p = (float)(r < 8 ? p0[r & 7] : p1[r & 7]);
                    pf[st][r >> 3][r & 7] = (__bf16)(p * (x[st][r] - d4[i]));
                }
            }
        }
    };
    f32x16 acc[D / 32];  // dV^T (P-wave) or dK^T (dS-wave): rows d, column = key
#pragma unroll
    for (int tt = 0; tt < D / 32; ++tt) acc[tt] = f32x16{};
    // dV^T += dO^T P (P-wave) or dK^T += Q^T dS (dS-wave) for the tile in
    // slot sl, A operands by transpose reads of the dO or Q tile.
    auto accumulate = [&](auto role, int sl) __attribute__((always_inline)) {
        const unsigned char* tb = decltype(role)::value ? dobuf[sl] : qbuf[sl];
#pragma unroll
        for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int base = (st * 32 + h2 * 16) * TL::kRowBytes;
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(tb + base + (t_base[0] ^ (tt << 6))));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(tb + base + (t_base[1] ^ (tt << 6))));
                    const s16x4 pair[2] = {lo, hi};
                    bf16x8 a;
                    __builtin_memcpy(&a, pair, sizeof(a));
                    acc[tt] = mfma(a, pf[st][h2], acc[tt]);
                }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kDkdvReadAhead, 0);
#pragma unroll
        for (int i = 0; i < D / 32 * kBc / 16 - kDkdvReadAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kDkdvReadAhead, 0);
    };

    // Prologue: tiles t0 and t0 + 1 resident (slots 0 and 1), then P(t0)
    // (P-wave) or dP(t0) (dS-wave).
    load_tile(t0, 0);
    if (t0 + 1 < nqt) load_tile(t0 + 1, 1);
    put_stats(0, fetch_stats(t0));
    if (t0 + 1 < nqt) put_stats(1, fetch_stats(t0 + 1));
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    clear_tails(t0, 0);
    if (t0 + 1 < nqt) clear_tails(t0 + 1, 1);
    __syncthreads();
    if (pwave) {
        scores(std::true_type{}, 0);
        probs(t0, 0, std::false_type{});
    } else {
        scores(std::false_type{}, 0);
    }

    // Step t, two phases per SIMD pair:
    //  phase 1: the P-wave runs dV(t) and S(t+1) on the matrix core while
    //           the dS-wave forms dS(t) and issues tile t+2's loads;
    //  phase 2: the dS-wave runs dK(t) and dP(t+1) while the P-wave issues
    //           its share of tile t+2 and forms P(t+1).
    // The phase barrier also orders P(t)'s reads before P(t+1)'s writes, so
    // one P buffer suffices; the step barrier publishes P(t+1) and tile t+2.
    // Each role runs its own copy of the loop. Steps whose tiles t+1 needs
    // no causal mask and lies inside N, with t + 2 < nqt, are straight-line
    // code, unrolled three at a time so that their slots are constants; the
    // values that cross a barrier there pass through empty volatile asm on
    // both sides of it, so the compiler keeps each phase's work in its phase.
    // Values crossing the step barrier: the accumulator and P(t+1) (P-wave)
    // or dP(t+1) (dS-wave); the phase barrier: the accumulator and S(t+1)
    // (P-wave) or dS(t) (dS-wave).
    auto pin = [&](auto role, auto mid) __attribute__((always_inline)) {
        auto& pfr = pf;  // named outside the discarded branch so both are captured
        auto& xr = x;
#pragma unroll
        for (int tt = 0; tt < D / 32; ++tt) asm volatile("" : "+v"(acc[tt]));
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) {
            if constexpr (decltype(role)::value != decltype(mid)::value)
                asm volatile("" : "+v"(pfr[st][0]), "+v"(pfr[st][1]));
            else
                asm volatile("" : "+v"(xr[st]));
        }
    };
    // First step whose tile t + 1 needs no causal mask for any key of the block.
    const int t_nomask = CAUSAL ? (k0 + kBwdRows - 1 + kBc - 1) / kBc - 1 : 0;
    const int t_full_end = min(N / kBc - 1, nqt - 2);  // straight-line steps t < t_full_end
    auto run = [&](auto role) __attribute__((always_inline)) {
        constexpr bool PW = decltype(role)::value;
        auto step = [&](auto full, int t, auto slot) __attribute__((always_inline)) {
            constexpr bool FULL = decltype(full)::value;
            const int s0 = slot;
            const int s1 = s0 == 2 ? 0 : s0 + 1;
            const int s2 = s0 == 0 ? 2 : s0 - 1;
            if constexpr (FULL) pin(role, std::false_type{});
            __syncthreads();
            if constexpr (FULL) pin(role, std::false_type{});
            float next_stats = 0.f;
            if constexpr (PW) {
                accumulate(role, s0);
                if (FULL || t + 1 < nqt) scores(role, s1);
            } else {
                dscores(s0);
                if (FULL || t + 2 < nqt) {
                    load_tile(t + 2, s2);
                    next_stats = fetch_stats(t + 2);
                }
            }
            if constexpr (FULL) pin(role, std::true_type{});
            __syncthreads();
            if constexpr (FULL) pin(role, std::true_type{});
            if constexpr (PW) {
                if (FULL || t + 2 < nqt) {
                    load_tile(t + 2, s2);
                    next_stats = fetch_stats(t + 2);
                }
                if (FULL || t + 1 < nqt) probs(t + 1, s1, full);
            } else {
                accumulate(role, s0);
                if (FULL || t + 1 < nqt) scores(role, s1);
            }
            if (FULL || t + 2 < nqt) {
                __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));  // this wave's loads of tile t+2
                clear_tails(t + 2, s2);
                put_stats(s2, next_stats);
            }
        };
        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;
        using C2 = std::integral_constant<int, 2>;
        int t = t0, sl = 0;
        // General steps up to the straight-line range, and on until slot 0.
        for (; t < nqt && (t < t_nomask || sl != 0); ++t, sl = sl == 2 ? 0 : sl + 1)
            step(std::false_type{}, t, sl);
        for (; t + 3 <= t_full_end; t += 3) {
            step(std::true_type{}, t, C0{});
            step(std::true_type{}, t + 1, C1{});
            step(std::true_type{}, t + 2, C2{});
        }
        for (; t < nqt; ++t, sl = sl == 2 ? 0 : sl + 1) step(std::false_type{}, t, sl);
    };
    if (pwave) run(std::true_type{});
    else run(std::false_type{});

    if (kj < N) {
        if (pwave) store_row<D>(dv + head_off + (size_t)kj * D, acc, 1.0f, lh);
        else store_row<D>(dk + head_off + (size_t)kj * D, acc, scale, lh);
    }
}

// ---------------------------------------------------------------- dq
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                      const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                      const float* __restrict__ lse, const float* __restrict__ delta,
                      __bf16* __restrict__ dq, int BH, int N, int nqb, float scale_log2,
                      float scale)
{
    using TL = Tile<D, kBwdWaves>;
    constexpr int L = TL::kLoadsPerWave;
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf[2][TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vbuf[2][TL::kBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int li = lane & 31;
    const int lh = lane >> 5;

    int qb, bh;
    block_coords<CAUSAL>(blockIdx.x, BH, nqb, qb, bh);
    const size_t head_off = (size_t)bh * (size_t)N * D;
    const __bf16* kh = k + head_off;
    const __bf16* vh = v + head_off;

    const int q0 = qb * kBwdRows;
    const int qw0 = q0 + wave * 32;
    const int qi = qw0 + li;

    // Q and dO rows of this lane's query as B operands.
    bf16x8 qf[D / 16], df[D / 16];
    {
        const __bf16* qrow = q + head_off + (size_t)qi * D;
        const __bf16* drow = dout + head_off + (size_t)qi * D;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            qf[c] = qi < N ? *reinterpret_cast<const bf16x8*>(qrow + c * 16 + lh * 8) : bf16x8{};
            df[c] = qi < N ? *reinterpret_cast<const bf16x8*>(drow + c * 16 + lh * 8) : bf16x8{};
        }
    }
    const float lse2 = qi < N ? lse[(size_t)bh * N + qi] * kLog2e : 0.f;
    const float dlt = qi < N ? delta[(size_t)bh * N + qi] : 0.f;
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    int ld_off[L];
#pragma unroll
    for (int it = 0; it < L; ++it) ld_off[it] = TL::load_offset(wave, it, lane);
    // Fragment offsets of chunk c and column block tt differ from those of
    // c = 0 and tt = 0 only in bits 5-7 and 6-7 (the swizzle permutes chunk
    // indices by XOR): f(c) = f(0) ^ (c << 5), t(tt, s) = t(0, s) ^ (tt << 6).
    // Only the base offsets stay live; the rest are rebuilt per tile.
    int f_base = TL::frag_offset(li, lh);
    int t_base[2] = {TL::tr_offset(0, 0, lane), TL::tr_offset(0, 1, lane)};

    const int nkb_all = (N + kBc - 1) / kBc;
    const int nkb = CAUSAL ? min(nkb_all, (q0 + kBwdRows - 1) / kBc + 1) : nkb_all;

    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

    issue_tile<TL>(kh, 0, N, kbuf[0], ld_off, wave);
    issue_tile<TL>(vh, 0, N, vbuf[0], ld_off, wave);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    clear_tile_tail<TL>(0, N, kbuf[0], tid);
    clear_tile_tail<TL>(0, N, vbuf[0], tid);
    __syncthreads();

    for (int kb = 0; kb < nkb; ++kb) {
        const int b = kb & 1;
        if (kb + 1 < nkb) {
            issue_tile<TL>(kh, kb + 1, N, kbuf[b ^ 1], ld_off, wave);
            issue_tile<TL>(vh, kb + 1, N, vbuf[b ^ 1], ld_off, wave);
        }
        const bool active = !CAUSAL || kb * kBc <= qw0 + 31;
        if (active) {
            const unsigned char* kt = kbuf[b];
            const unsigned char* vt = vbuf[b];
            asm volatile("" : "+v"(f_base), "+v"(t_base[0]), "+v"(t_base[1]));
            // S^T = K Q^T and dP^T = V dO^T: lane = query, 16 keys per sub-tile.
            f32x16 s[kBc / 32], dp[kBc / 32];
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st) {
                s[st] = f32x16{};
                dp[st] = f32x16{};
#pragma unroll
                for (int c = 0; c < D / 16; ++c) {
                    const int off = st * 32 * TL::kRowBytes + (f_base ^ (c << 5));
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + off);
                    const bf16x8 va = *reinterpret_cast<const bf16x8*>(vt + off);
                    s[st] = mfma(ka, qf[c], s[st]);
                    dp[st] = mfma(va, df[c], dp[st]);
                }
            }
            // K and V fragments a few MFMAs ahead, no further (VGPR budget).
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kDqReadAhead, 0);
#pragma unroll
            for (int i = 0; i < 2 * kBc / 32 * D / 16 - kDqReadAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kDqReadAhead, 0);
            // dS = P * (dP - D) as bf16 B operands; the mask is a separate
            // code path so that unmasked tiles carry no compares or branches.
            bf16x8 dsf[kBc / 32][2];
            auto make_ds = [&](auto masked) __attribute__((always_inline)) {
                constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
                for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][r], scale_log2, -lse2));
                        if constexpr (MASKED) {
                            const int j = kb * kBc + score_key(st, r, lh);
                            const bool ok = j < N && (!CAUSAL || j <= qi);
                            p = ok ? p : 0.f;
                        }
                        dsf[st][r >> 3][r & 7] = (__bf16)(p * (dp[st][r] - dlt));
                    }
            };
            if ((CAUSAL && kb * kBc + kBc - 1 > qw0) || kb * kBc + kBc > N)
                make_ds(std::true_type{});
            else
                make_ds(std::false_type{});
            // dQ^T += K^T dS^T, K^T by transpose reads of the K tile (two per MFMA).
#pragma unroll
            for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
                for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int base = (st * 32 + h2 * 16) * TL::kRowBytes;
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s16x4*)(kt + base + (t_base[0] ^ (tt << 6))));
                        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s16x4*)(kt + base + (t_base[1] ^ (tt << 6))));
                        const s16x4 pair[2] = {lo, hi};
                        bf16x8 ka;
                        __builtin_memcpy(&ka, pair, sizeof(ka));
                        acc[tt] = mfma(ka, dsf[st][h2], acc[tt]);
                    }
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kDqReadAhead, 0);
#pragma unroll
            for (int i = 0; i < D / 32 * kBc / 16 - kDqReadAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kDqReadAhead, 0);
        }
        if (kb + 1 < nkb) {
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
            clear_tile_tail<TL>(kb + 1, N, kbuf[b ^ 1], tid);
            clear_tile_tail<TL>(kb + 1, N, vbuf[b ^ 1], tid);
        }
        __syncthreads();
    }

    if (qi < N) store_row<D>(dq + head_off + (size_t)qi * D, acc, scale, lh);
}

// ---------------------------------------------------------------- dq, phased
// Grids of at least four rounds of workgroups (bwd_dq_phased): one workgroup
// per 256 queries of a head, 8 wave64s of 32 query rows in two
// phase-offset groups, as in the forward kernel (waves w and w + 4 share a
// SIMD). Per key tile j (64 keys) a wave runs
//   A(j): dS(j) = P(j) (dP(j) - D) from S(j) = Q K_j^T and dP(j) = dO V_j^T,
//         P recomputed as exp2(S c - lse2), masked entries 0, dS rounded to
//         bf16 (VALU and transcendental work only);
//   B(j): dQ^T += K_j^T dS(j)^T (K_j^T by transpose reads), then S(j+1) and
//         dP(j+1) (K and V fragments row-major): matrix work only.
// Group 1 runs one phase behind group 0 and every phase ends with a
// workgroup barrier, so on every SIMD one wave feeds the matrix core while
// the other runs the VALU work. S^T and dP^T come out of the 32x32x16 MFMA
// with one query per lane column, so dS is directly the B operand of the
// dQ product. K and V tiles go straight into two rings of four LDS slots
// (tile t in slot t % 4), loaded by the group in its VALU phase: in step j
// group 0 loads V_{j+3} and group 1 loads K_{j+3} (K_t is read in B(t-1)
// and B(t), up to global phase 2t + 2; V_t in B(t-1) only).
constexpr int kDqWaves = 8;
constexpr int kDqThreads = kDqWaves * 64;
constexpr int kDqRows = kDqWaves * 32;  // queries per workgroup
constexpr int kDqRing = 4;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_phased_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                             const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                             const float* __restrict__ lse, const float* __restrict__ delta,
                             __bf16* __restrict__ dq, int BH, int N, int nqb,
                             float scale_log2, float scale)
{
    using TL = Tile<D, kDqWaves>;
    using TG = Tile<D, kDqWaves / 2>;
    constexpr int L = TL::kLoadsPerWave;
    constexpr int LG = TG::kLoadsPerWave;  // = 2L
    __shared__ __attribute__((aligned(1024))) unsigned char kring[kDqRing][TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vring[kDqRing][TL::kBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int lane = tid & 63;
    const int li = lane & 31;
    const int lh = lane >> 5;

    int qb, bh;
    block_coords<CAUSAL>(blockIdx.x, BH, nqb, qb, bh);
    const size_t head_off = (size_t)bh * (size_t)N * D;
    const __bf16* kh = k + head_off;
    const __bf16* vh = v + head_off;

    const int q0 = qb * kDqRows;
    const int qw0 = q0 + wave * 32;
    const int qi = qw0 + li;


    bf16x8 qf[D / 16], df[D / 16];  // this lane's Q and dO rows (B operands), set in the prologue
    float lse2, dlt;                 // its lse * log2(e) and D
    const int nkb_all = (N + kBc - 1) / kBc;
    const int nkb = CAUSAL ? min(nkb_all, (q0 + kDqRows - 1) / kBc + 1) : nkb_all;

    int ld_off[L], gl_off[LG];
#pragma unroll
    for (int it = 0; it < L; ++it) ld_off[it] = TL::load_offset(wave, it, lane);
#pragma unroll
    for (int it = 0; it < LG; ++it) gl_off[it] = TG::load_offset(wave & 3, it, lane);
    // Buffer resource over tile t of `src`; a tile past the last one gets an
    // empty range (nothing is read) so that the loads are still issued and
    // the vmcnt arithmetic holds.
    auto tile_rsrc = [&](const __bf16* src, int t) __attribute__((always_inline)) {
        const int j0 = t * kBc;
        const bool real = t < nkb;
        const unsigned bytes = real ? (unsigned)min(kBc, N - j0) * TL::kRowBytes : 0u;
        return buffer_rsrc(real ? src + (size_t)j0 * D : src, bytes);
    };
    auto issue = [&](const __bf16* src, int t, unsigned char* dst) __attribute__((always_inline)) {
        const i32x4 rs = tile_rsrc(src, t);
#pragma unroll
        for (int it = 0; it < L; ++it)
            lds_dma16(rs, ld_off[it], lds_addr(dst + (wave * L + it) * 1024));
    };
    auto issue_grp = [&](const __bf16* src, int t, unsigned char* dst) __attribute__((always_inline)) {
        const i32x4 rs = tile_rsrc(src, t);
        unsigned lb = lds_addr(dst + (wave & 3) * LG * 1024);
        asm volatile("" : "+s"(lb));
#pragma unroll
        for (int it = 0; it < LG; ++it) lds_dma16(rs, gl_off[it], lb + it * 1024);
    };
    // Rows of a partial last tile past the sequence end are cleared once it
    // has landed: their weights are 0, and 0 * NaN would leak.
    auto clear_tail = [&](int t, unsigned char* dst) __attribute__((always_inline)) {
        const int rows = N - t * kBc;
        if (rows >= kBc) return;
        for (int x = tid; x < (kBc - rows) * TL::kChunks; x += kDqThreads) {
            const int row = rows + x / TL::kChunks;
            *reinterpret_cast<bf16x8*>(dst + row * TL::kRowBytes + (x % TL::kChunks) * 16) = bf16x8{};
        }
    };

    // Fragment offsets from three bases: chunk 2c + lh of a row sits at
    // base ^ (c << 5) and the transpose reads of column block tt at
    // base ^ (tt << 6) (the swizzle XORs chunk bits only and the ring bases
    // are 1024-aligned); ring slot and sub-tile offsets are immediates.
    unsigned kbase = lds_addr(kring[0]), vbase = lds_addr(vring[0]);
    asm volatile("" : "+s"(kbase), "+s"(vbase));
    unsigned k_row = kbase + TL::frag_offset(li, lh);
    unsigned v_row = vbase + TL::frag_offset(li, lh);
    unsigned k_tr[2] = {kbase + TL::tr_offset(0, 0, lane), kbase + TL::tr_offset(0, 1, lane)};

    f32x16 acc[D / 32];  // dQ^T: rows d, column = query
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    f32x16 sc[kBc / 32], dp[kBc / 32];  // S^T and dP^T of the tile whose dS runs next
    bf16x8 dsf[kBc / 32][2];             // dS of the current tile, from A(j) to B(j)

    // S^T = K Q^T and dP^T = V dO^T of the tile in ring slot `slot`; the K
    // and V fragments are read kDqReadAhead MFMAs ahead of their use.
    constexpr int kSPMfmas = 2 * (kBc / 32) * (D / 16);
    auto scores = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) {
            sc[st] = f32x16{};
            dp[st] = f32x16{};
        }
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st) {
                const unsigned off = slot * TL::kBytes + st * 32 * TL::kRowBytes;
                const bf16x8 ka = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                    (size_t)((k_row ^ ((unsigned)c << 5)) + off));
                const bf16x8 va = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                    (size_t)((v_row ^ ((unsigned)c << 5)) + off));
                sc[st] = mfma(ka, qf[c], sc[st]);
                dp[st] = mfma(va, df[c], dp[st]);
            }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kDqReadAhead, 0);
#pragma unroll
        for (int i = 0; i < kSPMfmas - kDqReadAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kDqReadAhead, 0);
    };
    // dQ^T += K^T dS^T for the tile in ring slot `slot`: two transpose reads
    // per MFMA, consecutive MFMAs on different accumulators.
    constexpr int kDqMfmas = (D / 32) * (kBc / 16);
    auto dq_update = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int tt = 0; tt < D / 32; ++tt) {
                    const unsigned off = slot * TL::kBytes + (st * 32 + h2 * 16) * TL::kRowBytes;
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(size_t)((k_tr[0] ^ ((unsigned)tt << 6)) + off));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(size_t)((k_tr[1] ^ ((unsigned)tt << 6)) + off));
                    const s16x4 pair[2] = {lo, hi};
                    bf16x8 ka;
                    __builtin_memcpy(&ka, pair, sizeof(ka));
                    acc[tt] = mfma(ka, dsf[st][h2], acc[tt]);
                }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kDqReadAhead, 0);
#pragma unroll
        for (int i = 0; i < kDqMfmas - kDqReadAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kDqReadAhead, 0);
    };

    // ---- prologue: this lane's Q and dO rows (B operands) and statistics,
    // then K_0..K_2 and V_0..V_2 in LDS, all landed before S(0) and dP(0)
    {
        const __bf16* qrow = q + head_off + (size_t)qi * D;
        const __bf16* drow = dout + head_off + (size_t)qi * D;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            qf[c] = qi < N ? *reinterpret_cast<const bf16x8*>(qrow + c * 16 + lh * 8) : bf16x8{};
            df[c] = qi < N ? *reinterpret_cast<const bf16x8*>(drow + c * 16 + lh * 8) : bf16x8{};
        }
    }
    lse2 = qi < N ? lse[(size_t)bh * N + qi] * kLog2e : 0.f;
    dlt = qi < N ? delta[(size_t)bh * N + qi] : 0.f;
    // Retire the row loads here, visibly to the compiler's wait-count pass.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    issue(kh, 0, kring[0]);
    issue(vh, 0, vring[0]);
    issue(kh, 1, kring[1]);
    issue(vh, 1, vring[1]);
    issue(kh, 2, kring[2]);
    issue(vh, 2, vring[2]);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    if (nkb <= 3) {  // the partial tile, if any, is among these
        clear_tail(nkb - 1, kring[nkb - 1]);
        clear_tail(nkb - 1, vring[nkb - 1]);
    }
    __syncthreads();
    scores(0);

    // Phases. Global phase s: group 0 runs A(s/2) for even s and B(s/2) for
    // odd s; group 1 runs one phase later. The group in its VALU phase loads
    // one tile: V_{s/2+3} in even phases (group 0), K_{(s+5)/2} in odd ones
    // (group 1), into the slot of the tile four back (V_{t-4} was last read in
    // phase 2t - 8, K_{t-4} in phase 2t - 6). A tile t is first read in phase
    // 2t - 1. Waits: at the end of its VALU phase a wave allows its loads of
    // that phase and the one two before in flight (vmcnt(2 LG)); at the end
    // of its MFMA phase only that step's (vmcnt(LG)). So group 1's K_t
    // (issued in phase 2t - 5) has landed at the end of phase 2t - 2, its
    // MFMA phase end, and group 0's V_t (issued in phase 2t - 6) at the end
    // of the same phase, its VALU phase end, and that phase's barrier
    // publishes both.
    auto phase_loads = [&](int s) __attribute__((always_inline)) {
        if ((s & 1) != grp) return;
        if ((s & 1) == 0) {
            const int t = s / 2 + 3;
            issue_grp(vh, t, vring[t & 3]);
        } else {
            const int t = (s + 5) / 2;
            issue_grp(kh, t, kring[t & 3]);
        }
    };
    // The partial last tile (if any), issued in phases 2 nkb - 8 (V) and
    // 2 nkb - 7 (K), is cleared at the end of phase 2 nkb - 4, after an extra
    // barrier (only the loading groups' waits cover it), one phase before it
    // is first read. Both groups reach that phase in the general steps.
    const int tail_phase = (nkb > 3 && N % kBc != 0 && nkb == nkb_all) ? 2 * nkb - 4 : -1;
    auto phase_end = [&](int s, auto mfma_phase) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(mfma_phase)::value) __builtin_amdgcn_s_waitcnt(wait_vmcnt(LG));
        else __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LG));
        if (s == tail_phase) {
            __syncthreads();
            clear_tail(nkb - 1, kring[(nkb - 1) & 3]);
            clear_tail(nkb - 1, vring[(nkb - 1) & 3]);
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto phase_end_plain = [&](auto mfma_phase) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(mfma_phase)::value) __builtin_amdgcn_s_waitcnt(wait_vmcnt(LG));
        else __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LG));
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };

    // A(j): dS of tile j from sc and dp. In the general steps (the tiles on
    // the causal diagonal and at the sequence end) every wave runs the masked
    // form, also where all of a wave's keys are masked (its dS is then 0):
    // the phase lasts as long as its slowest wave either way. Key
    // score_key(st, r, lh) is visible iff its lane-independent part
    // st*32 + (r/4)*8 + r%4 is at most one per-lane limit.
    auto phase_a = [&](auto full, int kb) __attribute__((always_inline)) {
        constexpr bool MASKED = !decltype(full)::value;
        if (MASKED && kb >= nkb) return;
        int lim = 0;
        if constexpr (MASKED) {
            lim = N - 1 - kb * kBc;
            if constexpr (CAUSAL) lim = min(lim, qi - kb * kBc);
            lim -= lh * 4;
            asm volatile("" : "+v"(lim));
        }
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[st][r], scale_log2, -lse2));
                if constexpr (MASKED) {
                    const int kc = st * 32 + (r >> 2) * 8 + (r & 3);
                    p = kc <= lim ? p : 0.f;
                }
                dsf[st][r >> 3][r & 7] = (__bf16)(p * (dp[st][r] - dlt));
            }
    };
    // B(j): dQ += K_j^T dS(j)^T, then S(j+1) and dP(j+1). The conditions are
    // uniform over the workgroup.
    auto phase_b = [&](auto full, int kb, int slot, int next_slot) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
        asm volatile("" : "+v"(k_row), "+v"(v_row), "+v"(k_tr[0]), "+v"(k_tr[1]));
        if (FULL || kb < nkb) dq_update(slot);
        if (FULL || kb + 1 < nkb) scores(next_slot);
    };
    // Values that cross a phase boundary pass through empty volatile asm on
    // both sides of its barrier in the straight-line steps: A -> B dS, B -> A
    // the next tile's S and dP and the accumulators.
    auto pin_a = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) asm volatile("" : "+v"(dsf[st][0]), "+v"(dsf[st][1]));
    };
    auto pin_b = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) asm volatile("" : "+v"(sc[st]), "+v"(dp[st]));
#pragma unroll
        for (int t = 0; t < D / 32; ++t) asm volatile("" : "+v"(acc[t]));
    };
    auto step = [&](auto ring, int kb) __attribute__((always_inline)) {
        constexpr int R = decltype(ring)::value;
        const int s = 2 * kb + grp;
        phase_loads(s);
        phase_a(std::false_type{}, kb);
        phase_end(s, std::false_type{});
        phase_b(std::false_type{}, kb, R, (R + 1) & 3);
        phase_end(s + 1, std::true_type{});
    };
    // Steps that every wave runs whole: tile j below the workgroup's first
    // query (causal) and inside N, so A(j) needs no mask; tile j + 1 below
    // nkb - 2, so every wave forms its scores in B(j) (the next step masks
    // them if it must) and the partial tile's clear is still ahead. Phase
    // 2 kb + grp is this wave's loading phase: group 0 loads V_{kb+3},
    // group 1 K_{kb+3}.
    auto step_full = [&](auto ring, int kb) __attribute__((always_inline)) {
        constexpr int R = decltype(ring)::value;
        if (grp == 0) issue_grp(vh, kb + 3, vring[(R + 3) & 3]);
        else issue_grp(kh, kb + 3, kring[(R + 3) & 3]);
        phase_a(std::true_type{}, kb);
        pin_a();
        phase_end_plain(std::false_type{});
        pin_a();
        phase_b(std::true_type{}, kb, R, (R + 1) & 3);
        pin_b();
        phase_end_plain(std::true_type{});
        pin_b();
    };

    if (grp == 1) phase_end(0, std::false_type{});  // group 1's idle first phase
    int kb = 0;
    const int kb_full = min(CAUSAL ? q0 / kBc : nkb - 1, min(N / kBc, nkb - 3));
    for (; kb + 4 <= kb_full; kb += 4) {
        step_full(std::integral_constant<int, 0>{}, kb);
        step_full(std::integral_constant<int, 1>{}, kb + 1);
        step_full(std::integral_constant<int, 2>{}, kb + 2);
        step_full(std::integral_constant<int, 3>{}, kb + 3);
    }
    // Four tiles per iteration; steps past the last tile only issue their
    // (empty) loads and meet the barriers.
    for (; kb < nkb; kb += 4) {
        step(std::integral_constant<int, 0>{}, kb);
        step(std::integral_constant<int, 1>{}, kb + 1);
        step(std::integral_constant<int, 2>{}, kb + 2);
        step(std::integral_constant<int, 3>{}, kb + 3);
    }
    // Group 0 stores its rows during group 1's last phase, then meets that
    // phase's barrier; no load may still be landing when the workgroup ends.
    if (grp == 0) {
        if (qi < N) store_row<D>(dq + head_off + (size_t)qi * D, acc, scale, lh);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    if (grp == 1 && qi < N) store_row<D>(dq + head_off + (size_t)qi * D, acc, scale, lh);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_one(const __bf16* q, const __bf16* k, const __bf16* v, const __bf16* o,
                          const float* lse, const __bf16* dout, __bf16* dq, __bf16* dk,
                          __bf16* dv, float* delta, int BH, int N, float scale_log2, float scale,
                          hipStream_t stream)
{
    const long long rows = (long long)BH * N;
    hipLaunchKernelGGL((fa_bwd_delta_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                       stream, o, dout, delta, rows);
    const int nblk = (N + kBwdRows - 1) / kBwdRows;
    const dim3 grid((unsigned)((long long)BH * nblk));
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL>), grid, dim3(kDkdvThreads), 0, stream, q, k,
                       v, dout, lse, delta, dk, dv, BH, N, nblk, scale_log2, scale);
    if (bwd_dq_phased(BH, N)) {
        const int nqb = (N + kDqRows - 1) / kDqRows;
        hipLaunchKernelGGL((fa_bwd_dq_phased_kernel<D, CAUSAL>),
                           dim3((unsigned)((long long)BH * nqb)), dim3(kDqThreads), 0, stream, q,
                           k, v, dout, lse, delta, dq, BH, N, nqb, scale_log2, scale);
    } else {
        hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL>), grid, dim3(kBwdThreads), 0, stream, q,
                           k, v, dout, lse, delta, dq, BH, N, nblk, scale_log2, scale);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* delta, int BH, int N, int d, float scale_log2, float scale,
                           bool causal, hipStream_t stream)
{
    auto c = [](const void* p) { return static_cast<const __bf16*>(p); };
    auto m = [](void* p) { return static_cast<__bf16*>(p); };
    if (d == 64)
        return causal ? launch_bwd_one<64, true>(c(q), c(k), c(v), c(o), lse, c(dout), m(dq), m(dk),
                                                 m(dv), delta, BH, N, scale_log2, scale, stream)
                      : launch_bwd_one<64, false>(c(q), c(k), c(v), c(o), lse, c(dout), m(dq),
                                                  m(dk), m(dv), delta, BH, N, scale_log2, scale,
                                                  stream);
    return causal ? launch_bwd_one<128, true>(c(q), c(k), c(v), c(o), lse, c(dout), m(dq), m(dk),
                                              m(dv), delta, BH, N, scale_log2, scale, stream)
                  : launch_bwd_one<128, false>(c(q), c(k), c(v), c(o), lse, c(dout), m(dq), m(dk),
                                               m(dv), delta, BH, N, scale_log2, scale, stream);
}

}  // namespace fa
