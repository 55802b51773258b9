// Attention forward with 8-bit (FP8 E4M3) Q, K and V on CDNA4 (gfx950).
//
// [FlashAttention: The GPU Memory Hack That Changed Everything
//  (ai.branddocks.com, episode 75), "FlashAttention-3: Hopper Architecture":
//  attention run in FP8 on the matrix units, about twice the FP16 rate, with
//  negligible quality loss]
// The method is the same tiled recurrence as the bf16 kernel (one running
// reference max per row, the output divided by the row sum once at the end);
// only the operand precision of the two products changes:
//  * Q, K, V arrive as E4M3 codes with one scale per tensor (value = scale *
//    code). S^T = K Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4 (64 of d per
//    instruction, fp32 accumulation); the Q and K scales fold into the
//    softmax constant c = scale * q_scale * k_scale * log2(e).
//  * w = exp2(s c - m + log2 48) = 48 p is formed in fp32; P is stored for
//    the second product as E4M3(w) (the factor keeps small weights out of
//    the subnormal range while the largest, 48 * 2^3 = 384, stays below
//    448, the largest E4M3 value) and the row sum adds the fp32 w.
//  * O^T += V^T P^T on the same instruction, 64 keys per instruction; V^T
//    comes from ds_read_b64_tr_b8 transpose reads of the V tile. The epilogue
//    divides by l (in units of 48 p) and multiplies by v_scale.
//
// gfx950 mapping (the bf16 kernel's structure, with FP8 tile sizes):
//  * One workgroup = 8 wave64s = 256 query rows, 32 per wave; waves w and
//    w+4 share a SIMD, so group 0 = waves 0-3 and group 1 = waves 4-7 put
//    one wave of each group on every SIMD. Per key tile j a wave runs A(j),
//    the softmax of tile j (VALU and transcendental work only), then B(j),
//    the scores of tile j+1 and O += P_j V_j (16 MFMAs and their LDS reads,
//    nothing else). Group 1 runs one phase behind group 0 and every phase
//    ends with a workgroup barrier, so on every SIMD one wave feeds the
//    matrix core while the other runs the softmax.
//  * Key tiles of 128 keys (16 KiB of K or V) through two rings of four
//    tiles in LDS (128 KiB), loaded with buffer_load_dwordx4 ... lds by the
//    four waves of the group in its softmax phase; a tile has four phases to
//    land. 128 keys make one MFMA phase 16 FP8 MFMAs, the same matrix-core
//    time as the bf16 kernel's 64-key phase.
//  * A row's reference max moves only when a tile's max passes it by more
//    than 3 (base 2), so p <= 8 and the output rescale, 64 multiplies per
//    lane, runs on about 1 wave-tile in 20 on long N(0,1) sequences (on
//    3 in 4 with an exact running max, on 1 in 2 with a slack of 0.75).
//  * Causal grids run one workgroup per pair of query blocks (the i-th
//    heaviest with the i-th lightest) as in the bf16 kernel.
// Within each 128-byte row the 16-byte chunks are XOR-swizzled so that both
// the row reads of K and the transpose reads of V are bank-conflict-free.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_common.h"
#include "fa_lds.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;

constexpr int kF8Waves = 8;             // two groups of four wave64s
constexpr int kF8Threads = kF8Waves * 64;
constexpr int kF8Rows = kF8Waves * 32;  // queries per workgroup
constexpr int kF8D = 128;               // head dimension (bytes per row)
constexpr int kF8Bc = 128;              // keys per K/V tile
constexpr int kF8Ring = 4;              // K (and V) tiles resident in LDS
// P is stored as E4M3(48 p), p <= 2^kF8Slack: 48 * 8 = 384 < 448.
constexpr float kF8Log2PScale = 5.584962500721156f;  // log2(48)
// Slack of the reference max, base-2 units (see above).
constexpr float kF8Slack = 3.0f;
// __builtin_amdgcn_sched_group_barrier instruction classes; fragment reads
// issued ahead of their MFMA, in MFMAs.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kF8ReadAhead = 3;

// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E4M3 and unit scales
// (E8M0 127 = 2^0).
__device__ inline f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// One tile of kF8Bc rows of a [rows][128] byte tensor in LDS.
struct Tile8 {
    static constexpr int kRowBytes = kF8D;
    static constexpr int kChunks = kRowBytes / 16;                     // 8
    static constexpr int kBytes = kF8Bc * kRowBytes;                   // 16 KiB
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;              // 8
    static constexpr int kLoads = kBytes / 1024;                       // 16
    // Physical chunk of logical chunk c in row r is c ^ swz(r). Bank group of
    // a 16-byte slot is (8 * (r % 2) + chunk) % 16. Row reads of 16
    // consecutive rows at one logical chunk need swz to be a bijection on the
    // 8 rows of each parity; the transpose reads (rows b + {0..3, 8..11} for
    // b % 4 == 0, two adjacent chunks) need its bits 1-2 to differ over the
    // four rows of each parity. This swz does both; it depends on row bits
    // 1-3 only, so rows 32 or 64 apart share it.
    __device__ static int swz(int r) {
        return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | ((r >> 2) & 1);
    }
    // Byte offset of wave-wide load n (0..15) for `lane`: load n fills tile
    // bytes [1024 n, 1024 n + 1024), lane i the 16-byte slot i there, i.e.
    // row 8 n + i / 8 at physical chunk i % 8.
    __device__ static int load_offset(int n, int lane) {
        const int row = n * kRowsPerLoad + lane / kChunks;
        return row * kRowBytes + (((lane % kChunks) ^ swz(row)) * 16);
    }
    __device__ static int frag_offset(int row, int chunk) {
        return row * kRowBytes + ((chunk ^ swz(row)) * 16);
    }
    // Transpose read r (0..3) of the 32-column block tt within a 64-key half
    // for `lane`: in each 16-lane group, lanes 2k and 2k+1 point at the two
    // 8-byte halves of one 16-byte slot of row k (k = 0..7) and lane j
    // receives byte j of the 8 rows. Row k is key b_r + k (k < 4) or
    // b_r + k + 4 (k >= 4), b_r = 32 (r / 2) + 16 (r % 2) + 4 h, h = lane / 32:
    // the keys that byte 8 r + k of the P operand holds (the score layout's
    // key order).
    __device__ static int tr_offset(int tt, int r, int lane) {
        const int j = lane & 15, k = j >> 1, half = j & 1;
        const int h = lane >> 5;
        const int row = 32 * (r >> 1) + 16 * (r & 1) + 4 * h + (k < 4 ? k : k + 4);
        const int chunk = tt * 2 + ((lane >> 4) & 1);
        return row * kRowBytes + ((chunk ^ swz(row)) * 16) + half * 8;
    }
};

template <bool CAUSAL, bool PAIRED>
__global__ __launch_bounds__(kF8Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                       const uint8_t* __restrict__ v, __bf16* __restrict__ o,
                       float* __restrict__ lse, int BH, int N, int nqb, float c_log2,
                       float out_scale)
{
    using TL = Tile8;
    constexpr int LW = TL::kLoads / kF8Waves;        // loads per wave, all eight loading
    constexpr int LG = TL::kLoads / (kF8Waves / 2);  // loads per wave, one group loading
    constexpr int kST = kF8Bc / 32;                  // 32-key sub-tiles per tile
    constexpr int kSMfmas = kST * (kF8D / 64);       // score MFMAs per tile
    constexpr int kPMfmas = (kF8D / 32) * (kF8Bc / 64);  // P.V MFMAs per tile
    __shared__ __attribute__((aligned(1024))) unsigned char kring[kF8Ring][TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vring[kF8Ring][TL::kBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int lane = tid & 63;
    const int li = lane & 31;
    const int lh = lane >> 5;

    int first, second, nitems, bh;
    if constexpr (PAIRED) {
        block_coords<CAUSAL>(blockIdx.x, BH, (nqb + 1) / 2, second, bh);
        first = nqb - 1 - second;
        nitems = first == second ? 1 : 2;
    } else {
        block_coords<CAUSAL>(blockIdx.x, BH, nqb, first, bh);
        second = first;
        nitems = 1;
    }
    for (int item = 0; item < nitems; ++item) {
    const int qb = item == 0 ? first : second;
    if (item) __syncthreads();  // the previous block's LDS reads are done
    const size_t head_off = (size_t)bh * (size_t)N * kF8D;
    const uint8_t* kh = k + head_off;
    const uint8_t* vh = v + head_off;
    const int q0 = qb * kF8Rows;
    const int qw0 = q0 + wave * 32;
    const int qi = qw0 + li;

    // This lane's query row as the B operand of S^T: bytes [64c + 32h, +32).
    i32x8 qf[kF8D / 64];
    {
        const uint8_t* qrow = q + head_off + (size_t)qi * kF8D;
#pragma unroll
        for (int c = 0; c < kF8D / 64; ++c) {
            i32x4 lo{}, hi{};
            if (qi < N) {
                lo = *reinterpret_cast<const i32x4*>(qrow + c * 64 + lh * 32);
                hi = *reinterpret_cast<const i32x4*>(qrow + c * 64 + lh * 32 + 16);
            }
            qf[c] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    }
    // Retire the Q loads here, visibly to the compiler's wait-count pass.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    const int nkb_all = (N + kF8Bc - 1) / kF8Bc;
    const int nkb = CAUSAL ? min(nkb_all, (q0 + kF8Rows - 1) / kF8Bc + 1) : nkb_all;
    // Last tile with a key visible to some row of this wave.
    const int last = CAUSAL ? min(nkb - 1, (qw0 + 31) / kF8Bc) : nkb - 1;
    // Tiles [0, nfull_w) need no mask for this wave.
    const int nfull_w = min(CAUSAL ? (qw0 + 1) / kF8Bc : nkb_all, N / kF8Bc);

    // Buffer resource over tile t of `src`; a tile past the last one gets an
    // empty range (nothing is read) so that the vmcnt arithmetic holds.
    auto tile_rsrc = [&](const uint8_t* src, int t) __attribute__((always_inline)) {
        const int j0 = t * kF8Bc;
        const bool real = t < nkb;
        const unsigned bytes = real ? (unsigned)min(kF8Bc, N - j0) * TL::kRowBytes : 0u;
        return buffer_rsrc(real ? src + (size_t)j0 * kF8D : src, bytes);
    };
    // This wave's share of tile t, all eight waves loading (prologue).
    auto issue = [&](const uint8_t* src, int t, unsigned char* dst) __attribute__((always_inline)) {
        const i32x4 rs = tile_rsrc(src, t);
#pragma unroll
        for (int it = 0; it < LW; ++it) {
            const int n = wave * LW + it;
            lds_dma16(rs, TL::load_offset(n, lane), lds_addr(dst + n * 1024));
        }
    };
    // This wave's share of tile t, the four waves of its group loading.
    auto issue_grp = [&](const uint8_t* src, int t, unsigned char* dst) __attribute__((always_inline)) {
        const i32x4 rs = tile_rsrc(src, t);
        unsigned lb = lds_addr(dst + (wave & 3) * LG * 1024);
        asm volatile("" : "+s"(lb));
#pragma unroll
        for (int it = 0; it < LG; ++it)
            lds_dma16(rs, TL::load_offset((wave & 3) * LG + it, lane), lb + it * 1024);
    };
    // Rows of a partial last V tile past the sequence end are cleared once
    // the tile has landed: their weights are 0, and 0 * NaN would leak.
    auto clear_tail = [&](int t, unsigned char* dst) __attribute__((always_inline)) {
        const int rows = N - t * kF8Bc;
        if (rows >= kF8Bc) return;
        for (int x = tid; x < (kF8Bc - rows) * TL::kChunks; x += kF8Threads)
            *reinterpret_cast<i32x4*>(dst + (rows + x / TL::kChunks) * TL::kRowBytes +
                                      (x % TL::kChunks) * 16) = i32x4{};
    };

    unsigned kbase = lds_addr(kring[0]), vbase = lds_addr(vring[0]);
    asm volatile("" : "+s"(kbase), "+s"(vbase));
    // K fragment of key row st*32 + li for MFMA chunk c: logical chunks
    // 4c + 2h and 4c + 2h + 1 (bytes 64c + 32h .. +31 of d). V^T transpose
    // reads per Tile8::tr_offset. The swizzle XORs chunk bits only, chunks
    // enter the offset at bits 4-6 and the ring bases are 1024-aligned, so
    // every fragment offset is one of two bases XOR a constant plus a
    // constant: k(c, x) = k0 ^ ((4c + x) << 4); v(tt, r) = (v0 ^ (tt << 5))
    // + row offset of read r (its rows differ from read 0's by 16 or 32 and
    // share their swizzle). Only the two bases stay live.
    unsigned k0 = kbase + TL::frag_offset(li, 2 * lh);
    unsigned v0 = vbase + TL::tr_offset(0, 0, lane);
    auto k_off = [&](int c, int x) __attribute__((always_inline)) {
        return k0 ^ ((unsigned)(4 * c + x) << 4);
    };
    auto v_off = [&](int tt, int r) __attribute__((always_inline)) {
        return (v0 ^ ((unsigned)tt << 5)) + (unsigned)((32 * (r >> 1) + 16 * (r & 1)) * TL::kRowBytes);
    };

    // K fragment of score MFMA i (sub-tile st = i % kST, d chunk c = i / kST)
    // from ring slot `slot`: two 16-byte reads.
    auto kfrag = [&](int slot, int i) __attribute__((always_inline)) {
        const int st = i % kST, c = i / kST;
        const unsigned off = slot * TL::kBytes + st * 32 * TL::kRowBytes;
        const i32x4 lo = *reinterpret_cast<const lds_i32x4*>((size_t)(k_off(c, 0) + off));
        const i32x4 hi = *reinterpret_cast<const lds_i32x4*>((size_t)(k_off(c, 1) + off));
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    // V^T fragment of P.V MFMA i (32-column block tt = i % 4, 64-key half
    // kh2 = i / 4) from ring slot `slot`: four transpose reads.
    auto vfrag = [&](int slot, int i) __attribute__((always_inline)) {
        const int tt = i % (kF8D / 32), half = i / (kF8D / 32);
        const unsigned off = slot * TL::kBytes + half * 64 * TL::kRowBytes;
        i32x8 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2*)(size_t)(v_off(tt, r) + off));
            a[2 * r] = x[0];
            a[2 * r + 1] = x[1];
        }
        return a;
    };

    f32x16 acc[kF8D / 32];  // O^T: rows d = 32 tt + 8 g + 4 h + i, column = query li
#pragma unroll
    for (int tt = 0; tt < kF8D / 32; ++tt) acc[tt] = f32x16{};
    float m_run = neg_inf();  // reference max, base-2 scaled domain
    float l_run = 0.f;        // this lane's share of the row sum, in units of 48 p
    f32x16 sc[kST];           // scores of the tile whose softmax runs next
    i32x8 pf[kF8Bc / 64];     // E4M3(48 p) of the current tile, one per 64-key half

    // Score MFMAs with their fragments read kF8ReadAhead MFMAs ahead, in
    // program order (so that the order stays pipelined even where the
    // scheduler keeps the source order).
    auto scores = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < kST; ++st) sc[st] = f32x16{};
        i32x8 fr[kF8ReadAhead];
#pragma unroll
        for (int i = 0; i < kF8ReadAhead; ++i) fr[i] = kfrag(slot, i);
#pragma unroll
        for (int i = 0; i < kSMfmas; ++i) {
            const i32x8 a = fr[i % kF8ReadAhead];
            if (i + kF8ReadAhead < kSMfmas) fr[i % kF8ReadAhead] = kfrag(slot, i + kF8ReadAhead);
            sc[i % kST] = mfma8(a, qf[i / kST], sc[i % kST]);
        }
    };
    // Scores of invisible keys (past N, or after the query when causal)
    // become -inf. Key score_key(st, r, lh) of the tile is visible iff its
    // lane-independent part st*32 + (r/4)*8 + r%4, a compile-time constant,
    // is at most one per-lane limit (so no per-key index is kept in a
    // register).
    auto mask = [&](int kb) __attribute__((always_inline)) {
        int lim = N - 1 - kb * kF8Bc;
        if constexpr (CAUSAL) lim = min(lim, qi - kb * kF8Bc);
        lim -= lh * 4;
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int st = 0; st < kST; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kc = st * 32 + (r >> 2) * 8 + (r & 3);
                sc[st][r] = kc <= lim ? sc[st][r] : neg_inf();
            }
    };

    // ---- prologue: K_0..K_3 and V_0, V_1 in LDS; scores of tile 0
    issue(kh, 0, kring[0]);
    issue(kh, 1, kring[1]);
    issue(vh, 0, vring[0]);
    issue(kh, 2, kring[2]);
    issue(vh, 1, vring[1]);
    issue(kh, 3, kring[3]);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    if (nkb <= 2) clear_tail(nkb - 1, vring[nkb - 1]);
    __syncthreads();
    scores(0);
    __syncthreads();  // every wave is done with K_0 before K_4 replaces it

    // Phases as in the bf16 kernel: global phase s, group 0 runs A(s/2) for
    // even s and B(s/2) for odd s, group 1 one phase later. Phase s starts
    // with one tile loaded by the group in its softmax phase: V_{s/2+2} in
    // even phases, K_{(s-1)/2+4} in odd ones, into the slot of the tile four
    // back; every phase ends with vmcnt(2 LG) and a barrier.
    auto phase_loads = [&](int s) __attribute__((always_inline)) {
        if ((s & 1) != grp) return;
        if ((s & 1) == 0) {
            const int t = s / 2 + 2;
            issue_grp(vh, t, vring[t & 3]);
        } else {
            const int t = (s - 1) / 2 + 4;
            issue_grp(kh, t, kring[t & 3]);
        }
    };
    // The same loads without a branch, for the main loop's steps: phase
    // s = 2 kb + grp is always this wave's softmax phase, so group 0 loads V
    // tiles and group 1 K tiles; tile t = kb + 2 (V) or kb + 4 (K) goes to
    // ring slot t % 4.
    auto step_loads = [&](int kb, int R) __attribute__((always_inline)) {
        const bool isk = grp != 0;
        const int t = kb + (isk ? 4 : 2);
        unsigned char* dst = isk ? kring[R] : vring[(R + 2) & 3];
        issue_grp(isk ? kh : vh, t, dst);
    };
    auto phase_end_plain = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LG));
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    const int tail_phase = (nkb > 2 && N % kF8Bc != 0 && nkb == nkb_all) ? 2 * nkb - 2 : -1;
    auto phase_end = [&](int s) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LG));
        if (s == tail_phase) {
            __syncthreads();
            clear_tail(nkb - 1, vring[(nkb - 1) & 3]);
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };

    // A(j): VALU only. Softmax of tile j: reference max and running sum,
    // E4M3 P, and O *= alpha when some row's reference moved.
    auto phase_a = [&](auto full, int kb) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
        if (!FULL) {
            if (kb > last) return;
            if (kb >= nfull_w) mask(kb);
        }
        // Row max of the lane's 64 scores in four v_max3 chains, then with
        // the partner lane (scores are finite or -inf).
        float mr4[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            float m = sc[c4][0];
#pragma unroll
            for (int r = 1; r < 15; r += 2)
                asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(m), "v"(sc[c4][r]), "v"(sc[c4][r + 1]));
            asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(m), "v"(sc[c4][15]));
            mr4[c4] = m;
        }
        float mraw;
        asm("v_max3_f32 %0, %1, %2, %3" : "=v"(mraw) : "v"(mr4[0]), "v"(mr4[1]), "v"(mr4[2]));
        asm("v_max_f32 %0, %1, %2" : "=v"(mraw) : "v"(mraw), "v"(mr4[3]));
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mraw), __float_as_uint(mraw),
                                                             false, false);
            asm("v_max_f32 %0, %1, %2" : "=v"(mraw) : "v"(__uint_as_float(sw[0])), "v"(__uint_as_float(sw[1])));
        }
        const float mtile = mraw > neg_inf() ? mraw * c_log2 : neg_inf();
        const bool grow = mtile > m_run + kF8Slack;  // tile 0 always moves it
        const float m_new = grow ? mtile : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        // w = exp2(s c - (m - log2 48)) = 48 p; E4M3(w) packed in the score
        // layout's key order: byte 16 st' + 4 g + i of pf[half] is key
        // score_key(2 half + st', 4 g + i).
        const float mb = m_run - kF8Log2PScale;
        float ls[4] = {-0.f, -0.f, -0.f, -0.f};
#pragma unroll
        for (int st = 0; st < kST; ++st)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float p4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p4[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[st][g * 4 + i], c_log2, -mb));
                    ls[i] += p4[i];
                }
                // bytes 0-1, then 2-3, of the dword (its old value is overwritten)
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], pf[st >> 1][(st & 1) * 4 + g],
                                                        false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], w, true);
                pf[st >> 1][(st & 1) * 4 + g] = w;
            }
        l_run = l_run * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int tt = 0; tt < kF8D / 32; ++tt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[tt][r] *= alpha;
        }
    };
    // B(j): MFMA work only. Scores of tile j+1 from K ring slot kslot, then
    // O^T += V_j^T P_j^T from V ring slot vslot.
    auto phase_b = [&](auto full, int kb, int kslot, int vslot) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
        asm volatile("" : "+v"(k0), "+v"(v0));  // rebuild the offsets here, not hoisted
        if (FULL || kb + 1 <= last) {
            scores(kslot);
            // two reads per fragment, kF8ReadAhead MFMAs ahead
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kF8ReadAhead, 0);
#pragma unroll
            for (int i = 0; i < kSMfmas - kF8ReadAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kF8ReadAhead, 0);
        }
        if (!FULL && kb > last) return;
        i32x8 fr[kF8ReadAhead];
#pragma unroll
        for (int i = 0; i < kF8ReadAhead; ++i) fr[i] = vfrag(vslot, i);
#pragma unroll
        for (int i = 0; i < kPMfmas; ++i) {
            const int tt = i % (kF8D / 32), half = i / (kF8D / 32);
            const i32x8 a = fr[i % kF8ReadAhead];
            if (i + kF8ReadAhead < kPMfmas) fr[i % kF8ReadAhead] = vfrag(vslot, i + kF8ReadAhead);
            acc[tt] = mfma8(a, pf[half], acc[tt]);
        }
        // four transpose reads per fragment, kF8ReadAhead MFMAs ahead
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4 * kF8ReadAhead, 0);
#pragma unroll
        for (int i = 0; i < kPMfmas - kF8ReadAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kF8ReadAhead, 0);
    };
    // The values that cross a phase boundary pass through empty volatile asm
    // on both sides of its barrier, so that their producers stay in the phase
    // that ends and their consumers in the phase that starts: the compiler
    // would otherwise move pure arithmetic (P.V MFMAs, exponentials) across
    // the barrier and break the pairing of the groups. A -> B: P, m, l;
    // B -> A: the next tile's scores and the output accumulators.
    auto pin_a = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < kF8Bc / 64; ++h) asm volatile("" : "+v"(pf[h]));
        asm volatile("" : "+v"(m_run), "+v"(l_run));
    };
    auto pin_b = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < kST; ++st) asm volatile("" : "+v"(sc[st]));
#pragma unroll
        for (int tt = 0; tt < kF8D / 32; ++tt) asm volatile("" : "+v"(acc[tt]));
    };
    // Tile j as this wave sees it: A(j) then B(j), each in its global phase
    // (group 1 one phase later than group 0); R = j mod 4 is a compile-time
    // constant, so every ring slot is a fixed LDS offset.
    auto step = [&](auto ring, int kb) __attribute__((always_inline)) {
        constexpr int R = decltype(ring)::value;
        const int s = 2 * kb + grp;
        // (In the causal kernels the steps' per-wave skips already keep the
        // phases apart, and pinning there doubles the live scores at the
        // skips' joins; the non-causal kernel pins as the full steps do.)
        phase_loads(s);
        phase_a(std::false_type{}, kb);
        if constexpr (!CAUSAL) pin_a();
        phase_end(s);
        if constexpr (!CAUSAL) pin_a();
        phase_loads(s + 1);
        phase_b(std::false_type{}, kb, (R + 1) & 3, R);
        if constexpr (!CAUSAL) pin_b();
        phase_end(s + 1);
        if constexpr (!CAUSAL) pin_b();
    };
    // A step that every wave of the workgroup runs in full: its tile j and
    // the next one lie wholly below the workgroup's first query (causal) and
    // inside the sequence, so nothing is masked or skipped and the step is
    // straight-line code (phase s + 1 is never this wave's loading phase,
    // and the tail clear lies in the last phases).
    auto step_full = [&](auto ring, int kb) __attribute__((always_inline)) {
        constexpr int R = decltype(ring)::value;
        step_loads(kb, R);
        phase_a(std::true_type{}, kb);
        pin_a();
        phase_end_plain();
        pin_a();
        phase_b(std::true_type{}, kb, (R + 1) & 3, R);
        pin_b();
        phase_end_plain();
        pin_b();
    };

    if (grp == 1) {  // group 1's idle first phase
        phase_loads(0);
        phase_end(0);
    }
    // Steps j < kb_full are full for every wave: tiles j and j + 1 lie below
    // the workgroup's first query (causal) and within N / 128. Four tiles per
    // iteration; the remaining steps, past the last tile (kb >= nkb) too, take
    // the general path, where steps past the last tile only issue their
    // (empty) loads and meet the barriers. kb_full <= nkb - 2 keeps the
    // phase of the partial tile's clear (2 nkb - 2, which group 1 reaches in
    // step nkb - 2) in the general path for both groups, so both meet its
    // extra barrier.
    const int kb_full = min(CAUSAL ? q0 / kF8Bc : nkb - 1, min(N / kF8Bc, nkb - 2));
    int kb = 0;
    for (; kb + 4 <= kb_full; kb += 4) {
        step_full(std::integral_constant<int, 0>{}, kb);
        step_full(std::integral_constant<int, 1>{}, kb + 1);
        step_full(std::integral_constant<int, 2>{}, kb + 2);
        step_full(std::integral_constant<int, 3>{}, kb + 3);
    }
    for (; kb < nkb; kb += 4) {
        step(std::integral_constant<int, 0>{}, kb);
        step(std::integral_constant<int, 1>{}, kb + 1);
        step(std::integral_constant<int, 2>{}, kb + 2);
        step(std::integral_constant<int, 3>{}, kb + 3);
    }
    // ---- epilogue: O = acc * v_scale / l, lse = (m2 + log2(l / 48)) * ln 2
    auto epilogue = [&]() __attribute__((always_inline)) {
        const float l_tot = sum_with_partner(l_run);
        if (qi < N) {
            const float inv = out_scale / l_tot;
            __bf16* orow = o + head_off + (size_t)qi * kF8D;
#pragma unroll
            for (int tt = 0; tt < kF8D / 32; ++tt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    store4(orow + tt * 32 + g * 8 + lh * 4, acc[tt][g * 4] * inv,
                           acc[tt][g * 4 + 1] * inv, acc[tt][g * 4 + 2] * inv,
                           acc[tt][g * 4 + 3] * inv);
            if (lh == 0)
                lse[(size_t)bh * N + qi] =
                    (m_run - kF8Log2PScale + log2f(l_tot)) * 0.69314718055994531f;
        }
    };
    if (grp == 0) {
        epilogue();
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    if (grp == 1) epilogue();
    }  // work items
}

// Causal grids pair query blocks as the bf16 kernel does (small grids, or
// N <= 8192).
constexpr long long kF8PairMaxGrid = 2 * 256;
constexpr int kF8PairMaxN = 8192;

}  // namespace

hipError_t launch_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int N, float c_log2, float out_scale, bool causal, hipStream_t stream)
{
    const int nqb = (N + kF8Rows - 1) / kF8Rows;
    const long long blocks = (long long)BH * nqb;
    auto qp = static_cast<const uint8_t*>(q);
    auto kp = static_cast<const uint8_t*>(k);
    auto vp = static_cast<const uint8_t*>(v);
    auto op = static_cast<__bf16*>(o);
    if (causal && nqb > 1 && (blocks <= kF8PairMaxGrid || N <= kF8PairMaxN)) {
        const dim3 grid((unsigned)((long long)BH * ((nqb + 1) / 2)));
        hipLaunchKernelGGL((fa_fwd_fp8_kernel<true, true>), grid, dim3(kF8Threads), 0, stream, qp,
                           kp, vp, op, lse, BH, N, nqb, c_log2, out_scale);
    } else if (causal) {
        hipLaunchKernelGGL((fa_fwd_fp8_kernel<true, false>), dim3((unsigned)blocks),
                           dim3(kF8Threads), 0, stream, qp, kp, vp, op, lse, BH, N, nqb, c_log2,
                           out_scale);
    } else {
        hipLaunchKernelGGL((fa_fwd_fp8_kernel<false, false>), dim3((unsigned)blocks),
                           dim3(kF8Threads), 0, stream, qp, kp, vp, op, lse, BH, N, nqb, c_log2,
                           out_scale);
    }
    return hipGetLastError();
}

}  // namespace fa
