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
//  * One workgroup = 8 wave64s = 256 query rows; each wave owns 32 rows. The
//    hardware places waves w and w+4 on the same SIMD (measured: every
//    workgroup, every CU), so group 0 = waves 0-3 and group 1 = waves 4-7
//    put one wave of each group on every SIMD.
//  * Per key tile j a wave runs two phases: A(j) = the softmax of tile j
//    (row max, exp2, row sum, bf16 P, output rescale: VALU and
//    transcendental work only) and B(j) = the scores of tile j+1 and
//    O += P_j V_j (32 MFMAs and their LDS reads, no other work). Group 1
//    runs one phase behind group 0 and every phase ends with a workgroup
//    barrier, so on each SIMD one wave feeds the matrix core while the other
//    runs the softmax: the two kinds of work overlap by construction instead
//    of by chance. Scheduling fences keep each instruction inside its phase.
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
//  * K and V tiles (64 keys) go from HBM straight into LDS with
//    buffer_load_dwordx4 ... lds (no VGPR staging) through two rings of four
//    tiles each (128 KiB at d = 128, one workgroup per CU). Every phase, the
//    four waves in their softmax phase load one tile (V in even phases, K in
//    odd ones), which has four phases (two tiles) to land before it is read;
//    the waves in their MFMA phase issue no memory instruction. Ring slot
//    and sub-tile offsets are instruction immediates: the loop is unrolled
//    by the ring size. Buffer-resource bounds make rows past the sequence
//    end read as 0.
//  * LDS rows hold 16-byte chunks XOR-swizzled by row, so that the K reads
//    (16 rows, same chunk) and the V transpose reads (4 rows x 4 chunks per
//    32 lanes) hit distinct banks.
//  * Softmax in base 2: p = exp2(s * scale*log2(e) - m) is one FMA and one
//    v_exp_f32 per score; the row max is taken on the raw scores. A row's
//    reference max m (the exponent offset of its running sum and output)
//    moves only when a tile's max exceeds it by more than kMaxSlack, so p
//    lies in (0, 2^kMaxSlack] and the acc *= alpha pass is skipped for a
//    wave in which no row's reference moved. The result is the same sum
//    regrouped: lse = m + log2(l) and O = acc / l hold for any m at or
//    below the true max.
//  * Causal: key tiles past the workgroup's last query are never loaded, a
//    wave skips tiles that lie wholly above its 32 rows, and the mask is
//    applied only on tiles that cross a wave's diagonal or the sequence end.
//    The tiles below the workgroup's diagonal run as straight-line steps
//    without those conditions, each phase one basic block whose crossing
//    values are pinned on both sides of the barrier.
//  * Grids that would leave CUs idle (fa_plan.cpp decides, fa_fwd_grid
//    reports): either 128-row blocks whose key tiles the two wave groups
//    split, with the two partial (max, sum, output) states merged at the end
//    [Flash Attention Optimization (aicomputerinstitute.com), "The fix: tile
//    the computation..."], or, for causal grids, query blocks grouped so that
//    every workgroup carries the heaviest block's work.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_common.h"
#include "fa_lds.h"

namespace fa {
namespace {

constexpr int kPPWaves = 8;                  // two groups of four wave64s
constexpr int kPPThreads = kPPWaves * 64;
constexpr int kRing = 4;                     // K (and V) tiles resident in LDS
// __builtin_amdgcn_sched_group_barrier instruction classes
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
// LDS reads issued ahead of the MFMA that consumes them, in MFMAs
// (measured flat from 2 to 8; 6 leaves the register budget unspilled).
constexpr int kReadAhead = 6;
// Slack of the reference max, base-2 units: the max moves (and the output is
// rescaled) only when a tile's max exceeds it by more than this. With an
// exact running max (slack 0) three waves in four rescale on every tile of
// the long-document workload; with 3 the rescale is rare and the forward is
// 4.8% faster. The cost is precision in rows that one key dominates: its
// weight 2^delta (delta <= 3) is rounded to bf16 for P V instead of being
// exactly 1 (measured max|dO| on the spiky workload 0.0163 against 0.0153;
// a slack of 8 gave 0.0263).
constexpr float kMaxSlack = 3.0f;
static_assert(kBrBf16 == kPPWaves * 32, "32 query rows per wave");

// KS = 1: each workgroup covers 256 query rows and both wave groups see every
// key tile. KS = 2 (grids too small to fill the CUs): a workgroup covers 128
// rows, waves w and w + 4 own the same 32 rows, group g takes the key tiles
// t = g (mod 2), and the two partial (max, sum, output) states of a row are
// merged at the end with two correction factors.
// Items of workgroup L of the balanced causal grid (see fwd_plan): in
// logical order, each head contributes {nqb-1} and {nqb-2-p, p} for
// p < (nqb-1)/2, and for even nqb every two heads share one workgroup of
// their middle blocks (nqb-2)/2, placed after the two heads' own; the
// logical order is spread over the XCDs in contiguous runs, as block_coords
// does. Heavier block first.
__device__ inline void balanced_items(int L, int BH, int nqb, int& bh0, int& qb0, int& bh1,
                                      int& qb1, int& nitems)
{
    const int per = 1 + (nqb - 1) / 2;
    const bool mid = nqb % 2 == 0;
    const int total = BH * per + (mid ? (BH + 1) / 2 : 0);
    const int idx = total % kXcds == 0 ? (L % kXcds) * (total / kXcds) + L / kXcds : L;
    const int grp_sz = mid ? 2 * per + 1 : per;       // WGs per head pair (even nqb) or head
    const int g = idx / grp_sz, r = idx - g * grp_sz;
    int h, j;
    if (mid) {
        const int h0 = 2 * g;
        const int heads = min(2, BH - h0);             // the last group may hold one head
        if (r == heads * per) {                        // the middle blocks of the group's heads
            bh0 = h0;
            qb0 = bh1 = qb1 = 0;
            qb0 = (nqb - 2) / 2;
            bh1 = h0 + 1;
            qb1 = qb0;
            nitems = heads;
            return;
        }
        h = h0 + r / per;
        j = r % per;
    } else {
        h = g;
        j = r;
    }
    bh0 = bh1 = h;
    if (j == 0) {
        qb0 = qb1 = nqb - 1;
        nitems = 1;
    } else {
        qb0 = nqb - 1 - j;  // nqb - 2 - p with p = j - 1
        qb1 = j - 1;
        nitems = 2;
    }
}

template <int D, bool CAUSAL, bool PAIRED, int KS, bool BAL>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                        const __bf16* __restrict__ v, __bf16* __restrict__ o,
                        float* __restrict__ lse, int BH, int N, int nqb, float scale_log2)
{
    static_assert(KS == 1 || (KS == 2 && !PAIRED), "key split only for one block per workgroup");
    static_assert(!BAL || PAIRED, "balanced groups are run by the paired kernel");
    constexpr int kRowsWG = kBrBf16 / KS;  // query rows per workgroup
    using TL = Tile<D, kPPWaves>;
    constexpr int L = TL::kLoadsPerWave;
    // Tile t of K lives in kring[t % 4], tile t of V in vring[t % 4]; rows
    // are swizzled (Tile::swz).
    __shared__ __attribute__((aligned(1024))) unsigned char kring[kRing][TL::kBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char vring[kRing][TL::kBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases in SGPRs
    const int grp = wave >> 2;  // waves w and w+4 share a SIMD
    const int wq = KS == 1 ? wave : (wave & 3);  // the wave's 32-row slot in the block
    const int lane = tid & 63;
    const int li = lane & 31;   // query column of this lane in the wave's 32
    const int lh = lane >> 5;   // which 8-element half of each 16-wide k slice

    // Work items: one query block per workgroup, or (PAIRED, causal) the two
    // blocks nqb-1-p and p of a head one after the other, so that every
    // workgroup has the same number of key tiles.
    int first, second, nitems, bh0, bh1;
    if constexpr (BAL) {
        balanced_items(blockIdx.x, BH, nqb, bh0, first, bh1, second, nitems);
    } else if constexpr (PAIRED) {
        block_coords<CAUSAL>(blockIdx.x, BH, (nqb + 1) / 2, second, bh0);
        first = nqb - 1 - second;
        nitems = first == second ? 1 : 2;
        bh1 = bh0;
    } else {
        block_coords<CAUSAL>(blockIdx.x, BH, nqb, first, bh0);
        second = first;
        nitems = 1;
        bh1 = bh0;
    }
    for (int item = 0; item < nitems; ++item) {
    const int qb = item == 0 ? first : second;
    const int bh = item == 0 ? bh0 : bh1;
    if (item) __syncthreads();  // the previous block's LDS reads are done
    const size_t head_off = (size_t)bh * (size_t)N * D;
    const __bf16* qh = q + head_off;
    const __bf16* kh = k + head_off;
    const __bf16* vh = v + head_off;

    const int q0 = qb * kRowsWG;
    const int qw0 = q0 + wq * 32;     // first query of this wave
    const int qi = qw0 + li;          // this lane's query row

    // Q fragment (B operand of S^T = K Q^T): row qi, d slice c*16 + lh*8 + 0..7.
    bf16x8 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qf[c] = qi < N ? *reinterpret_cast<const bf16x8*>(qh + (size_t)qi * D + c * 16 + lh * 8)
                       : bf16x8{};
    // Retire the Q loads here, visibly to the compiler's wait-count pass
    // (s_waitcnt vmcnt(0)); otherwise it keeps a vmcnt(0) inside the loop,
    // which would also wait for the tile loads in flight.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    const int nkb_all = (N + kBc - 1) / kBc;
    const int nkb = CAUSAL ? min(nkb_all, (q0 + kRowsWG - 1) / kBc + 1) : nkb_all;
    // Last tile with a key visible to some row of this wave.
    const int last = CAUSAL ? min(nkb - 1, (qw0 + 31) / kBc) : nkb - 1;

    // Direct loads. When a set of W waves fills a tile, load `it` of the
    // set's wave w fills LDS bytes [n*1024, n*1024 + 1024),
    // n = w*(kTileLoads/W) + it; lane i fills the 16-byte slot i there, i.e.
    // row n*kRowsPerLoad + i / kChunks, physical chunk i % kChunks, which
    // holds logical chunk (i % kChunks) ^ swz(row). The prologue's tiles are
    // loaded by all eight waves (L loads each); in the phase loop each tile is
    // loaded by the four waves of the group in its softmax phase (2L loads
    // each), so that a wave in its MFMA phase issues no memory instruction:
    // its first score MFMA does not queue behind the workgroup's tile loads
    // at the start of the phase (measured 3% faster than all eight waves
    // loading every phase).
    using TG = Tile<D, kPPWaves / 2>;
    constexpr int LG = TG::kLoadsPerWave;  // = 2L
    int ld_off[L], gl_off[LG];
#pragma unroll
    for (int it = 0; it < L; ++it) ld_off[it] = TL::load_offset(wave, it, lane);
#pragma unroll
    for (int it = 0; it < LG; ++it) gl_off[it] = TG::load_offset(wave & 3, it, lane);
    // Buffer resource over tile t of `src`. A tile past the last one gets an
    // empty range (nothing is read), so that the loads are still issued and
    // the vmcnt arithmetic of the phase loop holds.
    auto tile_rsrc = [&](const __bf16* src, int t) __attribute__((always_inline)) {
        const int j0 = t * kBc;
        const bool real = t < nkb;
        const unsigned bytes = real ? (unsigned)min(kBc, N - j0) * TL::kRowBytes : 0u;
        return buffer_rsrc(real ? src + (size_t)j0 * D : src, bytes);
    };
    // This wave's share of tile t of `src` into `dst`, all eight waves loading.
    auto issue = [&](const __bf16* src, int t, unsigned char* dst) __attribute__((always_inline)) {
        const i32x4 rs = tile_rsrc(src, t);
#pragma unroll
        for (int it = 0; it < L; ++it)
            lds_dma16(rs, ld_off[it], lds_addr(dst + (wave * L + it) * 1024));
    };
    // This wave's share of tile t, the four waves of its group loading.
    auto issue_grp = [&](const __bf16* src, int t, unsigned char* dst) __attribute__((always_inline)) {
        const i32x4 rs = tile_rsrc(src, t);
        if constexpr (PAIRED) {
            // LDS base of this wave's share, formed at the issue (not kept live)
            unsigned lb = lds_addr(dst + (wave & 3) * LG * 1024);
            asm volatile("" : "+s"(lb));
#pragma unroll
            for (int it = 0; it < LG; ++it) lds_dma16(rs, gl_off[it], lb + it * 1024);
        } else {
#pragma unroll
            for (int it = 0; it < LG; ++it)
                lds_dma16(rs, gl_off[it], lds_addr(dst + ((wave & 3) * LG + it) * 1024));
        }
    };
    // Rows of a partial last V tile past the sequence end must hold finite
    // values (their probabilities are 0, and 0 * NaN would leak); they are
    // cleared once the tile's loads have landed. Partial K rows need nothing:
    // their scores are replaced by -inf.
    auto clear_tail = [&](int t, unsigned char* dst) __attribute__((always_inline)) {
        const int rows = N - t * kBc;
        if (rows >= kBc) return;
        for (int x = tid; x < (kBc - rows) * TL::kChunks; x += kPPThreads) {
            const int row = rows + x / TL::kChunks;
            *reinterpret_cast<bf16x8*>(dst + row * TL::kRowBytes + (x % TL::kChunks) * 16) = bf16x8{};
        }
    };

    // LDS byte addresses of the two rings, hidden from constant folding: all
    // per-lane addresses below are ring base + lane offset in one VGPR, and
    // the ring slot and sub-tile offsets (< 64 KiB from the ring base) ride in
    // the instructions' 16-bit offset fields.
    unsigned kbase = lds_addr(kring[0]), vbase = lds_addr(vring[0]);
    asm volatile("" : "+s"(kbase), "+s"(vbase));

    // K fragment (A operand of S^T): key row st*32 + li, logical chunk 2c + lh.
    // V^T fragment (A operand of O^T += V^T P^T) by two transpose reads: for
    // read s (slots 4s..4s+3) lane l points at key 4*lh + (l % 16) / 4 + 8s of
    // the 16-key chunk and d = tt*32 + ((l / 16) % 2) * 16 + 4 * (l % 4).
    unsigned k_off[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) k_off[c] = kbase + TL::frag_offset(li, 2 * c + lh);
    unsigned v_off[D / 32][2];
#pragma unroll
    for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
        for (int s = 0; s < 2; ++s) v_off[tt][s] = vbase + TL::tr_offset(tt, s, lane);
    // The swizzle permutes 16-byte chunks by XOR and the ring bases are
    // 1024-aligned, so the offsets of chunk c and column block tt differ from
    // those of c = 0 and tt = 0 only by XOR: k(c) = k(0) ^ (c << 5),
    // v(tt, s) = v(0, s) ^ (tt << 6). The paired kernel, whose work-item loop
    // holds more registers, keeps only the three bases live and rebuilds the
    // rest in every phase; the one-block kernel keeps all offsets.
    auto k_frag = [&](int c) __attribute__((always_inline)) {
        if constexpr (PAIRED) return k_off[0] ^ ((unsigned)c << 5);
        else return k_off[c];
    };
    auto v_frag = [&](int tt, int s) __attribute__((always_inline)) {
        if constexpr (PAIRED) return v_off[0][s] ^ ((unsigned)tt << 6);
        else return v_off[tt][s];
    };

    // S^T tile of 64 keys from the K tile in ring slot `slot`: MFMA i uses
    // the K fragment of key row st*32 + li, d slice c*16 + lh*8, with
    // st = i % 2 and c = i / 2, so consecutive MFMAs alternate between the
    // two 32-key accumulators (no back-to-back accumulator dependency).
    constexpr int kKFrags = kBc / 32 * D / 16;
    auto scores = [&](int slot, f32x16 (&s)[kBc / 32]) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) s[st] = f32x16{};
#pragma unroll
        for (int i = 0; i < kKFrags; ++i) {
            const int st = i % (kBc / 32), c = i / (kBc / 32);
            const bf16x8 kf = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                (size_t)(k_frag(c) + slot * TL::kBytes + st * 32 * TL::kRowBytes));
            s[st] = mfma(kf, qf[c], s[st]);
        }
    };
    // Replace the scores of invisible keys (past N, or after the query when
    // causal) by -inf. Key score_key(st, r, lh) of the tile is visible iff
    // its lane-independent part st*32 + (r/4)*8 + r%4, a compile-time
    // constant, is at most one per-lane limit: written with per-key indices,
    // the mask had the compiler keep all 32 key indices in registers.
    auto mask = [&](int kb, f32x16 (&s)[kBc / 32]) {
        int lim = N - 1 - kb * kBc;
        if constexpr (CAUSAL) lim = min(lim, qi - kb * kBc);
        lim -= lh * 4;
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kc = st * 32 + (r >> 2) * 8 + (r & 3);
                s[st][r] = kc <= lim ? s[st][r] : neg_inf();
            }
    };

    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    float m_run = neg_inf();  // reference max, base-2 scaled domain
    float l_run = 0.f;        // this lane's share of the running sum

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
    f32x16 sc[kBc / 32];  // scores of the tile whose softmax runs next
    scores(KS == 1 ? 0 : grp, sc);  // KS = 2: group g starts with tile g
    __syncthreads();  // every wave is done with K_0 (K_1) before K_4 (K_5) replaces it

    // Phases. Global phase s: group 0 runs A(s/2) for even s and B(s/2) for
    // odd s; group 1 runs one phase later. A(j) is VALU work only (softmax of
    // tile j, rescale of the output); B(j) is MFMA work only (scores of tile
    // j+1 from K_{j+1}, then O += P_j V_j), so on every SIMD one wave feeds
    // the matrix core while the other runs the softmax.
    // Loads: phase s starts with one tile, V_{s/2+2} in even phases and
    // K_{(s-1)/2+4} in odd ones, loaded by the group whose softmax phase it
    // is (group s % 2; 2L loads per wave) into the ring slot of the tile four
    // back (its last reader, group 1's B, ended two phases earlier). A wave
    // thus issues 2L loads every other phase, and every phase ends with
    // vmcnt(4L): at the end of phase s the wave's loads of phases s and s-2
    // may still be in flight, those of phase s-4 have landed, and the
    // barrier publishes them. K_t is first read in phase 2t-1, V_t in phase
    // 2t+1.
    // KS = 2: tiles are consumed twice as fast (K_t is read in phase t - 1 and
    // V_t in phase t + 1, by group t % 2), so every phase loads one K and one
    // V tile: K_{s+4} into the slot of K_s (last read in phase s - 1) and
    // V_{s+2} into the slot of V_{s-2} (last read in phase s - 1), both first
    // read in phase s + 3. The loading group issues 4L loads per wave every
    // other phase, so the same vmcnt(4L) at every phase end leaves only the
    // current phase's loads in flight and publishes those of phase s - 2.
    auto phase_loads = [&](int s) __attribute__((always_inline)) {
        if ((s & 1) != grp) return;
        if constexpr (KS == 2) {
            issue_grp(kh, s + 4, kring[(s + 4) & 3]);
            issue_grp(vh, s + 2, vring[(s + 2) & 3]);
            return;
        }
        if ((s & 1) == 0) {
            const int t = s / 2 + 2;
            issue_grp(vh, t, vring[t & 3]);
        } else {
            const int t = (s - 1) / 2 + 4;
            issue_grp(kh, t, kring[t & 3]);
        }
    };
    // The partial last V tile, if any, was issued in phase 2*nkb - 6 (when
    // nkb > 2) and has landed at the end of phase 2*nkb - 2, one phase before
    // it is first read; it is cleared there, after a barrier (only the
    // loading group's waits cover it). The scheduling fences keep every
    // instruction inside its phase: the compiler would otherwise move MFMAs
    // and VALU work across the barrier and break the pairing of the groups.
    // (KS = 2: V_{nkb-1} is issued in phase nkb - 3, read in phase nkb.)
    const int tail_phase = (nkb > 2 && N % kBc != 0 && nkb == nkb_all)
                               ? (KS == 1 ? 2 * nkb - 2 : nkb - 1) : -1;
    auto phase_end = [&](int s) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(4 * L));
        if (s == tail_phase) {
            __syncthreads();
            clear_tail(nkb - 1, vring[(nkb - 1) & 3]);
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };

    // Tiles [0, nfull_w) need no mask for this wave: all their keys are < N
    // and (causal) <= the wave's first query.
    const int nfull_w = min(CAUSAL ? (qw0 + 1) / kBc : nkb_all, N / kBc);
    bf16x8 pf[kBc / 32][2];  // P of the current tile, from A(j) to B(j)

    // A(j): VALU only. Softmax of tile j (scores in sc): reference max and
    // running sum, bf16 P, and O *= alpha (skipped when no row's reference
    // moved: alpha == 1).
    auto phase_a = [&](auto full, int kb) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
        if (!FULL) {
            if (kb > last) return;
            if (kb >= nfull_w) mask(kb, sc);
        }
        // Row max of the lane's 32 scores in four v_max3 chains, then with the
        // partner lane. The scores are finite or -inf; written as instructions
        // because fmaxf would add a canonicalizing move per MFMA result.
        float mr4[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const int st = c4 >> 1, r0 = (c4 & 1) * 8;
            float m = sc[st][r0];
#pragma unroll
            for (int r = 1; r < 7; r += 2)
                asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(m), "v"(sc[st][r0 + r]), "v"(sc[st][r0 + r + 1]));
            asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(m), "v"(sc[st][r0 + 7]));
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
        // scale >= 0, so the scaled max is scale_log2 * raw max
        const float mtile = mraw > neg_inf() ? mraw * scale_log2 : neg_inf();
        const bool grow = mtile > m_run + kMaxSlack;  // -inf + slack = -inf: tile 0 always moves it
        const float m_new = grow ? mtile : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        bf16x8 p1[1][kBc / 32][2];
        // p = exp2(s c - m) in bf16 for P V, its fp32 sum in four partial
        // chains that start at -0 (so the first add folds away)
        float lsum;
        {
            float ls[4] = {-0.f, -0.f, -0.f, -0.f};
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const float p = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(sc[st][h2 * 8 + r], scale_log2, -m_run));
                        ls[r & 3] += p;
                        p1[0][st][h2][r] = (__bf16)p;
                    }
            lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
        }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) {
            pf[st][0] = p1[0][st][0];
            pf[st][1] = p1[0][st][1];
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
        }
    };
    constexpr int kPVMfmas = D / 32 * kBc / 16;
    // B(j): MFMA work only. Scores of tile j+1 from K ring slot kslot, then
    // O^T += V_j^T P_j^T from V ring slot vslot.
    auto phase_b = [&](auto full, int kb, int kslot, int vslot) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
        if constexpr (PAIRED) asm volatile("" : "+v"(k_off[0]), "+v"(v_off[0][0]), "+v"(v_off[0][1]));
        if (FULL || kb + KS <= last) {  // the wave's next tile is kb + KS
            scores(kslot, sc);
            // K fragments kReadAhead MFMAs ahead, no further (VGPR budget).
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReadAhead, 0);
#pragma unroll
            for (int i = 0; i < kKFrags - kReadAhead; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kReadAhead, 0);
        }
        if (!FULL && kb > last) return;
        // 16-key chunk outer, 32-column block inner: consecutive MFMAs update
        // different accumulators.
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int tt = 0; tt < D / 32; ++tt) {
                    const unsigned off = vslot * TL::kBytes + (st * 32 + h2 * 16) * TL::kRowBytes;
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(size_t)(v_frag(tt, 0) + off));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(size_t)(v_frag(tt, 1) + off));
                    const s16x4 lohi[2] = {lo, hi};
                    bf16x8 vf;
                    __builtin_memcpy(&vf, lohi, sizeof(vf));
                    acc[tt] = mfma(vf, pf[st][h2], acc[tt]);
                }
        // V fragments (two transpose reads each) kReadAhead MFMAs ahead.
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kReadAhead, 0);
#pragma unroll
        for (int i = 0; i < kPVMfmas - kReadAhead; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kReadAhead, 0);
    };
    // The values that cross a phase boundary pass through empty volatile asm
    // on both sides of its barrier, so that their producers stay in the phase
    // that ends and their consumers in the phase that starts (the compiler
    // sees no dependence on the barrier and otherwise moves pure arithmetic,
    // P.V MFMAs or the next exponentials, across it): A -> B: P, m, l;
    // B -> A: the next tile's scores and the output accumulators.
    auto pin_a = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) asm volatile("" : "+v"(pf[st][0]), "+v"(pf[st][1]));
        asm volatile("" : "+v"(m_run), "+v"(l_run));
    };
    auto pin_b = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < kBc / 32; ++st) asm volatile("" : "+v"(sc[st]));
#pragma unroll
        for (int t = 0; t < D / 32; ++t) asm volatile("" : "+v"(acc[t]));
    };
    // Tile j as this wave sees it: A(j) then B(j), each in its global phase
    // (group 1 one phase later than group 0). R = j mod 4 is a compile-time
    // constant, so every ring slot is a fixed LDS offset. This general step
    // keeps the per-wave conditions (tiles past the wave's last one, masked
    // tiles, the partial tile's clear); pinning here as well measured even.
    auto step = [&](auto ring, int kb) __attribute__((always_inline)) {
        constexpr int R = decltype(ring)::value;
        const int s = 2 * kb + grp;
        phase_loads(s);
        phase_a(std::false_type{}, kb);
        phase_end(s);
        phase_loads(s + 1);
        phase_b(std::false_type{}, kb, (R + 1) & 3, R);
        phase_end(s + 1);
    };
    // Steps that every wave runs whole (tiles j and j + 1 below the
    // workgroup's first query when causal, inside N, and before the phase of
    // the partial tile's clear) as straight-line code: no mask, no skip, and
    // the loads without a branch (phase 2 kb + grp is always this wave's
    // loading phase: group 0 loads V_{kb+2}, group 1 K_{kb+4}). With the
    // pins, one basic block per phase: 4.5% faster on the long-document
    // workload, 8% on non-causal N = 4096, bitwise-equal outputs.
    auto phase_end_plain = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(4 * L));
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto step_full = [&](auto ring, int kb) __attribute__((always_inline)) {
        constexpr int R = decltype(ring)::value;
        {
            const bool isk = grp != 0;
            issue_grp(isk ? kh : vh, kb + (isk ? 4 : 2), isk ? kring[R] : vring[(R + 2) & 3]);
        }
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
    if constexpr (KS == 1) {
    // Steps j < kb_full are full; kb_full <= nkb - 2 keeps the phase of the
    // partial tile's clear (2 nkb - 2, which group 1 reaches in step nkb - 2)
    // in the general path for both groups, so both meet its extra barrier.
    int kb = 0;
    const int kb_full = min(CAUSAL ? q0 / kBc : nkb - 1, min(N / kBc, nkb - 2));
    for (; kb + 4 <= kb_full; kb += 4) {
        step_full(std::integral_constant<int, 0>{}, kb);
        step_full(std::integral_constant<int, 1>{}, kb + 1);
        step_full(std::integral_constant<int, 2>{}, kb + 2);
        step_full(std::integral_constant<int, 3>{}, kb + 3);
    }
    // Four tiles per iteration; steps past the last tile (kb >= nkb) only
    // issue their (empty) loads and meet the barriers.
    for (; kb < nkb; kb += 4) {
        step(std::integral_constant<int, 0>{}, kb);
        step(std::integral_constant<int, 1>{}, kb + 1);
        step(std::integral_constant<int, 2>{}, kb + 2);
        step(std::integral_constant<int, 3>{}, kb + 3);
    }
    } else {
    // KS = 2: step j of group g is tile t = 2j + g, with A(t) in phase t and
    // B(t) (scores of tile t + 2, then P_t V_t) in phase t + 1. Both groups
    // run ceil(nkb / 2) steps; a group past its last tile only issues its
    // (empty) loads and meets the barriers.
    for (int j = 0; 2 * j < nkb; ++j) {
        const int t = 2 * j + grp;
        phase_loads(t);
        phase_a(std::false_type{}, t);
        phase_end(t);
        phase_loads(t + 1);
        phase_b(std::false_type{}, t, (t + 2) & 3, t & 3);
        phase_end(t + 1);
    }
    }
    // ---- epilogue: O = acc / l, lse = (m2 + log2 l) * ln 2
    auto epilogue = [&]() __attribute__((always_inline)) {
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
    };
    if constexpr (KS == 1) {
    // Group 0's outputs are final after its last MFMA phase: it stores them in
    // the phase in which group 1 runs its last MFMA phase (no tile is loaded
    // or read by group 0 there any more), then meets that phase's barrier.
    if (grp == 0) {
        epilogue();
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    }
    // No load may still be landing in LDS when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    if (grp == 1) epilogue();
    } else {
    // KS = 2: group 0 meets the barrier of group 1's last phase; then, with
    // every load landed and every ring read done, group 1 hands its (m, l,
    // acc) to group 0 through the K ring (lane-major 16-byte slots) and the
    // V ring, and group 0 merges the two states of each row with the factors
    // 2^(m_g - m), m = max(m_0, m_1), and stores the rows.
    if (grp == 0) {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __syncthreads();
    static_assert(kPPWaves / 2 * (D / 32) * 4 * 64 * 16 <= kRing * TL::kBytes, "exchange fits the K ring");
    float* xm = reinterpret_cast<float*>(vring[0]);  // [wave slot][m, l][lane]
    auto xacc = [&](int tt, int g) __attribute__((always_inline)) {
        return reinterpret_cast<f32x4*>(kring[0] + (((wq * (D / 32) + tt) * 4 + g) * 64 + lane) * 16);
    };
    if (grp == 1) {
        xm[(wq * 2 + 0) * 64 + lane] = m_run;
        xm[(wq * 2 + 1) * 64 + lane] = l_run;
#pragma unroll
        for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *xacc(tt, g) = f32x4{acc[tt][g * 4 + 0], acc[tt][g * 4 + 1], acc[tt][g * 4 + 2],
                                     acc[tt][g * 4 + 3]};
    }
    __syncthreads();
    if (grp == 0) {
        const float m1 = xm[(wq * 2 + 0) * 64 + lane];
        const float l1 = xm[(wq * 2 + 1) * 64 + lane];
        const float m = fmaxf(m_run, m1);
        // a group that saw no visible key of the row has m = -inf, l = 0, acc = 0
        const float a0 = m_run > neg_inf() ? __builtin_amdgcn_exp2f(m_run - m) : 0.f;
        const float a1 = m1 > neg_inf() ? __builtin_amdgcn_exp2f(m1 - m) : 0.f;
        l_run = l_run * a0 + l1 * a1;
        m_run = m;
#pragma unroll
        for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 x = *xacc(tt, g);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[tt][g * 4 + i] = acc[tt][g * 4 + i] * a0 + x[i] * a1;
            }
        epilogue();
    }
    }
    }  // work items
}

template <int D, bool CAUSAL>
hipError_t launch_one(const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o, float* lse,
                      int BH, int N, float scale_log2, hipStream_t stream)
{
    const FwdPlan pl = fwd_plan(BH, N, CAUSAL);
    const dim3 grid((unsigned)pl.grid);
    if (pl.key_split == 2)
        hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, false, 2, false>), grid, dim3(kPPThreads),
                           0, stream, q, k, v, o, lse, BH, N, pl.nqb, scale_log2);
    else if (CAUSAL && pl.balanced)
        hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, CAUSAL, 1, CAUSAL>), grid,
                           dim3(kPPThreads), 0, stream, q, k, v, o, lse, BH, N, pl.nqb, scale_log2);
    else if (CAUSAL && pl.paired)
        hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, CAUSAL, 1, false>), grid, dim3(kPPThreads),
                           0, stream, q, k, v, o, lse, BH, N, pl.nqb, scale_log2);
    else
        hipLaunchKernelGGL((fa_fwd_bf16_kernel<D, CAUSAL, false, 1, false>), grid, dim3(kPPThreads),
                           0, stream, q, k, v, o, lse, BH, N, pl.nqb, scale_log2);
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
