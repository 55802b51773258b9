// Attention forward with 8-bit (FP8 E4M3) Q, K and V on CDNA4 (gfx950).
//
// [FlashAttention: The GPU Memory Hack That Changed Everything
//  (ai.branddocks.com, episode 75), "FlashAttention-3: Hopper Architecture":
//  attention run in FP8 on the matrix units, about twice the FP16 rate, with
//  negligible quality loss]
// The method is the same tiled, single-running-max recurrence as the bf16
// kernel; only the operand precision of the two products changes:
//  * Q, K, V arrive as E4M3 codes with one scale per tensor (value = scale *
//    code). S^T = K Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4 (64 of d per
//    instruction, fp32 accumulation); the Q and K scales fold into the
//    softmax constant c = scale * q_scale * k_scale * log2(e).
//  * p = exp2(s c - m) is in (0, 1]; P is stored for the second product as
//    E4M3 of 256 * p (the factor keeps small weights out of the subnormal
//    range; 256 <= 448, the largest code), and the row sum l takes the fp32 p.
//  * O^T += V^T P^T on the same instruction, 64 keys per instruction; V^T
//    comes from ds_read_b64_tr_b8 transpose reads of the V tile. The epilogue
//    divides by 256 l and multiplies by v_scale.
//
// Layout: 4 waves of 32 query rows (128 per workgroup), K and V tiles of 64
// keys x 128 bytes double-buffered in LDS and loaded by buffer_load ... lds;
// within each 128-byte row the 16-byte chunks are XOR-swizzled so that both
// the row reads of K and the transpose reads of V are bank-conflict-free.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.h"
#include "fa_lds.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kF8Waves = 4;
constexpr int kF8Threads = kF8Waves * 64;
constexpr int kF8Rows = kF8Waves * 32;  // queries per workgroup
constexpr int kF8D = 128;               // head dimension (bytes per row)
constexpr float kPScale = 256.0f;       // P is stored as E4M3(256 p)

// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E4M3 and unit scales
// (E8M0 127 = 2^0).
__device__ inline f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// One 64-key tile of a [rows][128] byte tensor in LDS.
struct Tile8 {
    static constexpr int kRowBytes = kF8D;
    static constexpr int kChunks = kRowBytes / 16;                     // 8
    static constexpr int kBytes = kBc * kRowBytes;                     // 8 KiB
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;              // 8
    static constexpr int kLoadsPerWave = kBytes / 1024 / kF8Waves;     // 2
    // Physical chunk of logical chunk c in row r is c ^ swz(r). Bank group of
    // a 16-byte slot is (8 * (r % 2) + chunk) % 16. Row reads of 16
    // consecutive rows at one logical chunk need swz to be a bijection on the
    // 8 rows of each parity; the transpose reads (rows b + {0..3, 8..11} for
    // b % 4 == 0, two adjacent chunks) need its bits 1-2 to differ over the
    // four rows of each parity. This swz does both.
    __device__ static int swz(int r) {
        return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | ((r >> 2) & 1);
    }
    __device__ static int load_offset(int wave, int it, int lane) {
        const int n = wave * kLoadsPerWave + it;
        const int row = n * kRowsPerLoad + lane / kChunks;
        return row * kRowBytes + (((lane % kChunks) ^ swz(row)) * 16);
    }
    __device__ static int frag_offset(int row, int chunk) {
        return row * kRowBytes + ((chunk ^ swz(row)) * 16);
    }
    // Transpose read r (0..3) of the 32-column block tt for `lane`: in each
    // 16-lane group, lanes 2k and 2k+1 point at the two 8-byte halves of one
    // 16-byte slot of row k (k = 0..7) and lane j receives byte j of the 8
    // rows. Row k is key b_r + k (k < 4) or b_r + k + 4 (k >= 4), b_r =
    // 32 (r / 2) + 16 (r % 2) + 4 h, h = lane / 32: the keys that byte
    // 8 r + k of the P operand holds (the score layout's key order).
    __device__ static int tr_offset(int tt, int r, int lane) {
        const int j = lane & 15, k = j >> 1, half = j & 1;
        const int h = lane >> 5;
        const int row = 32 * (r >> 1) + 16 * (r & 1) + 4 * h + (k < 4 ? k : k + 4);
        const int chunk = tt * 2 + ((lane >> 4) & 1);
        return row * kRowBytes + ((chunk ^ swz(row)) * 16) + half * 8;
    }
};

template <bool CAUSAL>
__global__ __launch_bounds__(kF8Threads) __attribute__((amdgpu_waves_per_eu(CAUSAL ? 3 : 2, CAUSAL ? 3 : 2)))
void fa_fwd_fp8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                       const uint8_t* __restrict__ v, __bf16* __restrict__ o,
                       float* __restrict__ lse, int BH, int N, int nqb, float c_log2,
                       float out_scale)
{
    using TL = Tile8;
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

    int ld_off[L];
#pragma unroll
    for (int it = 0; it < L; ++it) ld_off[it] = TL::load_offset(wave, it, lane);
    // K fragment of key row st*32 + li: logical chunks 4c + 2h and 4c + 2h + 1.
    int k_off[kF8D / 64][2];
#pragma unroll
    for (int c = 0; c < kF8D / 64; ++c)
#pragma unroll
        for (int x = 0; x < 2; ++x) k_off[c][x] = TL::frag_offset(li, 4 * c + 2 * lh + x);
    int v_off[kF8D / 32][4];
#pragma unroll
    for (int tt = 0; tt < kF8D / 32; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) v_off[tt][r] = TL::tr_offset(tt, r, lane);

    auto issue = [&](const uint8_t* src, int t, unsigned char* dst) __attribute__((always_inline)) {
        const int j0 = t * kBc;
        const unsigned bytes = (unsigned)min(kBc, N - j0) * TL::kRowBytes;
        const i32x4 rs = buffer_rsrc(src + (size_t)j0 * kF8D, bytes);
#pragma unroll
        for (int it = 0; it < L; ++it)
            lds_dma16(rs, ld_off[it], lds_addr(dst + (wave * L + it) * 1024));
    };
    // Rows past the sequence end are cleared once the tile has landed: their
    // weights are 0, and 0 * NaN would leak.
    auto clear_tail = [&](int t, unsigned char* dst) __attribute__((always_inline)) {
        const int rows = N - t * kBc;
        if (rows >= kBc) return;
        for (int x = tid; x < (kBc - rows) * TL::kChunks; x += kF8Threads)
            *reinterpret_cast<i32x4*>(dst + (rows + x / TL::kChunks) * TL::kRowBytes +
                                      (x % TL::kChunks) * 16) = i32x4{};
    };

    const int nkb_all = (N + kBc - 1) / kBc;
    const int nkb = CAUSAL ? min(nkb_all, (q0 + kF8Rows - 1) / kBc + 1) : nkb_all;

    f32x16 acc[kF8D / 32];  // O^T: rows d = 32 tt + 8 g + 4 h + i, column = query li
#pragma unroll
    for (int tt = 0; tt < kF8D / 32; ++tt) acc[tt] = f32x16{};
    float m = neg_inf();  // running row max of s * c (both partner lanes agree)
    float l = 0.f;        // this lane's share of the row sum

    issue(kh, 0, kbuf[0]);
    issue(vh, 0, vbuf[0]);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    clear_tail(0, kbuf[0]);
    clear_tail(0, vbuf[0]);
    __syncthreads();

    for (int kb = 0; kb < nkb; ++kb) {
        const int b = kb & 1;
        if (kb + 1 < nkb) {
            issue(kh, kb + 1, kbuf[b ^ 1]);
            issue(vh, kb + 1, vbuf[b ^ 1]);
        }
        // Causal: a wave whose rows all precede the tile's first key skips it.
        const bool active = !CAUSAL || kb * kBc <= qw0 + 31;
        if (active) {
            const unsigned char* kt = kbuf[b];
            const unsigned char* vt = vbuf[b];
            // S^T for the tile's 64 keys: lane = query, 16 keys per sub-tile.
            f32x16 s[kBc / 32];
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st) {
                s[st] = f32x16{};
#pragma unroll
                for (int c = 0; c < kF8D / 64; ++c) {
                    const int base = st * 32 * TL::kRowBytes;
                    const i32x4 lo = *reinterpret_cast<const i32x4*>(kt + base + k_off[c][0]);
                    const i32x4 hi = *reinterpret_cast<const i32x4*>(kt + base + k_off[c][1]);
                    const i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    s[st] = mfma8(a, qf[c], s[st]);
                }
            }
            // Mask keys past the sequence end and, causal, after this row.
            const bool need_mask = (CAUSAL && kb * kBc + kBc - 1 > qw0) || kb * kBc + kBc > N;
            if (need_mask) {
#pragma unroll
                for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = kb * kBc + score_key(st, r, lh);
                        if (j >= N || (CAUSAL && j > qi)) s[st][r] = neg_inf();
                    }
            }
            // Running max over both partner lanes (the row's two key halves).
            float mx = neg_inf();
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
            mx = max_with_partner(mx * c_log2);
            const float m_new = fmaxf(m, mx);
            // Every row sees key 0 in tile 0, so m_new is finite from there on.
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            m = m_new;
            // p = exp2(s c - m), E4M3(256 p) packed in the score layout's key
            // order: byte 16 st + 4 g + i of this lane is key score_key(st, 4g + i).
            i32x8 pf;
            float lsum = 0.f;
            const float mb = m - 8.0f;  // exp2(s c - (m - 8)) = 256 p
#pragma unroll
            for (int st = 0; st < kBc / 32; ++st)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float p4[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = s[st][g * 4 + i];
                        p4[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c_log2, -mb));
                        lsum += p4[i];
                    }
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p4[0], p4[1], 0, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(p4[2], p4[3], w, true);
                    pf[st * 4 + g] = w;
                }
            l = l * alpha + lsum * (1.0f / kPScale);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
                for (int tt = 0; tt < kF8D / 32; ++tt) acc[tt] *= alpha;
            }
            // O^T += V^T P^T: V^T by four transpose reads per 32-row block.
#pragma unroll
            for (int tt = 0; tt < kF8D / 32; ++tt) {
                i32x8 a;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_i32x2*)(vt + v_off[tt][r]));
                    a[2 * r] = x[0];
                    a[2 * r + 1] = x[1];
                }
                acc[tt] = mfma8(a, pf, acc[tt]);
            }
        }
        if (kb + 1 < nkb) {
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));  // this wave's loads of tile kb+1
            clear_tail(kb + 1, kbuf[b ^ 1]);
            clear_tail(kb + 1, vbuf[b ^ 1]);
        }
        __syncthreads();
    }

    // Keep the accumulators' last products in uniform control flow.
#pragma unroll
    for (int tt = 0; tt < kF8D / 32; ++tt) asm volatile("" : "+v"(acc[tt]));
    const float lt = sum_with_partner(l);
    const float inv = out_scale / (kPScale * lt);  // l in units of p; acc in units of 256 p
    if (qi < N) {
        __bf16* orow = o + head_off + (size_t)qi * kF8D;
#pragma unroll
        for (int tt = 0; tt < kF8D / 32; ++tt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store4(orow + tt * 32 + g * 8 + lh * 4, acc[tt][g * 4] * inv,
                       acc[tt][g * 4 + 1] * inv, acc[tt][g * 4 + 2] * inv,
                       acc[tt][g * 4 + 3] * inv);
        if (lh == 0)
            lse[(size_t)bh * N + qi] = (m + __builtin_amdgcn_logf(lt)) * 0.6931471805599453f;
    }
}

}  // namespace

hipError_t launch_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int N, float c_log2, float out_scale, bool causal, hipStream_t stream)
{
    const int nqb = (N + kF8Rows - 1) / kF8Rows;
    const dim3 grid((unsigned)((long long)BH * nqb));
    auto qp = static_cast<const uint8_t*>(q);
    auto kp = static_cast<const uint8_t*>(k);
    auto vp = static_cast<const uint8_t*>(v);
    auto op = static_cast<__bf16*>(o);
    if (causal)
        hipLaunchKernelGGL((fa_fwd_fp8_kernel<true>), grid, dim3(kF8Threads), 0, stream, qp, kp,
                           vp, op, lse, BH, N, nqb, c_log2, out_scale);
    else
        hipLaunchKernelGGL((fa_fwd_fp8_kernel<false>), grid, dim3(kF8Threads), 0, stream, qp, kp,
                           vp, op, lse, BH, N, nqb, c_log2, out_scale);
    return hipGetLastError();
}

}  // namespace fa
