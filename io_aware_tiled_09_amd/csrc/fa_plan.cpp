// Launch shapes of the bf16 forward (host code: the kernel file launches by
// it, the C ABI reports it) and the choice of the backward's dQ kernel.
#include "fa_kernels.h"

namespace fa {
namespace {

// Causal grids run one workgroup per pair of query blocks (the i-th
// heaviest with the i-th lightest) when the grid is small or N <= 8192: with
// one block each, the heavy blocks (many key tiles) and the light ones land
// unevenly on the CUs. The paired kernel measured 1-17% faster for d = 128
// causal at N <= 8192 on grids of 1024-2048 blocks, and even at N = 16384,
// so longer sequences keep one block per workgroup.
constexpr long long kPairMaxGrid = 2 * 256;  // 256 CUs on MI355X
constexpr int kPairMaxN = 8192;
// A grid of fewer workgroups than CUs leaves CUs idle; if the grid of
// 128-row blocks whose key range the two wave groups split (KS = 2) still
// fits one workgroup per CU, that grid runs instead: each workgroup then
// has half the key tiles per group. A larger key-split grid runs in more
// than one round of workgroups, and the fixed cost of each workgroup (its
// prologue, the first tiles' latency, the epilogue) outweighs the shorter
// loop (measured on B8 H12 N1024 d64 causal: 768 key-split workgroups
// 43.0 us, 384 unpaired blocks 41.6 us, 192 paired blocks 31.4 us).
constexpr long long kCUs = 256;
// Causal grids whose pairs leave CUs idle and which the key split would run
// in more than one round group the query blocks so that every workgroup
// has exactly the heaviest block's work: block q of a head costs q + 1 units
// (4 key tiles each), and the workgroups are {nqb-1}, {nqb-2-p, p} and, when
// nqb is even, the middle blocks (nqb-2)/2 of two heads. nqb units per
// workgroup instead of the pairs' nqb + 1, and about half a workgroup more
// per head (GPT-2 shape: 240 workgroups of 4 units against 192 of 5).
long long balanced_grid(long long BH, int nqb)
{
    const long long per = 1 + (nqb - 1) / 2;
    return BH * per + (nqb % 2 == 0 ? (BH + 1) / 2 : 0);
}

}  // namespace

FwdPlan fwd_plan(long long BH, int N, bool causal)
{
    FwdPlan pl;
    pl.balanced = false;
    pl.key_split = 1;
    pl.rows = kBrBf16;
    pl.nqb = (N + kBrBf16 - 1) / kBrBf16;
    const long long blocks = BH * pl.nqb;
    pl.paired = causal && pl.nqb > 1 && (blocks <= kPairMaxGrid || N <= kPairMaxN);
    pl.grid = pl.paired ? BH * ((pl.nqb + 1) / 2) : blocks;
    const int nqb2 = (N + kBrBf16 / 2 - 1) / (kBrBf16 / 2);
    if (pl.grid < kCUs && BH * nqb2 <= kCUs && BH * nqb2 > pl.grid) {
        pl.key_split = 2;
        pl.paired = false;
        pl.rows = kBrBf16 / 2;
        pl.nqb = nqb2;
        pl.grid = BH * nqb2;
    } else if (causal && pl.nqb > 1 && pl.grid < kCUs && balanced_grid(BH, pl.nqb) <= kCUs) {
        pl.paired = true;
        pl.balanced = true;
        pl.grid = balanced_grid(BH, pl.nqb);
    }
    return pl;
}

// The phased dQ kernel (256 queries and one workgroup per CU, two
// phase-offset wave groups) runs grids of at least four rounds of
// workgroups; smaller grids run the 128-query kernel with two workgroups per
// CU, whose workgroups overlap one another's prologue and epilogue. Measured
// (whole backward call, gradients bitwise equal; 128-query -> phased):
// B2 H32 N8192 d128 causal (2048 workgroups of 256 queries) 3421 -> 3345-3353
// us, B1 H32 N16384 causal (2048) 6399 -> 6231 us, B2 H32 N4096 non-causal
// (1024) 1676 -> 1634 us; B4 H16 N2048 d128 causal (512) 297.2 -> 303.3 us,
// B8 H16 N1024 d64 causal (512) 139.2 -> 140.2 us, B8 H12 N1024 d64 causal
// (384) 111.4 -> 116.9 us, B4 H12 N512 d64 (96) 28.4 -> 32.4 us.
bool bwd_dq_phased(long long BH, int N)
{
    return BH * ((N + 255) / 256) >= 4 * kCUs;
}

}  // namespace fa
