// Launch shape of the bf16 forward (host code: the kernel file launches by
// it, the C ABI reports it).
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

}  // namespace

FwdPlan fwd_plan(long long BH, int N, bool causal)
{
    FwdPlan pl;
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
    }
    return pl;
}

}  // namespace fa
