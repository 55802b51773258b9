// Host-only driver for the C ABI's argument checks (io_aware_tiled_09_amd/
// csrc/fa_api.cpp), built with AddressSanitizer and UBSan by
// tests/test_asan.py. The kernel launchers are replaced by stubs that count
// their calls and touch no memory, so every entry point runs its checks on
// fake device addresses without a GPU: a call either returns a status before
// any launch, or reaches exactly one stub.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>

#include "fa.h"
#include "../../io_aware_tiled_09_amd/csrc/fa_kernels.h"

static int g_launches = 0;

namespace fa {
hipError_t launch_bf16(const void*, const void*, const void*, void*, float*, int, int, int, float,
                       bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_f32(const float*, const float*, const float*, float*, float*, int, int, int,
                      float, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const float*,
                           const void*, void*, void*, void*, float*, int, int, int, float, float,
                           bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fp8(const void*, const void*, const void*, void*, float*, int, int, float, float,
                      bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const void*, const void*, const void*, const int*, const int*, void*,
                         float*, float*, int, int, int, int, int, int, int, float, hipStream_t) {
    ++g_launches; return hipSuccess;
}
static float g_scratch_stand_in[4];
hipError_t bwd_scratch(float** out) { *out = g_scratch_stand_in; return hipSuccess; }
}  // namespace fa

static int g_fail = 0;
#define EXPECT(call, status, launches)                                                     \
    do {                                                                                   \
        const int before = g_launches;                                                     \
        const int got = (call);                                                            \
        if (got != (status) || g_launches - before != (launches)) {                        \
            printf("FAIL line %d: status %d (want %d), launches %d (want %d)\n", __LINE__, \
                   got, (status), g_launches - before, (launches));                        \
            ++g_fail;                                                                      \
        }                                                                                  \
    } while (0)

int main()
{
    const uintptr_t A = 0x7F0000000000ull, MB = 1u << 20;
    auto P = [&](uintptr_t off) { return reinterpret_cast<void*>(A + off); };
    auto F = [&](uintptr_t off) { return reinterpret_cast<float*>(A + off); };
    auto I = [&](uintptr_t off) { return reinterpret_cast<int*>(A + off); };
    // forward, bf16 and fp32
    EXPECT(fa_fwd(P(0), P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), 2, 4, 333, 128, 0.1f, 1, nullptr), FA_OK, 1);
    EXPECT(fa_fwd(nullptr, P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), 2, 4, 333, 128, 0.1f, 1, nullptr), FA_ERR_NULL_PTR, 0);
    EXPECT(fa_fwd(P(0), P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), -1, 4, 333, 128, 0.1f, 1, nullptr), FA_ERR_BAD_SHAPE, 0);
    EXPECT(fa_fwd(P(0), P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), 2, 4, 333, 96, 0.1f, 1, nullptr), FA_ERR_UNSUPPORTED_HEAD_DIM, 0);
    EXPECT(fa_fwd(P(0), P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), 2, 4, 333, 128, -0.1f, 1, nullptr), FA_ERR_BAD_SCALE, 0);
    EXPECT(fa_fwd(P(8), P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), 2, 4, 333, 128, 0.1f, 1, nullptr), FA_ERR_MISALIGNED, 0);
    EXPECT(fa_fwd(P(0), P(64 * MB), P(128 * MB), P(0), F(256 * MB), 2, 4, 333, 128, 0.1f, 1, nullptr), FA_ERR_ALIASING, 0);
    EXPECT(fa_fwd(P(0), P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), 65536, 65536, 128, 64, 0.1f, 1, nullptr), FA_ERR_TOO_LARGE, 0);
    EXPECT(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 333, 128, 0.1f, 1, nullptr), FA_OK, 0);
    EXPECT(fa_fwd_f32((float*)P(0), (float*)P(64 * MB), (float*)P(128 * MB), (float*)P(192 * MB), F(256 * MB), 1, 1, 256, 64, 0.125f, 0, nullptr), FA_OK, 1);
    EXPECT(fa_fwd_f32((float*)P(0), (float*)P(64 * MB), (float*)P(128 * MB), (float*)P(192 * MB), F(64 * MB + 4), 1, 1, 256, 64, 0.125f, 0, nullptr), FA_ERR_ALIASING, 0);
    // FP8
    // (64 MiB of codes per input, 128 MiB of bf16 output)
    EXPECT(fa_fwd_fp8(P(0), P(256 * MB), P(512 * MB), P(768 * MB), F(1024 * MB), 2, 32, 8192, 128, 0.088f, 0.01f, 0.01f, 0.01f, 1, nullptr), FA_OK, 1);
    EXPECT(fa_fwd_fp8(P(0), P(256 * MB), P(512 * MB), P(768 * MB), F(800 * MB), 2, 32, 8192, 128, 0.088f, 0.01f, 0.01f, 0.01f, 1, nullptr), FA_ERR_ALIASING, 0);
    EXPECT(fa_fwd_fp8(P(0), P(256 * MB), P(512 * MB), P(768 * MB), F(1024 * MB), 2, 32, 8192, 64, 0.088f, 0.01f, 0.01f, 0.01f, 1, nullptr), FA_ERR_UNSUPPORTED_HEAD_DIM, 0);
    EXPECT(fa_fwd_fp8(P(0), P(256 * MB), P(512 * MB), P(768 * MB), F(1024 * MB), 2, 32, 8192, 128, 0.088f, 0.0f, 0.01f, 0.01f, 1, nullptr), FA_ERR_BAD_SCALE, 0);
    // backward, with a workspace and with the static scratch
    EXPECT(fa_bwd(P(0), P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), P(320 * MB), P(384 * MB), P(448 * MB), P(512 * MB), F(576 * MB), 1, 2, 100, 64, 0.125f, 1, nullptr), FA_OK, 1);
    EXPECT(fa_bwd(P(0), P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), P(320 * MB), P(384 * MB), P(448 * MB), P(512 * MB), F(256 * MB), 1, 2, 100, 64, 0.125f, 1, nullptr), FA_ERR_ALIASING, 0);
    EXPECT(fa_bwd_noalloc(P(0), P(64 * MB), P(128 * MB), P(192 * MB), F(256 * MB), P(320 * MB), P(384 * MB), P(448 * MB), P(512 * MB), 1, 2, 100, 64, 0.125f, 1, nullptr), FA_OK, 1);
    const uintptr_t G = 1024 * MB;
    EXPECT(fa_bwd_noalloc(P(0), P(G), P(2 * G), P(3 * G), F(4 * G), P(5 * G), P(6 * G), P(7 * G), P(8 * G), 1, 1, 4194305, 64, 0.125f, 1, nullptr), FA_ERR_SCRATCH_LIMIT, 0);
    // decode
    const size_t ws = fa_decode_workspace_bytes(3, 8, 128, 16, 10);
    EXPECT(fa_decode_paged(P(0), P(64 * MB), P(128 * MB), I(192 * MB), I(193 * MB), P(194 * MB), F(195 * MB), P(196 * MB), ws, 3, 8, 2, 128, 40, 16, 10, 0.1f, nullptr), FA_OK, 1);
    EXPECT(fa_decode_paged(P(0), P(64 * MB), P(128 * MB), I(192 * MB), I(193 * MB), P(194 * MB), F(195 * MB), P(196 * MB), ws - 1, 3, 8, 2, 128, 40, 16, 10, 0.1f, nullptr), FA_ERR_WORKSPACE, 0);
    EXPECT(fa_decode_paged(P(0), P(64 * MB), P(128 * MB), I(192 * MB), I(193 * MB), P(194 * MB), F(195 * MB), P(196 * MB), ws, 3, 8, 3, 128, 40, 16, 10, 0.1f, nullptr), FA_ERR_BAD_SHAPE, 0);
    // launch shape (host arithmetic only)
    {
        int rows = 0, paired = 0;
        const long long g1 = fa_fwd_grid(4, 12, 512, 0, &rows, &paired);
        const long long g2 = fa_fwd_grid(2, 32, 8192, 1, &rows, &paired);
        const long long g3 = fa_fwd_grid(1 << 16, 1 << 14, 1 << 20, 0, nullptr, nullptr);
        const long long g4 = fa_fwd_grid(-1, 2, 3, 1, nullptr, nullptr);
        if (g1 != 192 || g2 != 1024 || rows != 256 || paired != 1 || g3 != -FA_ERR_TOO_LARGE ||
            g4 != -FA_ERR_BAD_SHAPE) {
            printf("FAIL: fa_fwd_grid %lld %lld %lld %lld\n", g1, g2, g3, g4);
            ++g_fail;
        }
    }
    // every status has a description
    for (int s = 0; s <= 11; ++s)
        if (!fa_status_string(s) || !fa_status_string(s)[0]) { printf("FAIL: status %d\n", s); ++g_fail; }
    printf("%s: %d launches reached the stubs\n", g_fail ? "FAILED" : "ok", g_launches);
    return g_fail ? 1 : 0;
}
