// Internal interface between the C ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime_api.h>

namespace fa {

constexpr int kWaves = 4;            // wave64s per workgroup
constexpr int kBr = kWaves * 32;     // query rows per workgroup (32 per wave)
constexpr int kBc = 64;              // keys per K/V tile
constexpr int kBrBf16 = 256;         // query rows per workgroup of the bf16 kernel (8 waves)

// Enqueue one forward pass on `stream`. Shapes are assumed validated:
// BH = B*H >= 1, N >= 1, d in {64, 128}, BH*ceil(N/kBr) < 2^31.
// scale_log2 = softmax scale * log2(e) >= 0.
hipError_t launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                       int BH, int N, int d, float scale_log2, bool causal, hipStream_t stream);
// Grid of the bf16 forward for a shape: rows per query block (256, or 128
// when the two wave groups split the key range), whether causal blocks run
// in pairs, and the number of workgroups.
struct FwdPlan {
    int key_split;      // 1 or 2
    bool paired;
    bool balanced;      // causal blocks grouped so that every workgroup has nqb units of work
    int rows;           // query rows per block
    int nqb;            // query blocks per head
    long long grid;     // workgroups
};
FwdPlan fwd_plan(long long BH, int N, bool causal);
// Whether the backward's dQ runs the phased 256-query kernel (else the
// 128-query one).
bool bwd_dq_phased(long long BH, int N);
hipError_t launch_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                      int BH, int N, int d, float scale_log2, bool causal, hipStream_t stream);
// Backward pass (bf16 tensors, fp32 lse); delta: BH*N floats of workspace.
// scale_log2 as above; scale = the softmax scale itself (>= 0).
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* delta, int BH, int N, int d, float scale_log2, float scale,
                           bool causal, hipStream_t stream);

// Static device scratch of the allocation-free backward (fa_scratch.hip):
// room for the D values of B*H*N <= kBwdScratchRows rows (16 MiB per GPU).
// bwd_scratch() returns the current device's address of it, looked up once
// per device; it allocates nothing.
constexpr long long kBwdScratchRows = 1LL << 22;
hipError_t bwd_scratch(float** out);

// FP8 E4M3 forward (d = 128): q, k, v hold E4M3 codes; c_log2 = scale *
// q_scale * k_scale * log2(e) > 0; out_scale = v_scale.
hipError_t launch_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                      int N, float c_log2, float out_scale, bool causal, hipStream_t stream);

// Decode over a paged KV cache. Keys per split workgroup, and the number of
// split slots per (sequence, head) in the workspace.
constexpr int kSplit = 512;
inline int decode_max_splits(int max_pages, int page_size) {
    return (int)(((long long)max_pages * page_size + kSplit - 1) / kSplit);
}
// q, o: bf16 [B][H][d]; caches: bf16 [num_pages][H_kv][page_size][d];
// ws: fp32 workspace of B*H*max_splits*(d + 2) floats; c_log2 = scale*log2(e).
// Validated: d in {64, 128}, H / H_kv in {1, 2, 4, 8}, page_size % 16 == 0.
hipError_t launch_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int* page_table, const int* seq_lens, void* o, float* lse,
                         float* ws, int B, int H, int H_kv, int d, int num_pages, int page_size,
                         int max_pages, float c_log2, hipStream_t stream);

}  // namespace fa
