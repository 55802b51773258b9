// LDS tile layout and HBM -> LDS direct loads shared by the bf16 forward and
// backward kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>

#include "fa_common.h"

namespace fa {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// One tile of kBc rows of a [rows][D] bf16 tensor (K, V, Q or dO) in LDS,
// loaded by WAVES waves with 16-byte-per-lane direct loads.
template <int D, int WAVES>
struct Tile {
    static constexpr int kRowBytes = D * 2;                 // one row, bf16
    static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
    static constexpr int kBytes = kBc * kRowBytes;          // one tile
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;   // rows per wave-wide load
    static constexpr int kLoadsPerWave = kBytes / 1024 / WAVES;
    static_assert(kLoadsPerWave * 1024 * WAVES == kBytes, "tile must split over waves");

    // Physical 16-byte chunk slot of logical chunk c in tile row r is c ^ swz(r).
    // D = 128 (16 chunks/row, rows 256 B apart): a bijection of r mod 16 whose
    //   value over 4 consecutive rows differs in bits 2-3.
    // D = 64 (8 chunks/row, rows 128 B apart, so row parity picks the bank
    //   half): a bijection of (r >> 1) mod 8 whose value over rows r, r+2
    //   differs in bit 2.
    // Reads of 16 rows at one logical chunk (row-major fragments) and the
    // transpose reads (4 rows x 4 chunks per 32 lanes) then hit distinct banks.
    __device__ static int swz(int r) {
        if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
        else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    }
    // Byte offset, in the tile, of this wave's direct load `it` for `lane`:
    // load n = wave*kLoadsPerWave + it fills tile bytes [n*1024, n*1024+1024),
    // lane i the 16-byte slot i there, i.e. row n*kRowsPerLoad + i/kChunks at
    // physical chunk i % kChunks, which holds logical chunk (i % kChunks) ^ swz(row).
    __device__ static int load_offset(int wave, int it, int lane) {
        const int n = wave * kLoadsPerWave + it;
        const int row = n * kRowsPerLoad + lane / kChunks;
        const int lchunk = (lane % kChunks) ^ swz(row);
        return row * kRowBytes + lchunk * 16;
    }
    // Byte offset of the row-major fragment read (16 bytes: d = chunk*8..+7)
    // of `row` at logical chunk `chunk`.
    __device__ static int frag_offset(int row, int chunk) {
        return row * kRowBytes + ((chunk ^ swz(row)) * 16);
    }
    // Byte offset of transpose read s (0, 1) for the 32-column block tt: lane
    // l points at row 4*lh + (l % 16) / 4 + 8s of a 16-row chunk and column
    // d0 = tt*32 + ((l / 16) % 2) * 16 + 4 * (l % 4); in each 16-lane group,
    // lanes 4k..4k+3 supply 16 consecutive columns of row k and lane i receives
    // column i of the 4 rows, so two reads give a lane the 8 rows
    // {4h..4h+3, 8+4h..8+4h+3} of one column (h = lane / 32).
    __device__ static int tr_offset(int tt, int s, int lane) {
        const int lh = lane >> 5;
        const int row = 4 * lh + (lane % 16) / 4 + 8 * s;
        const int d0 = tt * 32 + ((lane / 16) % 2) * 16 + 4 * (lane % 4);
        return row * kRowBytes + (((d0 / 8) ^ swz(row)) * 16) + (d0 % 8) * 2;
    }
};

// s_waitcnt immediate (gfx9 encoding) with only vmcnt constrained (n < 16):
// expcnt and lgkmcnt keep their maximum values.
constexpr int wait_vmcnt(int n) { return 0x0F70 | n; }

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
// other buffers as dependent on it; kernels wait for these loads explicitly
// (vmcnt) before the barrier that publishes a tile. The LDS base goes in
// M0 as an input operand of the asm ("{m0}"), so the compiler itself sets M0
// and knows what it holds.
__device__ inline void lds_dma16(i32x4 rsrc, unsigned voff, unsigned lds_base) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "{m0}"(lds_base) : "memory");
}

}  // namespace fa
