// LDS tiles shared by the backward and split-KV kernels: a swizzled layout
// that serves both row reads and transposed reads, a whole-row global loader
// for it, and the transposed-read offsets.
#pragma once

#include "common.h"

namespace attn {

// LDS tile of rows x D bf16 (row-major, 16-byte chunks), read two ways: a
// row read (16 bytes of one row per lane: 16 lanes on 16 consecutive rows)
// and a transposed read (ds_read_b64_tr_b16: 16 lanes on 4 consecutive rows,
// 32 bytes of each).  Chunk c of row r sits at chunk position c ^ swz(r),
// which keeps both patterns free of bank conflicts.
template <int D>
struct SwzTile {
    static constexpr int CPR = D / 8;
    __device__ static int swz(int r) {
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    }
    // element offset of 8-aligned column col of row r
    __device__ static int at(int r, int col) { return r * D + ((((col >> 3) ^ swz(r))) << 3) + (col & 7); }
};

// Rows [r0, r0 + ROWS) of a [S, D] bf16 matrix -> registers, 16 bytes per
// thread per instruction, D/8 lanes per row (whole cache lines); rows past S
// are zero.  store() writes them to a SwzTile.
template <int D, int ROWS, int NT>
struct RowTile {
    static constexpr int CPR = D / 8;
    static constexpr int CH = ROWS * CPR / NT;
    static_assert(CH * NT == ROWS * CPR, "tile/thread mismatch");
    u32x4 r[CH];
    __device__ __forceinline__ void load(const uint16_t* base, int r0, int S, int tid) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + NT * i, row = r0 + c / CPR;
            r[i] = row < S ? *(const u32x4*)(base + (int64_t)row * D + (c % CPR) * 8) : u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(uint16_t* t, int tid) const {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + NT * i;
            *(u32x4*)(t + SwzTile<D>::at(c / CPR, (c % CPR) * 8)) = r[i];
        }
    }
};

__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int half) {
    const u32x4 w = {pack_bf16x2(x[8 * half + 0], x[8 * half + 1]), pack_bf16x2(x[8 * half + 2], x[8 * half + 3]),
                     pack_bf16x2(x[8 * half + 4], x[8 * half + 5]), pack_bf16x2(x[8 * half + 6], x[8 * half + 7])};
    return as_bf16x8(w);
}

// Per-lane offsets of the transposed read of a 16-row block (rows 16kb + ..)
// of a SwzTile: lane j of 16-lane group G reads row 4(G/2) + j/4 (k-slots
// 0-3) and that row + 8 (k-slots 4-7), columns 32db + 16(G%2) + 4(j%4) .. +3.
// Adding 16 rows leaves the swizzle unchanged, so block kb is + 16 kb D.
template <int D>
struct TrOffsets {
    static constexpr int DB = D / 32;
    int lo[DB], hi[DB];
    __device__ __forceinline__ void init(int lane) {
        const int G = lane >> 4, j = lane & 15;
        const int r = 4 * (G >> 1) + (j >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int col = db * 32 + (G & 1) * 16 + 4 * (j & 3);
            lo[db] = SwzTile<D>::at(r, col);
            hi[db] = SwzTile<D>::at(r + 8, col);
        }
    }
    __device__ __forceinline__ bf16x8 read(const uint16_t* t, int kb, int db) const {
        return tr_read_pair(t + kb * 16 * D + lo[db], t + kb * 16 * D + hi[db]);
    }
};

// A wave's 32 x D output tile, held as transposed 32x32 MFMA accumulators
// acc[db] (lane l32 = output row, register 4j + e = column 32 db + 8 j + 4 g
// + e), times the lane's scale, to bf16 rows dst + r D for r < nrows (the 32
// rows are contiguous in memory).  Goes through 32 D 2 bytes of LDS owned by
// the wave so that every store instruction writes whole rows, 16 bytes per
// lane: stores of 8 bytes per lane spread over 32 rows cost several times
// more.  In LDS, 16-byte chunk c of row r sits at c ^ ((r / RPL) % CPO) (RPL
// rows share one 256-byte bank line), with its two 8-byte halves swapped for
// rows 16-31: the 32 lanes of one write (one row each, same chunk and half)
// then cover all 64 banks once, and the reads (16 lanes per 256 bytes) too.
template <int D, int BATCH = 32 * D * 2 / 16 / 64>
__device__ __forceinline__ void store_rows_via_lds(char* stage, const f32x16 (&acc)[D / 32], float scale,
                                                   uint16_t* dst, int nrows, int lane) {
    constexpr int RB = D * 2;     // bytes per row
    constexpr int CPO = RB / 16;  // 16-byte chunks per row
    constexpr int RPL = 256 / RB; // rows per 256-byte bank line
    const int l32 = lane & 31, g = lane >> 5;
    const int wswz = (l32 / RPL) % CPO, whalf = g ^ ((l32 >> 4) & 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x2 w = {pack_bf16x2(acc[db][4 * j] * scale, acc[db][4 * j + 1] * scale),
                             pack_bf16x2(acc[db][4 * j + 2] * scale, acc[db][4 * j + 3] * scale)};
            const int c = db * 4 + j;
            *(u32x2*)(stage + l32 * RB + ((c ^ wswz) * 16) + whalf * 8) = w;
        }
    }
    // the wave's own LDS writes complete before its reads (in order).  BATCH
    // read-backs are in flight at a time (fewer registers for callers that
    // hold much else).
#pragma unroll
    for (int i0 = 0; i0 < 32 * CPO / 64; i0 += BATCH) {
#pragma unroll
        for (int i = i0; i < i0 + BATCH; ++i) {
            const int pos = i * 64 + lane, r = pos / CPO, c = pos % CPO;
            u32x4 x = *(const u32x4*)(stage + r * RB + ((c ^ ((r / RPL) % CPO)) * 16));
            if ((r >> 4) & 1) x = u32x4{x[2], x[3], x[0], x[1]};
            if (r < nrows) *(u32x4*)(dst + (int64_t)r * D + c * 8) = x;
        }
        if (i0 + BATCH < 32 * CPO / 64) __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace attn
