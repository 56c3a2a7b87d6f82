// Staging of key and value tiles from HBM into LDS, shared by the fused
// forward and the unfused P.V product.
//
// Keys are stored row-major, Ks[key][d] (row stride D + 8 elements), because
// the Q.K^T product reads 8 consecutive d of one key per lane.
//
// Values are stored transposed, Vt[d][key] (row stride BN + 8), because the
// P.V product reads 8 keys of one d per lane.  The transpose happens in
// registers: a thread loads 4 consecutive keys x 8 consecutive d (four 16-byte
// loads), regroups them into 8 columns of 4 keys and writes each column with
// one 8-byte LDS store.
#pragma once

#include "common.h"

namespace attn {

template <int D, int BN, int NT>
struct KTile {
    static constexpr int KPAD = D + 8;
    static constexpr int CPR = D / 8;              // 16-byte chunks per key row
    static constexpr int CH = BN * CPR / NT;       // chunks per thread
    static_assert(CH >= 1 && BN * CPR % NT == 0, "tile/thread mismatch");
    u32x4 r[CH];

    __device__ __forceinline__ void load(const uint16_t* kb, int n0, int S, int tid) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + NT * i;
            const int key = n0 + c / CPR;
            const int col = c % CPR;
            r[i] = (key < S) ? *(const u32x4*)(kb + (int64_t)key * D + col * 8) : u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(uint16_t* Ks, int tid) const {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + NT * i;
            *(u32x4*)(Ks + (c / CPR) * KPAD + (c % CPR) * 8) = r[i];
        }
    }
};

// PERMUTE selects the key order inside each 16-key group of a Vt row.
//  false: natural order (key j at column j).
//  true:  4-key chunks in the order 0, 2, 1, 3, i.e. keys
//         0-3, 8-11, 4-7, 12-15.  Lane half g of a 32x32x16 MFMA then finds
//         the 8 keys its P operand holds (keys 4g..4g+3 and 8+4g..8+4g+3 of
//         the group, the row order of the 32x32 accumulator) contiguous.
template <int D, int BN, int NT, bool PERMUTE>
struct VTile {
    static constexpr int VPAD = BN + 8;
    static constexpr int KG = BN / 4;             // 4-key groups per tile
    static constexpr int UNITS = KG * (D / 8);    // (4 keys x 8 d) blocks per tile
    static_assert(UNITS <= NT, "one block per thread at most");
    u32x4 r[4];

    __device__ __forceinline__ bool active(int tid) const { return tid < UNITS; }

    __device__ __forceinline__ void load(const uint16_t* vb, int n0, int S, int tid) {
        if (tid >= UNITS) return;
        const int kg = tid % KG;
        const int dc = tid / KG;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int key = n0 + kg * 4 + rr;
            r[rr] = (key < S) ? *(const u32x4*)(vb + (int64_t)key * D + dc * 8) : u32x4{0, 0, 0, 0};
        }
    }

    __device__ __forceinline__ static int column(int kg) {
        if (!PERMUTE) return kg * 4;
        const int c4 = kg & 3;
        return (kg >> 2) * 16 + (((c4 & 1) << 1) | (c4 >> 1)) * 4;
    }

    __device__ __forceinline__ void store(uint16_t* Vt, int tid) const {
        if (tid >= UNITS) return;
        const int kg = tid % KG;
        const int dc = tid / KG;
        const int col = column(kg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            const uint32_t x0 = r[0][w], x1 = r[1][w], x2 = r[2][w], x3 = r[3][w];
            uint32_t lo, hi;
            if (e & 1) {
                lo = (x0 >> 16) | (x1 & 0xffff0000u);
                hi = (x2 >> 16) | (x3 & 0xffff0000u);
            } else {
                lo = (x0 & 0xffffu) | (x1 << 16);
                hi = (x2 & 0xffffu) | (x3 << 16);
            }
            *(u32x2*)(Vt + (dc * 8 + e) * VPAD + col) = u32x2{lo, hi};
        }
    }
};

}  // namespace attn
