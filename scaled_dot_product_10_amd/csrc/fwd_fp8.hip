// Fused attention forward with fp8 (OCP E4M3, "e4m3fn") operands on the
// gfx950 fp8 matrix cores: q, k, v are e4m3 codes with one float scale each
// (value = code * scale); the probabilities are rounded to e4m3 for the P.V
// product; scores, sums and the output accumulate in float32; out is bf16.
//
// The FP8 remark of the ai-manual.ru tutorial (section 6: on H100 SDPA runs
// in FP8 for about another 2x) is the idea; v_mfma_scale_f32_32x32x64_f8f6f4
// (unit block scales) does 32x32x64 per instruction, twice the bf16 rate.
//
// Layout and schedule: 128 queries per workgroup (32 per wave), 64-key tiles
// of K and V through LDS (whole-row loads, the next tile in registers while
// the current one is multiplied).  Per tile and wave:
//   S^T = K.Q^T: A = K rows from LDS (32 bytes of d per lane), B = Q (kept in
//     registers); two 32-key blocks.
//   softmax: exact running max per query (so every p <= 1), p scaled by 2^8
//     (so the small ones stay in e4m3's normal range) and rounded to e4m3;
//     the sum l adds the rounded values back, so out is an exact convex
//     combination of v rows under the weights actually used.
//   O^T += V^T.P^T: A = V^T via ds_read_b64_tr_b8, B = the 32 e4m3 weights a
//     lane holds (its two 16-key halves of the S^T accumulators).
// The k order of an fp8 product only has to agree between A and B within each
// half-wave; the transposed V reads are arranged to match the accumulator's
// key order (rows 8(r/4) + 4g + r%4 of each 32-key block).
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int NT = 256;  // 4 waves
constexpr int BM = 128;  // queries per workgroup
constexpr int BN = 64;   // keys per tile
constexpr float kPScale = 256.0f;  // p in (0, 1] is stored as p * 2^8 (<= 256 < 448)

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

struct Fp8Params {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    uint16_t* out;
    float* lse;
    int Hq, Hkv, S, group, nq;
    uint32_t total;
    float c;      // softmax scale * q_scale * k_scale * log2(e)
    float vs;     // v_scale
};

// 32x32x64 e4m3 x e4m3 -> f32 (block scales 2^0)
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// LDS tile: rows x D bytes, 16-byte chunks; chunk c of row r at c ^ swz(r).
// Row reads (16 lanes on 16 rows) and the transposed byte reads (16 lanes on
// 8 rows) both hit distinct banks.
template <int D>
struct Fp8Tile {
    static constexpr int CPR = D / 16;  // chunks per row
    __device__ static int swz(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
    __device__ static int at(int r, int chunk) { return r * D + ((chunk ^ swz(r)) << 4); }
};

// BN rows [r0, r0 + BN) of a [S, D] byte matrix -> registers -> LDS; rows past S are zero
template <int D>
struct Fp8Rows {
    static constexpr int CPR = D / 16;
    static constexpr int CH = BN * CPR / NT;
    static_assert(CH >= 1 && CH * NT == BN * CPR, "tile/thread mismatch");
    u32x4 r[CH];
    __device__ __forceinline__ void load(const uint8_t* base, int r0, int S, int tid) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + NT * i, row = r0 + c / CPR;
            r[i] = row < S ? *(const u32x4*)(base + (int64_t)row * D + (c % CPR) * 16) : u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(uint8_t* t, int tid) const {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + NT * i;
            *(u32x4*)(t + Fp8Tile<D>::at(c / CPR, c % CPR)) = r[i];
        }
    }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void fwd_fp8_kernel(Fp8Params p) {
    constexpr int KS = D / 64;  // k-steps of the Q.K^T product
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    using T = Fp8Tile<D>;
    __shared__ __attribute__((aligned(16))) uint8_t Ks[BN * D];
    __shared__ __attribute__((aligned(16))) uint8_t Vs[BN * D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const uint32_t L = xcd_remap(blockIdx.x, p.total);
    const int bh = (int)(L / (uint32_t)p.nq);
    const int tile = CAUSAL ? p.nq - 1 - (int)(L % (uint32_t)p.nq) : (int)(L % (uint32_t)p.nq);
    const int b = bh / p.Hq, h = bh % p.Hq, kvh = h / p.group;
    const int S = p.S;
    const int m0 = tile * BM;
    const int qw = m0 + wave * 32;
    const int qi = qw + l32;
    const int64_t row0 = (int64_t)bh * S;
    const uint8_t* kb = p.k + ((int64_t)b * p.Hkv + kvh) * S * D;
    const uint8_t* vb = p.v + ((int64_t)b * p.Hkv + kvh) * S * D;

    // Q operand: query qi, d = 64 ks + 32 g .. +31
    i32x8 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
        if (qi < S) {
            const uint8_t* src = p.q + (row0 + qi) * D + ks * 64 + g * 32;
            lo = *(const u32x4*)src;
            hi = *(const u32x4*)(src + 16);
        }
        qreg[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    // K row read of row l32 (+32 sb), chunks 4 ks + 2 g and + 1
    int koff[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        koff[ks][0] = T::at(l32, 4 * ks + 2 * g);
        koff[ks][1] = T::at(l32, 4 * ks + 2 * g + 1);
    }
    // transposed V read u (bytes 8u..8u+7 of the A operand): source lane
    // s = lane % 16 names key row 16u + 8(t/4) + 4g + t%4 (t = s/2) and the 8
    // bytes at d = 32 db + 16 (G%2) + 8 (s%2) of it, where G = lane / 16; the
    // 16 lanes of G then each receive one d (32 db + 16 (G%2) + lane % 16) for
    // the 8 keys.  Adding 16 rows leaves the swizzle unchanged.
    int voff[DB];
    {
        const int G = lane >> 4, s = lane & 15, t = s >> 1, par = s & 1;
        const int r = 8 * (t >> 2) + 4 * (G >> 1) + (t & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) voff[db] = T::at(r, 2 * db + (G & 1)) + 8 * par;
    }

    const float c = p.c;
    float m = -INFINITY;  // running max of s * c for query qi
    float l = 0.f;        // running sum of the rounded 2^8 p over this lane's keys
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

    const int qlast = min(m0 + BM, S) - 1;
    const int ntiles = CAUSAL ? qlast / BN + 1 : (S + BN - 1) / BN;
    Fp8Rows<D> tk, tv;
    tk.load(kb, 0, S, tid);
    tv.load(vb, 0, S, tid);
    for (int n = 0; n < ntiles; ++n) {
        const int n0 = n * BN;
        __syncthreads();  // previous tile consumed
        tk.store(Ks, tid);
        tv.store(Vs, tid);
        __syncthreads();
        if (n + 1 < ntiles) {
            tk.load(kb, n0 + BN, S, tid);
            tv.load(vb, n0 + BN, S, tid);
        }
        if (CAUSAL && n0 > qw + 31) continue;  // every key after every query of the wave
        f32x16 sacc[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            sacc[sb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a0 = *(const u32x4*)(Ks + sb * 32 * D + koff[ks][0]);
                const u32x4 a1 = *(const u32x4*)(Ks + sb * 32 * D + koff[ks][1]);
                const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                sacc[sb] = mfma_fp8(a, qreg[ks], sacc[sb]);
            }
        }
        // accumulator row r of block sb: key n0 + 32 sb + 8(r/4) + 4g + r%4
        float t = -INFINITY;
        const bool edge = (CAUSAL && n0 + BN - 1 > qw) || n0 + BN > S;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (edge) {
                    const int key = n0 + sb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if ((CAUSAL && key > qi) || key >= S) sacc[sb][r] = -INFINITY;
                }
                t = fmaxf(t, sacc[sb][r]);
            }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
        const float mn = fmaxf(m, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c);
        const float mref = mn == -INFINITY ? 0.f : mn;  // nothing visible yet: p = 0, nothing to rescale
        const float alpha = fast_exp2(m - mref);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        // p * 2^8 -> e4m3, packed in the accumulator's order (byte 16 sb + r)
        i32x8 pb;
        const float moff = mref - 8.0f;  // 2^(s c - m) * 2^8
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int sb = w >> 2, r = (w & 3) * 4;
            int x = 0;
            x = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(fmaf(sacc[sb][r], c, -moff)),
                                                fast_exp2(fmaf(sacc[sb][r + 1], c, -moff)), x, false);
            x = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(fmaf(sacc[sb][r + 2], c, -moff)),
                                                fast_exp2(fmaf(sacc[sb][r + 3], c, -moff)), x, true);
            pb[w] = x;
            l += (__builtin_amdgcn_cvt_f32_fp8(x, 0) + __builtin_amdgcn_cvt_f32_fp8(x, 1)) +
                 (__builtin_amdgcn_cvt_f32_fp8(x, 2) + __builtin_amdgcn_cvt_f32_fp8(x, 3));
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            i32x8 a;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(Vs + u * 16 * D + voff[db]));
                a[2 * u] = x[0];
                a[2 * u + 1] = x[1];
            }
            oacc[db] = mfma_fp8(a, pb, oacc[db]);
        }
    }

    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    const float ltot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    if (qi < S) {
        const float inv = p.vs / ltot;
        uint16_t* orow = p.out + (row0 + qi) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = db * 32 + j * 8 + g * 4;
                *(u32x2*)(orow + d0) = u32x2{pack_bf16x2(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv),
                                             pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv)};
            }
        }
        if (p.lse && g == 0) p.lse[row0 + qi] = (m + __log2f(ltot) - 8.0f) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const Fp8Params& prm, hipStream_t stream) {
    Fp8Params arg = prm;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&fwd_fp8_kernel<D, CAUSAL>, dim3(prm.total), dim3(NT), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream) {
    Fp8Params prm;
    prm.q = (const uint8_t*)a.q;
    prm.k = (const uint8_t*)a.k;
    prm.v = (const uint8_t*)a.v;
    prm.out = (uint16_t*)a.out;
    prm.lse = a.lse;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.S = a.S;
    prm.group = a.Hq / a.Hkv;
    prm.nq = (a.S + BM - 1) / BM;
    prm.total = (uint32_t)((int64_t)a.B * a.Hq * prm.nq);
    prm.c = a.scale * a.q_scale * a.k_scale * kLog2e;
    prm.vs = a.v_scale;
    if (a.D == 128) return a.causal ? launch<128, true>(prm, stream) : launch<128, false>(prm, stream);
    return a.causal ? launch<64, true>(prm, stream) : launch<64, false>(prm, stream);
}

}  // namespace attn
