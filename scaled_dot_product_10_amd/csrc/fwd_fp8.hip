// Fused attention forward with fp8 (OCP E4M3, "e4m3fn") operands on the
// gfx950 fp8 matrix cores: q, k, v are e4m3 codes with one float scale each
// (value = code * scale); the probabilities are rounded to e4m3 for the P.V
// product; scores, sums and the output accumulate in float32; out is bf16.
//
// The FP8 remark of the ai-manual.ru tutorial (section 6: on H100 SDPA runs
// in FP8 for about another 2x) is the idea; v_mfma_scale_f32_32x32x64_f8f6f4
// (unit block scales) does 32x32x64 per instruction, twice the bf16 rate.
//
// The schedule is the bf16 kernel's (fwd_bf16.hip): 8 waves, 256 queries per
// workgroup (32 per wave), 64-key tiles of K and V brought into LDS by
// global_load_lds_dwordx4 and double-buffered, and two wave groups one phase
// apart, so on every SIMD one wave runs the matrix products of a tile while
// its partner runs the softmax of the next:
//   M phase:  S(n+1)^T = K(n+1).Q^T (A = K rows from LDS, 32 bytes of d per
//             lane; B = Q in registers), O^T += V(n)^T.P(n)^T (A = V^T through
//             ds_read_b64_tr_b8; B = the 32 e4m3 weights a lane holds), and
//             one more product of an all-ones A with P(n)^T whose every row is
//             the tile's sum of the rounded weights (the row sum l, without a
//             vector-ALU decode of the e4m3 bytes).
//   V phase:  mask, then 2^(s c - mc + 7) rounded to e4m3, against a storage
//             reference mc (an integer, in scaled log2 units) that is only
//             raised, to floor(tile max), when some score exceeds it by more
//             than 1.75: every stored value stays below 2^8.75 < 448 (the
//             largest e4m3 value).  O and l accumulate against a second
//             integer reference ma <= mc; the P.V and l products take P with
//             the E8M0 block scale 2^(mc - ma) of the MFMA (one per lane, i.e.
//             per query and 32-key block), so raising mc costs no rescaling.
//             Only when mc - ma would pass 64 are O and l multiplied by
//             2^(ma - mc) and ma moved up (the first tile always does this).
// The k order of an fp8 product only has to agree between A and B within each
// half-wave; the transposed V reads give each lane the keys of the S^T
// accumulator rows (8(r/4) + 4g + r%4 of each 32-key block) in that order.
#include "common.h"
#include "launch.h"
#include "lds_dma.h"
#include "lds_tiles.h"

namespace attn {
namespace {

constexpr int BM = 256;  // queries per workgroup
constexpr int BN = 64;   // keys per tile
constexpr int NW = 8;    // waves (two per SIMD)
constexpr int NT = NW * 64;
constexpr float kBias = 7.0f;    // stored weight 2^(s c - mc + kBias)
constexpr float kRaise = 1.75f;  // s c - mc <= kRaise, so stored <= 2^8.75 < 448
constexpr int kMaxShift = 64;    // mc - ma <= 64 keeps O and l far inside float range

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
    uint32_t hgrp;  // causal: heads whose tiles one XCD runs together (0: plain order)
    float c;        // softmax scale * q_scale * k_scale * log2(e)
    float vs;       // v_scale
};

constexpr int kSlotsPerXcd = 32;  // 32 CUs per XCD, one workgroup per CU

// 32x32x64 e4m3 x e4m3 -> f32 (block scales 2^0)
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// the same with B scaled by the E8M0 exponent in byte 0 of sb (2^(sb - 127)):
// lane l's scale applies to column l % 32, k block l / 32 of B (checked on
// the hardware)
__device__ __forceinline__ f32x16 mfma_fp8_sb(const i32x8& a, const i32x8& b, const f32x16& c, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// LDS tile: BN rows x D bytes, 16-byte chunks; chunk c of row r at c ^ swz(r).
// 64 banks of 4 bytes span 256 bytes: two 128-byte rows (D = 128) or four
// 64-byte rows (D = 64).  Row reads (16 lanes on 16 rows, one chunk) need the
// rows that share a bank span to take distinct chunks.  A transposed byte read
// serves 32 lanes at once: 8 rows {0..3, 8..11} (or {4..7, 12..15}) x the two
// chunks 2j, 2j+1, so those rows that share a bank span must also take
// distinct chunk pairs, i.e. distinct swz >> 1.  At D = 128 with
// h = (r >> 1) & 7, swz = (h2, h0, h1) (a bit permutation of h) meets both.
template <int D>
struct Tile8 {
    static constexpr int CPR = D / 16;
    static constexpr int BYTES = BN * D;           // 8 KB (D=128) / 4 KB (D=64)
    static constexpr int CHUNKS = BYTES / 1024;    // DMA instructions per tile
    static_assert(CHUNKS >= 1 && CHUNKS <= NW, "one DMA instruction per wave at most");
    __device__ static int swz(int r) {
        if (D == 64) return (r >> 2) & 3;
        const int h = (r >> 1) & 7;
        return (h & 4) | ((h & 1) << 1) | ((h >> 1) & 1);
    }
    __device__ static int at(int r, int chunk) { return r * D + ((chunk ^ swz(r)) << 4); }
};

// DMA of one K or V tile: wave w (< CHUNKS) fills LDS positions
// p = 64 w + lane, i.e. row p / CPR at chunk position p % CPR, which holds
// chunk (p % CPR) ^ swz(row); rows past the sequence repeat row S-1 (their
// keys are masked).
template <int D>
struct DmaPlan8 {
    using T = Tile8<D>;
    uint32_t off;
    __device__ __forceinline__ void init(int wave, int lane) {
        const int pos = wave * 64 + lane;
        const int r = pos / T::CPR;
        off = (uint32_t)(r * D + (((pos % T::CPR) ^ T::swz(r)) << 4));
    }
    __device__ __forceinline__ void issue(const uint8_t* base, int n0, int S, uint8_t* tile, int wave) const {
        if (wave >= T::CHUNKS) return;
        const uint8_t* tb = base + (int64_t)n0 * D;
        const uint32_t l0 = lds_addr(tile) + (uint32_t)wave * 1024u;
        if (n0 + BN <= S) {
            dma16(tb, off, l0);
        } else {
            const int r = (int)(off / D);
            const int last = S - 1 - n0;
            dma16(tb, off - (uint32_t)((r - min(r, last)) * D), l0);
        }
    }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT) void fwd_fp8_kernel(Fp8Params p) {
    using T = Tile8<D>;
    constexpr int KS = D / 64;  // k-steps of the Q.K^T product
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    // K and V buffers; after the last barrier, the output staging area
    constexpr int SMEM = 4 * T::BYTES > NW * 32 * D * 2 ? 4 * T::BYTES : NW * 32 * D * 2;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
    auto Kbuf = [&](int i) __attribute__((always_inline)) { return smem + (i & 1) * T::BYTES; };
    auto Vbuf = [&](int i) __attribute__((always_inline)) { return smem + (2 + (i & 1)) * T::BYTES; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const uint32_t L = xcd_remap(blockIdx.x, p.total);
    int bh, tile;
    if (CAUSAL) {
        if (p.hgrp > 0 && blockIdx.x < p.total / 8u * 8u) {
            // groups of hgrp heads fill one XCD, longest tiles first (as in the bf16 kernel)
            const uint32_t per = p.total / 8u;
            const uint32_t loc = L % per;
            const uint32_t gsz = p.hgrp * (uint32_t)p.nq;
            const uint32_t r = loc % gsz;
            tile = p.nq - 1 - (int)(r / p.hgrp);
            bh = (int)((L - loc) / (uint32_t)p.nq + (loc / gsz) * p.hgrp + r % p.hgrp);
        } else {
            bh = (int)(L / (uint32_t)p.nq);
            tile = p.nq - 1 - (int)(L % (uint32_t)p.nq);
        }
    } else {
        bh = (int)(L / (uint32_t)p.nq);
        tile = (int)(L % (uint32_t)p.nq);
    }
    const int b = bh / p.Hq, h = bh % p.Hq, kvh = h / p.group;
    const int S = p.S;
    const int m0 = tile * BM;
    const int64_t row0 = (int64_t)bh * S;
    const uint8_t* kb = p.k + ((int64_t)b * p.Hkv + kvh) * S * D;
    const uint8_t* vb = p.v + ((int64_t)b * p.Hkv + kvh) * S * D;
    const int qwmin = m0 + wave * 32;
    const int qwmax = qwmin + 31;
    const int qi = qwmin + l32;
    const int qlast = min(m0 + BM, S) - 1;
    const int ntiles = (S + BN - 1) / BN;
    const int nend = CAUSAL ? min(ntiles, qlast / BN + 1) : ntiles;

    DmaPlan8<D> dma;
    dma.init(wave, lane);
    dma.issue(kb, 0, S, Kbuf(0), wave);
    dma.issue(vb, 0, S, Vbuf(0), wave);
    if (nend > 1) dma.issue(kb, BN, S, Kbuf(1), wave);

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
    // K row reads: row l32 (+32 for the second key block), chunks 4 ks + 2 g, + 1
    int koff[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        koff[ks][0] = T::at(l32, 4 * ks + 2 * g);
        koff[ks][1] = T::at(l32, 4 * ks + 2 * g + 1);
    }
    // transposed V read u (A bytes 8u..8u+7): source lane s = lane % 16 names
    // key row 16u + 8(t/4) + 4g + t%4 (t = s/2) and its 8 bytes at
    // d = 32 db + 16 (G%2) + 8 (s%2), G = lane / 16; each lane of G then holds
    // d = 32 db + lane % 32 for those 8 keys.  +16 rows keeps the swizzle.
    int voff[DB];
    {
        const int G = lane >> 4, s = lane & 15, t = s >> 1, par = s & 1;
        const int r = 8 * (t >> 2) + 4 * (G >> 1) + (t & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) voff[db] = T::at(r, 2 * db + (G & 1)) + 8 * par;
    }
    i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                  0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0
    // opaque from here on: kept in registers, not rebuilt before every l product
    asm volatile("" : "+v"(ones));

    const float c = p.c;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    f32x16 lacc = f32x16{};  // every row: running sum of the weights (against ma)
    // references of query qi in scaled log2 units (integers once the first
    // tile has set them; a finite start so that no exponent argument is
    // inf - inf): ma for O and l, mc = ma + kx for the stored weights
    float ma = -1e30f, mc = -1e30f;
    int sbv = 127;  // E8M0 scale 2^kx of the stored weights in the P products
    f32x16 sacc[2];
    i32x8 pb = {};  // each V phase overwrites every byte

    // S^T = K.Q^T for the tile in Kt
    auto qk = [&](const uint8_t* Kt) __attribute__((always_inline)) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            sacc[sb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a0 = *(const u32x4*)(Kt + sb * 32 * D + koff[ks][0]);
                const u32x4 a1 = *(const u32x4*)(Kt + sb * 32 * D + koff[ks][1]);
                const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                sacc[sb] = mfma_fp8(a, qreg[ks], sacc[sb]);
            }
        }
    };

    // 2^(s c - mc + kBias) -> e4m3, byte 16 sb + r of the B operand
    auto exp_pack = [&](float mref) __attribute__((always_inline)) {
        const float moff = mref - kBias;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int sb = w >> 2, r = (w & 3) * 4;
            int x = pb[w];  // both halves are overwritten; no zeroing
            x = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(fmaf(sacc[sb][r], c, -moff)),
                                                fast_exp2(fmaf(sacc[sb][r + 1], c, -moff)), x, false);
            x = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(fmaf(sacc[sb][r + 2], c, -moff)),
                                                fast_exp2(fmaf(sacc[sb][r + 3], c, -moff)), x, true);
            pb[w] = x;
        }
    };

    // softmax of tile n0 (from sacc)
    auto softmax = [&](int n0) __attribute__((always_inline)) {
        if ((CAUSAL && n0 + BN - 1 > qwmin) || n0 + BN > S) {
            // register r of key block sb holds key n0 + 4g + kofs, kofs =
            // 32 sb + 8 (r / 4) + r % 4: masked when kofs passes hi, the
            // offset of this lane's last visible key (its query, or S - 1)
            const int hi = (CAUSAL ? min(qi, S - 1) : S - 1) - (n0 + g * 4);
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (sb * 32 + (r >> 2) * 8 + (r & 3) > hi) sacc[sb][r] = -INFINITY;
        }
        // lane max of the 32 scores: a chain of three-way maxima
        float tmax;
        {
            float u[11];
#pragma unroll
            for (int i = 0; i < 10; ++i) {
                const float a0 = i < 5 ? sacc[0][3 * i] : sacc[1][3 * (i - 5)];
                const float a1 = i < 5 ? sacc[0][3 * i + 1] : sacc[1][3 * (i - 5) + 1];
                const float a2 = i < 5 ? sacc[0][3 * i + 2] : sacc[1][3 * (i - 5) + 2];
                u[i] = fmaxf(fmaxf(a0, a1), a2);
            }
            u[10] = fmaxf(sacc[0][15], sacc[1][15]);
            const float v0 = fmaxf(fmaxf(u[0], u[1]), u[2]), v1 = fmaxf(fmaxf(u[3], u[4]), u[5]);
            const float v2 = fmaxf(fmaxf(u[6], u[7]), u[8]), v3 = fmaxf(u[9], u[10]);
            tmax = fmaxf(fmaxf(v0, v1), fmaxf(v2, v3));
        }
        if (__builtin_amdgcn_ballot_w64(tmax * c > mc + kRaise)) {
            // raise mc to floor of the row's tile max (both half-waves of a
            // query take the same value, so they keep one reference)
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
            const float mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
            mc = mt > mc + kRaise ? floorf(mt) : mc;
            sbv = 127 + (int)fminf(mc - ma, (float)(kMaxShift + 1));
        }
        if (__builtin_amdgcn_ballot_w64(mc - ma > (float)kMaxShift)) {
            // move ma up to mc: O and l by an exact power of two (0 on the
            // first tile)
            const float alpha = ldexpf(1.0f, (int)fmaxf(ma - mc, -256.0f));
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            lacc *= alpha;
            ma = mc;
            sbv = 127;
        }
        exp_pack(mc);
    };

    auto active = [&](int n) __attribute__((always_inline)) { return !CAUSAL || n * BN <= qwmax; };

    phase_barrier(true);

    // M(n): S(n+1) = K(n+1).Q^T, O += P(n).V(n), l += P(n).1; operands read
    // AHEAD products in advance.  For the last tile the S(n+1) product reads
    // the (stale, in-bounds) other K buffer and its result is never used.
    auto mphase = [&](int n) __attribute__((always_inline)) {
        if (!active(n)) return;
        constexpr int NQK = 2 * KS, NP = NQK + DB, AHEAD = 3;
        const uint8_t* Kt = Kbuf(n + 1);
        const uint8_t* Vt = Vbuf(n);
        auto rd = [&](int i) __attribute__((always_inline)) {
            i32x8 a;
            if (i < NQK) {
                const int sb = i / KS, ks = i % KS;
                const u32x4 a0 = *(const u32x4*)(Kt + sb * 32 * D + koff[ks][0]);
                const u32x4 a1 = *(const u32x4*)(Kt + sb * 32 * D + koff[ks][1]);
                a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            } else {
                const int db = i - NQK;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(Vt + u * 16 * D + voff[db]));
                    a[2 * u] = x[0];
                    a[2 * u + 1] = x[1];
                }
            }
            return a;
        };
        __builtin_amdgcn_s_setprio(1);
        sacc[0] = f32x16{};  // the V phase has consumed S(n)
        sacc[1] = f32x16{};
        i32x8 buf[AHEAD];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) buf[i] = rd(i);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const i32x8 a = buf[i % AHEAD];
            if (i + AHEAD < NP) buf[i % AHEAD] = rd(i + AHEAD);
            if (i < NQK) {
                sacc[i / KS] = mfma_fp8(a, qreg[i % KS], sacc[i / KS]);
            } else {
                oacc[i - NQK] = mfma_fp8_sb(a, pb, oacc[i - NQK], sbv);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        lacc = mfma_fp8_sb(ones, pb, lacc, sbv);
        __builtin_amdgcn_s_setprio(0);
    };
    auto vphase = [&](int n) __attribute__((always_inline)) {
        if (active(n)) softmax(n * BN);
    };
    auto dma_step = [&](int k) __attribute__((always_inline)) {
        if (k + 1 < nend) dma.issue(kb, (k + 1) * BN, S, Kbuf(k + 1), wave);
        if (k < nend) dma.issue(vb, k * BN, S, Vbuf(k), wave);
    };

    // phase schedule of the bf16 kernel: group 0 one phase ahead of group 1
    if (grp == 0) {
        qk(Kbuf(0));
        phase_barrier(false);
        for (int n = 0; n < nend; ++n) {
            vphase(n);
            phase_barrier(true);
            dma_step(n + 1);
            mphase(n);
            phase_barrier(false);
        }
        phase_barrier(true);
    } else {
        phase_barrier(false);
        qk(Kbuf(0));
        phase_barrier(true);
        for (int n = 0; n < nend; ++n) {
            dma_step(n + 1);
            vphase(n);
            phase_barrier(false);
            mphase(n);
            phase_barrier(true);
        }
    }

    // O through this wave's share of the (now idle) LDS, so that the stores
    // cover whole rows of the wave's 32 contiguous output rows (as in the
    // bf16 kernel)
    const float l = lacc[0];
    const float inv = p.vs / l;
    store_rows_via_lds<D>((char*)smem + wave * 32 * D * 2, oacc, inv, p.out + (row0 + qwmin) * D, S - qwmin, lane);
    if (qi < S && p.lse && g == 0) p.lse[row0 + qi] = (ma + __log2f(l) - kBias) * kLn2;
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
    prm.hgrp = 0;
    const uint32_t per = prm.total / 8u;
    if (a.causal && per > 0 && per % (uint32_t)prm.nq == 0) {
        const uint32_t heads_here = per / (uint32_t)prm.nq;
        uint32_t g = (uint32_t)(kSlotsPerXcd / prm.nq > 1 ? kSlotsPerXcd / prm.nq : 1);
        if (g > heads_here) g = heads_here;
        while (heads_here % g) --g;
        prm.hgrp = g;
    }
    if (a.D == 128) return a.causal ? launch<128, true>(prm, stream) : launch<128, false>(prm, stream);
    return a.causal ? launch<64, true>(prm, stream) : launch<64, false>(prm, stream);
}

}  // namespace attn
