// Fused causal attention forward, bfloat16 in/out, float32 accumulation.
//
// Computes out = softmax(scale * q k^T + mask) v one query tile at a time,
// streaming key/value tiles through LDS and keeping the softmax online (a
// running row max m and row sum l, with the output rescaled whenever m
// grows), so the S x S score matrix never leaves the chip.  This is the
// tiling-plus-online-softmax idea described in the Flash backend section of
// the Hugging Face "Profiling in PyTorch (Part 3)" article; the structure of
// a resident query block, a loop over key/value blocks and a float32
// accumulator follows the fused kernel sketch in section 4 of the
// ai-manual.ru tutorial, with the online softmax and causal masking that the
// sketch leaves out.
//
// Work decomposition (gfx950, wave64):
//   workgroup = 4 waves = 128 queries of one (batch, head); wave w owns 32.
//   Each loop step handles BN = 64 keys:
//     S^T = K . Q^T    on v_mfma_f32_32x32x16_bf16.  A = K rows from LDS,
//                      B = the wave's Q rows, held in VGPRs for the whole
//                      loop.  In the 32x32 result lane l holds one query
//                      (l % 32) and 16 keys, so row max / row sum are
//                      in-lane plus one exchange with lane l ^ 32.
//     online softmax   p = 2^(s*c - m*c) with c = scale*log2(e).
//     O^T += V^T . P^T on the same MFMA.  B = P^T straight from the S^T
//                      accumulator (converted to bf16), A = V^T from the
//                      transposed LDS tile, stored in the key order the
//                      accumulator produces.  O^T keeps one query per lane,
//                      so the rescale by exp2(m_old - m_new) is per-lane.
//   Causal: key tiles past the workgroup's last query are never loaded, a
//   wave skips the MFMAs of tiles past its own last query, and only tiles
//   that straddle the diagonal (or the end of the sequence) apply the mask.
//   Causal workgroups start with the longest (last) query tiles.
#include "common.h"
#include "kv_tile.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BM = 128;   // queries per workgroup
constexpr int BN = 64;    // keys per loop step
constexpr int NT = 256;   // threads per workgroup

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    float* lse;
    int Hq, Hkv, S, group, nq;
    uint32_t total;
    float c;  // scale * log2(e), > 0
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void fwd_bf16_kernel(Params p) {
    constexpr int KS = D / 16;  // k-steps of the Q.K^T product
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    using KT = KTile<D, BN, NT>;
    using VT = VTile<D, BN, NT, true>;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KT::KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VT::VPAD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const uint32_t L = xcd_remap(blockIdx.x, p.total);
    const int bh = (int)(L / (uint32_t)p.nq);
    int tile = (int)(L % (uint32_t)p.nq);
    if (CAUSAL) tile = p.nq - 1 - tile;  // longest tiles first
    const int b = bh / p.Hq;
    const int h = bh % p.Hq;
    const int kvh = h / p.group;
    const int S = p.S;
    const int m0 = tile * BM;

    const int64_t row0 = (int64_t)bh * S;  // first row of this (b, h) in [B*Hq*S]
    const uint16_t* qb = p.q + row0 * D;
    const int64_t kvrow0 = ((int64_t)b * p.Hkv + kvh) * S;
    const uint16_t* kb = p.k + kvrow0 * D;
    const uint16_t* vb = p.v + kvrow0 * D;

    const int qwmin = m0 + wave * 32;
    const int qwmax = qwmin + 31;
    const int qi = qwmin + l32;  // this lane's query

    // Q operand (B of S^T = K.Q^T): query qi, d = 16*ks + 8*g .. +7.
    bf16x8 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0, 0, 0, 0};
        if (qi < S) x = *(const u32x4*)(qb + (int64_t)qi * D + ks * 16 + g * 8);
        qreg[ks] = as_bf16x8(x);
    }

    const int qlast = min(m0 + BM, S) - 1;
    const int ntiles = (S + BN - 1) / BN;
    const int nend = CAUSAL ? min(ntiles, qlast / BN + 1) : ntiles;
    const float c = p.c;

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float mrow = -INFINITY;  // running max of raw scores q.k for query qi
    float lrow = 0.f;        // running sum of p over this lane's keys

    KT kt;
    VT vt;
    kt.load(kb, 0, S, tid);
    vt.load(vb, 0, S, tid);
    kt.store(Ks, tid);
    vt.store(Vt, tid);
    __syncthreads();

    for (int n = 0; n < nend; ++n) {
        const int n0 = n * BN;
        const bool has_next = n + 1 < nend;
        if (has_next) {
            kt.load(kb, n0 + BN, S, tid);
            vt.load(vb, n0 + BN, S, tid);
        }
        if (!CAUSAL || n0 <= qwmax) {
            // ---- S^T = K . Q^T : two 32-key blocks ------------------------
            f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const bf16x8 a = *(const bf16x8*)(Ks + (sb * 32 + l32) * KT::KPAD + ks * 16 + g * 8);
                    sacc[sb] = mfma32x32x16(a, qreg[ks], sacc[sb]);
                }
            }
            // ---- mask: keys after the query, keys past the end -------------
            if ((CAUSAL && n0 + BN - 1 > qwmin) || n0 + BN > S) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = n0 + sb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                        if ((CAUSAL && key > qi) || key >= S) sacc[sb][r] = -INFINITY;
                    }
                }
            }
            // ---- online softmax --------------------------------------------
            float mt = sacc[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sacc[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[1][r]);
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float mnew = fmaxf(mrow, mt);  // finite: key 0 is in the first tile
            const float mc = mnew * c;
            const float alpha = fast_exp2(fmaf(mrow, c, -mc));
            float psum = 0.f;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = fast_exp2(fmaf(sacc[sb][r], c, -mc));
                    sacc[sb][r] = pr;
                    psum += pr;
                }
            }
            lrow = fmaf(lrow, alpha, psum);
            mrow = mnew;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

            // ---- O^T += V^T . P^T -----------------------------------------
            // 16-key block kb = 2*sb + hh uses accumulator registers 8*hh..8*hh+7.
            bf16x8 pb[4];
#pragma unroll
            for (int kb16 = 0; kb16 < 4; ++kb16) {
                const int sb = kb16 >> 1, hh = kb16 & 1;
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf16x2(sacc[sb][hh * 8 + 2 * e], sacc[sb][hh * 8 + 2 * e + 1]);
                pb[kb16] = as_bf16x8(w);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int kb16 = 0; kb16 < 4; ++kb16) {
                    const bf16x8 a = *(const bf16x8*)(Vt + (db * 32 + l32) * VT::VPAD + kb16 * 16 + g * 8);
                    oacc[db] = mfma32x32x16(a, pb[kb16], oacc[db]);
                }
            }
        }
        __syncthreads();  // every wave is done with this tile's LDS
        if (has_next) {
            kt.store(Ks, tid);
            vt.store(Vt, tid);
            __syncthreads();
        }
    }

    // ---- epilogue: O / l, lse ------------------------------------------------
    const float ltot = lrow + __shfl_xor(lrow, 32);
    if (qi < S) {
        const float inv = 1.0f / ltot;
        uint16_t* orow = p.out + (row0 + qi) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = db * 32 + j * 8 + g * 4;
                const u32x2 w = {pack_bf16x2(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv),
                                 pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv)};
                *(u32x2*)(orow + d0) = w;
            }
        }
        if (p.lse && g == 0) p.lse[row0 + qi] = (mrow * c + __log2f(ltot)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const Params& prm, hipStream_t stream) {
    Params arg = prm;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&fwd_bf16_kernel<D, CAUSAL>, dim3(prm.total), dim3(NT), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
    Params prm;
    prm.q = (const uint16_t*)a.q;
    prm.k = (const uint16_t*)a.k;
    prm.v = (const uint16_t*)a.v;
    prm.out = (uint16_t*)a.out;
    prm.lse = a.lse;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.S = a.S;
    prm.group = a.Hq / a.Hkv;
    prm.nq = (a.S + BM - 1) / BM;
    prm.total = (uint32_t)((int64_t)a.B * a.Hq * prm.nq);
    prm.c = a.scale * kLog2e;
    if (a.D == 128) return a.causal ? launch<128, true>(prm, stream) : launch<128, false>(prm, stream);
    return a.causal ? launch<64, true>(prm, stream) : launch<64, false>(prm, stream);
}

}  // namespace attn
