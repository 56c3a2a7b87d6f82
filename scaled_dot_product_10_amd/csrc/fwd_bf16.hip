// Fused causal attention forward, bfloat16 in/out, float32 accumulation.
//
// Computes out = softmax(scale * q k^T + mask) v one query tile at a time,
// streaming key/value tiles through LDS and keeping the softmax online (a
// running row max m and row sum l), so the S x S score matrix never leaves
// the chip.  This is the tiling-plus-online-softmax idea described in the
// Flash backend section of the Hugging Face "Profiling in PyTorch (Part 3)"
// article; the structure of a resident query block, a loop over key/value
// blocks and a float32 accumulator follows the fused kernel sketch in
// section 4 of the ai-manual.ru tutorial, with the online softmax and causal
// masking that the sketch leaves out.
//
// Work decomposition (gfx950, wave64, two workgroups per CU):
//   workgroup = 4 waves = 128 queries of one (batch, head); wave w owns 32.
//   Each loop step handles BN = 64 keys:
//     S^T = K . Q^T    v_mfma_f32_32x32x16_bf16.  A = K rows read from LDS,
//                      B = the wave's Q rows, held in VGPRs for the whole
//                      loop.  In the 32x32 result lane l holds one query
//                      (l % 32) and 16 keys, so row max / row sum are
//                      in-lane plus one exchange with lane l ^ 32.
//     online softmax   p = 2^(s*c - m*c), c = scale*log2(e).  m is only moved
//                      when a row max exceeds it by more than 2^8 in p units
//                      (p stays <= 256, far from float32 overflow), so the
//                      rescale of O by 2^((m_old - m_new) c) is rare.
//     O^T += V^T . P^T same MFMA.  B = P^T straight from the S^T accumulator
//                      (converted to bf16).  A = V^T comes from the row-major
//                      V tile through ds_read_b64_tr_b16, which hands each
//                      lane 4 keys of one d; the keys it picks match the
//                      order of the S^T accumulator rows.
//   Memory pipeline: K and V tiles go HBM -> LDS with global_load_lds_dwordx4
//   (no register staging), double-buffered; K(n+2) and V(n+1) are in flight
//   while tile n is computed, and one barrier per step publishes them.  The
//   product S(n+1) = K(n+1).Q^T is issued before the softmax of tile n, so the
//   matrix cores have independent work while the vector ALUs run the softmax.
//   LDS rows are XOR-swizzled in 16-byte chunks so every operand read is
//   free of bank conflicts.
//   Causal: key tiles past the workgroup's last query are never loaded, a
//   wave skips the products of tiles past its own last query, and only tiles
//   that straddle the diagonal (or the end of the sequence) apply the mask.
//   Causal workgroups start with the longest query tiles.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BM = 128;   // queries per workgroup
constexpr int BN = 64;    // keys per loop step
constexpr int NT = 256;   // threads per workgroup
constexpr float kRescaleLog2 = 8.0f;  // move m only when p would exceed 2^8

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    float* lse;
    int Hq, Hkv, S, group, nq;
    uint32_t total;
    float c;    // scale * log2(e), > 0
    float thr;  // kRescaleLog2 / c: rescale threshold in raw score units
};

// LDS tile layout: BN rows x D bf16, 16-byte chunks.  Chunk c of row r sits
// at chunk position r*CPR + (c ^ swizzle(r)).
template <int D>
struct Tile {
    static constexpr int CPR = D / 8;                 // chunks per row
    static constexpr int BYTES = BN * D * 2;          // 16 KB (D=128) / 8 KB (D=64)
    static constexpr int DMA_PER_WAVE = BYTES / 1024 / 4;
    // K: the 16 rows one operand read touches per 16-lane phase land on 16
    // different bank groups (rows of 128 bytes alternate bank halves).
    __device__ static int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    // V: the 4 rows one transposed read touches per 16-lane phase land on 4
    // different 64-byte bank groups.
    __device__ static int vswz(int r) { return 4 * (D == 128 ? (r & 3) : ((r >> 1) & 1)); }
};

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One global_load_lds_dwordx4: 64 lanes x 16 bytes from global memory into 1 KB
// of LDS at lds (wave-uniform), lane L filling bytes [16L, 16L+16).  Issued as
// inline assembly so the compiler does not treat every later LDS read as
// dependent on it; completion is awaited explicitly (s_waitcnt vmcnt(0)) before
// the barrier that publishes the tile.  M0 is a reserved register that the
// compiler loads right before each of its own uses, so setting it here is safe.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}

// Issue this wave's share of the DMA of one K or V tile (rows n0..n0+BN-1).
// Each global_load_lds_dwordx4 fills 1 KB of LDS, lane L writing bytes
// [16L, 16L+16) of it; the lane fetches whichever global chunk belongs at
// that swizzled position.  Rows past the end of the sequence repeat row S-1
// (those keys are masked, and their P is 0).
template <int D, bool IS_V>
__device__ __forceinline__ void dma_tile(const uint16_t* base, int n0, int S, char* tile, int wave, int lane) {
    using T = Tile<D>;
#pragma unroll
    for (int i = 0; i < T::DMA_PER_WAVE; ++i) {
        const int inst = wave * T::DMA_PER_WAVE + i;
        const int p = inst * 64 + lane;
        const int r = p / T::CPR;
        const int c = (p % T::CPR) ^ (IS_V ? T::vswz(r) : T::kswz(r));
        const int key = min(n0 + r, S - 1);
        dma16(base + (int64_t)key * D + c * 8, lds_addr(tile) + inst * 1024);
    }
}

__device__ __forceinline__ void wait_dma_and_barrier() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

__device__ __forceinline__ bf16x8 tr_read_pair(const char* p0, const char* p1) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
    const short __attribute__((ext_vector_type(8))) x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, x);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void fwd_bf16_kernel(Params p) {
    using T = Tile<D>;
    constexpr int KS = D / 16;  // k-steps of the Q.K^T product
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    constexpr int ROWB = T::CPR * 16;  // bytes per tile row
    __shared__ __attribute__((aligned(1024))) char smem[4 * T::BYTES];
    char* Kb[2] = {smem, smem + T::BYTES};
    char* Vb[2] = {smem + 2 * T::BYTES, smem + 3 * T::BYTES};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const uint32_t L = xcd_remap(blockIdx.x, p.total);
    int bh, tile;
    if (CAUSAL) {
        // tile-major within each XCD's range: the longest tiles of every head first
        const uint32_t per = p.total / 8u;
        const uint32_t heads_here = per / (uint32_t)p.nq;
        if (blockIdx.x < per * 8u && heads_here > 0 && per % (uint32_t)p.nq == 0) {
            const uint32_t base = L - L % per;
            const uint32_t loc = L % per;
            tile = p.nq - 1 - (int)(loc / heads_here);
            bh = (int)(base / (uint32_t)p.nq + loc % heads_here);
        } else {
            bh = (int)(L / (uint32_t)p.nq);
            tile = p.nq - 1 - (int)(L % (uint32_t)p.nq);
        }
    } else {
        bh = (int)(L / (uint32_t)p.nq);
        tile = (int)(L % (uint32_t)p.nq);
    }
    const int b = bh / p.Hq;
    const int h = bh % p.Hq;
    const int kvh = h / p.group;
    const int S = p.S;
    const int m0 = tile * BM;

    const int64_t row0 = (int64_t)bh * S;
    const uint16_t* qb = p.q + row0 * D;
    const int64_t kvrow0 = ((int64_t)b * p.Hkv + kvh) * S;
    const uint16_t* kb = p.k + kvrow0 * D;
    const uint16_t* vb = p.v + kvrow0 * D;

    const int qwmin = m0 + wave * 32;
    const int qwmax = qwmin + 31;
    const int qi = qwmin + l32;

    const int qlast = min(m0 + BM, S) - 1;
    const int ntiles = (S + BN - 1) / BN;
    const int nend = CAUSAL ? min(ntiles, qlast / BN + 1) : ntiles;

    // ---- prologue: K(0), V(0), K(1) in flight while Q is loaded -------------
    dma_tile<D, false>(kb, 0, S, Kb[0], wave, lane);
    dma_tile<D, true>(vb, 0, S, Vb[0], wave, lane);
    if (nend > 1) dma_tile<D, false>(kb, BN, S, Kb[1], wave, lane);

    // Q operand (B of S^T = K.Q^T): query qi, d = 16*ks + 8*g .. +7.
    bf16x8 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0, 0, 0, 0};
        if (qi < S) x = *(const u32x4*)(qb + (int64_t)qi * D + ks * 16 + g * 8);
        qreg[ks] = as_bf16x8(x);
    }

    // per-lane LDS byte offsets of the operand reads
    int koff[KS];  // K row l32 (+32 for the second key block), chunk 2ks+g
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = l32 * ROWB + (((2 * ks + g) ^ T::kswz(l32)) * 16);
    int voff[DB];  // transposed V read: lane j of 16-lane group G fetches row 4*(G/2) + j/4,
                   // d = 32*db + 16*(G%2) + 4*(j%4) .. +3
    {
        const int G = lane >> 4, j = lane & 15;
        const int r = 4 * (G >> 1) + (j >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d0 = db * 32 + (G & 1) * 16 + 4 * (j & 3);
            voff[db] = r * ROWB + (((d0 >> 3) ^ T::vswz(r)) * 16) + (d0 & 7) * 2;
        }
    }

    const float c = p.c;
    const float thr = p.thr;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float mrow = -INFINITY;  // running reference max of raw scores for query qi
    float lrow = 0.f;        // running sum of p over this lane's keys

    auto qk = [&](f32x16(&s)[2], const char* Kt) {
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const bf16x8 a = *(const bf16x8*)(Kt + koff[ks] + sb * 32 * ROWB);
                s[sb] = mfma32x32x16(a, qreg[ks], s[sb]);
            }
        }
    };

    // Mask tile n's scores (diagonal / tail tiles only), take the row max and
    // move the reference max m when the new max exceeds it by more than the
    // threshold (then O and l are rescaled by 2^((m_old - m_new) c)).
    auto rowmax = [&](f32x16(&s)[2], int n0, auto need_mask) {
        if (need_mask) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = n0 + sb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                    if ((CAUSAL && key > qi) || key >= S) s[sb][r] = -INFINITY;
                }
            }
        }
        float mt = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[1][r]);
        return fmaxf(mt, __shfl_xor(mt, 32));
    };
    auto update_max = [&](float mt) {
        const bool upd = mt > mrow + thr;
        if (__builtin_amdgcn_ballot_w64(upd)) {
            const float mnew = upd ? mt : mrow;
            const float alpha = fast_exp2((mrow - mnew) * c);
            lrow *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            mrow = mnew;
        }
    };

    // p = 2^(s c - m c) -> bf16 P^T operand; 16-key block kb16 = accumulator
    // registers 8*(kb16&1).. of key block kb16>>1.
    auto exp_pack = [&](f32x16(&s)[2], bf16x8(&pb)[4]) {
        const float mc = mrow * c;
        float psum = 0.f;
#pragma unroll
        for (int kb16 = 0; kb16 < 4; ++kb16) {
            const int sb = kb16 >> 1, hh = kb16 & 1;
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(fmaf(s[sb][hh * 8 + 2 * e], c, -mc));
                const float p1 = fast_exp2(fmaf(s[sb][hh * 8 + 2 * e + 1], c, -mc));
                psum += p0 + p1;
                w[e] = pack_bf16x2(p0, p1);
            }
            pb[kb16] = as_bf16x8(w);
        }
        lrow += psum;
    };

    // O^T += V^T . P^T ; 16-key block kb16 uses rows 16*kb16 .. +15 of the tile
    auto pv = [&](const bf16x8(&pb)[4], const char* Vt) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int kb16 = 0; kb16 < 4; ++kb16) {
                const char* base = Vt + voff[db] + kb16 * 16 * ROWB;
                const bf16x8 a = tr_read_pair(base, base + 8 * ROWB);
                oacc[db] = mfma32x32x16(a, pb[kb16], oacc[db]);
            }
        }
    };

    // Tiles whose every key is visible to every query of the workgroup and
    // that lie fully inside the sequence: [0, nfull).
    const int nfull = min(CAUSAL ? (m0 + 1) / BN : S / BN, S / BN);
    // Step n is "fast" when tile n+1 is such a tile: then exp(n), S(n+1), PV(n)
    // and max(n+1) form one branch-free block the scheduler can interleave.
    const int nfast = max(0, min(nfull, nend) - 1);

    // One step: on entry S(n) is in scur (masked, its max folded into m) and
    // tiles n (K, V) and n+1 (K) are in LDS.
    auto step = [&](int n, f32x16(&scur)[2], f32x16(&snext)[2], auto fast) {
        const int n0 = n * BN;
        if (n + 2 < nend) dma_tile<D, false>(kb, n0 + 2 * BN, S, Kb[n & 1], wave, lane);
        if (n + 1 < nend) dma_tile<D, true>(vb, n0 + BN, S, Vb[(n + 1) & 1], wave, lane);
        bf16x8 pb[4];
        if (fast) {
            exp_pack(scur, pb);
            qk(snext, Kb[(n + 1) & 1]);
            pv(pb, Vb[n & 1]);
            update_max(rowmax(snext, n0 + BN, std::false_type{}));
        } else {
            const bool cur = !CAUSAL || n0 <= qwmax;
            const bool nxt = n + 1 < nend && (!CAUSAL || n0 + BN <= qwmax);
            if (cur) exp_pack(scur, pb);
            if (nxt) qk(snext, Kb[(n + 1) & 1]);
            if (cur) pv(pb, Vb[n & 1]);
            if (nxt) update_max(rowmax(snext, n0 + BN, std::true_type{}));
        }
        wait_dma_and_barrier();
    };

    wait_dma_and_barrier();
    f32x16 s0[2], s1[2];
    qk(s0, Kb[0]);
    update_max(rowmax(s0, 0, std::true_type{}));
    // fast steps in pairs (keeps s0 as the current buffer at every even n),
    // then the remaining steps on the general path
    int n = 0;
    for (; n + 1 < nfast; n += 2) {
        step(n, s0, s1, std::true_type{});
        step(n + 1, s1, s0, std::true_type{});
    }
    for (; n < nend; n += 2) {
        step(n, s0, s1, std::false_type{});
        if (n + 1 < nend) step(n + 1, s1, s0, std::false_type{});
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
    prm.thr = kRescaleLog2 / prm.c;
    if (a.D == 128) return a.causal ? launch<128, true>(prm, stream) : launch<128, false>(prm, stream);
    return a.causal ? launch<64, true>(prm, stream) : launch<64, false>(prm, stream);
}

}  // namespace attn
