// Fused causal attention forward, float32 throughout.
//
// Same method as the bfloat16 kernel (key/value tiles through LDS, online
// softmax, nothing of size S x S in device memory) on plain float32 vector
// ALU arithmetic.  This is the path for float32 inputs, where the bfloat16
// matrix cores do not apply; it is a correctness path, sized for short
// sequences, where the time is latency rather than arithmetic.
//
// Layout: a workgroup of eight waves owns QW queries (16 at D = 64, 8 at
// D = 128).  Each query takes DS = D / 16 adjacent lanes, each holding 16 of
// its d's of q and of the output accumulator; a dot product is the lane's
// 16-term partial sum plus DPP adds over the query's lanes (quad swaps, then
// a half-row mirror at D = 128).  The eight waves (two per SIMD) split the
// key range: wave w takes the 16-key steps n = w, w + 8, ..., each through
// its own K/V buffers in LDS (a lane reads its 16 d's of a key as four
// 16-byte reads), with the next step's tile loaded into registers while the
// current one is used, so the loop has no workgroup barrier.  At the end
// waves 1-7 hand (m, l, o) to wave 0 through LDS (over the K/V buffers),
// which merges the eight partial softmaxes.  Small query groups spread short
// sequences over many compute units: a 128-query head takes 8 workgroups.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int NWF = 8;   // waves per workgroup (split of the key range)
constexpr int BNF = 16;  // keys per step
constexpr int DLF = 16;  // d's per lane

struct Params {
    const float* q;
    const float* k;
    const float* v;
    float* out;
    float* lse;
    int Hq, Hkv, S, group, nq;
    float c;  // scale * log2(e), > 0
};

template <int D>
struct F32Shape {
    static constexpr int DS = D / DLF;       // lanes per query
    static constexpr int QW = 64 / DS;       // queries per workgroup
    static constexpr int TF = BNF * D;       // floats of one K or V step tile
    static constexpr int LPT = TF / 64 / 4;  // 16-byte loads per lane per tile
};

// sum over the DS adjacent lanes of one query (DPP within rows of 16 lanes)
template <int DS>
__device__ __forceinline__ float query_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
    if (DS == 8)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // half-row mirror
    return x;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * NWF) void fwd_f32_kernel(Params p) {
    using F = F32Shape<D>;
    constexpr int DS = F::DS, QW = F::QW, DL = DLF, TF = F::TF, LPT = F::LPT;
    static_assert(DS == 4 || DS == 8, "4 or 8 lanes per query");
    // per wave: K, V of its step; after the loop: o, m, l of waves 1..NWF-1
    constexpr int KVF = NWF * 2 * TF, REDF = (NWF - 1) * (DL + 2) * 64;
    __shared__ __attribute__((aligned(16))) float lds[KVF > REDF ? KVF : REDF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    auto red = [&](int w, int i) __attribute__((always_inline)) -> float& { return lds[(w * (DL + 2) + i) * 64 + lane]; };
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x / p.nq;
    int tile = blockIdx.x % p.nq;
    if (CAUSAL) tile = p.nq - 1 - tile;
    const int b = bh / p.Hq;
    const int h = bh % p.Hq;
    const int kvh = h / p.group;
    const int S = p.S;
    const int m0 = tile * QW;
    const int qi = m0 + lane / DS;      // this lane's query
    const int d0 = (lane % DS) * DL;    // its first d
    const int64_t row0 = (int64_t)bh * S;
    const int64_t kvrow0 = ((int64_t)b * p.Hkv + kvh) * S;

    // q: rows past the end repeat row S - 1 (their results are never stored)
    float q[DL];
    {
        const float* qp = p.q + (row0 + min(qi, S - 1)) * D + d0;
#pragma unroll
        for (int d = 0; d < DL; d += 4) {
            const f32x4 x = *(const f32x4*)(qp + d);
            q[d] = x[0];
            q[d + 1] = x[1];
            q[d + 2] = x[2];
            q[d + 3] = x[3];
        }
    }
    float o[DL];
#pragma unroll
    for (int d = 0; d < DL; ++d) o[d] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float c = p.c;

    const int qlast = min(m0 + QW, S) - 1;
    const int ntiles = (S + BNF - 1) / BNF;
    const int nend = CAUSAL ? min(ntiles, qlast / BNF + 1) : ntiles;

    // Step tile n of K and V into registers: lane t's 16-byte load i covers
    // floats (i * 64 + t) * 4 .. +3 of the tile (rows past S read as zero)
    f32x4 kr[LPT], vr[LPT];
    auto load = [&](int n) __attribute__((always_inline)) {
        const int n0 = n * BNF;
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int f = (i * 64 + lane) * 4;
            const int r = f / D;
            const bool ok = n0 + r < S;
            const int64_t off = (kvrow0 + n0 + (ok ? r : 0)) * D + f % D;
            kr[i] = ok ? *(const f32x4*)(p.k + off) : f32x4{0.f, 0.f, 0.f, 0.f};
            vr[i] = ok ? *(const f32x4*)(p.v + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    float* Ks = lds + wave * 2 * TF;
    float* Vs = Ks + TF;
    if (wave < nend) load(wave);
    for (int n = wave; n < nend; n += NWF) {
        // this wave's buffers are free: its reads of the previous step are
        // done (LDS operations of one wave complete in order)
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            *(f32x4*)(Ks + (i * 64 + lane) * 4) = kr[i];
            *(f32x4*)(Vs + (i * 64 + lane) * 4) = vr[i];
        }
        __builtin_amdgcn_wave_barrier();
        if (n + NWF < nend) load(n + NWF);
        const int n0 = n * BNF;

        float s[BNF];
        float mt = -INFINITY;
#pragma unroll
        for (int j0 = 0; j0 < BNF; j0 += 4) {  // four keys at a time: independent chains
            float dot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < DL; d += 4) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const f32x4 kk = *(const f32x4*)(Ks + (j0 + u) * D + d0 + d);
                    dot[u] = fmaf(q[d], kk[0], dot[u]);
                    dot[u] = fmaf(q[d + 1], kk[1], dot[u]);
                    dot[u] = fmaf(q[d + 2], kk[2], dot[u]);
                    dot[u] = fmaf(q[d + 3], kk[3], dot[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float x = query_sum<DS>(dot[u]);
                const int key = n0 + j0 + u;
                s[j0 + u] = ((CAUSAL && key > qi) || key >= S) ? -INFINITY : x;
                mt = fmaxf(mt, s[j0 + u]);
            }
        }
        const float mnew = fmaxf(m, mt);
        if (mnew != -INFINITY) {  // else the whole step is masked for this lane
            // (s - m) * c: exactly 0 for the largest score, so its weight is exactly 1
            const float alpha = fast_exp2((m - mnew) * c);
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < BNF; ++j) {
                s[j] = fast_exp2((s[j] - mnew) * c);
                psum += s[j];
            }
            l = fmaf(l, alpha, psum);
            m = mnew;
#pragma unroll
            for (int d = 0; d < DL; d += 4) {
                float a0 = o[d] * alpha, a1 = o[d + 1] * alpha, a2 = o[d + 2] * alpha, a3 = o[d + 3] * alpha;
#pragma unroll
                for (int j = 0; j < BNF; ++j) {
                    const f32x4 vv = *(const f32x4*)(Vs + j * D + d0 + d);
                    a0 = fmaf(s[j], vv[0], a0);
                    a1 = fmaf(s[j], vv[1], a1);
                    a2 = fmaf(s[j], vv[2], a2);
                    a3 = fmaf(s[j], vv[3], a3);
                }
                o[d] = a0;
                o[d + 1] = a1;
                o[d + 2] = a2;
                o[d + 3] = a3;
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // merge: o = sum_w o_w 2^((m_w - M) c), l likewise, M = max_w m_w (a
    // wave that saw no key of this query has m_w = -inf and weight 0)
    __syncthreads();  // every wave is done with its K/V buffers
    if (wave > 0) {
#pragma unroll
        for (int d = 0; d < DL; ++d) red(wave - 1, d) = o[d];
        red(wave - 1, DL) = m;
        red(wave - 1, DL + 1) = l;
    }
    __syncthreads();
    if (wave > 0) return;
    float mm = m;
#pragma unroll
    for (int w = 0; w < NWF - 1; ++w) mm = fmaxf(mm, red(w, DL));
    const float a = m == -INFINITY ? 0.f : fast_exp2((m - mm) * c);
    l *= a;
#pragma unroll
    for (int d = 0; d < DL; ++d) o[d] *= a;
#pragma unroll
    for (int w = 0; w < NWF - 1; ++w) {
        const float mw = red(w, DL);
        const float aw = mw == -INFINITY ? 0.f : fast_exp2((mw - mm) * c);
        l = fmaf(red(w, DL + 1), aw, l);
#pragma unroll
        for (int d = 0; d < DL; ++d) o[d] = fmaf(red(w, d), aw, o[d]);
    }
    if (qi < S) {
        const float inv = 1.0f / l;
        float* orow = p.out + (row0 + qi) * D + d0;
#pragma unroll
        for (int d = 0; d < DL; d += 4) *(f32x4*)(orow + d) = f32x4{o[d], o[d + 1], o[d + 2], o[d + 3]} * inv;
        if (p.lse && d0 == 0) p.lse[row0 + qi] = (mm * c + __log2f(l)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const Params& prm, int blocks, hipStream_t stream) {
    Params arg = prm;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&fwd_f32_kernel<D, CAUSAL>, dim3(blocks), dim3(64 * NWF), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
    Params prm;
    prm.q = (const float*)a.q;
    prm.k = (const float*)a.k;
    prm.v = (const float*)a.v;
    prm.out = (float*)a.out;
    prm.lse = a.lse;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.S = a.S;
    prm.group = a.Hq / a.Hkv;
    const int qw = a.D == 128 ? F32Shape<128>::QW : F32Shape<64>::QW;
    prm.nq = (a.S + qw - 1) / qw;
    prm.c = a.scale * kLog2e;
    const int blocks = (int)((int64_t)a.B * a.Hq * prm.nq);
    if (a.D == 128) return a.causal ? launch<128, true>(prm, blocks, stream) : launch<128, false>(prm, blocks, stream);
    return a.causal ? launch<64, true>(prm, blocks, stream) : launch<64, false>(prm, blocks, stream);
}

}  // namespace attn
