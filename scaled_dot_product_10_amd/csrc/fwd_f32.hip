// Fused causal attention forward, float32 throughout.
//
// Same method as the bfloat16 kernel (key/value tiles through LDS, online
// softmax, nothing of size S x S in device memory) on plain float32 vector
// ALU arithmetic: one lane per query, 64 queries per workgroup, 16 keys per
// step.  This is the path for float32 inputs, where the bfloat16 matrix
// cores do not apply; it is a correctness path, not a throughput one.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int BMF = 64;  // queries per workgroup (one wave)
constexpr int BNF = 16;  // keys per step

struct Params {
    const float* q;
    const float* k;
    const float* v;
    float* out;
    float* lse;
    int Hq, Hkv, S, group, nq;
    float c;  // scale * log2(e), > 0
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(BMF) void fwd_f32_kernel(Params p) {
    __shared__ float Qs[BMF][D + 1];  // +1: lanes read different rows of one column
    __shared__ float Ks[BNF][D];
    __shared__ float Vs[BNF][D];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x / p.nq;
    int tile = blockIdx.x % p.nq;
    if (CAUSAL) tile = p.nq - 1 - tile;
    const int b = bh / p.Hq;
    const int h = bh % p.Hq;
    const int kvh = h / p.group;
    const int S = p.S;
    const int m0 = tile * BMF;
    const int qi = m0 + tid;
    const int64_t row0 = (int64_t)bh * S;
    const int64_t kvrow0 = ((int64_t)b * p.Hkv + kvh) * S;

    for (int idx = tid; idx < BMF * D; idx += BMF) {
        const int r = idx / D, d = idx % D;
        Qs[r][d] = (m0 + r < S) ? p.q[(row0 + m0 + r) * D + d] : 0.f;
    }

    float o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float c = p.c;

    const int qlast = min(m0 + BMF, S) - 1;
    const int ntiles = (S + BNF - 1) / BNF;
    const int nend = CAUSAL ? min(ntiles, qlast / BNF + 1) : ntiles;

    for (int n = 0; n < nend; ++n) {
        const int n0 = n * BNF;
        __syncthreads();  // previous tile consumed (and Qs written, first time)
        for (int idx = tid; idx < BNF * D; idx += BMF) {
            const int r = idx / D, d = idx % D;
            const bool ok = n0 + r < S;
            Ks[r][d] = ok ? p.k[(kvrow0 + n0 + r) * D + d] : 0.f;
            Vs[r][d] = ok ? p.v[(kvrow0 + n0 + r) * D + d] : 0.f;
        }
        __syncthreads();

        float s[BNF];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < BNF; ++j) {
            float dot = 0.f;
#pragma unroll 16
            for (int d = 0; d < D; ++d) dot = fmaf(Qs[tid][d], Ks[j][d], dot);
            const int key = n0 + j;
            s[j] = ((CAUSAL && key > qi) || key >= S) ? -INFINITY : dot;
            mt = fmaxf(mt, s[j]);
        }
        const float mnew = fmaxf(m, mt);
        if (mnew == -INFINITY) continue;  // whole step masked for this lane
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
        for (int d = 0; d < D; ++d) {
            float acc = o[d] * alpha;
#pragma unroll
            for (int j = 0; j < BNF; ++j) acc = fmaf(s[j], Vs[j][d], acc);
            o[d] = acc;
        }
    }

    if (qi < S) {
        const float inv = 1.0f / l;
        float* orow = p.out + (row0 + qi) * D;
#pragma unroll
        for (int d = 0; d < D; d += 4) *(f32x4*)(orow + d) = f32x4{o[d], o[d + 1], o[d + 2], o[d + 3]} * inv;
        if (p.lse) p.lse[row0 + qi] = (m * c + __log2f(l)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const Params& prm, int blocks, hipStream_t stream) {
    Params arg = prm;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&fwd_f32_kernel<D, CAUSAL>, dim3(blocks), dim3(BMF), args, 0, stream);
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
    prm.nq = (a.S + BMF - 1) / BMF;
    prm.c = a.scale * kLog2e;
    const int blocks = (int)((int64_t)a.B * a.Hq * prm.nq);
    if (a.D == 128) return a.causal ? launch<128, true>(prm, blocks, stream) : launch<128, false>(prm, blocks, stream);
    return a.causal ? launch<64, true>(prm, blocks, stream) : launch<64, false>(prm, blocks, stream);
}

}  // namespace attn
