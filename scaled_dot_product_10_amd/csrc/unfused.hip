// The unfused pipeline, one kernel per step, mirroring the naive attention of
// the Hugging Face "Profiling in PyTorch (Part 3)" article ("Naive
// Attention" section): (1) scores = q k^T, (2)-(4) scale, mask with -inf and
// softmax, (5) out = attn v.  Scores and probabilities are materialised in
// caller-owned buffers of size B*H*S*S, which is exactly the memory traffic
// the fused kernel avoids.
//
// The bfloat16 products use the same 32x32x16 MFMA as the fused kernel.  The
// float32 variants run a plain LDS-tiled vector-ALU matrix product.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// Step 1, bfloat16: scores[bh][i][j] = sum_d q[bh][i][d] k[bkv][j][d], float32.
// 128 x 128 output tile per workgroup; wave (wi, wj) owns 64 x 64 = 2 x 2
// MFMA blocks.  The 128-row Q and K tiles are loaded whole rows at a time
// (D/8 lanes per row, so every load instruction covers whole cache lines)
// into swizzled LDS, from which A = k rows (j = lane % 32) and B = q rows
// (i = lane % 32) are read; a lane's accumulators then hold runs of 4
// consecutive keys of one query.  The operand area is then reused: each wave
// passes its 32 x 64 half-blocks through a private part of it and stores them
// row by row, 16 lanes writing one row's 256 contiguous bytes, 16 bytes each,
// so the score stores also cover whole cache lines.
// ---------------------------------------------------------------------------
constexpr int QK_T = 128;
constexpr int QK_STAGE_LD = 68;  // floats per staged row: 64 keys + 4 (spreads rows over the banks)

struct QkParams {
    const uint16_t* q;
    const uint16_t* k;
    float* scores;
    int Hq, Hkv, S, group, nt;
    uint32_t total;
};

template <int D>
__global__ __launch_bounds__(256) void qk_gemm_bf16_kernel(QkParams p) {
    constexpr int KS = D / 16;
    constexpr int CPR = D / 8;                  // 16-byte chunks per row
    constexpr int LCH = QK_T * CPR / 256;       // chunks per thread per operand tile
    constexpr int TILE = QK_T * D;              // elements per operand tile
    constexpr int STAGE_BYTES = 4 * 32 * QK_STAGE_LD * 4;
    constexpr int SMEM = 2 * TILE * 2 > STAGE_BYTES ? 2 * TILE * 2 : STAGE_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];
    uint16_t* Qs = (uint16_t*)smem;
    uint16_t* Ks = Qs + TILE;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const uint32_t L = xcd_remap(blockIdx.x, p.total);
    const uint32_t nt2 = (uint32_t)p.nt * p.nt;
    const int bh = (int)(L / nt2);
    const int rem = (int)(L % nt2);
    const int ti = rem / p.nt, tj = rem % p.nt;
    const int b = bh / p.Hq, h = bh % p.Hq, kvh = h / p.group;
    const int S = p.S;
    const uint16_t* qb = p.q + ((int64_t)bh * S + ti * QK_T) * D;
    const uint16_t* kb = p.k + (((int64_t)b * p.Hkv + kvh) * S + tj * QK_T) * D;
    // chunk c of row r sits at chunk position c ^ swz(r): the 16 rows one
    // operand read touches land on different banks
    auto swz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
    {
        u32x4 rq[LCH], rk[LCH];
#pragma unroll
        for (int i = 0; i < LCH; ++i) {
            const int c = tid + 256 * i, r = c / CPR, col = (c % CPR) * 8;
            rq[i] = ti * QK_T + r < S ? *(const u32x4*)(qb + r * D + col) : u32x4{0, 0, 0, 0};
            rk[i] = tj * QK_T + r < S ? *(const u32x4*)(kb + r * D + col) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < LCH; ++i) {
            const int c = tid + 256 * i, r = c / CPR, pos = r * D + (((c % CPR) ^ swz(r)) * 8);
            *(u32x4*)(Qs + pos) = rq[i];
            *(u32x4*)(Ks + pos) = rk[i];
        }
    }
    __syncthreads();
    const int ib = ti * QK_T + (wave >> 1) * 64;
    const int jb = tj * QK_T + (wave & 1) * 64;
    const int rq0 = (wave >> 1) * 64 + l32, rk0 = (wave & 1) * 64 + l32;

    f32x16 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        bf16x8 a[2], bb[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int rq = rq0 + 32 * x, rk = rk0 + 32 * x;
            a[x] = *(const bf16x8*)(Qs + rq * D + (((2 * ks + g) ^ swz(rq)) * 8));
            bb[x] = *(const bf16x8*)(Ks + rk * D + (((2 * ks + g) ^ swz(rk)) * 8));
        }
        // acc[x][y] = K-block y . Q-block x^T: lane l holds query ib + 32x + l % 32
        // and keys jb + 32y + 8(r/4) + 4(l/32) + r%4 in accumulator r.
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) acc[x][y] = mfma32x32x16(bb[y], a[x], acc[x][y]);
    }
    __syncthreads();  // operand tiles consumed; their space now stages the output

    float* st = (float*)smem + wave * 32 * QK_STAGE_LD;
    float* sb = p.scores + (int64_t)bh * S * S;
    const bool full = jb + 64 <= S && (S & 3) == 0;
    const int rr = lane >> 4;        // row within a group of 4 staged rows
    const int cc = (lane & 15) * 4;  // first of the lane's 4 keys
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(f32x4*)(st + l32 * QK_STAGE_LD + y * 32 + q4 * 8 + g * 4) =
                    f32x4{acc[x][y][4 * q4], acc[x][y][4 * q4 + 1], acc[x][y][4 * q4 + 2], acc[x][y][4 * q4 + 3]};
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int r = 4 * t + rr;
            const int i = ib + x * 32 + r;
            const f32x4 v = *(const f32x4*)(st + r * QK_STAGE_LD + cc);
            if (i < S) {
                float* dst = sb + (int64_t)i * S + jb + cc;
                if (full) {
                    __builtin_nontemporal_store(v, (f32x4*)dst);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (jb + cc + e < S) __builtin_nontemporal_store(v[e], dst + e);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// ---------------------------------------------------------------------------
// Step 1 and step 5, float32: C[bh][i][j] = sum_k A[bh][i][k] * Bm(k, j) with
// Bm(k, j) = B[bkv][j][k] (BT, for q k^T) or B[bkv][k][j] (for p v).
// 64 x 64 tile per workgroup, 16 x 16 threads, 4 x 4 outputs per thread.
// ---------------------------------------------------------------------------
struct SgemmParams {
    const float* A;
    const float* Bm;
    float* C;
    int M, N, K;          // C is M x N, contraction length K
    int Hq, Hkv, group;
    int tn, tiles;        // tiles along N, tiles per bh
    uint32_t total;
};

template <bool BT>
__global__ __launch_bounds__(256) void sgemm_f32_kernel(SgemmParams p) {
    constexpr int T = 64, KC = 16;
    __shared__ float As[KC][T + 1];
    __shared__ float Bs[KC][T + 1];
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const uint32_t L = blockIdx.x;
    const int bh = (int)(L / (uint32_t)p.tiles);
    const int rem = (int)(L % (uint32_t)p.tiles);
    const int i0 = (rem / p.tn) * T, j0 = (rem % p.tn) * T;
    const int b = bh / p.Hq, h = bh % p.Hq, kvh = h / p.group;
    const float* A = p.A + (int64_t)bh * p.M * p.K;
    const float* Bm = p.Bm + ((int64_t)b * p.Hkv + kvh) * (int64_t)p.N * p.K;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += KC) {
        for (int idx = tid; idx < KC * T; idx += 256) {
            // As[kk][ii] = A[i0+ii][k0+kk]; Bs[kk][jj] = Bm(k0+kk, j0+jj)
            const int ii = idx / KC, kk = idx % KC;
            const int i = i0 + ii, k = k0 + kk;
            As[kk][ii] = (i < p.M && k < p.K) ? A[(int64_t)i * p.K + k] : 0.f;
            if (BT) {
                const int j = j0 + ii;
                Bs[kk][ii] = (j < p.N && k < p.K) ? Bm[(int64_t)j * p.K + k] : 0.f;
            } else {
                const int kk2 = idx / T, jj = idx % T;
                const int k2 = k0 + kk2, j = j0 + jj;
                Bs[kk2][jj] = (j < p.N && k2 < p.K) ? Bm[(int64_t)k2 * p.N + j] : 0.f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
            float a[4], bv[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) a[x] = As[kk][ty + 16 * x];
#pragma unroll
            for (int y = 0; y < 4; ++y) bv[y] = Bs[kk][tx + 16 * y];
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], bv[y], acc[x][y]);
        }
        __syncthreads();
    }
    float* C = p.C + (int64_t)bh * p.M * p.N;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int i = i0 + ty + 16 * x;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            const int j = j0 + tx + 16 * y;
            if (i < p.M && j < p.N) C[(int64_t)i * p.N + j] = acc[x][y];
        }
    }
}

// ---------------------------------------------------------------------------
// Steps 2-4: p = softmax(scale * x) over the unmasked keys of each row; masked
// entries are written as 0 and never read.  One wave per row.
// Fast path (S % 4 == 0, S <= 64*4*NCH): the row stays in registers, read
// once with 16-byte loads, written once.  General path: two passes (online
// max/sum, then normalise and write).
// ---------------------------------------------------------------------------
struct SmParams {
    const float* x;
    void* p;
    float* lse;
    int S;
    int64_t rows;
    float c;  // scale * log2(e)
    int causal;
};

template <typename OutT>
__device__ __forceinline__ void store4(OutT* dst, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* dst, f32x4 v) {
    __builtin_nontemporal_store(v, (f32x4*)dst);
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* dst, f32x4 v) {
    const u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    __builtin_nontemporal_store(w, (u32x2*)dst);
}
template <typename OutT>
__device__ __forceinline__ void store1(OutT* dst, float v);
template <>
__device__ __forceinline__ void store1<float>(float* dst, float v) { *dst = v; }
template <>
__device__ __forceinline__ void store1<uint16_t>(uint16_t* dst, float v) {
    *dst = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
}

template <int NCH, typename OutT>
__global__ __launch_bounds__(256) void softmax_rows_kernel(SmParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.rows) return;  // whole wave
    const int S = p.S;
    const int i = (int)(row % S);
    const int lim = p.causal ? i + 1 : S;  // keys j < lim are visible
    const float* x = p.x + row * S;
    OutT* out = (OutT*)p.p + row * S;
    const float c = p.c;

    f32x4 v[NCH];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
        const int j0 = 4 * (lane + 64 * t);
        f32x4 e = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (j0 < lim) {
            e = __builtin_nontemporal_load((const f32x4*)(x + j0));
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (j0 + u >= lim) e[u] = -INFINITY;
        }
        v[t] = e;
        mx = fmaxf(fmaxf(mx, fmaxf(e[0], e[1])), fmaxf(e[2], e[3]));
    }
    mx = wave_max(mx);
    const float mc = mx * c;
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[t][u] = fast_exp2(fmaf(v[t][u], c, -mc));
            sum += v[t][u];
        }
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
        const int j0 = 4 * (lane + 64 * t);
        if (j0 < S) store4<OutT>(out + j0, v[t] * inv);
    }
    if (p.lse && lane == 0) p.lse[row] = (mc + __log2f(sum)) * kLn2;
}

template <typename OutT>
__global__ __launch_bounds__(256) void softmax_rows_general_kernel(SmParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.rows) return;
    const int S = p.S;
    const int i = (int)(row % S);
    const int lim = p.causal ? i + 1 : S;
    const float* x = p.x + row * S;
    OutT* out = (OutT*)p.p + row * S;
    const float c = p.c;
    // pass 1: per-lane running max and sum (scaled log2 units), then combine
    float m = -INFINITY, s = 0.f;
    for (int j = lane; j < lim; j += 64) {
        const float t = x[j] * c;
        const float mn = fmaxf(m, t);
        s = s * fast_exp2(m - mn) + fast_exp2(t - mn);
        m = mn;
    }
    const float M = wave_max(m);
    const float tot = wave_sum(m == -INFINITY ? 0.f : s * fast_exp2(m - M));
    const float inv = 1.0f / tot;
    // pass 2
    for (int j = lane; j < S; j += 64) {
        const float pv = (j < lim) ? fast_exp2(fmaf(x[j], c, -M)) * inv : 0.f;
        store1<OutT>(out + j, pv);
    }
    if (p.lse && lane == 0) p.lse[row] = (M + __log2f(tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// Step 5, bfloat16: out[bh][i][d] = sum_j p[bh][i][j] v[bkv][j][d].
// Computed as out^T = V^T . P^T on the 32x32x16 MFMA, 128 queries per
// workgroup (32 per wave), 64 keys per step.  Both tiles are read from global
// memory whole rows at a time (8 lanes per 128-byte P row segment, D/8 lanes
// per V row), which keeps every load instruction on whole cache lines, and
// pass through LDS: P rows as they are (the B operand is 8 consecutive keys
// of one query), V rows swizzled and read back transposed.  The next step's
// tiles are in flight in registers while a step multiplies.
// ---------------------------------------------------------------------------
constexpr int PV_BM = 128, PV_BN = 64;

struct PvParams {
    const uint16_t* p;
    const uint16_t* v;
    uint16_t* out;
    int Hq, Hkv, S, group, nq;
    uint32_t total;
};

template <int D, bool ALIGNED>
__global__ __launch_bounds__(256, 2) void pv_gemm_bf16_kernel(PvParams p) {
    constexpr int DB = D / 32;
    constexpr int PPAD = PV_BN + 8;
    constexpr int CPR = D / 8;                   // 16-byte chunks per V row
    constexpr int VCH = PV_BN * CPR / 256;       // V chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t Vs[PV_BN * D];
    __shared__ __attribute__((aligned(16))) uint16_t Ps[PV_BM * PPAD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const uint32_t L = xcd_remap(blockIdx.x, p.total);
    const int bh = (int)(L / (uint32_t)p.nq);
    const int tile = (int)(L % (uint32_t)p.nq);
    const int b = bh / p.Hq, h = bh % p.Hq, kvh = h / p.group;
    const int S = p.S;
    const int qi = tile * PV_BM + wave * 32 + l32;
    const uint16_t* pbase = p.p + ((int64_t)bh * S + tile * PV_BM) * S;
    const uint16_t* vb = p.v + ((int64_t)b * p.Hkv + kvh) * S * D;
    auto vswz = [](int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
    u32x4 pr[4], vr[VCH];
    auto load = [&](int n) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, r = c >> 3, key = n * PV_BN + (c & 7) * 8;
            u32x4 w = {0, 0, 0, 0};
            if (tile * PV_BM + r < S) {
                const uint16_t* src = pbase + (int64_t)r * S + key;
                if (ALIGNED) {
                    if (key < S) w = *(const u32x4*)src;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t x = (key + e < S) ? src[e] : 0u;
                        w[e >> 1] |= (e & 1) ? (x << 16) : x;
                    }
                }
            }
            pr[i] = w;
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = tid + 256 * i, key = n * PV_BN + c / CPR;
            vr[i] = key < S ? *(const u32x4*)(vb + (int64_t)key * D + (c % CPR) * 8) : u32x4{0, 0, 0, 0};
        }
    };
    int voff[DB];  // transposed read: lane j of 16-lane group G takes rows 8(G/2) + j/4 (+4),
                   // d = 32db + 16(G%2) + 4(j%4) .. +3
    {
        const int G = lane >> 4, j = lane & 15;
        const int r = 8 * (G >> 1) + (j >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d0 = db * 32 + (G & 1) * 16 + 4 * (j & 3);
            voff[db] = r * D + (((d0 >> 3) ^ vswz(r)) * 8) + (d0 & 7);
        }
    }
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    const int ntiles = (S + PV_BN - 1) / PV_BN;
    load(0);
    for (int n = 0; n < ntiles; ++n) {
        __syncthreads();  // previous tile consumed
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            *(u32x4*)(Ps + (c >> 3) * PPAD + (c & 7) * 8) = pr[i];
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = tid + 256 * i, r = c / CPR;
            *(u32x4*)(Vs + r * D + (((c % CPR) ^ vswz(r)) * 8)) = vr[i];
        }
        __syncthreads();
        if (n + 1 < ntiles) load(n + 1);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 bb = *(const bf16x8*)(Ps + (wave * 32 + l32) * PPAD + kb * 16 + g * 8);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint16_t* base = Vs + voff[db] + kb * 16 * D;
                oacc[db] = mfma32x32x16(tr_read_pair(base, base + 4 * D), bb, oacc[db]);
            }
        }
    }
    if (qi < S) {
        uint16_t* orow = p.out + ((int64_t)bh * S + qi) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = db * 32 + j * 8 + g * 4;
                *(u32x2*)(orow + d0) = u32x2{pack_bf16x2(oacc[db][4 * j], oacc[db][4 * j + 1]),
                                             pack_bf16x2(oacc[db][4 * j + 2], oacc[db][4 * j + 3])};
            }
        }
    }
}

template <typename K, typename P>
hipError_t launch1(K kernel, dim3 grid, dim3 block, const P& prm, hipStream_t stream) {
    P arg = prm;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)kernel, grid, block, args, 0, stream);
}

hipError_t launch_sgemm(bool bt, const float* A, const float* Bm, float* C, int B, int Hq, int Hkv,
                        int M, int N, int K, hipStream_t stream) {
    SgemmParams prm;
    prm.A = A;
    prm.Bm = Bm;
    prm.C = C;
    prm.M = M;
    prm.N = N;
    prm.K = K;
    prm.Hq = Hq;
    prm.Hkv = Hkv;
    prm.group = Hq / Hkv;
    prm.tn = (N + 63) / 64;
    prm.tiles = ((M + 63) / 64) * prm.tn;
    prm.total = (uint32_t)((int64_t)B * Hq * prm.tiles);
    if (bt) return launch1(&sgemm_f32_kernel<true>, dim3(prm.total), dim3(256), prm, stream);
    return launch1(&sgemm_f32_kernel<false>, dim3(prm.total), dim3(256), prm, stream);
}

template <typename OutT>
hipError_t launch_softmax(const SoftmaxArgs& a, hipStream_t stream) {
    SmParams prm;
    prm.x = a.scores;
    prm.p = a.p;
    prm.lse = a.lse;
    prm.S = a.S;
    prm.rows = (int64_t)a.B * a.H * a.S;
    prm.c = a.scale * kLog2e;
    prm.causal = a.causal;
    const dim3 grid((unsigned)((prm.rows + 3) / 4)), block(256);
    const int chunks = (a.S + 255) / 256;  // float4 chunks per lane
    if (a.S % 4 == 0) {
        if (chunks <= 1) return launch1(&softmax_rows_kernel<1, OutT>, grid, block, prm, stream);
        if (chunks <= 2) return launch1(&softmax_rows_kernel<2, OutT>, grid, block, prm, stream);
        if (chunks <= 4) return launch1(&softmax_rows_kernel<4, OutT>, grid, block, prm, stream);
        if (chunks <= 8) return launch1(&softmax_rows_kernel<8, OutT>, grid, block, prm, stream);
        if (chunks <= 16) return launch1(&softmax_rows_kernel<16, OutT>, grid, block, prm, stream);
        if (chunks <= 32) return launch1(&softmax_rows_kernel<32, OutT>, grid, block, prm, stream);
    }
    return launch1(&softmax_rows_general_kernel<OutT>, grid, block, prm, stream);
}

}  // namespace

hipError_t launch_qk_gemm_bf16(const QkArgs& a, hipStream_t stream) {
    QkParams prm;
    prm.q = (const uint16_t*)a.q;
    prm.k = (const uint16_t*)a.k;
    prm.scores = a.scores;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.S = a.S;
    prm.group = a.Hq / a.Hkv;
    prm.nt = (a.S + QK_T - 1) / QK_T;
    prm.total = (uint32_t)((int64_t)a.B * a.Hq * prm.nt * prm.nt);
    if (a.D == 128) return launch1(&qk_gemm_bf16_kernel<128>, dim3(prm.total), dim3(256), prm, stream);
    return launch1(&qk_gemm_bf16_kernel<64>, dim3(prm.total), dim3(256), prm, stream);
}

hipError_t launch_qk_gemm_f32(const QkArgs& a, hipStream_t stream) {
    return launch_sgemm(true, (const float*)a.q, (const float*)a.k, a.scores, a.B, a.Hq, a.Hkv, a.S, a.S, a.D,
                        stream);
}

hipError_t launch_masked_softmax_bf16(const SoftmaxArgs& a, hipStream_t stream) {
    return launch_softmax<uint16_t>(a, stream);
}

hipError_t launch_masked_softmax_f32(const SoftmaxArgs& a, hipStream_t stream) {
    return launch_softmax<float>(a, stream);
}

hipError_t launch_pv_gemm_bf16(const PvArgs& a, hipStream_t stream) {
    PvParams prm;
    prm.p = (const uint16_t*)a.p;
    prm.v = (const uint16_t*)a.v;
    prm.out = (uint16_t*)a.out;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.S = a.S;
    prm.group = a.Hq / a.Hkv;
    prm.nq = (a.S + PV_BM - 1) / PV_BM;
    prm.total = (uint32_t)((int64_t)a.B * a.Hq * prm.nq);
    const bool aligned = a.S % 8 == 0;
    if (a.D == 128)
        return aligned ? launch1(&pv_gemm_bf16_kernel<128, true>, dim3(prm.total), dim3(256), prm, stream)
                       : launch1(&pv_gemm_bf16_kernel<128, false>, dim3(prm.total), dim3(256), prm, stream);
    return aligned ? launch1(&pv_gemm_bf16_kernel<64, true>, dim3(prm.total), dim3(256), prm, stream)
                   : launch1(&pv_gemm_bf16_kernel<64, false>, dim3(prm.total), dim3(256), prm, stream);
}

hipError_t launch_pv_gemm_f32(const PvArgs& a, hipStream_t stream) {
    return launch_sgemm(false, (const float*)a.p, (const float*)a.v, (float*)a.out, a.B, a.Hq, a.Hkv, a.S, a.D,
                        a.S, stream);
}

}  // namespace attn
