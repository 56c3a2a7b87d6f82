// Split-KV attention forward for short query counts (a decode step against a
// key/value cache), bfloat16.
//
// q is [B, Hq, Sq, D] with Sq small; k, v are [B, Hkv, Skv, D] with Skv >= Sq.
// The queries are the last Sq positions of the sequence, so with causal = 1
// query i sees keys 0 .. Skv - Sq + i.  The sketch kernel of the ai-manual.ru
// tutorial (section 4) gives one program a whole query block and every key;
// its list of what the sketch lacks names split-k, the step taken here: with
// few queries, one program per query block would leave most of the GPU idle,
// so the key axis is cut into nsplit ranges that run in parallel, each
// producing a partial result (out normalised over its range, and its range's
// log-sum-exp), and a second kernel merges them:
//   lse = ln sum_s e^{lse_s},   out = sum_s e^{lse_s - lse} out_s.
//
// splitkv_bf16_kernel: workgroup = (b, key/value head g, block of 32 packed
//   query rows, split).  The rows are the (query head of g's group, query)
//   pairs, so a GQA group's heads share every K/V tile.  Q is the MFMA B
//   operand (row r = lane % 32) for the whole split; 128-key chunks of K and V
//   pass through LDS (whole-row loads, the next chunk in flight while the
//   current one is processed), each wave takes 32 keys of a chunk and
//   keeps its own running max, sum and O^T; the four waves merge through LDS
//   at the end.  The kernel is bound by the K/V read: its arithmetic is a
//   small fraction of the matrix cores' rate.
// splitkv_merge_kernel: one workgroup per row.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "lds_tiles.h"

namespace attn {
namespace {

constexpr int NT = 256;        // 4 waves
constexpr int ROWS = 32;       // packed query rows per workgroup (MFMA columns)
constexpr int CHUNK = 128;     // keys per workgroup step (32 per wave)
constexpr int kMaxMergeSplits = 4096;  // splits the merge holds in LDS (the entry point's limit)

struct SkvParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* opart;  // [nsplit][B*Hq*Sq][D]
    float* lpart;  // [nsplit][B*Hq*Sq]
    int Hq, Hkv, Sq, Skv, group;
    int nsplit;
    int klen;      // keys per split, a multiple of CHUNK
    int nrb;       // row blocks per (b, g)
    int64_t rtot;  // B * Hq * Sq
    uint32_t total;
    float c;       // scale * log2(e)
    int causal;
};

template <int D>
__global__ __launch_bounds__(NT, 2) void splitkv_bf16_kernel(SkvParams p) {
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    using TKV = RowTile<D, CHUNK, NT>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * CHUNK * D];  // K chunk, V chunk
    uint16_t* Ks = smem;
    uint16_t* Vs = smem + CHUNK * D;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    // grid order: split fastest, so the splits of one row block run side by side
    const uint32_t L = blockIdx.x;
    const int split = (int)(L % (uint32_t)p.nsplit);
    const uint32_t u = L / (uint32_t)p.nsplit;
    const int rb = (int)(u % (uint32_t)p.nrb);
    const int bg = (int)(u / (uint32_t)p.nrb);
    const int b = bg / p.Hkv, kvh = bg % p.Hkv;
    const int Sq = p.Sq, Skv = p.Skv;
    const int nrows = p.group * Sq;  // packed rows of this (b, g)

    // this lane's packed row r -> (query head, query index)
    const int r = rb * ROWS + l32;
    const bool rvalid = r < nrows;
    const int hq = kvh * p.group + (rvalid ? r / Sq : 0);
    const int qi = rvalid ? r % Sq : 0;
    const int64_t grow = ((int64_t)b * p.Hq + hq) * Sq + qi;  // row of q / out / partials
    const int klast = p.causal ? Skv - Sq + qi : Skv - 1;     // last key this row sees

    bf16x8 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0, 0, 0, 0};
        if (rvalid) x = *(const u32x4*)(p.q + grow * D + ks * 16 + g * 8);
        qreg[ks] = as_bf16x8(x);
    }
    int roff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[ks] = SwzTile<D>::at(wave * 32 + l32, (2 * ks + g) * 8);
    TrOffsets<D> tr;
    tr.init(lane);

    const int64_t kv0 = ((int64_t)b * p.Hkv + kvh) * Skv;
    const uint16_t* kb = p.k + kv0 * D;
    const uint16_t* vb = p.v + kv0 * D;
    const int k_lo = split * p.klen;
    const int k_hi = min(k_lo + p.klen, Skv);
    const float c = p.c;

    float m = -INFINITY;  // running max of s * c over this wave's keys (per row)
    float l = 0.f;        // running sum of 2^(s c - m), this lane's keys
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

    // The split's chunks are taken in a rotated order, different per
    // workgroup, so that workgroups streaming equally aligned slices do not
    // hit the same memory channels in step.  The next chunk is loaded into
    // registers while the current one is processed.
    const int nch = (k_hi - k_lo + CHUNK - 1) / CHUNK;
    const int rot = nch > 0 ? (int)((L * 7u) % (uint32_t)nch) : 0;
    auto chunk = [&](int i) __attribute__((always_inline)) {
        const int j = i + rot;
        return k_lo + (j < nch ? j : j - nch) * CHUNK;
    };
    TKV tk, tv;
    if (nch > 0) {
        tk.load(kb, chunk(0), k_hi, tid);  // rows at or past k_hi are zero (and masked below)
        tv.load(vb, chunk(0), k_hi, tid);
    }
    for (int i = 0; i < nch; ++i) {
        const int k0 = chunk(i);
        __syncthreads();  // previous chunk consumed
        tk.store(Ks, tid);
        tv.store(Vs, tid);
        __syncthreads();
        if (i + 1 < nch) {
            tk.load(kb, chunk(i + 1), k_hi, tid);
            tv.load(vb, chunk(i + 1), k_hi, tid);
        }
        const int kw = k0 + wave * 32;  // this wave's first key
        if (kw >= k_hi) continue;
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc = mfma32x32x16(*(const bf16x8*)(Ks + roff[ks]), qreg[ks], sacc);
        // accumulator row e: key kw + 8(e/4) + 4g + e%4
        float t = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = kw + 8 * (e >> 2) + 4 * g + (e & 3);
            if (key >= k_hi || key > klast) sacc[e] = -INFINITY;
            t = fmaxf(t, sacc[e]);
        }
        // the other half-wave holds the other 16 keys of the same row
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
        const float mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
        const float mn = fmaxf(m, mt);
        const float mref = mn == -INFINITY ? 0.f : mn;  // every key so far masked: p = 0, no rescale
        const float alpha = fast_exp2(m - mref);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        m = mn;
        f32x16 pv;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            pv[e] = fast_exp2(fmaf(sacc[e], c, -mref));
            l += pv[e];
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const bf16x8 pb = pack8(pv, half);
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] = mfma32x32x16(tr.read(Vs + wave * 32 * D, half, db), pb, oacc[db]);
        }
    }

    // ---- merge the four waves' partial results through LDS ------------------
    // red[w][d][row] = wave w's O^T (consecutive rows on consecutive banks);
    // ml = per wave and row: m, then l
    __shared__ float ml[2][4][ROWS];
    __syncthreads();
    float* red = (float*)smem;
    static_assert(4 * ROWS * D * 4 <= 2 * CHUNK * D * 2, "merge area fits");
    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    const float ltot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    if (g == 0) {
        ml[0][wave][l32] = m;
        ml[1][wave][l32] = ltot;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int d = db * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
            red[(wave * D + d) * ROWS + l32] = oacc[db][e];
        }
    __syncthreads();
    // thread -> row tid % 32 and D/8 consecutive d
    constexpr int DPT = D / 8;
    const int rr = tid % ROWS, d0 = (tid / ROWS) * DPT;
    const int r2 = rb * ROWS + rr;
    if (r2 < nrows) {
        const int64_t row = ((int64_t)b * p.Hq + kvh * p.group + r2 / Sq) * Sq + r2 % Sq;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[0][w][rr]);
        float wsc[4], Ls = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            wsc[w] = M == -INFINITY ? 0.f : fast_exp2(ml[0][w][rr] - M);
            Ls += wsc[w] * ml[1][w][rr];
        }
        const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
        float* dst = p.opart + ((int64_t)split * p.rtot + row) * D + d0;
#pragma unroll
        for (int e = 0; e < DPT; ++e) {
            float o = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) o += wsc[w] * red[(w * D + d0 + e) * ROWS + rr];
            dst[e] = o * inv;
        }
        if (d0 == 0) p.lpart[(int64_t)split * p.rtot + row] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
    }
}

// out = sum_s e^{lse_s - lse} out_s, lse = ln sum_s e^{lse_s}; one thread per (row, d)
// Workgroup-wide max / sum of one value per thread (all NT threads call it).
__device__ __forceinline__ float block_reduce(float x, bool is_max, float* scratch) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float y = __shfl_xor(x, o, 64);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) scratch[wave] = x;
    __syncthreads();
    float r = scratch[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) r = is_max ? fmaxf(r, scratch[w]) : r + scratch[w];
    __syncthreads();  // scratch reusable
    return r;
}

// One workgroup per row: the split weights w_s = e^{lse_s - M} are computed
// once (all threads load lse values side by side) and kept in LDS; then
// thread t sums w_s out_s[d] over the splits s = t / D (mod NT / D) for
// d = t % D, four independent partial sums deep, and the NT / D parts are
// added through LDS.  The loads are latency-bound, not bandwidth-bound, so
// what matters is how many are in flight at once.
template <int D>
__global__ __launch_bounds__(NT) void splitkv_merge_kernel(const float* opart, const float* lpart, uint16_t* out,
                                                             float* lse, int64_t rows, int nsplit) {
    constexpr int P = NT / D;  // parts per d
    __shared__ float wsh[kMaxMergeSplits];
    __shared__ float red[NT];
    __shared__ float scratch[NT / 64];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    float M = -INFINITY;
    for (int s = tid; s < nsplit; s += NT) M = fmaxf(M, lpart[(int64_t)s * rows + row]);
    M = block_reduce(M, true, scratch);
    float Lpart = 0.f;
    for (int s = tid; s < nsplit; s += NT) {
        const float w = M == -INFINITY ? 0.f : __expf(lpart[(int64_t)s * rows + row] - M);
        wsh[s] = w;
        Lpart += w;
    }
    const float Ls = block_reduce(Lpart, false, scratch);  // its barriers also publish wsh
    const int d = tid % D, part = tid / D;
    const float* base = opart + row * D + d;
    const int64_t step = rows * D;  // one split further
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    int s = part;
    for (; s + 3 * P < nsplit; s += 4 * P) {
        o0 += wsh[s] * base[(int64_t)s * step];
        o1 += wsh[s + P] * base[(int64_t)(s + P) * step];
        o2 += wsh[s + 2 * P] * base[(int64_t)(s + 2 * P) * step];
        o3 += wsh[s + 3 * P] * base[(int64_t)(s + 3 * P) * step];
    }
    for (; s < nsplit; s += P) o0 += wsh[s] * base[(int64_t)s * step];
    red[tid] = (o0 + o1) + (o2 + o3);
    __syncthreads();
    if (part == 0) {
        float o = red[d];
#pragma unroll
        for (int j = 1; j < P; ++j) o += red[d + j * D];
        const float v = Ls > 0.f ? o / Ls : 0.f;
        out[row * D + d] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
        if (lse && d == 0) lse[row] = Ls > 0.f ? M + __logf(Ls) : -INFINITY;
    }
}

template <typename K, typename P>
hipError_t launch1(K kernel, uint32_t grid, const P& prm, hipStream_t stream) {
    P arg = prm;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)kernel, dim3(grid), dim3(NT), args, 0, stream);
}

// Scratch of the allocation-free entry point: the partial outputs and
// log-sum-exps of every split, in the layout of the caller's workspace.  One
// copy per GPU, held for the life of the process; every call on a GPU
// shares it (concurrent calls on one GPU race).  Each call's split kernel
// writes every slot its merge reads, so nothing needs clearing between calls.
static __device__ __align__(256) float scratch[kSplitkvScratchFloats];

}  // namespace

// Device address of this GPU's scratch: looked up once per device (with that
// device current) and kept; the array's host-side name is not a device
// address and must never reach a kernel.
hipError_t splitkv_scratch(hipStream_t stream, float** ptr) {
    static std::mutex mu;
    static float* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (e2 != hipSuccess) return e2;
        if (!a) return hipErrorInvalidSymbol;
        addr[dev] = (float*)a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

int splitkv_row_blocks(int Hq, int Hkv, int Sq) { return (Hq / Hkv * Sq + ROWS - 1) / ROWS; }
int splitkv_chunk() { return CHUNK; }

hipError_t launch_splitkv_bf16(const SplitKvArgs& a, hipStream_t stream) {
    SkvParams prm;
    prm.q = (const uint16_t*)a.q;
    prm.k = (const uint16_t*)a.k;
    prm.v = (const uint16_t*)a.v;
    const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
    prm.opart = a.workspace;
    prm.lpart = a.workspace + (int64_t)a.nsplit * rows * a.D;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.Sq = a.Sq;
    prm.Skv = a.Skv;
    prm.group = a.Hq / a.Hkv;
    prm.nsplit = a.nsplit;
    const int per = (a.Skv + a.nsplit - 1) / a.nsplit;
    prm.klen = (per + CHUNK - 1) / CHUNK * CHUNK;
    prm.nrb = splitkv_row_blocks(a.Hq, a.Hkv, a.Sq);
    prm.rtot = rows;
    prm.total = (uint32_t)((int64_t)a.B * a.Hkv * prm.nrb * a.nsplit);
    prm.c = a.scale * kLog2e;
    prm.causal = a.causal;
    hipError_t e = a.D == 128 ? launch1(&splitkv_bf16_kernel<128>, prm.total, prm, stream)
                              : launch1(&splitkv_bf16_kernel<64>, prm.total, prm, stream);
    if (e != hipSuccess) return e;
    const uint32_t mgrid = (uint32_t)rows;  // one workgroup per row
    const float* op = prm.opart;
    const float* lp = prm.lpart;
    uint16_t* out = (uint16_t*)a.out;
    float* lse = a.lse;
    int64_t nrow = rows;
    int ns = a.nsplit;
    void* args[] = {(void*)&op, (void*)&lp, (void*)&out, (void*)&lse, (void*)&nrow, (void*)&ns};
    return hipLaunchKernel(a.D == 128 ? (const void*)&splitkv_merge_kernel<128> : (const void*)&splitkv_merge_kernel<64>,
                           dim3(mgrid), dim3(NT), args, 0, stream);
}

}  // namespace attn
