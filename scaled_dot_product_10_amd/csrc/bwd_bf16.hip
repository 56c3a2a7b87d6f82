// Attention backward, bfloat16 in and out, float32 accumulation.
//
// The gradients are the chain-rule derivative of the forward
// out_i = sum_j p_ij v_j, p_ij = exp(s_ij - lse_i), s_ij = scale q_i . k_j
// (the forward formula of the ainews.cool deep-dive, causal mask as in the
// Hugging Face article's "Naive Attention" section; the ai-manual.ru
// tutorial, section 6, warns that the flash backward is the delicate part):
//
//   delta_i = dout_i . out_i                     (= sum_j p_ij dp_ij)
//   dp_ij   = dout_i . v_j
//   ds_ij   = p_ij (dp_ij - delta_i)
//   dv_j    = sum_i p_ij dout_i
//   dk_j    = scale sum_i ds_ij q_i
//   dq_i    = scale sum_j ds_ij k_j
//
// Three kernels, none of which writes an S x S matrix: p is recomputed on
// chip from the forward's lse in both main kernels.
//   bwd_delta_kernel   delta_i, one pass over out and dout.
//   bwd_dkdv_kernel    a workgroup owns 128 keys of one key/value head and
//                      sweeps every query (of every query head of its group)
//                      that sees them: S = Q K^T and dP = dO V^T with K, V in
//                      LDS, then dV^T += dO^T P and dK^T += Q^T dS with Q and
//                      dO read transposed from LDS; two waves share each
//                      32-key column block, one per half of a query tile.
//   bwd_dq_kernel      a workgroup owns 128 queries and sweeps their keys:
//                      S^T = K Q^T and dP^T = V dO^T with Q, dO in
//                      registers, then dQ^T += K^T dS^T with K read
//                      transposed from LDS.
// dq is computed by its own kernel rather than by atomic adds from the dK/dV
// sweep: two more products per tile, but no read-modify-write traffic and a
// deterministic result.
//
// MFMA layouts are those of v_mfma_f32_32x32x16_bf16 (common.h).  In both
// main kernels the probabilities and ds come out of an accumulator whose
// lane owns one column; a 16-row block of it is exactly the B operand of the
// next product when the A operand's k order is the accumulator's row order
// (rows 4g..4g+3 and 8+4g..8+4g+3 for lane half g), which the transposed
// LDS read provides.
#include "common.h"
#include "launch.h"
#include "lds_dma.h"
#include "lds_tiles.h"

namespace attn {
namespace {

constexpr int NT = 256;       // 4 waves (delta, dQ)
constexpr int KEYS_WG = 128;  // keys per dK/dV workgroup (32 per wave)
constexpr int QRY_TILE = 64;  // queries per step of the dK/dV sweep
constexpr int QRY_WG = 128;   // queries per dQ workgroup (32 per wave)
constexpr int KEY_TILE = 64;  // keys per step of the dQ sweep

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* out;
    const uint16_t* dout;
    const float* lse;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* delta;
    int B, Hq, Hkv, S, group;
    int ntiles;      // workgroups per head (key tiles or query tiles)
    uint32_t total;  // workgroups in the grid
    float c;         // scale * log2(e)
    float scale;
    int causal;
};

// ---------------------------------------------------------------------------
// delta_i = sum_d dout[i][d] out[i][d]; D/8 lanes per row, 16 bytes each.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NT) void bwd_delta_kernel(BwdParams p, int64_t rows) {
    constexpr int LPR = D / 8;         // lanes per row
    constexpr int RPB = NT / LPR;      // rows per block
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
    const int col = (tid % LPR) * 8;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = *(const u32x4*)(p.out + row * D + col);
        const u32x4 b = *(const u32x4*)(p.dout + row * D + col);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a0 = __uint_as_float(a[e] << 16), a1 = __uint_as_float(a[e] & 0xffff0000u);
            const float b0 = __uint_as_float(b[e] << 16), b1 = __uint_as_float(b[e] & 0xffff0000u);
            acc = fmaf(a0, b0, fmaf(a1, b1, acc));
        }
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (row < rows && tid % LPR == 0) p.delta[row] = acc;
}

// DMA of one 64-row tile (K, V, Q or dO) into a SwzTile by NW waves: instruction i of wave w fills
// LDS chunk positions p = (w PER + i) 64 + lane, i.e. row p / CPR at chunk
// position p % CPR, which holds chunk (p % CPR) ^ swz(row); rows past the
// end of the sequence repeat row S-1 (those keys are masked, those queries
// have lse = +inf and weight 0).
template <int D, int NW>
struct SwzDma {
    static constexpr int CPR = D / 8;
    static constexpr int PER = 64 * CPR / 64 / NW;  // instructions per wave
    static_assert(PER >= 1 && PER * NW * 64 == 64 * CPR, "whole tile, whole instructions");
    uint32_t off[PER];
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int pos = (wave * PER + i) * 64 + lane;
            const int r = pos / CPR;
            off[i] = (uint32_t)(r * D * 2 + (((pos % CPR) ^ SwzTile<D>::swz(r)) * 16));
        }
    }
    __device__ __forceinline__ void issue(const uint16_t* base, int n0, int S, uint16_t* tile, int wave) const {
        const uint16_t* tb = base + (int64_t)n0 * D;
        const uint32_t l0 = lds_addr(tile) + (uint32_t)(wave * PER) * 1024u;
        const int last = S - 1 - n0;  // last valid row of this tile
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int r = (int)(off[i] / (D * 2));
            const uint32_t o = n0 + 64 <= S ? off[i] : off[i] - (uint32_t)((r - min(r, last)) * D * 2);
            dma16(tb, o, l0 + i * 1024);
        }
    }
};

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup = (b, kv head g, 128-key tile) of 8 waves, two per SIMD;
// waves w and w + 4 own keys n0 + 32 (w % 4) .. +31 (lane l32 = key) and take
// the first and second 32 queries of every 64-query tile.  The workgroup
// sweeps the query heads of the group and their 64-query tiles from the first
// one that sees the keys.  K and V of the workgroup's keys stay in LDS (the
// B operands of S = Q K^T and dP = dO V^T are read from there), which keeps
// each wave, with its dK^T and dV^T accumulators, within 256 registers; at
// one wave per SIMD with K and V in registers (392 registers) the products
// and the exponentials of a wave could not overlap.  At the end waves 4-7
// add their partial dK^T, dV^T into waves 0-3 through LDS.
// ---------------------------------------------------------------------------
constexpr int NT2 = 512;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT2) void bwd_dkdv_kernel(BwdParams p) {
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    using TK = RowTile<D, KEYS_WG, NT2>;
    static_assert(QRY_TILE == 64, "one SwzDma tile per query tile");
    __shared__ __attribute__((aligned(1024))) uint16_t KVs[2 * KEYS_WG * D];   // K rows, then V rows
    __shared__ __attribute__((aligned(1024))) uint16_t QOs[4 * QRY_TILE * D];  // Q(buf 0), Q(1), dO(0), dO(1)
    __shared__ __attribute__((aligned(16))) float LDs[2][2][QRY_TILE];         // [buf]: lse * log2(e) (+inf past S), delta
    uint16_t* Ks = KVs;
    uint16_t* Vs = KVs + KEYS_WG * D;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the DMA's LDS address is scalar
    const int l32 = lane & 31, g = lane >> 5;
    const int kq = wave & 3;   // key quarter of the workgroup
    const int xh = wave >> 2;  // which 32 queries of each 64-query tile
    const uint32_t L = xcd_remap(blockIdx.x, p.total);
    const int bg = (int)(L / (uint32_t)p.ntiles);
    const int tile = (int)(L % (uint32_t)p.ntiles);  // ascending: longest sweeps first under the mask
    const int b = bg / p.Hkv, kvh = bg % p.Hkv;
    const int S = p.S;
    const int n0 = tile * KEYS_WG;
    const int key = n0 + kq * 32 + l32;
    const uint16_t* kb = p.k + (int64_t)bg * S * D;
    const uint16_t* vb = p.v + (int64_t)bg * S * D;
    {
        TK tk, tv;
        tk.load(kb, n0, S, tid);  // rows past S are zero
        tv.load(vb, n0, S, tid);
        tk.store(Ks, tid);
        tv.store(Vs, tid);
    }
    int roff[KS], koff[KS];  // row l32 of this wave's query block / key quarter, chunk 2ks + g
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        roff[ks] = SwzTile<D>::at(xh * 32 + l32, (2 * ks + g) * 8);
        koff[ks] = SwzTile<D>::at(kq * 32 + l32, (2 * ks + g) * 8);
    }
    TrOffsets<D> tr;
    tr.init(lane);

    f32x16 dvacc[DB], dkacc[DB];  // dV^T, dK^T: rows d, column = key
#pragma unroll
    for (int db = 0; db < DB; ++db) dvacc[db] = dkacc[db] = f32x16{};

    const int nqt = (S + QRY_TILE - 1) / QRY_TILE;
    const int qt0 = CAUSAL ? n0 / QRY_TILE : 0;
    const int steps = (nqt - qt0) * p.group;  // (head, query tile) pairs
    const float c = p.c;
    const float kLog2eF = kLog2e;

    // Q, dO tiles by DMA into two buffers; lse and delta of the next tile go
    // through registers and are stored after the current tile's products
    SwzDma<D, NT2 / 64> dma;
    dma.init(wave, lane);
    float lnext = 0.f, dnext = 0.f;
    auto fetch = [&](int s, int buf) __attribute__((always_inline)) {
        const int h = kvh * p.group + s / (nqt - qt0);
        const int m0 = (qt0 + s % (nqt - qt0)) * QRY_TILE;
        const int64_t rowb = ((int64_t)b * p.Hq + h) * S;
        dma.issue(p.q + rowb * D, m0, S, QOs + buf * QRY_TILE * D, wave);
        dma.issue(p.dout + rowb * D, m0, S, QOs + (2 + buf) * QRY_TILE * D, wave);
        if (tid < QRY_TILE) {
            const int i = m0 + tid;
            lnext = i < S ? p.lse[rowb + i] * kLog2eF : INFINITY;
            dnext = i < S ? p.delta[rowb + i] : 0.f;
        }
    };
    if (steps > 0) {
        fetch(0, 0);
        if (tid < QRY_TILE) {
            LDs[0][0][tid] = lnext;
            LDs[0][1][tid] = dnext;
        }
    }
    for (int s = 0; s < steps; ++s) {
        const int m0 = (qt0 + s % (nqt - qt0)) * QRY_TILE;
        const int buf = s & 1;
        // tile s has landed for every wave (and, at s = 0, K and V are
        // stored); every wave is done with buffer buf ^ 1 (tile s - 1)
        phase_barrier(true);
        if (s + 1 < steps) fetch(s + 1, buf ^ 1);
        const uint16_t* Qs = QOs + buf * QRY_TILE * D;
        const uint16_t* Os = QOs + (2 + buf) * QRY_TILE * D;
        const float* Ls = LDs[buf][0];
        const float* Ds = LDs[buf][1];
        auto publish_next = [&]() __attribute__((always_inline)) {
            if (s + 1 < steps && tid < QRY_TILE) {
                LDs[buf ^ 1][0][tid] = lnext;
                LDs[buf ^ 1][1][tid] = dnext;
            }
        };
        const int qb = m0 + xh * 32;  // first query of this wave's block
        // unless every query of the block is before every key of the wave
        if (!CAUSAL || qb + 31 >= n0 + kq * 32) {
            f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 aq = *(const bf16x8*)(Qs + roff[ks]);
                const bf16x8 ao = *(const bf16x8*)(Os + roff[ks]);
                const bf16x8 bk = *(const bf16x8*)(Ks + koff[ks]);
                const bf16x8 bv = *(const bf16x8*)(Vs + koff[ks]);
                sacc = mfma32x32x16(aq, bk, sacc);
                dpacc = mfma32x32x16(ao, bv, dpacc);
            }
            // row r of the accumulators: query qb + 8(r/4) + 4g + r%4, masked
            // (causal) when its offset 8(r/4) + r%4 is below lo
            const int lo = key - qb - 4 * g;
            f32x16 pv, dsv;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int rl = xh * 32 + q4 * 8 + g * 4;
                const f32x4 l4 = *(const f32x4*)(Ls + rl);
                const f32x4 d4 = *(const f32x4*)(Ds + rl);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = q4 * 4 + e;
                    float pr = fast_exp2(fmaf(sacc[r], c, -l4[e]));
                    if (CAUSAL && q4 * 8 + e < lo) pr = 0.f;
                    pv[r] = pr;
                    dsv[r] = pr * (dpacc[r] - d4[e]);
                }
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const bf16x8 pb = pack8(pv, half);
                const bf16x8 db8 = pack8(dsv, half);
                const int kblk = xh * 2 + half;  // 16-query block of the tile
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dvacc[db] = mfma32x32x16(tr.read(Os, kblk, db), pb, dvacc[db]);
                    dkacc[db] = mfma32x32x16(tr.read(Qs, kblk, db), db8, dkacc[db]);
                }
            }
        }
        publish_next();
    }

    // waves 4-7 hand their partial sums to waves 0-3: dV^T, then dK^T,
    // through the K/V area (4 waves x DB x 16 x 64 floats = 32 KB at D = 128)
    float* red = (float*)KVs;
    static_assert(4 * DB * 16 * 64 * 4 <= 2 * KEYS_WG * D * 2, "reduction area fits");
    // (the last tile's K/V reads end before the first barrier below)
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        f32x16* acc = pass == 0 ? dvacc : dkacc;
        __syncthreads();  // last reads of the area done
        if (xh == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) red[((kq * DB + db) * 16 + e) * 64 + lane] = acc[db][e];
        }
        __syncthreads();
        if (xh == 0) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[db][e] += red[((kq * DB + db) * 16 + e) * 64 + lane];
        }
    }
    if (xh == 0 && key < S) {
        uint16_t* dkr = p.dk + ((int64_t)bg * S + key) * D;
        uint16_t* dvr = p.dv + ((int64_t)bg * S + key) * D;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = db * 32 + j * 8 + g * 4;
                *(u32x2*)(dkr + d0) = u32x2{pack_bf16x2(dkacc[db][4 * j] * sc, dkacc[db][4 * j + 1] * sc),
                                            pack_bf16x2(dkacc[db][4 * j + 2] * sc, dkacc[db][4 * j + 3] * sc)};
                *(u32x2*)(dvr + d0) = u32x2{pack_bf16x2(dvacc[db][4 * j], dvacc[db][4 * j + 1]),
                                            pack_bf16x2(dvacc[db][4 * j + 2], dvacc[db][4 * j + 3])};
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = (b, h, 128-query tile), longest (last) tiles first; wave w
// owns queries m0 + 32w .. +31 (lane l32 = query).  Sweeps 64-key tiles,
// which reach LDS by global_load_lds_dwordx4 (no register staging) into two
// buffers: tile t+1 is in flight while tile t is multiplied, with one
// barrier per tile.
// ---------------------------------------------------------------------------
// At most 256 registers, so two waves share each SIMD (measured 16% faster
// overall than one wave per SIMD).

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(BwdParams p) {
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    __shared__ __attribute__((aligned(1024))) uint16_t KVs[4 * KEY_TILE * D];  // K(buf 0), K(buf 1), V(0), V(1)
    auto Kbuf = [&](int t) __attribute__((always_inline)) { return KVs + (t & 1) * KEY_TILE * D; };
    auto Vbuf = [&](int t) __attribute__((always_inline)) { return KVs + (2 + (t & 1)) * KEY_TILE * D; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the DMA's LDS address is scalar
    const int l32 = lane & 31, g = lane >> 5;
    const uint32_t L = xcd_remap(blockIdx.x, p.total);
    const int bh = (int)(L / (uint32_t)p.ntiles);
    const int tile = p.ntiles - 1 - (int)(L % (uint32_t)p.ntiles);
    const int b = bh / p.Hq, h = bh % p.Hq, kvh = h / p.group;
    const int S = p.S;
    const int m0 = tile * QRY_WG;
    const int qw = m0 + wave * 32;  // first query of this wave
    const int qi = qw + l32;
    const int64_t rowb = (int64_t)bh * S;
    const uint16_t* kb = p.k + ((int64_t)b * p.Hkv + kvh) * S * D;
    const uint16_t* vb = p.v + ((int64_t)b * p.Hkv + kvh) * S * D;

    bf16x8 qreg[KS], oreg[KS];  // B operands: column = this lane's query, k = d
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
        if (qi < S) {
            a = *(const u32x4*)(p.q + (rowb + qi) * D + ks * 16 + g * 8);
            c = *(const u32x4*)(p.dout + (rowb + qi) * D + ks * 16 + g * 8);
        }
        qreg[ks] = as_bf16x8(a);
        oreg[ks] = as_bf16x8(c);
    }
    const float l2 = qi < S ? p.lse[rowb + qi] * kLog2e : INFINITY;
    const float dl = qi < S ? p.delta[rowb + qi] : 0.f;
    int roff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[ks] = SwzTile<D>::at(l32, (2 * ks + g) * 8);
    TrOffsets<D> tr;
    tr.init(lane);

    f32x16 dqacc[DB];  // dQ^T: rows d, column = query
#pragma unroll
    for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

    const int qlast = min(m0 + QRY_WG, S) - 1;
    const int nkt = CAUSAL ? qlast / KEY_TILE + 1 : (S + KEY_TILE - 1) / KEY_TILE;
    const float c = p.c;
    SwzDma<D, NT / 64> dma;
    dma.init(wave, lane);
    dma.issue(kb, 0, S, Kbuf(0), wave);
    dma.issue(vb, 0, S, Vbuf(0), wave);
    for (int t = 0; t < nkt; ++t) {
        const int k0 = t * KEY_TILE;
        // tile t has landed for every wave, and every wave is done with the
        // buffers of tile t-1, which tile t+1 now fills
        phase_barrier(true);
        if (t + 1 < nkt) {
            dma.issue(kb, k0 + KEY_TILE, S, Kbuf(t + 1), wave);
            dma.issue(vb, k0 + KEY_TILE, S, Vbuf(t + 1), wave);
        }
        const uint16_t* Ks = Kbuf(t);
        const uint16_t* Vs = Vbuf(t);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int kb0 = k0 + sb * 32;
            if (CAUSAL && kb0 > qw + 31) continue;  // every key after every query of the wave
            f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ak = *(const bf16x8*)(Ks + sb * 32 * D + roff[ks]);
                const bf16x8 av = *(const bf16x8*)(Vs + sb * 32 * D + roff[ks]);
                sacc = mfma32x32x16(ak, qreg[ks], sacc);
                dpacc = mfma32x32x16(av, oreg[ks], dpacc);
            }
            // row r: key kb0 + 8(r/4) + 4g + r%4, masked when its offset
            // 8(r/4) + r%4 passes hi (past this lane's query or past S)
            const int hi = (CAUSAL ? min(qi, S - 1) : S - 1) - kb0 - 4 * g;
            f32x16 dsv;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pr = fast_exp2(fmaf(sacc[r], c, -l2));
                if (8 * (r >> 2) + (r & 3) > hi) pr = 0.f;
                dsv[r] = pr * (dpacc[r] - dl);
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const bf16x8 db8 = pack8(dsv, half);
#pragma unroll
                for (int db = 0; db < DB; ++db) dqacc[db] = mfma32x32x16(tr.read(Ks, sb * 2 + half, db), db8, dqacc[db]);
            }
        }
    }
    if (qi < S) {
        uint16_t* r = p.dq + (rowb + qi) * D;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = db * 32 + j * 8 + g * 4;
                *(u32x2*)(r + d0) = u32x2{pack_bf16x2(dqacc[db][4 * j] * sc, dqacc[db][4 * j + 1] * sc),
                                          pack_bf16x2(dqacc[db][4 * j + 2] * sc, dqacc[db][4 * j + 3] * sc)};
            }
        }
    }
}

template <typename K>
hipError_t launch(K kernel, uint32_t grid, const BwdParams& prm, hipStream_t stream, int threads = NT) {
    BwdParams arg = prm;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)kernel, dim3(grid), dim3(threads), args, 0, stream);
}

template <typename K>
hipError_t launch_delta(K kernel, int64_t rows, int rpb, const BwdParams& prm, hipStream_t stream) {
    BwdParams arg = prm;
    int64_t n = rows;
    void* args[] = {&arg, &n};
    return hipLaunchKernel((const void*)kernel, dim3((uint32_t)((rows + rpb - 1) / rpb)), dim3(NT), args, 0, stream);
}

template <int D>
hipError_t run(BwdParams prm, const BwdArgs& a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.S;
    hipError_t e = launch_delta(&bwd_delta_kernel<D>, rows, NT / (D / 8), prm, stream);
    if (e != hipSuccess) return e;
    prm.ntiles = (a.S + KEYS_WG - 1) / KEYS_WG;
    prm.total = (uint32_t)((int64_t)a.B * a.Hkv * prm.ntiles);
    e = a.causal ? launch(&bwd_dkdv_kernel<D, true>, prm.total, prm, stream, NT2)
                 : launch(&bwd_dkdv_kernel<D, false>, prm.total, prm, stream, NT2);
    if (e != hipSuccess) return e;
    prm.ntiles = (a.S + QRY_WG - 1) / QRY_WG;
    prm.total = (uint32_t)((int64_t)a.B * a.Hq * prm.ntiles);
    return a.causal ? launch(&bwd_dq_kernel<D, true>, prm.total, prm, stream)
                    : launch(&bwd_dq_kernel<D, false>, prm.total, prm, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
    BwdParams prm;
    prm.q = (const uint16_t*)a.q;
    prm.k = (const uint16_t*)a.k;
    prm.v = (const uint16_t*)a.v;
    prm.out = (const uint16_t*)a.out;
    prm.dout = (const uint16_t*)a.dout;
    prm.lse = a.lse;
    prm.dq = (uint16_t*)a.dq;
    prm.dk = (uint16_t*)a.dk;
    prm.dv = (uint16_t*)a.dv;
    prm.delta = a.delta;
    prm.B = a.B;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.S = a.S;
    prm.group = a.Hq / a.Hkv;
    prm.ntiles = 0;
    prm.total = 0;
    prm.c = a.scale * kLog2e;
    prm.scale = a.scale;
    prm.causal = a.causal;
    return a.D == 128 ? run<128>(prm, a, stream) : run<64>(prm, a, stream);
}

}  // namespace attn
