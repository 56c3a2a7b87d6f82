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
// Work decomposition (gfx950, wave64):
//   workgroup = 8 waves = 256 queries of one (batch, head); wave w owns 32.
//   The hardware puts waves w and w+4 on the same SIMD.
//   For each tile of BN = 64 keys a wave runs two phases:
//     M phase (matrix cores):  S(n+1)^T = K(n+1).Q^T and O^T += V(n)^T.P(n)^T,
//                      32 v_mfma_f32_32x32x16_bf16 with their LDS reads.
//     V phase (vector ALUs):   mask and row max of S(n), then
//                      p = 2^(s c - m c) (c = scale*log2(e)), row sums, and
//                      P(n) packed to bf16.
//   Waves 0-3 run one phase ahead of waves 4-7, with a workgroup barrier
//   after every phase, so on every SIMD one wave issues matrix products while
//   its partner does the softmax: the matrix cores and the vector ALUs work
//   at the same time instead of taking turns.
//   S^T (not S) is computed so that lane l holds one query (l % 32) and 16
//   keys: row max / row sum are in-lane plus one exchange with lane l ^ 32,
//   and P^T is directly the B operand of the second product.  V^T comes from
//   the row-major V tile through ds_read_b64_tr_b16, which hands each lane 4
//   keys of one d, in the key order of the S^T accumulator rows.
//   The reference max m only moves when some lane's sum of p over a tile
//   exceeds 2^12 (so every p stays <= 2^12, far from float32 overflow), so
//   rescaling O is rare.
//   Memory pipeline: K and V tiles go HBM -> LDS with global_load_lds_dwordx4
//   (no register staging), double-buffered, each in flight for two phases.
//   LDS rows are XOR-swizzled in 16-byte chunks so every operand read is free
//   of bank conflicts.
//   Causal: key tiles past the workgroup's last query are never loaded, a
//   wave skips the work of tiles past its own last query, and only tiles that
//   straddle the diagonal (or the end of the sequence) apply the mask.
//   Causal workgroups start with the longest query tiles.  Grids whose
//   (head, query tile) items fill whole rounds of compute units run the
//   persistent form below instead: one workgroup per compute unit over a
//   fixed item list, the key/value stream running on across items.
//   Sliding window (LOCAL): key tiles before every query's window are
//   skipped like tiles past the diagonal, and the visible ones run in a
//   rotated order so that query tiles that start together read each key
//   tile they share at the same time, through the XCD's L2.
//   Block mask (one flag per 64 queries x 64 keys): each wave group (two
//   64-query blocks) first lists the key tiles either of its blocks may see,
//   and streams that list through K/V buffers of its own in the same phase
//   schedule; a wave gives P = 0 to the listed tiles its own block may not
//   see, and skips their products when the next tile does not need them.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"
#include "lds_tiles.h"

namespace attn {
namespace {

constexpr int BM = 256;   // queries per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int NW = 8;     // waves per workgroup (two per SIMD)
constexpr int NT = NW * 64;
constexpr float kMaxTileSum = 4096.0f;  // bound on one lane tile sum of p (so p <= 2^12)
constexpr int kMaskBlock = 64;          // block-mask granularity (queries and keys); == BN
constexpr int kMaxMaskTiles = 2048;     // key tiles a block-masked launch may have (S <= 131072)
static_assert(kMaskBlock == BN && BM % kMaskBlock == 0 && BM / kMaskBlock <= 8, "mask blocks vs tiles");

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    float* lse;
    int Hq, Hkv, S, group, nq;
    uint32_t total;
    uint32_t hgrp;  // causal: heads whose tiles one XCD runs together (0: plain order)
    float c;        // scale * log2(e), > 0
    int window;     // LOCAL: keys each query sees (its own and window - 1 before it)
    // BLOCK: flag (b, h, qb, kb) at bmask[b * bm_sb + h * bm_sh + qb * nkb + kb]
    const uint8_t* bmask;
    int64_t bm_sb, bm_sh;
    int nkb;
    // optional: kStampWords words per workgroup (see WgStamp)
    uint64_t* stamps;
};

// Per-workgroup record of a stamped launch, written by lane 0 of wave 0:
// shader-clock counter and 100 MHz real-time counter when the workgroup
// starts and when that wave has stored its output, the hardware placement
// registers, and the (batch * head, query tile) it ran.
struct WgStamp {
    uint64_t t0, r0;
    __device__ __forceinline__ void start() {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    __device__ __forceinline__ void finish(uint64_t* all, int bh, int tile) const {
        const uint64_t t1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        uint64_t* s = all + (uint64_t)blockIdx.x * kStampWords;
        s[0] = t0;
        s[1] = r0;
        s[2] = t1;
        s[3] = r1;
        s[4] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID: wave, SIMD, CU, shader array, engine
        s[5] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID: which of the 8 dies
        s[6] = (uint64_t)bh;
        s[7] = (uint64_t)tile;
    }
};

// Workgroups one XCD holds at once: 32 CUs per XCD, one 8-wave workgroup per CU.
constexpr int kSlotsPerXcd = 32;
// Grids of at most this many 256-query workgroups (one per CU) take the
// key-split form: their time is the longest workgroup's.
constexpr int64_t kSplitMaxWorkgroups = 8 * kSlotsPerXcd;

// LDS tile layout: BN rows x D bf16, 16-byte chunks.  Chunk c of row r sits
// at chunk position r*CPR + (c ^ swizzle(r)).
template <int D>
struct Tile {
    static constexpr int CPR = D / 8;                 // chunks per row
    static constexpr int BYTES = BN * D * 2;          // 16 KB (D=128) / 8 KB (D=64)
    // K: the 16 rows one operand read touches per 16-lane phase land on 16
    // different bank groups (rows of 128 bytes alternate bank halves).
    __device__ static int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    // V: the 4 rows one transposed read touches per 16-lane phase land on 4
    // different 64-byte bank groups.
    __device__ static int vswz(int r) { return 4 * (D == 128 ? (r & 3) : ((r >> 1) & 1)); }
};

// Per-lane source offsets of the DMA of one K or V tile.  Instruction i of
// wave w fills LDS chunk positions p = (w*PER + i)*64 + lane; position p holds
// chunk c = (p % CPR) ^ swizzle(r) of tile row r = p / CPR, so the lane fetches
// byte offset r*2D + 16c from the tile's first row.
template <int D, bool IS_V, int NWV = NW>
struct DmaPlan {
    using T = Tile<D>;
    static constexpr int PER = T::BYTES / 1024 / NWV;  // 1 KB instructions per wave and tile
    uint32_t off[PER];
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int p = (wave * PER + i) * 64 + lane;
            const int r = p / T::CPR;
            const int c = (p % T::CPR) ^ (IS_V ? T::vswz(r) : T::kswz(r));
            off[i] = (uint32_t)(r * D * 2 + c * 16);
        }
    }
    // Rows of a tile whose first row is at tb into LDS at byte address l0 (the
    // whole tile's), this wave's share; with full = false, rows past row
    // `last` of the tile repeat that row.
    __device__ __forceinline__ void issue_at(const uint16_t* tb, bool full, int last, uint32_t l0, int wave) const {
        const uint32_t lw = l0 + (uint32_t)(wave * PER) * 1024u;
        if (full) {
#pragma unroll
            for (int i = 0; i < PER; ++i) dma16(tb, off[i], lw + i * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int r = (int)(off[i] / (D * 2));
                dma16(tb, off[i] - (uint32_t)((r - min(r, last)) * D * 2), lw + i * 1024);
            }
        }
    }
    // rows n0 .. n0+BN-1 of the head starting at base; rows past the end of
    // the sequence repeat row S-1 (those keys are masked and their P is 0)
    __device__ __forceinline__ void issue(const uint16_t* base, int n0, int S, char* tile, int wave) const {
        const uint16_t* tb = base + (int64_t)n0 * D;
        const uint32_t l0 = lds_addr(tile) + (uint32_t)(wave * PER) * 1024u;
        if (n0 + BN <= S) {
#pragma unroll
            for (int i = 0; i < PER; ++i) dma16(tb, off[i], l0 + i * 1024);
        } else {
            const int last = S - 1 - n0;  // last valid row of this tile
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int r = (int)(off[i] / (D * 2));
                const uint32_t o = off[i] - (uint32_t)((r - min(r, last)) * D * 2);
                dma16(tb, o, l0 + i * 1024);
            }
        }
    }
};

// LOCAL (with CAUSAL): sliding window, query i sees keys i - window + 1 .. i.
// The workgroup starts at the first key tile its first query sees; a wave
// skips the tiles before its own window (the phases still run, so the
// schedule is the causal one), and tiles that straddle a window's left edge
// are masked like the diagonal.
// BLOCK: the loop runs over positions 0 .. npos-1 of the workgroup's list of
// key tiles (tile number and one flag per query block); buffers alternate by
// position.  Otherwise position n is tile n.
// SPLIT (grids too small to fill the chip with 256-query workgroups): a
// workgroup takes 128 queries; waves w and w+4 take the same 32 queries,
// waves 0-3 the first half of the key tiles and waves 4-7 the second half,
// each group with its own K/V buffers, in the same phase schedule.  At the
// end waves 4-7 hand their (m, l, O) to their partners through LDS, which
// merge them (the split-KV combination: both scaled to the larger m).  The
// longest workgroup then runs half as many tiles.
template <int D, bool CAUSAL, bool LOCAL, bool BLOCK, bool SPLIT>
__global__ __launch_bounds__(NT) void fwd_bf16_kernel(Params p) {
    static_assert(!LOCAL || CAUSAL, "a sliding window is a causal mask");
    static_assert(!(LOCAL && BLOCK), "one mask kind at a time");
    static_assert(!SPLIT || (!LOCAL && !BLOCK), "the key split is for plain (causal or full) attention");
    constexpr int BMK = SPLIT ? BM / 2 : BM;  // queries per workgroup
    using T = Tile<D>;
    constexpr int KS = D / 16;  // k-steps of the Q.K^T product
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    constexpr int ROWB = T::CPR * 16;  // bytes per tile row
    // SPLIT and BLOCK: each wave group streams its own key tiles
    constexpr bool GBUF = SPLIT || BLOCK;
    __shared__ __attribute__((aligned(1024))) char smem[(GBUF ? 8 : 4) * T::BYTES];
    // BLOCK: one list of key tiles per wave group, the tiles that one of its
    // two query blocks may see (bits 0-23 tile, bit 24 + j: query block j of
    // the workgroup may see it)
    constexpr int LSTRIDE = kMaxMaskTiles + 2;
    __shared__ uint32_t blist[BLOCK ? 2 * LSTRIDE : 1];
    __shared__ int bcount[BLOCK ? 2 * NW : 1];
    // K buffers at [0, 2*BYTES), V buffers at [2*BYTES, 4*BYTES) (SPLIT and
    // BLOCK: one such set per wave group)
    const int gofs = GBUF ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 8) * 4 * T::BYTES : 0;
    auto Kbuf = [&](int i) __attribute__((always_inline)) { return smem + gofs + (i & 1) * T::BYTES; };
    auto Vbuf = [&](int i) __attribute__((always_inline)) { return smem + gofs + (2 + (i & 1)) * T::BYTES; };

    const int tid = threadIdx.x;
    const bool stamping = p.stamps != nullptr && tid == 0;
    WgStamp stamp;
    if (stamping) stamp.start();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;  // 0: waves 0-3 (one phase ahead), 1: waves 4-7
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const uint32_t L = xcd_remap(blockIdx.x, p.total);
    int bh, tile;
    if (CAUSAL) {
        if (p.hgrp > 0 && blockIdx.x < p.total / 8u * 8u) {
            // Each XCD's range is cut into groups of hgrp heads whose tiles
            // together fill the XCD; inside a group the longest tiles go
            // first.  All tiles of a group start together and read the same
            // K/V tiles in step, and the next group's long tiles take the CUs
            // its short tiles free, so every CU ends up with the same work.
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
    const int b = bh / p.Hq;
    const int h = bh % p.Hq;
    const int kvh = h / p.group;
    const int S = p.S;
    const int m0 = tile * BMK;

    const int64_t row0 = (int64_t)bh * S;
    const uint16_t* qb = p.q + row0 * D;
    const int64_t kvrow0 = ((int64_t)b * p.Hkv + kvh) * S;
    const uint16_t* kb = p.k + kvrow0 * D;
    const uint16_t* vb = p.v + kvrow0 * D;

    const int qwmin = m0 + (SPLIT ? (wave & 3) : wave) * 32;
    const int qwmax = qwmin + 31;
    const int qi = qwmin + l32;

    const int qlast = min(m0 + BMK, S) - 1;
    const int ntiles = (S + BN - 1) / BN;
    const int nall = CAUSAL ? min(ntiles, qlast / BN + 1) : ntiles;  // key tiles of the workgroup
    // SPLIT: each group runs nend positions; group 1's position n is tile
    // toff + n, which may lie past the last tile (an idle position)
    int nend = SPLIT ? (nall + 1) / 2 : nall;
    const int toff = SPLIT && grp ? nend : 0;
    const int nbeg = LOCAL ? max(0, m0 - p.window + 1) / BN : 0;
    // LOCAL: the workgroup's key tiles nbeg .. nend-1 run in rotated order,
    // position nbeg + i taking tile nbeg + (i + rot) mod cnt with rot such
    // that the tile is congruent to i modulo cnt.  Workgroups whose windows
    // have the same length (all but the first few query tiles) and that
    // start together then read the same key tile at the same time wherever
    // their windows overlap, so their K/V reads meet in the XCD's L2 (in
    // ascending order neighbouring query tiles would be four tiles apart).
    const int lcnt = LOCAL ? nend - nbeg : 1;
    const int lrot = LOCAL ? (lcnt - nbeg % lcnt) % lcnt : 0;

    if (BLOCK) {
        // For each wave group, list the tiles below nend that one of its two
        // query blocks may see, in order: flags per thread, then a ballot /
        // popcount compaction per list.  Both groups then run max(count)
        // positions; the shorter list is padded with entries that name no
        // tile (never valid) and no query block.
        const int qb0 = m0 / kMaskBlock;
        const int nqb = min(BM / kMaskBlock, (S - m0 + kMaskBlock - 1) / kMaskBlock);
        const uint8_t* mrow = p.bmask + (int64_t)b * p.bm_sb + (int64_t)h * p.bm_sh + (int64_t)qb0 * p.nkb;
        int base[2] = {0, 0};
        for (int t0 = 0; t0 < nend; t0 += NT) {
            const int t = t0 + tid;
            uint32_t bits = 0;
            if (t < nend) {
#pragma unroll
                for (int j = 0; j < BM / kMaskBlock; ++j)
                    if (j < nqb && mrow[(int64_t)j * p.nkb + t]) bits |= 1u << j;
            }
            int within[2];
#pragma unroll
            for (int gl = 0; gl < 2; ++gl) {
                const uint64_t bal = __builtin_amdgcn_ballot_w64(((bits >> (2 * gl)) & 3u) != 0);
                within[gl] = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                if (lane == 0) bcount[gl * NW + wave] = __builtin_popcountll(bal);
            }
            __syncthreads();
#pragma unroll
            for (int gl = 0; gl < 2; ++gl) {
                int before = 0, total = 0;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const int cw = bcount[gl * NW + w];
                    before += w < wave ? cw : 0;
                    total += cw;
                }
                if ((bits >> (2 * gl)) & 3u) blist[gl * LSTRIDE + base[gl] + before + within[gl]] = (uint32_t)t | (bits << 24);
                base[gl] += total;
            }
            __syncthreads();
        }
        nend = max(base[0], base[1]);
#pragma unroll
        for (int gl = 0; gl < 2; ++gl)
            for (int i = base[gl] + tid; i < nend + 2; i += NT) blist[gl * LSTRIDE + i] = 0xffffffu;
        __syncthreads();
        if (nend == 0) {  // no key visible to any query of this workgroup
            if (qi < S) {
                uint16_t* orow = p.out + (row0 + qi) * D;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int j = 0; j < 4; ++j) *(u32x2*)(orow + db * 32 + j * 8 + g * 4) = u32x2{0u, 0u};
                if (p.lse && g == 0) p.lse[row0 + qi] = -INFINITY;
            }
            if (stamping) stamp.finish(p.stamps, bh, tile);
            return;
        }
    }
    // Entry of position n (BLOCK: the list entry; otherwise n itself), read
    // once per loop iteration; the key tile it names, and whether this wave's
    // query block may see that tile.
    auto ent = [&](int n) __attribute__((always_inline)) {
        if (LOCAL) {
            int i = n - nbeg + lrot;  // < 2 lcnt + 2 for the positions the loop names
            i -= i >= lcnt ? lcnt : 0;
            i -= i >= lcnt ? lcnt : 0;
            return (uint32_t)(nbeg + i);
        }
        return BLOCK ? __builtin_amdgcn_readfirstlane(blist[grp * LSTRIDE + n]) : (uint32_t)(n + toff);
    };
    auto tile_of = [&](uint32_t e) __attribute__((always_inline)) { return BLOCK ? (int)(e & 0xffffffu) : (int)e; };
    // SPLIT, BLOCK: the position names a tile of the workgroup (BLOCK's
    // padding entries name none)
    auto valid = [&](uint32_t e) __attribute__((always_inline)) { return !GBUF || tile_of(e) < nall; };
    auto wave_sees = [&](uint32_t e) __attribute__((always_inline)) {
        return !BLOCK || ((e >> (24 + wave / 2)) & 1u) != 0;
    };

    // ---- prologue: K(nbeg), V(nbeg), K(nbeg+1) in flight while Q is loaded --
    const int dw = GBUF ? (wave & 3) : wave;  // wave's share of its group's tile loads
    DmaPlan<D, false, GBUF ? NW / 2 : NW> kdma;
    DmaPlan<D, true, GBUF ? NW / 2 : NW> vdma;
    kdma.init(dw, lane);
    vdma.init(dw, lane);
    if (valid(ent(nbeg))) {
        kdma.issue(kb, tile_of(ent(nbeg)) * BN, S, Kbuf(nbeg), dw);
        vdma.issue(vb, tile_of(ent(nbeg)) * BN, S, Vbuf(nbeg), dw);
    }
    if (nbeg + 1 < nend && valid(ent(nbeg + 1))) kdma.issue(kb, tile_of(ent(nbeg + 1)) * BN, S, Kbuf(nbeg + 1), dw);

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
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    // Running reference max of query qi in scaled log2 units (m * c).  It
    // starts at a finite -1e30 rather than -inf so that no exponent argument
    // is ever inf - inf (this file is built without NaN semantics): on the
    // first tile every unmasked p overflows to +inf, which the tile-sum check
    // catches, and masked ones give 2^-inf = 0.
    float mc = -1e30f;
    float lrow = 0.f;        // running sum of p over this lane's keys
    f32x16 sacc[2];          // S^T of the tile in flight (two 32-key blocks)
    bf16x8 pb[4];            // P^T of the tile in flight, bf16 (four 16-key blocks)

    // S^T = K.Q^T for the tile in Kt.  Operands are read two products ahead;
    // the scheduling fences stop the compiler from hoisting further reads
    // (which would only raise register pressure).
    auto qk = [&](const char* Kt) __attribute__((always_inline)) {
        constexpr int NP = 2 * KS;  // products: (ks, sb) pairs
        auto rd = [&](int i) __attribute__((always_inline)) { return *(const bf16x8*)(Kt + koff[i >> 1] + (i & 1) * 32 * ROWB); };
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
        bf16x8 a0 = rd(0), a1 = rd(1);
#pragma unroll
        for (int i = 0; i < NP; i += 2) {
            bf16x8 n0, n1;
            if (i + 2 < NP) {
                n0 = rd(i + 2);
                n1 = rd(i + 3);
            }
            sacc[0] = mfma32x32x16(a0, qreg[i >> 1], sacc[0]);
            sacc[1] = mfma32x32x16(a1, qreg[i >> 1], sacc[1]);
            __builtin_amdgcn_sched_barrier(0);
            a0 = n0;
            a1 = n1;
        }
    };

    // O^T += V^T . P^T ; 16-key block kb16 uses rows 16*kb16 .. +15 of the tile.
    // Same read-ahead scheme as qk: the next key block's operands are in flight
    // while the current one is multiplied.
    auto pv = [&](const char* Vt) __attribute__((always_inline)) {
        auto rd = [&](int i) __attribute__((always_inline)) {  // product i = (kb16, db) = (i / DB, i % DB)
            const char* base = Vt + voff[i % DB] + (i / DB) * 16 * ROWB;
            return tr_read_pair(base, base + 8 * ROWB);
        };
        constexpr int NP = 4 * DB;
        bf16x8 a0 = rd(0), a1 = rd(1);
#pragma unroll
        for (int i = 0; i < NP; i += 2) {
            bf16x8 n0, n1;
            if (i + 2 < NP) {
                n0 = rd(i + 2);
                n1 = rd(i + 3);
            }
            oacc[i % DB] = mfma32x32x16(a0, pb[i / DB], oacc[i % DB]);
            oacc[(i + 1) % DB] = mfma32x32x16(a1, pb[(i + 1) / DB], oacc[(i + 1) % DB]);
            __builtin_amdgcn_sched_barrier(0);
            a0 = n0;
            a1 = n1;
        }
    };

    // p = 2^(s c - m c) for the current reference m -> bf16 P^T operand; returns
    // this lane's sum of p.  The sum is taken on the float32 p with plain adds:
    // v_dot2_f32_bf16 on the packed P would run on the matrix cores and wait
    // behind the partner wave's products, whereas adds overlap them.  It
    // differs from the sum of the bf16-rounded weights by a relative 2^-8 at
    // most (bf16 keeps 8 significant bits; far less on average).
    // 16-key block kb16 = accumulator registers 8*(kb16&1).. of key block kb16>>1.
    auto exp_pack = [&](float mref) __attribute__((always_inline)) {
        float ps[4] = {0.f, 0.f, 0.f, 0.f};  // independent partial sums
#pragma unroll
        for (int kb16 = 0; kb16 < 4; ++kb16) {
            const int sb = kb16 >> 1, hh = kb16 & 1;
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(fmaf(sacc[sb][hh * 8 + 2 * e], c, -mref));
                const float p1 = fast_exp2(fmaf(sacc[sb][hh * 8 + 2 * e + 1], c, -mref));
                w[e] = pack_bf16x2(p0, p1);
                ps[e] += p0 + p1;
            }
            pb[kb16] = as_bf16x8(w);
        }
        return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };

    // Softmax of tile n0 against the running reference max m.  Fast path: the
    // exponentials with the current m.  The reference only has to keep p
    // bounded: when some lane's tile sum exceeds 2^12 (or is inf, as on the
    // first tile, where m starts at -1e30 and every visible p overflows) the
    // slow path takes the tile's row max
    // (exchanged between the two half-waves that share each query, so they keep
    // one reference), moves m, rescales O and l by 2^((m_old - m_new) c) and
    // redoes the exponentials, after which every p <= 1.
    auto softmax_impl = [&](int n0, auto may_mask) __attribute__((always_inline)) {
        if (may_mask && ((CAUSAL && n0 + BN - 1 > qwmin) || n0 + BN > S || (LOCAL && n0 <= qwmax - p.window))) {
            // register r of key block sb holds key n0 + 4g + kofs, kofs =
            // 32 sb + 8 (r / 4) + r % 4: masked when kofs passes hi (this
            // lane's query, or S - 1) or, LOCAL, when kofs <= lo (a key
            // before the row's window)
            const int hi = (CAUSAL ? min(qi, S - 1) : S - 1) - (n0 + g * 4);
            const int lo = LOCAL ? qi - p.window - (n0 + g * 4) : 0;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kofs = sb * 32 + (r >> 2) * 8 + (r & 3);
                    if (kofs > hi || (LOCAL && kofs <= lo)) sacc[sb][r] = -INFINITY;
                }
            }
        }
        float lt = exp_pack(mc);
        if (__builtin_amdgcn_ballot_w64(!(lt <= kMaxTileSum))) {
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = fmaxf(sacc[0][i], sacc[1][i]);
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                for (int i = 0; i < w; ++i) t[i] = fmaxf(t[i], t[i + w]);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[0]), __float_as_uint(t[0]), false, false);
            const float mnew = fmaxf(mc, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c);
            const float alpha = fast_exp2(mc - mnew);  // 0 on the first tile
            lrow *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            mc = mnew;
            lt = exp_pack(mc);
        }
        lrow += lt;
    };
    auto softmax = [&](int n0) __attribute__((always_inline)) { softmax_impl(n0, std::true_type{}); };

    auto active = [&](uint32_t e) __attribute__((always_inline)) {
        return valid(e) && (!CAUSAL || tile_of(e) * BN <= qwmax);
    };
    // LOCAL: the tile holds a key this wave's first query sees (tiles before
    // every query's window are skipped, like tiles past the diagonal)
    auto in_window = [&](uint32_t e) __attribute__((always_inline)) {
        return !LOCAL || tile_of(e) * BN + BN - 1 > qwmin - p.window;
    };

    phase_barrier(true);

    // M(n), n >= 0: S(n+1) = K(n+1).Q^T and O += P(n).V(n) as one software
    // pipeline of 2*KS + 4*DB products whose LDS operands are read AHEAD
    // products in advance (the scheduling fences stop the compiler from
    // hoisting reads further, which would only cost registers).  One code
    // path: for the last tile the S(n+1) product reads the (stale, in-bounds)
    // other K buffer and its result is never used.
    auto mphase = [&](int n, uint32_t e0, uint32_t e1) __attribute__((always_inline)) {
        // P(n) is all zero for a tile this wave does not see: only S(n+1), if
        // it counts (LOCAL's rotated order puts such tiles anywhere; in
        // ascending order a tile past the diagonal is followed by no other)
        if (!active(e0) || (LOCAL && !in_window(e0))) {
            if (LOCAL && active(e1) && in_window(e1)) qk(Kbuf(n + 1));
            return;
        }
        // BLOCK: a listed tile this wave's block may not see has P = 0 (set in
        // the V phase); the phase runs only for the next tile's S product
        if (BLOCK && !wave_sees(e0) && !(active(e1) && wave_sees(e1))) return;
        constexpr int NQK = 2 * KS, NPV = 4 * DB, NP = NQK + NPV, AHEAD = 4;
        const char* Kt = Kbuf(n + 1);
        const char* Vt = Vbuf(n);
        auto rd = [&](int i) __attribute__((always_inline)) {
            if (i < NQK) return *(const bf16x8*)(Kt + koff[i >> 1] + (i & 1) * 32 * ROWB);
            const int j = i - NQK;  // (kb16, db) = (j / DB, j % DB)
            const char* base = Vt + voff[j % DB] + (j / DB) * 16 * ROWB;
            return tr_read_pair(base, base + 8 * ROWB);
        };
        __builtin_amdgcn_s_setprio(1);
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
        bf16x8 buf[AHEAD];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) buf[i] = rd(i);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const bf16x8 a = buf[i % AHEAD];
            if (i + AHEAD < NP) buf[i % AHEAD] = rd(i + AHEAD);
            if (i < NQK) {
                sacc[i & 1] = mfma32x32x16(a, qreg[i >> 1], sacc[i & 1]);
            } else {
                const int j = i - NQK;
                oacc[j % DB] = mfma32x32x16(a, pb[j / DB], oacc[j % DB]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // V(n): softmax of tile n (from S(n) of the previous M phase)
    // BLOCK: a listed tile this wave's block may not see gets P = 0
    auto vphase = [&](uint32_t e0) __attribute__((always_inline)) {
        if (active(e0) && in_window(e0)) {
            if (wave_sees(e0)) {
                softmax(tile_of(e0) * BN);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) pb[i] = bf16x8{};
            }
        }
    };
    // DMA of K(k+1) and V(k) at the start of phase 2k (k >= 1); ek, ek1 the
    // entries of positions k, k+1
    auto dma_step = [&](int k, uint32_t ek, uint32_t ek1) __attribute__((always_inline)) {
        if (k + 1 < nend && valid(ek1)) kdma.issue(kb, tile_of(ek1) * BN, S, Kbuf(k + 1), dw);
        if (k < nend && valid(ek)) vdma.issue(vb, tile_of(ek) * BN, S, Vbuf(k), dw);
    };

    // Phase schedule (barrier after every phase; odd phases also wait for the
    // tile DMA started at the preceding even phase):
    //   phase       0      2n+1    2n+2    ...  2nend+1
    //   group 0   M(-1)    V(n)    M(n)         -
    //   group 1     -      M(n-1)  V(n)         M(nend-1)
    // with M(n) and V(n) as above, so group 0 runs one phase ahead and on every
    // SIMD one wave issues matrix products while the other runs the softmax.
    // K(m) is read in phases 2m and 2m+1, V(m) in phases 2m+2 and 2m+3.  The
    // DMA of K(k+1) and V(k) starts at phase 2k into the buffers of K(k-1) and
    // V(k-2), whose last readers finished in phase 2k-1, and is awaited before
    // the barrier that ends phase 2k+1.
    if (grp == 0) {
        qk(Kbuf(nbeg));
        phase_barrier(false);
        for (int n = nbeg; n < nend; ++n) {
            const uint32_t e0 = ent(n), e1 = ent(n + 1), e2 = ent(n + 2);
            vphase(e0);
            phase_barrier(true);
            dma_step(n + 1, e1, e2);
            mphase(n, e0, e1);
            phase_barrier(false);
        }
        phase_barrier(true);
    } else {
        phase_barrier(false);
        qk(Kbuf(nbeg));
        phase_barrier(true);
        for (int n = nbeg; n < nend; ++n) {
            const uint32_t e0 = ent(n), e1 = ent(n + 1), e2 = ent(n + 2);
            dma_step(n + 1, e1, e2);
            vphase(e0);
            phase_barrier(false);
            mphase(n, e0, e1);
            phase_barrier(true);
        }
    }

    // ---- epilogue: O / l, lse ------------------------------------------------
    // O goes through this wave's share of the K/V buffers (idle after the last
    // barrier) so that the stores cover whole rows: the wave's 32 rows are
    // contiguous in out, and each store instruction writes 1 KB (D = 128) of
    // them instead of 8 bytes per lane in 32 different rows.
    if (SPLIT) {
        // waves 4-7 hand (m, l, O) to their partners above group 0's output
        // staging; the partners scale both halves to the larger m and add
        constexpr int STG = (NW / 2) * 32 * D * 2;  // group 0's staging area
        constexpr int WREG = DB * 16 * 64;          // floats of one wave's O
        static_assert(STG + (NW / 2) * (WREG + 128) * 4 <= 8 * T::BYTES, "merge area fits");
        float* mreg = (float*)(smem + STG) + (wave & 3) * (WREG + 128);
        if (grp == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) mreg[(db * 16 + r) * 64 + lane] = oacc[db][r];
            mreg[WREG + lane] = mc;
            mreg[WREG + 64 + lane] = lrow;
        }
        __syncthreads();
        if (grp == 1) return;
        const float m1 = mreg[WREG + lane], l1 = mreg[WREG + 64 + lane];
        const float mm = fmaxf(mc, m1);
        const float a0 = fast_exp2(mc - mm), a1 = fast_exp2(m1 - mm);  // 0 for a half that saw no key
        lrow = lrow * a0 + l1 * a1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = oacc[db][r] * a0 + mreg[(db * 16 + r) * 64 + lane] * a1;
        mc = mm;
    }
    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lrow), __float_as_uint(lrow), false, false);
    const float ltot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    // BLOCK: a query block that sees no listed tile has l = 0: out 0, lse -inf
    const bool seen = !BLOCK || ltot > 0.f;
    const float inv = seen ? 1.0f / ltot : 0.f;
    static_assert(NW * 32 * D * 2 <= 4 * T::BYTES, "staging fits the K/V buffers");
    store_rows_via_lds<D>(smem + wave * 32 * D * 2, oacc, inv, p.out + (row0 + qwmin) * D, S - qwmin, lane);
    if (qi < S && p.lse && g == 0) p.lse[row0 + qi] = seen ? (mc + __log2f(ltot)) * kLn2 : -INFINITY;
    if (stamping) stamp.finish(p.stamps, bh, tile);
}

// ---------------------------------------------------------------------------
// Persistent form (plain causal or full attention, S >= BM): one workgroup per
// compute unit runs a fixed list of (head, query tile) items back to back.
// The key/value tile stream and the two wave groups' phase schedule run on
// across item boundaries, so an item's start costs no pipeline fill: while
// the last tiles of one item are processed, the first key/value tiles of the
// next are already in flight, and its Q rows wait in LDS (each wave brings in
// its own 32 rows by LDS DMA during the previous item and copies them into
// registers at that item's last softmax phase).  The previous item's output
// is normalised and stored during the next item's first softmax phase.
//
// Items (R = rounds, G workgroups; the hardware deals workgroups round-robin
// over the 8 XCDs, so workgroup w runs on XCD w % 8):
// - causal, with (G/8) % nq == 0: item i of workgroup w = 8c + x is tile
//   j = c % nq (i even) or nq-1-j (i odd, key tiles in descending order) of
//   head (2R x + i) hpr + c / nq, hpr = (G/8) / nq.  Every workgroup runs
//   4 (nq + 1) key tiles per two items, and in each item round an XCD holds
//   all tiles of hpr heads: a head's items start together (ascending) or end
//   together (descending), so each head has one read front and its
//   key/value tiles are read once, in step, through the XCD's L2.
// - causal otherwise: unit j of a head = its tiles nq-1-j and j (the second
//   in descending order); full attention: unit j = tile j.  Workgroup w runs
//   unit (x R + r) G/8 + c in round r: an XCD's workgroups take consecutive
//   units, the tiles of a few heads.
struct PersistParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    float* lse;
    int Hq, Hkv, S, group, nq;
    int units;   // units per head (causal nq / 2, full nq)
    int rounds;  // units per workgroup
    int hpr;     // causal, > 0: heads per item round (see item_bh_tile); 0: pairs of one head
    int window;  // sliding window (LOCAL): keys q - window + 1 .. q
    float c;     // scale * log2(e), > 0
    uint64_t* stamps;
};

// A zero the compiler cannot see through.  Per-lane addresses used once per
// item (Q DMA, output staging) are derived from lane | opaque_zero() inside
// the loop, so they are computed where they are used instead of being
// hoisted out of the loop and held in registers for the whole kernel.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}
// The same for wave-uniform values: values used only at item boundaries are
// recomputed there from S | opaque_szero() instead of being held in scalar
// registers across the loop.
__device__ __forceinline__ int opaque_szero() {
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}

template <int D, bool CAUSAL, bool LOCAL = false>
__global__ __launch_bounds__(NT) void fwd_bf16_persist_kernel(PersistParams p) {
    static_assert(!LOCAL || CAUSAL, "a sliding window is a causal mask");
    using T = Tile<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int ROWB = T::CPR * 16;
    constexpr int QWB = 32 * D * 2;  // bytes of one wave's 32 Q rows
    constexpr int QPER = QWB / 1024; // its DMA instructions
    __shared__ __attribute__((aligned(1024))) char smem[4 * T::BYTES + NW * QWB];
    auto Kbuf = [&](int i) __attribute__((always_inline)) { return smem + (i & 1) * T::BYTES; };
    auto Vbuf = [&](int i) __attribute__((always_inline)) { return smem + (2 + (i & 1)) * T::BYTES; };

    const int tid = threadIdx.x;
    const bool stamping = p.stamps != nullptr && tid == 0;
    WgStamp stamp;
    if (stamping) stamp.start();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    char* const qst = smem + 4 * T::BYTES + wave * QWB;  // this wave's Q rows (K-tile layout)
    const int S = p.S;
    const int nitems = p.rounds * (CAUSAL && !LOCAL ? 2 : 1);
    const uint32_t G = gridDim.x;
    // XCD x (blockIdx % 8) runs units [x U/8, (x+1) U/8) of all U = rounds G:
    // consecutive heads, G/8 units per round

    // item i of this workgroup -> (b * Hq + h, query tile); key tiles it runs
    auto item_bh_tile = [&](int i, int& bh, int& tile) __attribute__((always_inline)) {
        const uint32_t w = blockIdx.x | (uint32_t)opaque_szero();
        if (LOCAL) {
            // item round i of XCD x: all nq tiles of hpr heads, workgroup c
            // tile (c + i nq / R) % nq: over its R items a workgroup meets
            // tiles spread over the sequence, so the short first tiles (whose
            // windows are cut by the sequence start) fall to different ones
            const int nq = p.nq, c = (int)(w / 8u);
            bh = ((int)(w % 8u) * p.rounds + i) * p.hpr + c / nq;
            tile = (c % nq + i * nq / p.rounds) % nq;
            return;
        }
        if (CAUSAL && p.hpr > 0) {
            // item round i of XCD x: its G/8 workgroups take all nq tiles of
            // hpr heads, workgroup c tile j = c % nq in even rounds and
            // nq-1-j in odd ones (descending), so each head has one read
            // front and every workgroup the same 4 (nq + 1) key tiles per
            // two rounds
            const int nq = p.nq, c = (int)(w / 8u), j = c % nq;
            bh = ((int)(w % 8u) * p.rounds * 2 + i) * p.hpr + c / nq;
            tile = (i & 1) ? nq - 1 - j : j;
            return;
        }
        const int r = CAUSAL ? i >> 1 : i;
        const uint32_t L = ((w % 8u) * (uint32_t)p.rounds + (uint32_t)r) * (G / 8u) + w / 8u;
        bh = (int)(L / (uint32_t)p.units);
        const int j = (int)(L % (uint32_t)p.units);
        tile = CAUSAL ? ((i & 1) ? j : p.nq - 1 - j) : j;
    };
    auto item_tiles = [&](int tile) __attribute__((always_inline)) {
        const int Sx = S | opaque_szero(), nt = (Sx + BN - 1) / BN;
        return CAUSAL ? min(nt, (min(tile * BM + BM, Sx) - 1) / BN + 1) : nt;
    };
    // LOCAL: an item's key tiles lbeg .. lend-1 (the window of its first
    // query to its diagonal), run in rotated order from tile lbeg + rot, the
    // one congruent to 0 modulo their count: the workgroups of a head that
    // start an item round together then read the same tile at the same time
    auto local_beg = [&](int tile_) __attribute__((always_inline)) {
        return max(0, tile_ * BM - (p.window | opaque_szero()) + 1) / BN;
    };
    auto local_first = [&](int beg, int cnt) __attribute__((always_inline)) { return beg + (cnt - beg % cnt) % cnt; };
    // The stream position: position k of the current item (nk key tiles,
    // head bh, query tile), at key tile kt, moving by dk; the next item's
    // head, query tile, key tile count and direction.  Every item has at
    // least 4 key tiles, so the two positions after the current one lie in
    // these two items.  The second item of a causal pair runs its key tiles
    // in descending order: pair j's second item starts when its first ends,
    // at a time that depends on j, but it then reads at every moment the
    // same key tile as the second items of the head's other pairs, so a
    // head's workgroups read at most two key tiles at a time (the ascending
    // and the descending front) and the XCD's L2 serves the other reads.
    int it = 0, k = 0, nk, bh, tile, kt = 0, dk = 1;  // the next item's direction: CAUSAL ? -dk : dk
    int lbeg = 0, lend = 0;  // LOCAL: the current item's key tiles
    int nbh = 0, ntile = 0;
    auto kv_of = [&](int bh_) __attribute__((always_inline)) {
        const int b = bh_ / p.Hq, h = bh_ % p.Hq;
        return ((int64_t)b * p.Hkv + h / p.group) * S * D;  // element offset of the head's key 0
    };
    item_bh_tile(0, bh, tile);
    nk = item_tiles(tile);
    if (LOCAL) {
        lbeg = local_beg(tile);
        lend = nk;
        nk = lend - lbeg;
        kt = local_first(lbeg, nk);
    }
    bool has_next = nitems > 1;
    if (has_next) item_bh_tile(1, nbh, ntile);
    // DMA sources: K of position n+2 and V of position n+1 (tile pointers
    // that move one tile per position, cstep bytes in the current item and
    // CAUSAL ? -cstep : cstep in the next, and jump to the next item's first
    // key tile at the crossing)
    constexpr int64_t TSTEP = (int64_t)BN * D;  // elements per key tile
    const int64_t kv0 = kv_of(bh);
    int64_t cstep = TSTEP * 2;
    // element offset of the next item's first key tile (the last one when it
    // runs in descending order)
    auto first_tile = [&]() __attribute__((always_inline)) {
        if (LOCAL) return kv_of(nbh);  // LOCAL: the next item's head; tiles are placed by index
        return kv_of(nbh) + (CAUSAL && dk > 0 ? (int64_t)(item_tiles(ntile) - 1) * TSTEP : 0);
    };
    int64_t knext = has_next ? first_tile() : 0;
    const char* kp = (const char*)(p.k + kv0 + 2 * TSTEP);
    const char* vp = (const char*)(p.v + kv0 + TSTEP);
    int64_t kvcur = kv0;  // LOCAL: the current item's head (element offset of key 0)
    auto advance_item = [&]() __attribute__((always_inline)) {
        ++it;
        bh = nbh;
        tile = ntile;
        nk = item_tiles(tile);
        if (CAUSAL && !LOCAL) {
            dk = -dk;
            cstep = -cstep;
        }
        k = 0;
        kt = dk < 0 ? nk - 1 : 0;
        if (LOCAL) {
            lbeg = local_beg(tile);
            lend = nk;
            nk = lend - lbeg;
            kt = local_first(lbeg, nk);
            kvcur = knext;
        }
        has_next = it + 1 < nitems;
        if (has_next) {
            item_bh_tile(it + 1, nbh, ntile);
            knext = first_tile();
        }
    };

    DmaPlan<D, false> kdma;
    DmaPlan<D, true> vdma;
    kdma.init(wave, lane);
    vdma.init(wave, lane);
    // DMA of this wave's 32 Q rows (first row r0 of head bh_) into qst, laid
    // out like a K tile (row r, chunk c at c ^ kswz(r)); rows past the end of
    // the sequence repeat row S - 1 (their results are never stored)
    auto q_dma = [&](int bh_, int tile_) __attribute__((always_inline)) {
        const int ln = lane | opaque_zero();  // offsets computed here, not held across the loop
        const int r0 = tile_ * BM + wave * 32;
        const uint16_t* base = p.q + ((int64_t)bh_ * S + min(r0, S - 1)) * D;
        const int last = S - 1 - min(r0, S - 1);  // last row of the 32 inside the sequence
        const uint32_t l0 = lds_addr(qst);
#pragma unroll
        for (int i = 0; i < QPER; ++i) {
            const int pos = i * 64 + ln;
            const int r = pos / T::CPR;
            const int cc = (pos % T::CPR) ^ T::kswz(r);
            dma16(base, (uint32_t)(min(r, last) * D * 2 + cc * 16), l0 + i * 1024);
        }
    };

    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = l32 * ROWB + (((2 * ks + g) ^ T::kswz(l32)) * 16);
    int voff[DB];
    {
        const int Gq = lane >> 4, j = lane & 15;
        const int r = 4 * (Gq >> 1) + (j >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d0 = db * 32 + (Gq & 1) * 16 + 4 * (j & 3);
            voff[db] = r * ROWB + (((d0 >> 3) ^ T::vswz(r)) * 16) + (d0 & 7) * 2;
        }
    }
    bf16x8 qreg[KS];
    // Q rows from LDS into the operand registers (once per item).
    auto q_read = [&]() __attribute__((always_inline)) {
        const int z = opaque_zero();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = *(const bf16x8*)(qst + (koff[ks] | z));
    };

    // ---- prologue: Q of the first item, K(0), V(0), K(1) ---------------------
    q_dma(bh, tile);
    {
        // LOCAL: the first two tiles of the rotated order
        const int t0 = LOCAL ? kt : 0, t1 = LOCAL ? (kt + 1 < lend ? kt + 1 : lbeg) : 1;
        kdma.issue(p.k + kv0, t0 * BN, S, Kbuf(0), wave);
        vdma.issue(p.v + kv0, t0 * BN, S, Vbuf(0), wave);
        kdma.issue(p.k + kv0, t1 * BN, S, Kbuf(1), wave);  // the item has 4 or more key tiles
    }
    phase_barrier(true);
    q_read();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    const float c = p.c;
    // the item whose softmax and output this wave is on
    int qwmin = tile * BM + wave * 32;
    int qi = qwmin + l32;
    int wbh = bh;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float mc = -1e30f;  // reference max (see fwd_bf16_kernel); finite, so no inf - inf
    float lrow = 0.f;
    f32x16 sacc[2];
    bf16x8 pb[4];

    auto qk = [&](const char* Kt) __attribute__((always_inline)) {
        constexpr int NP = 2 * KS;
        auto rd = [&](int i) __attribute__((always_inline)) { return *(const bf16x8*)(Kt + koff[i >> 1] + (i & 1) * 32 * ROWB); };
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
        bf16x8 a0 = rd(0), a1 = rd(1);
#pragma unroll
        for (int i = 0; i < NP; i += 2) {
            bf16x8 n0, n1;
            if (i + 2 < NP) {
                n0 = rd(i + 2);
                n1 = rd(i + 3);
            }
            sacc[0] = mfma32x32x16(a0, qreg[i >> 1], sacc[0]);
            sacc[1] = mfma32x32x16(a1, qreg[i >> 1], sacc[1]);
            __builtin_amdgcn_sched_barrier(0);
            a0 = n0;
            a1 = n1;
        }
    };
    auto pv = [&](const char* Vt) __attribute__((always_inline)) {
        auto rd = [&](int i) __attribute__((always_inline)) {
            const char* base = Vt + voff[i % DB] + (i / DB) * 16 * ROWB;
            return tr_read_pair(base, base + 8 * ROWB);
        };
        constexpr int NP = 4 * DB;
        bf16x8 a0 = rd(0), a1 = rd(1);
#pragma unroll
        for (int i = 0; i < NP; i += 2) {
            bf16x8 n0, n1;
            if (i + 2 < NP) {
                n0 = rd(i + 2);
                n1 = rd(i + 3);
            }
            oacc[i % DB] = mfma32x32x16(a0, pb[i / DB], oacc[i % DB]);
            oacc[(i + 1) % DB] = mfma32x32x16(a1, pb[(i + 1) / DB], oacc[(i + 1) % DB]);
            __builtin_amdgcn_sched_barrier(0);
            a0 = n0;
            a1 = n1;
        }
    };
    auto exp_pack = [&](float mref) __attribute__((always_inline)) {
        float ps[4];
#pragma unroll
        for (int kb16 = 0; kb16 < 4; ++kb16) {
            const int sb = kb16 >> 1, hh = kb16 & 1;
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(fmaf(sacc[sb][hh * 8 + 2 * e], c, -mref));
                const float p1 = fast_exp2(fmaf(sacc[sb][hh * 8 + 2 * e + 1], c, -mref));
                w[e] = pack_bf16x2(p0, p1);
                ps[e] = kb16 == 0 ? p0 + p1 : ps[e] + (p0 + p1);
            }
            pb[kb16] = as_bf16x8(w);
        }
        return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    // softmax of key tile n0 of the current item (see fwd_bf16_kernel);
    // masked: the tile has keys past this wave's diagonal or past the end
    auto softmax = [&](int n0, bool masked) __attribute__((always_inline)) {
        if (masked) {
            // accumulator register r of key block sb holds key n0 + kofs + 4g,
            // kofs = 32 sb + 8 (r / 4) + r % 4; it is masked when kofs > hi.
            // The sign of hi - kofs selects -inf bit by bit (v_bfi), so no
            // lane masks are held in scalar registers.
            // LOCAL: also masked when kofs <= lo (key before the row's window)
            const int hi = (CAUSAL ? min(qi, S - 1) : S - 1) - (n0 + g * 4);
            const int lo = LOCAL ? qi - p.window - (n0 + g * 4) : 0;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kofs = sb * 32 + (r >> 2) * 8 + (r & 3);
                    uint32_t m = (uint32_t)((hi - kofs) >> 31);  // all ones when masked
                    if (LOCAL) m |= (uint32_t)((kofs - lo - 1) >> 31);
                    sacc[sb][r] = __uint_as_float((__float_as_uint(sacc[sb][r]) & ~m) | (0xff800000u & m));
                }
            }
        }
        float lt = exp_pack(mc);
        if (__builtin_amdgcn_ballot_w64(!(lt <= kMaxTileSum))) {
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = fmaxf(sacc[0][i], sacc[1][i]);
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                for (int i = 0; i < w; ++i) t[i] = fmaxf(t[i], t[i + w]);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[0]), __float_as_uint(t[0]), false, false);
            const float mnew = fmaxf(mc, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c);
            const float alpha = fast_exp2(mc - mnew);
            lrow *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            mc = mnew;
            lt = exp_pack(mc);
        }
        lrow += lt;
    };
    // O / l and lse of the current item.  O goes through this wave's Q
    // staging area, which is free between the copy of the next item's Q into
    // the registers (last softmax phase of this item) and the DMA of the Q
    // after it (issued after this), so that every store writes whole rows.
    auto epilogue = [&]() __attribute__((always_inline)) {
        const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lrow), __float_as_uint(lrow), false, false);
        const float ltot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
        const int64_t row0 = (int64_t)wbh * S;
        store_rows_via_lds<D, 2>(qst, oacc, 1.0f / ltot, p.out + (row0 + qwmin) * D, S - qwmin, lane | opaque_zero());
        if (qi < S && p.lse && g == 0) p.lse[row0 + qi] = (mc + __log2f(ltot)) * kLn2;
    };
    // Per item and wave: last key tile this wave sees (kact) and first key
    // tile that needs the element mask (kmask: the diagonal tile under the
    // causal mask, the partial last tile of a ragged sequence).  Every row
    // of the wave sees the first key of each tile up to kact, so a
    // descending item's first tile already gives every row a finite max.
    // ncommon: number of positions k with 2 <= k < nk - 3 (the DMA's common
    // case: whole tiles in this item)
    // LOCAL: kwin, the first key tile holding a key of this wave's windows,
    // and kwfull, the first tile inside every row's window.
    int kact, kmask, ncommon, kwin = 0, kwfull = 0;
    auto set_limits = [&]() __attribute__((always_inline)) {
        kact = CAUSAL ? (qwmin + 31) / BN : nk - 1;
        const int Sx = S | opaque_szero();
        const int ktail = Sx / BN;  // the partial last key tile, or one past the last
        kmask = CAUSAL ? min((qwmin + 1) / BN, ktail) : ktail;
        ncommon = max(nk - 5, 0);
        if (LOCAL) {
            const int W = p.window | opaque_szero();
            kwin = max(qwmin - W + 1, 0) / BN;
            kwfull = (max(qwmin + 31 - W + 1, 0) + BN - 1) / BN;
        }
    };
    // LOCAL: this wave sees key tile t (it holds a key of one of its windows)
    auto sees = [&](int t) __attribute__((always_inline)) { return (unsigned)(t - kwin) <= (unsigned)(kact - kwin); };
    set_limits();
    // V phase of position (it, k).  The rare events are tested with one range
    // check: at an item's first tile (k = 0) the previous item's output goes
    // out and the state restarts; at its last tile (k = nk - 1) the next
    // item's Q rows (in LDS since two or more phases) go into the registers,
    // after this item's last S product (previous M phase) and before the next
    // one's first (next M phase).
    auto vphase = [&]() __attribute__((always_inline)) {
        if ((unsigned)(k - 1) >= (unsigned)(nk - 2)) {
            if (k == 0) {
                if (it > 0) {
                    epilogue();
                    qwmin = tile * BM + wave * 32;
                    qi = qwmin + l32;
                    wbh = bh;
                    set_limits();
#pragma unroll
                    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
                    mc = -1e30f;
                    lrow = 0.f;
                }
            } else if (has_next) {
                q_read();
            }
        }
        if (LOCAL ? sees(kt) : (!CAUSAL || kt <= kact)) {
            softmax(kt * BN, kt >= kmask || (LOCAL && kt < kwfull));
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) pb[i] = bf16x8{};  // see the M phase
        }
    };
    // DMA at the start of phase 2n+2: K of position n+2, V of position n+1,
    // and the next item's Q rows once the Q staging area is free: after the
    // previous item's output has gone through it, i.e. after the V phase of
    // the item's first tile (group 0 issues its DMA after that V phase, group
    // 1 before it, so group 1 takes the second tile).  Buffers alternate with
    // the position's parity: K buffer (n+2) & 1 = n & 1, V buffer (n+1) & 1.
    // Common case (2 <= k < nk - 3): both tiles and the next iteration's
    // inside this item, whole tiles, no Q DMA.
    const int qdma_k = grp;
    const uint32_t lbase = lds_addr(smem);
    uint32_t kb_off = 0;  // (n & 1) * tile bytes
    // LOCAL: key tile of position k + d (d = 1, 2) of the current item, or of
    // the next item's position k + d - nk, and its head
    auto local_pos = [&](int d, int& t, int64_t& hb) __attribute__((always_inline)) {
        if (k + d < nk) {
            t = kt + d;
            if (t >= lend) t -= nk;
            hb = kvcur;
        } else {
            const int nb = local_beg(ntile), nn = item_tiles(ntile) - nb;
            t = local_first(nb, nn) + (k + d - nk);
            if (t >= nb + nn) t -= nn;
            hb = knext;
        }
    };
    auto dma = [&]() __attribute__((always_inline)) {
        const uint32_t lk = lbase + kb_off;
        const uint32_t lv = lbase + 2u * T::BYTES + (kb_off ^ (uint32_t)T::BYTES);
        if (LOCAL) {
            // whole tiles (the sequence is a whole number of query tiles)
            int t;
            int64_t hb;
            if (k + 2 < nk || has_next) {
                local_pos(2, t, hb);
                kdma.issue_at(p.k + hb + (int64_t)t * TSTEP, true, 0, lk, wave);
            }
            if (k + 1 < nk || has_next) {
                local_pos(1, t, hb);
                vdma.issue_at(p.v + hb + (int64_t)t * TSTEP, true, 0, lv, wave);
            }
            if (k == qdma_k && has_next) q_dma(nbh, ntile);
        } else if ((unsigned)(k - 2) < (unsigned)ncommon) {
            kdma.issue_at((const uint16_t*)kp, true, 0, lk, wave);
            vdma.issue_at((const uint16_t*)vp, true, 0, lv, wave);
            kp += cstep;
            vp += cstep;
        } else {
            // key tiles of positions n+2 and n+1, in this item or the next
            const int kn = k + 2 - nk;
            const bool ndesc = CAUSAL && dk > 0;
            const int nnk = ndesc ? item_tiles(ntile) : 0;
            const int kk = kn < 0 ? kt + 2 * dk : (ndesc ? nnk - 1 - kn : kn);
            const int vk = k + 1 < nk ? kt + dk : (ndesc ? nnk - 1 : 0);
            if (k + 2 < nk || has_next)
                kdma.issue_at((const uint16_t*)kp, kk * BN + BN <= S, S - 1 - kk * BN, lk, wave);
            if (k + 1 < nk || has_next)
                vdma.issue_at((const uint16_t*)vp, vk * BN + BN <= S, S - 1 - vk * BN, lv, wave);
            if (k == qdma_k && has_next) q_dma(nbh, ntile);
            // sources of the next iteration (positions n+3 and n+2)
            const int64_t nstep = CAUSAL ? -cstep : cstep;
            kp = k + 3 < nk ? kp + cstep : (k + 3 == nk ? (const char*)(p.k + knext) : kp + nstep);
            vp = k + 2 < nk ? vp + cstep : (k + 2 == nk ? (const char*)(p.v + knext) : vp + nstep);
        }
        kb_off ^= (uint32_t)T::BYTES;
    };
    int np = 0;  // parity of the position: buffers of the M phase's reads
    // M phase of position (it, k): S of the next position and O += P V of
    // this one, as one software pipeline.  It runs when this wave sees key
    // tile kt, when it sees the next position's tile (a descending item's
    // position before the first tile the wave sees), or at an item's last
    // position when another item follows: a wave that does not see tile kt
    // has P = 0 (set in its V phase), so its product adds nothing.  An S
    // product nobody uses (a tile the wave does not see, or after the last
    // position, on the stale but in-bounds other buffer) is harmless.
    auto mphase = [&]() __attribute__((always_inline)) {
        if (LOCAL) {
            // the rotated order puts tiles this wave does not see anywhere:
            // the phase runs for this tile, or for the next one's S product
            if (!sees(kt) && !(k + 1 < nk ? sees(kt + 1 < lend ? kt + 1 : lbeg) : has_next)) return;
        } else if (CAUSAL && kt > kact - (dk >> 1) && !(k == nk - 1 && has_next)) {
            // descending items also need the M phase of the position before
            // the first tile the wave sees (kact + 1), for that tile's S product
            return;
        }
        __builtin_amdgcn_s_setprio(1);
        {
            constexpr int NQK = 2 * KS, NPV = 4 * DB, NP = NQK + NPV, AHEAD = 4;
            const char* Kt = Kbuf(np + 1);
            const char* Vt = Vbuf(np);
            auto rd = [&](int i) __attribute__((always_inline)) {
                if (i < NQK) return *(const bf16x8*)(Kt + koff[i >> 1] + (i & 1) * 32 * ROWB);
                const int j = i - NQK;
                const char* base = Vt + voff[j % DB] + (j / DB) * 16 * ROWB;
                return tr_read_pair(base, base + 8 * ROWB);
            };
            sacc[0] = f32x16{};
            sacc[1] = f32x16{};
            bf16x8 buf[AHEAD];
#pragma unroll
            for (int i = 0; i < AHEAD; ++i) buf[i] = rd(i);
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const bf16x8 a = buf[i % AHEAD];
                if (i + AHEAD < NP) buf[i % AHEAD] = rd(i + AHEAD);
                if (i < NQK) {
                    sacc[i & 1] = mfma32x32x16(a, qreg[i >> 1], sacc[i & 1]);
                } else {
                    const int j = i - NQK;
                    oacc[j % DB] = mfma32x32x16(a, pb[j / DB], oacc[j % DB]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // next position; false past the last
    auto advance = [&]() __attribute__((always_inline)) {
        np ^= 1;
        kt += dk;
        if (LOCAL && kt == lend) kt = lbeg;
        if (++k < nk) return true;
        if (!has_next) return false;
        advance_item();
        return true;
    };

    // Phase schedule: as in fwd_bf16_kernel, over the whole stream.
    if (grp == 0) {
        qk(Kbuf(0));
        phase_barrier(false);
        do {
            vphase();
            phase_barrier(true);
            dma();
            mphase();
            phase_barrier(false);
        } while (advance());
        phase_barrier(true);
    } else {
        phase_barrier(false);
        qk(Kbuf(0));
        phase_barrier(true);
        do {
            dma();
            vphase();
            phase_barrier(false);
            mphase();
            phase_barrier(true);
        } while (advance());
    }
    epilogue();
    if (stamping) {
        int bh0, tile0;
        item_bh_tile(0, bh0, tile0);
        stamp.finish(p.stamps, bh0, tile0);
    }
}

template <int D, bool CAUSAL, bool LOCAL = false>
hipError_t launch_persist(const PersistParams& prm, uint32_t grid, hipStream_t stream) {
    PersistParams arg = prm;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&fwd_bf16_persist_kernel<D, CAUSAL, LOCAL>, dim3(grid), dim3(NT), args, 0,
                           stream);
}

// Compute units of the stream's device (cached per device).
int device_cus(hipStream_t stream) {
    static int cus[kMaxDevices] = {};
    int dev = 0;
    if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 0;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int D, bool CAUSAL, bool LOCAL = false, bool BLOCK = false, bool SPLIT = false>
hipError_t launch(const Params& prm, hipStream_t stream) {
    Params arg = prm;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&fwd_bf16_kernel<D, CAUSAL, LOCAL, BLOCK, SPLIT>, dim3(prm.total), dim3(NT),
                           args, 0, stream);
}

}  // namespace

int64_t fwd_bf16_max_workgroups(int B, int Hq, int S) {
    // the key-split form takes BM / 2 queries per workgroup, the others BM
    return (int64_t)B * Hq * ((S + BM / 2 - 1) / (BM / 2));
}

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
    // plain attention with at most one 256-query workgroup per CU: 128-query
    // workgroups with the key range split between the wave groups.  Causal:
    // the longest tile sets the time, and the split halves it.  Without the
    // mask every workgroup is as long, and the split pays only while the
    // doubled grid still runs in one round.
    const bool windowed = a.causal && a.window > 0 && a.window < a.S;
    const int64_t g256 = (int64_t)a.B * a.Hq * ((a.S + BM - 1) / BM);
    const bool split = !a.bmask && !windowed && a.S > BM &&
                       g256 <= (a.causal ? kSplitMaxWorkgroups : kSplitMaxWorkgroups / 2);
    const int bmk = split ? BM / 2 : BM;
    prm.nq = (a.S + bmk - 1) / bmk;
    prm.total = (uint32_t)((int64_t)a.B * a.Hq * prm.nq);
    prm.c = a.scale * kLog2e;
    prm.window = a.window;
    prm.bmask = a.bmask;
    prm.bm_sb = a.bmask_stride_b;
    prm.bm_sh = a.bmask_stride_h;
    prm.nkb = (a.S + kMaskBlock - 1) / kMaskBlock;
    prm.stamps = (uint64_t*)a.stamps;
    prm.hgrp = 0;
    const uint32_t per = prm.total / 8u;
    if (per > 0 && per % (uint32_t)prm.nq == 0) {
        const uint32_t heads_here = per / (uint32_t)prm.nq;
        uint32_t g = (uint32_t)(kSlotsPerXcd / prm.nq > 1 ? kSlotsPerXcd / prm.nq : 1);
        if (g > heads_here) g = heads_here;
        while (heads_here % g) --g;
        prm.hgrp = g;
    }
    if (a.bmask) {
        if (a.D == 128) return a.causal ? launch<128, true, false, true>(prm, stream) : launch<128, false, false, true>(prm, stream);
        return a.causal ? launch<64, true, false, true>(prm, stream) : launch<64, false, false, true>(prm, stream);
    }
    // a window of at least S keys hides nothing the causal mask shows
    if (windowed) {
        // persistent form: whole query tiles (every item then has 4 or more
        // key tiles), whole rounds of tiles, and the tiles of whole heads on
        // each XCD's compute units
        const int cus = device_cus(stream);
        const int64_t units = (int64_t)a.B * a.Hq * prm.nq;
        if (a.S % BM == 0 && cus >= 8 && cus % 8 == 0 && (cus / 8) % prm.nq == 0 && units % cus == 0 &&
            units / cus <= (1 << 20)) {
            PersistParams pp;
            pp.q = prm.q;
            pp.k = prm.k;
            pp.v = prm.v;
            pp.out = prm.out;
            pp.lse = prm.lse;
            pp.Hq = prm.Hq;
            pp.Hkv = prm.Hkv;
            pp.S = prm.S;
            pp.group = prm.group;
            pp.nq = prm.nq;
            pp.units = prm.nq;
            pp.rounds = (int)(units / cus);
            pp.hpr = cus / 8 / prm.nq;
            pp.window = a.window;
            pp.c = prm.c;
            pp.stamps = prm.stamps;
            return a.D == 128 ? launch_persist<128, true, true>(pp, cus, stream)
                              : launch_persist<64, true, true>(pp, cus, stream);
        }
        return a.D == 128 ? launch<128, true, true>(prm, stream) : launch<64, true, true>(prm, stream);
    }
    // Persistent form: plain attention, every item at least one 256-query
    // tile long (so each has 4 or more key tiles), causal query tiles in
    // pairs, and whole rounds of units over the compute units.
    if (!a.bmask && !windowed && !split && a.S >= BM && !(a.causal && prm.nq % 2)) {
        const int cus = device_cus(stream);
        const int64_t units = (int64_t)a.B * a.Hq * (a.causal ? prm.nq / 2 : prm.nq);
        if (cus >= 8 && cus % 8 == 0 && units % cus == 0 && units / cus <= (1 << 20)) {
            PersistParams pp;
            pp.q = prm.q;
            pp.k = prm.k;
            pp.v = prm.v;
            pp.out = prm.out;
            pp.lse = prm.lse;
            pp.Hq = prm.Hq;
            pp.Hkv = prm.Hkv;
            pp.S = prm.S;
            pp.group = prm.group;
            pp.nq = prm.nq;
            pp.units = a.causal ? prm.nq / 2 : prm.nq;
            pp.rounds = (int)(units / cus);
            // causal: item rounds of whole heads when an XCD's workgroups
            // hold the tiles of whole heads
            pp.hpr = a.causal && (cus / 8) % prm.nq == 0 ? cus / 8 / prm.nq : 0;
            pp.window = 0;
            pp.c = prm.c;
            pp.stamps = prm.stamps;
            if (a.D == 128)
                return a.causal ? launch_persist<128, true>(pp, cus, stream) : launch_persist<128, false>(pp, cus, stream);
            return a.causal ? launch_persist<64, true>(pp, cus, stream) : launch_persist<64, false>(pp, cus, stream);
        }
    }
    if (split) {
        if (a.D == 128)
            return a.causal ? launch<128, true, false, false, true>(prm, stream)
                            : launch<128, false, false, false, true>(prm, stream);
        return a.causal ? launch<64, true, false, false, true>(prm, stream) : launch<64, false, false, false, true>(prm, stream);
    }
    if (a.D == 128) return a.causal ? launch<128, true>(prm, stream) : launch<128, false>(prm, stream);
    return a.causal ? launch<64, true>(prm, stream) : launch<64, false>(prm, stream);
}

}  // namespace attn
