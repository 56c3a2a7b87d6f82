// C ABI of libattn (declared in include/attn.h): argument checks, then one
// kernel launch per call (three for the backward).  Checks run before any HIP call, so a rejected call
// has no side effect at all.
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "attn.h"
#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxGrid = 0x7fffffff;  // workgroups per launch

bool bad_dims(int B, int Hq, int Hkv, int S) {
    return B < 1 || Hq < 1 || Hkv < 1 || S < 1 || Hq % Hkv != 0;
}

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

// Byte ranges [p, p + n) overlap?
bool overlap(const void* p, int64_t n, const void* q, int64_t m) {
    if (!p || !q || n <= 0 || m <= 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

// Product of sizes, or -1 if it does not fit in int64 with room to spare.
int64_t prod(std::initializer_list<int64_t> xs) {
    int64_t r = 1;
    for (int64_t x : xs) {
        if (x <= 0) return -1;
        if (r > (int64_t(1) << 62) / x) return -1;
        r *= x;
    }
    return r;
}

attn_status hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
}

// Shared checks of the fused forward.  esz = element bytes.
attn_status check_fwd(const void* q, const void* k, const void* v, const void* out, const float* lse, int B,
                      int Hq, int Hkv, int S, int D, float scale, int causal, int esz) {
    if (!q || !k || !v || !out) return ATTN_ERR_NULL_POINTER;
    if (bad_dims(B, Hq, Hkv, S)) return ATTN_ERR_BAD_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_BAD_SCALE;
    const int64_t nq = prod({B, Hq, S, D, esz});
    const int64_t nkv = prod({B, Hkv, S, D, esz});
    const int64_t nl = prod({B, Hq, S, 4});
    if (nq < 0 || nkv < 0 || nl < 0) return ATTN_ERR_BAD_SHAPE;
    if (prod({B, Hq, (S + 63) / 64}) > kMaxGrid) return ATTN_ERR_BAD_SHAPE;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
        misaligned(lse, 4))
        return ATTN_ERR_MISALIGNED;
    if (overlap(out, nq, q, nq) || overlap(out, nq, k, nkv) || overlap(out, nq, v, nkv) ||
        overlap(lse, nl, q, nq) || overlap(lse, nl, k, nkv) || overlap(lse, nl, v, nkv) ||
        overlap(lse, nl, out, nq))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

attn_status check_qk(const void* q, const void* k, const float* scores, int B, int Hq, int Hkv, int S, int D,
                     int esz) {
    if (!q || !k || !scores) return ATTN_ERR_NULL_POINTER;
    if (bad_dims(B, Hq, Hkv, S)) return ATTN_ERR_BAD_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    const int64_t nq = prod({B, Hq, S, D, esz});
    const int64_t nk = prod({B, Hkv, S, D, esz});
    const int64_t ns = prod({B, Hq, S, S, 4});
    if (nq < 0 || nk < 0 || ns < 0) return ATTN_ERR_BAD_SHAPE;
    const int64_t t = (S + 127) / 128, t64 = (S + 63) / 64;
    if (prod({B, Hq, t, t}) > kMaxGrid || prod({B, Hq, t64, t64}) > kMaxGrid) return ATTN_ERR_BAD_SHAPE;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(scores, 16)) return ATTN_ERR_MISALIGNED;
    if (overlap(scores, ns, q, nq) || overlap(scores, ns, k, nk)) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

attn_status check_softmax(const float* scores, const void* p, const float* lse, int B, int H, int S, float scale,
                          int causal, int esz) {
    if (!scores || !p) return ATTN_ERR_NULL_POINTER;
    if (B < 1 || H < 1 || S < 1) return ATTN_ERR_BAD_SHAPE;
    if (causal != 0 && causal != 1) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_BAD_SCALE;
    const int64_t ns = prod({B, H, S, S, 4});
    const int64_t np = prod({B, H, S, S, esz});
    const int64_t nl = prod({B, H, S, 4});
    if (ns < 0 || np < 0 || nl < 0) return ATTN_ERR_BAD_SHAPE;
    if (prod({B, H, (S + 3) / 4}) > kMaxGrid) return ATTN_ERR_BAD_SHAPE;
    if (misaligned(scores, 16) || misaligned(p, 16) || misaligned(lse, 4)) return ATTN_ERR_MISALIGNED;
    if (overlap(p, np, scores, ns) || overlap(lse, nl, scores, ns) || overlap(lse, nl, p, np))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

attn_status check_pv(const void* p, const void* v, const void* out, int B, int Hq, int Hkv, int S, int D, int esz) {
    if (!p || !v || !out) return ATTN_ERR_NULL_POINTER;
    if (bad_dims(B, Hq, Hkv, S)) return ATTN_ERR_BAD_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    const int64_t np = prod({B, Hq, S, S, esz});
    const int64_t nv = prod({B, Hkv, S, D, esz});
    const int64_t no = prod({B, Hq, S, D, esz});
    if (np < 0 || nv < 0 || no < 0) return ATTN_ERR_BAD_SHAPE;
    if (prod({B, Hq, (S + 63) / 64, 2}) > kMaxGrid) return ATTN_ERR_BAD_SHAPE;
    if (misaligned(p, 16) || misaligned(v, 16) || misaligned(out, 16)) return ATTN_ERR_MISALIGNED;
    if (overlap(out, no, p, np) || overlap(out, no, v, nv)) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

attn_status check_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, const void* dq, const void* dk, const void* dv, const float* delta, int B,
                      int Hq, int Hkv, int S, int D, float scale, int causal) {
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !delta) return ATTN_ERR_NULL_POINTER;
    if (bad_dims(B, Hq, Hkv, S)) return ATTN_ERR_BAD_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_BAD_SCALE;
    const int64_t nq = prod({B, Hq, S, D, 2});
    const int64_t nkv = prod({B, Hkv, S, D, 2});
    const int64_t nl = prod({B, Hq, S, 4});
    if (nq < 0 || nkv < 0 || nl < 0) return ATTN_ERR_BAD_SHAPE;
    if (prod({B, Hq, (S + 15) / 16}) > kMaxGrid) return ATTN_ERR_BAD_SHAPE;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
        misaligned(dout, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) ||
        misaligned(lse, 4) || misaligned(delta, 4))
        return ATTN_ERR_MISALIGNED;
    struct Range {
        const void* p;
        int64_t n;
    };
    const Range ins[] = {{q, nq}, {k, nkv}, {v, nkv}, {out, nq}, {dout, nq}, {lse, nl}};
    const Range outs[] = {{dq, nq}, {dk, nkv}, {dv, nkv}, {delta, nl}};
    for (const Range& o : outs) {
        for (const Range& i : ins)
            if (overlap(o.p, o.n, i.p, i.n)) return ATTN_ERR_ALIAS;
        for (const Range& o2 : outs)
            if (&o2 != &o && overlap(o.p, o.n, o2.p, o2.n)) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

attn::FwdArgs fwd_args(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                       int S, int D, float scale, int causal) {
    attn::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.S = S;
    a.D = D;
    a.scale = scale;
    a.causal = causal;
    a.window = 0;
    return a;
}

}  // namespace

extern "C" {

attn_status attn_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                          int Hkv, int S, int D, float scale, int causal, void* stream) {
    const attn_status st = check_fwd(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, 2);
    if (st != ATTN_OK) return st;
    return hip_status(attn::launch_fwd_bf16(fwd_args(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal),
                                            (hipStream_t)stream));
}

attn_status attn_fwd_bf16_stamped(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                                  int Hq, int Hkv, int S, int D, float scale, int causal, uint64_t* stamps,
                                  void* stream) {
    const attn_status st = check_fwd(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, 2);
    if (st != ATTN_OK) return st;
    if (!stamps) return ATTN_ERR_NULL_POINTER;
    if (misaligned(stamps, 8)) return ATTN_ERR_MISALIGNED;
    const int64_t ns = prod({attn::fwd_bf16_max_workgroups(B, Hq, S), attn::kStampWords, 8});
    if (ns < 0) return ATTN_ERR_BAD_SHAPE;
    const int64_t nq = prod({B, Hq, S, D, 2});
    const int64_t nkv = prod({B, Hkv, S, D, 2});
    const int64_t nl = prod({B, Hq, S, 4});
    if (overlap(stamps, ns, q, nq) || overlap(stamps, ns, k, nkv) || overlap(stamps, ns, v, nkv) ||
        overlap(stamps, ns, out, nq) || overlap(stamps, ns, lse, nl))
        return ATTN_ERR_ALIAS;
    attn::FwdArgs a = fwd_args(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal);
    a.stamps = (unsigned long long*)stamps;
    return hip_status(attn::launch_fwd_bf16(a, (hipStream_t)stream));
}

size_t attn_fwd_bf16_stamp_bytes(int B, int Hq, int S) {
    if (B < 1 || Hq < 1 || S < 1) return 0;
    const int64_t n = prod({attn::fwd_bf16_max_workgroups(B, Hq, S), attn::kStampWords, 8});
    return n < 0 ? 0 : (size_t)n;
}

attn_status attn_fwd_local_bf16(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                                int Hkv, int S, int D, float scale, int window, void* stream) {
    const attn_status st = check_fwd(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, 1, 2);
    if (st != ATTN_OK) return st;
    if (window < 1) return ATTN_ERR_UNSUPPORTED;
    attn::FwdArgs a = fwd_args(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, 1);
    a.window = window;
    return hip_status(attn::launch_fwd_bf16(a, (hipStream_t)stream));
}

attn_status attn_fwd_blockmask_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                    const uint8_t* block_mask, int64_t mask_stride_b, int64_t mask_stride_h, int B,
                                    int Hq, int Hkv, int S, int D, float scale, int causal, void* stream) {
    const attn_status st = check_fwd(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, 2);
    if (st != ATTN_OK) return st;
    if (!block_mask) return ATTN_ERR_NULL_POINTER;
    if (S > ATTN_MASK_MAX_S) return ATTN_ERR_UNSUPPORTED;
    if (mask_stride_b < 0 || mask_stride_h < 0) return ATTN_ERR_BAD_SHAPE;
    const int64_t nb = (S + ATTN_MASK_BLOCK - 1) / ATTN_MASK_BLOCK;
    // bytes from block_mask to one past its last flag
    const int64_t lim = int64_t(1) << 60;
    if (mask_stride_b > lim / B || mask_stride_h > lim / Hq) return ATTN_ERR_BAD_SHAPE;
    const int64_t extent = (int64_t)(B - 1) * mask_stride_b + (int64_t)(Hq - 1) * mask_stride_h + nb * nb;
    const int64_t no = prod({B, Hq, S, D, 2});
    const int64_t nl = prod({B, Hq, S, 4});
    if (overlap(out, no, block_mask, extent) || overlap(lse, nl, block_mask, extent)) return ATTN_ERR_ALIAS;
    attn::FwdArgs a = fwd_args(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal);
    a.bmask = block_mask;
    a.bmask_stride_b = mask_stride_b;
    a.bmask_stride_h = mask_stride_h;
    return hip_status(attn::launch_fwd_bf16(a, (hipStream_t)stream));
}

attn_status attn_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                         int S, int D, float scale, float q_scale, float k_scale, float v_scale, int causal,
                         void* stream) {
    if (!q || !k || !v || !out) return ATTN_ERR_NULL_POINTER;
    if (bad_dims(B, Hq, Hkv, S)) return ATTN_ERR_BAD_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return ATTN_ERR_UNSUPPORTED;
    for (float x : {scale, q_scale, k_scale, v_scale})
        if (!isfinite(x) || !(x > 0.f)) return ATTN_ERR_BAD_SCALE;
    if (!isfinite(scale * q_scale * k_scale * 1.4426950408889634f)) return ATTN_ERR_BAD_SCALE;
    const int64_t nq8 = prod({B, Hq, S, D});
    const int64_t nkv8 = prod({B, Hkv, S, D});
    const int64_t no = prod({B, Hq, S, D, 2});
    const int64_t nl = prod({B, Hq, S, 4});
    if (nq8 < 0 || nkv8 < 0 || no < 0 || nl < 0) return ATTN_ERR_BAD_SHAPE;
    if (prod({B, Hq, (S + 127) / 128}) > kMaxGrid) return ATTN_ERR_BAD_SHAPE;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) || misaligned(lse, 4))
        return ATTN_ERR_MISALIGNED;
    if (overlap(out, no, q, nq8) || overlap(out, no, k, nkv8) || overlap(out, no, v, nkv8) ||
        overlap(lse, nl, q, nq8) || overlap(lse, nl, k, nkv8) || overlap(lse, nl, v, nkv8) || overlap(lse, nl, out, no))
        return ATTN_ERR_ALIAS;
    attn::Fp8Args a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.S = S;
    a.D = D;
    a.scale = scale;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.causal = causal;
    return hip_status(attn::launch_fwd_fp8(a, (hipStream_t)stream));
}

attn_status attn_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse, int B, int Hq,
                         int Hkv, int S, int D, float scale, int causal, void* stream) {
    const attn_status st = check_fwd(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal, 4);
    if (st != ATTN_OK) return st;
    return hip_status(attn::launch_fwd_f32(fwd_args(q, k, v, out, lse, B, Hq, Hkv, S, D, scale, causal),
                                           (hipStream_t)stream));
}

static attn_status qk_common(const void* q, const void* k, float* scores, int B, int Hq, int Hkv, int S, int D,
                             void* stream, int esz) {
    const attn_status st = check_qk(q, k, scores, B, Hq, Hkv, S, D, esz);
    if (st != ATTN_OK) return st;
    attn::QkArgs a;
    a.q = q;
    a.k = k;
    a.scores = scores;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.S = S;
    a.D = D;
    return hip_status(esz == 2 ? attn::launch_qk_gemm_bf16(a, (hipStream_t)stream)
                               : attn::launch_qk_gemm_f32(a, (hipStream_t)stream));
}

attn_status attn_qk_gemm_bf16(const void* q, const void* k, float* scores, int B, int Hq, int Hkv, int S, int D,
                              void* stream) {
    return qk_common(q, k, scores, B, Hq, Hkv, S, D, stream, 2);
}

attn_status attn_qk_gemm_f32(const float* q, const float* k, float* scores, int B, int Hq, int Hkv, int S, int D,
                             void* stream) {
    return qk_common(q, k, scores, B, Hq, Hkv, S, D, stream, 4);
}

static attn_status softmax_common(const float* scores, void* p, float* lse, int B, int H, int S, float scale,
                                  int causal, void* stream, int esz) {
    const attn_status st = check_softmax(scores, p, lse, B, H, S, scale, causal, esz);
    if (st != ATTN_OK) return st;
    attn::SoftmaxArgs a;
    a.scores = scores;
    a.p = p;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.S = S;
    a.scale = scale;
    a.causal = causal;
    return hip_status(esz == 2 ? attn::launch_masked_softmax_bf16(a, (hipStream_t)stream)
                               : attn::launch_masked_softmax_f32(a, (hipStream_t)stream));
}

attn_status attn_masked_softmax_bf16(const float* scores, void* p, float* lse, int B, int H, int S, float scale,
                                     int causal, void* stream) {
    return softmax_common(scores, p, lse, B, H, S, scale, causal, stream, 2);
}

attn_status attn_masked_softmax_f32(const float* scores, float* p, float* lse, int B, int H, int S, float scale,
                                    int causal, void* stream) {
    return softmax_common(scores, p, lse, B, H, S, scale, causal, stream, 4);
}

static attn_status pv_common(const void* p, const void* v, void* out, int B, int Hq, int Hkv, int S, int D,
                             void* stream, int esz) {
    const attn_status st = check_pv(p, v, out, B, Hq, Hkv, S, D, esz);
    if (st != ATTN_OK) return st;
    attn::PvArgs a;
    a.p = p;
    a.v = v;
    a.out = out;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.S = S;
    a.D = D;
    return hip_status(esz == 2 ? attn::launch_pv_gemm_bf16(a, (hipStream_t)stream)
                               : attn::launch_pv_gemm_f32(a, (hipStream_t)stream));
}

attn_status attn_pv_gemm_bf16(const void* p, const void* v, void* out, int B, int Hq, int Hkv, int S, int D,
                              void* stream) {
    return pv_common(p, v, out, B, Hq, Hkv, S, D, stream, 2);
}

attn_status attn_pv_gemm_f32(const float* p, const float* v, float* out, int B, int Hq, int Hkv, int S, int D,
                             void* stream) {
    return pv_common(p, v, out, B, Hq, Hkv, S, D, stream, 4);
}

constexpr int kMaxSplits = 4096;

static int64_t splitkv_ws_floats(int B, int Hq, int Sq, int D, int nsplit) {
    return prod({nsplit, B, Hq, Sq, D + 1});
}

// Checks shared by the two split-KV entry points; workspace may be null
// (the allocation-free one) and is then not checked for alignment or overlap.
static attn_status check_splitkv(const void* q, const void* k, const void* v, const void* out, const float* lse,
                          const float* workspace, int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                          int causal, int nsplit) {
    if (!q || !k || !v || !out) return ATTN_ERR_NULL_POINTER;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < Sq || Hq % Hkv != 0) return ATTN_ERR_BAD_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return ATTN_ERR_UNSUPPORTED;
    if (nsplit < 1 || nsplit > kMaxSplits) return ATTN_ERR_UNSUPPORTED;
    if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_BAD_SCALE;
    const int64_t nq = prod({B, Hq, Sq, D, 2});
    const int64_t nkv = prod({B, Hkv, Skv, D, 2});
    const int64_t nl = prod({B, Hq, Sq, 4});
    const int64_t nws = splitkv_ws_floats(B, Hq, Sq, D, nsplit);
    if (nq < 0 || nkv < 0 || nl < 0 || nws < 0 || nws > (int64_t(1) << 60) / 4) return ATTN_ERR_BAD_SHAPE;
    if (prod({B, Hkv, attn::splitkv_row_blocks(Hq, Hkv, Sq), nsplit}) > kMaxGrid ||
        prod({B, Hq, Sq}) > kMaxGrid)  // the merge runs one workgroup per query row
        return ATTN_ERR_BAD_SHAPE;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
        misaligned(workspace, 16) || misaligned(lse, 4))
        return ATTN_ERR_MISALIGNED;
    const int64_t nwb = nws * 4;
    if (overlap(out, nq, q, nq) || overlap(out, nq, k, nkv) || overlap(out, nq, v, nkv) ||
        overlap(lse, nl, q, nq) || overlap(lse, nl, k, nkv) || overlap(lse, nl, v, nkv) || overlap(lse, nl, out, nq) ||
        overlap(workspace, nwb, q, nq) || overlap(workspace, nwb, k, nkv) || overlap(workspace, nwb, v, nkv) ||
        overlap(workspace, nwb, out, nq) || overlap(workspace, nwb, lse, nl))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

static attn::SplitKvArgs splitkv_args(const void* q, const void* k, const void* v, void* out, float* lse, float* workspace,
                               int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal, int nsplit) {
    attn::SplitKvArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.workspace = workspace;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Sq = Sq;
    a.Skv = Skv;
    a.D = D;
    a.scale = scale;
    a.causal = causal;
    a.nsplit = nsplit;
    return a;
}

attn_status attn_fwd_splitkv_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                  float* workspace, int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                                  int causal, int nsplit, void* stream) {
    if (!workspace) return ATTN_ERR_NULL_POINTER;
    const attn_status st =
        check_splitkv(q, k, v, out, lse, workspace, B, Hq, Hkv, Sq, Skv, D, scale, causal, nsplit);
    if (st != ATTN_OK) return st;
    return hip_status(attn::launch_splitkv_bf16(
        splitkv_args(q, k, v, out, lse, workspace, B, Hq, Hkv, Sq, Skv, D, scale, causal, nsplit),
        (hipStream_t)stream));
}

attn_status attn_fwd_splitkv_bf16_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                          int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                                          int nsplit, void* stream) {
    const attn_status st =
        check_splitkv(q, k, v, out, lse, nullptr, B, Hq, Hkv, Sq, Skv, D, scale, causal, nsplit);
    if (st != ATTN_OK) return st;
    if (splitkv_ws_floats(B, Hq, Sq, D, nsplit) > attn::kSplitkvScratchFloats) return ATTN_ERR_TOO_LARGE;
    float* ws = nullptr;
    const hipError_t e = attn::splitkv_scratch((hipStream_t)stream, &ws);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(attn::launch_splitkv_bf16(
        splitkv_args(q, k, v, out, lse, ws, B, Hq, Hkv, Sq, Skv, D, scale, causal, nsplit), (hipStream_t)stream));
}

size_t attn_splitkv_noalloc_max_bytes(void) { return (size_t)attn::kSplitkvScratchFloats * 4; }

size_t attn_splitkv_workspace_bytes(int B, int Hq, int Sq, int D, int nsplit) {
    if (nsplit < 1 || nsplit > kMaxSplits || (D != 64 && D != 128)) return 0;
    const int64_t n = splitkv_ws_floats(B, Hq, Sq, D, nsplit);
    return n < 0 || n > (int64_t(1) << 60) / 4 ? 0 : (size_t)n * 4;
}

int attn_splitkv_default_splits(int B, int Hq, int Hkv, int Sq, int Skv) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || Hq % Hkv != 0) return 0;
    // about two workgroups per compute unit (256 CUs), at least one key chunk per split
    const int64_t units = (int64_t)B * Hkv * attn::splitkv_row_blocks(Hq, Hkv, Sq);
    const int64_t want = (512 + units - 1) / units;
    const int64_t chunks = (Skv + attn::splitkv_chunk() - 1) / attn::splitkv_chunk();
    int64_t n = want < chunks ? want : chunks;
    if (n > kMaxSplits) n = kMaxSplits;
    return (int)(n < 1 ? 1 : n);
}

attn_status attn_bwd_bf16(const void* q, const void* k, const void* v, const void* out, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv,
                          int S, int D, float scale, int causal, void* stream) {
    const attn_status st = check_bwd(q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, S, D, scale, causal);
    if (st != ATTN_OK) return st;
    attn::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.S = S;
    a.D = D;
    a.scale = scale;
    a.causal = causal;
    return hip_status(attn::launch_bwd_bf16(a, (hipStream_t)stream));
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int S) {
    const int64_t n = prod({B, Hq, S, 4});
    return n < 0 ? 0 : (size_t)n;
}

size_t attn_scores_bytes(int B, int Hq, int S) {
    const int64_t n = prod({B, Hq, S, S, 4});
    return n < 0 ? 0 : (size_t)n;
}

size_t attn_probs_bytes(int B, int Hq, int S, int elem_bytes) {
    if (elem_bytes != 2 && elem_bytes != 4) return 0;
    const int64_t n = prod({B, Hq, S, S, elem_bytes});
    return n < 0 ? 0 : (size_t)n;
}

const char* attn_status_str(attn_status s) {
    switch (s) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_NULL_POINTER: return "ATTN_ERR_NULL_POINTER: a required pointer is NULL";
        case ATTN_ERR_BAD_SHAPE: return "ATTN_ERR_BAD_SHAPE: a size < 1, Hq % Hkv != 0, or a size overflows";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: D must be 64 or 128 and causal 0 or 1";
        case ATTN_ERR_BAD_SCALE: return "ATTN_ERR_BAD_SCALE: scale must be finite and > 0";
        case ATTN_ERR_MISALIGNED: return "ATTN_ERR_MISALIGNED: tensors need 16-byte alignment (lse 4)";
        case ATTN_ERR_ALIAS: return "ATTN_ERR_ALIAS: an output overlaps an input";
        case ATTN_ERR_HIP: return "ATTN_ERR_HIP: kernel launch failed";
        case ATTN_ERR_TOO_LARGE: return "ATTN_ERR_TOO_LARGE: the call needs more than the library's fixed scratch";
    }
    return "unknown attn_status";
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
