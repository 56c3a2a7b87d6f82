/*
 * attn.h -- libattn: causal scaled dot-product attention forward for AMD
 * MI355X (gfx950), as a plain C ABI.
 *
 * The operation is the one the four attention-profiling pages describe:
 *
 *     out = softmax(scale * q k^T + mask) v
 *
 * (the formula in the ainews.cool article's technical deep-dive; the five-step
 * causal pipeline -- q k^T, times scale, masked_fill with -inf where key j is
 * after query i, softmax over keys, times v -- in the "Naive Attention"
 * section of the Hugging Face "Profiling in PyTorch (Part 3)" article).
 *
 * Two ways to compute it are exported:
 *   - attn_fwd_*: one fused kernel.  Keys and values stream through on-chip
 *     memory in tiles and the softmax is computed online, so the S x S score
 *     matrix never reaches device memory (the tiling idea of the Flash
 *     backend section of the Hugging Face article).
 *   - the unfused trio attn_qk_gemm_* -> attn_masked_softmax_* ->
 *     attn_pv_gemm_*, three kernels that materialise scores and
 *     probabilities in caller-owned buffers, mirroring the naive pipeline.
 * and, for training, attn_bwd_bf16: the gradients of the fused forward.
 *
 * Conventions shared by every call
 *   Layout     q and out are [B, Hq, S, D]; k and v are [B, Hkv, S, D];
 *              scores and probabilities are [B, Hq, S, S]; lse is [B, Hq, S].
 *              All row-major and contiguous, D (or the key axis) fastest:
 *              the native [B, H, S, D] layout the cuDNN section of the
 *              Hugging Face article praises, with no transposes.
 *   Heads      Grouped-query attention: query head h reads key/value head
 *              h / (Hq / Hkv).  Hq must be a multiple of Hkv; Hkv = 1 is
 *              multi-query attention, Hkv = Hq ordinary multi-head.
 *   Mask       causal = 1 masks key j for query i when j > i (one shared
 *              sequence length S, so top-left and bottom-right alignment
 *              coincide); causal = 0 masks nothing.  Masked logits are -inf
 *              and get weight exactly 0.
 *   lse        Natural log of sum_j exp(scale * q_i . k_j) over unmasked j,
 *              float32.  Not on the pages; kept for a later backward pass or
 *              a merge of partial results.
 *   dtype      The _bf16 calls take and return bfloat16 tensors (passed as
 *              void*) and accumulate in float32; the probabilities handed to
 *              the second product are rounded to bfloat16 (round to nearest
 *              even).  The _f32 calls are float32 throughout.
 *   Sizes      B, Hq, Hkv, S >= 1; D must be 64 or 128.
 *   Memory     Every pointer is device memory owned by the caller.  The
 *              library allocates nothing, keeps no state between calls and is
 *              safe to call from several host threads.  q, k, v, out, scores
 *              and p must be 16-byte aligned; lse 4-byte aligned.  Outputs
 *              must not overlap inputs.
 *   Streams    stream is a hipStream_t passed as void*; NULL means the null
 *              stream.  Calls are asynchronous: they enqueue kernels and
 *              return.  A kernel fault shows up at the caller's next
 *              synchronisation, as usual for HIP.
 *   Errors     Arguments are checked before anything is enqueued; a failed
 *              check returns its code, launches nothing and leaves every
 *              output untouched.  ATTN_ERR_HIP means the launch itself
 *              failed; attn_last_hip_error() gives the HIP error code
 *              (per host thread).
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL_POINTER = 1, /* a required pointer is NULL                          */
    ATTN_ERR_BAD_SHAPE = 2,    /* a size < 1, Hq % Hkv != 0, or a size overflows      */
    ATTN_ERR_UNSUPPORTED = 3,  /* D not in {64, 128}, causal not in {0, 1}, or a     */
                               /* variant's own limit (stated with the variant)       */
    ATTN_ERR_BAD_SCALE = 4,    /* scale is not finite, or not > 0                     */
    ATTN_ERR_MISALIGNED = 5,   /* a tensor pointer breaks the alignment rule          */
    ATTN_ERR_ALIAS = 6,        /* an output overlaps an input                         */
    ATTN_ERR_HIP = 7,          /* the HIP launch failed; see attn_last_hip_error()    */
    ATTN_ERR_TOO_LARGE = 8     /* the call needs more than the library's fixed       */
                               /* scratch (allocation-free entry points only)         */
} attn_status;

/* ---------------------------------------------------------------------------
 * Fused forward (the hot path).
 *
 * out[b,h,i,:] = sum_j w_ij v[b,g,j,:],  w_ij = exp(s_ij - lse_i),
 * s_ij = scale * q[b,h,i,:] . k[b,g,j,:],  g = h / (Hq/Hkv),
 * over the unmasked j; lse[b,h,i] = ln sum_j exp(s_ij).
 *
 * q, k, v, out: bfloat16 (attn_fwd_bf16) or float32 (attn_fwd_f32).
 * lse: float32 [B,Hq,S], or NULL to skip writing it.
 * One kernel launch, no workspace.  The usual scale is 1/sqrt(D) (the scale
 * of the NaiveCausalAttention class in the Hugging Face article).
 * ------------------------------------------------------------------------- */
attn_status attn_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                          int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                          void* stream);
attn_status attn_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                         int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                         void* stream);

/* ---------------------------------------------------------------------------
 * Stamped fused forward (bfloat16): a measurement aid.
 *
 * Runs exactly the kernel attn_fwd_bf16 runs, with the same arguments and
 * results, and in addition each workgroup w writes ATTN_STAMP_WORDS 64-bit
 * words at stamps[w * ATTN_STAMP_WORDS]: the shader-clock counter and the
 * 100 MHz real-time counter when it starts, the same two when its first wave
 * has stored its output, its HW_ID and XCC_ID hardware registers (compute
 * unit and die it ran on), and the (batch * Hq + head) and query tile it
 * computed.  The ratio of the clock-counter span to the real-time span is the
 * shader clock the kernel ran at, so its throughput can be set against the
 * matrix cores' peak at that clock as well as at the nominal 2.4 GHz (the
 * pages report per-op utilisation beside latency: the ainews.cool per-op
 * table).  stamps: device memory of attn_fwd_bf16_stamp_bytes(B, Hq, S)
 * bytes, 8-byte aligned, not overlapping any other argument; records of
 * workgroups the launch does not have are left as they were (a launch uses
 * at most B * Hq * ceil(S / 128) workgroups).  One kernel launch.
 * ------------------------------------------------------------------------- */
#define ATTN_STAMP_WORDS 8
attn_status attn_fwd_bf16_stamped(const void* q, const void* k, const void* v, void* out, float* lse,
                                  int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                                  uint64_t* stamps, void* stream);
/* Bytes of attn_fwd_bf16_stamped's stamp records, or 0 on a bad size. */
size_t attn_fwd_bf16_stamp_bytes(int B, int Hq, int S);

/* ---------------------------------------------------------------------------
 * Fused forward with fp8 operands (OCP E4M3, "e4m3fn").
 *
 * q [B,Hq,S,D], k and v [B,Hkv,S,D]: one byte per element, e4m3fn codes;
 * the value of an element is decode(code) * q_scale (k_scale, v_scale), one
 * float scale per tensor.  out: bfloat16 [B,Hq,S,D]; lse: float32 [B,Hq,S] or
 * NULL.  Computes the same attention as attn_fwd_bf16 on those values, with
 * the products on the fp8 matrix cores (twice the bf16 rate): q k^T exactly
 * (fp8 products, float32 sums), the probabilities rounded to e4m3 (stored
 * against a power-of-two reference, 2^7 to 2^8.75 for the row max) for the
 * product with v, and out normalised by the sum of the rounded
 * probabilities.  The ai-manual.ru tutorial (section 6) names FP8 as the next
 * factor of two after bf16.  scale, q_scale, k_scale, v_scale: finite, > 0.
 * The codes must be finite values (not 0x7f / 0xff, e4m3fn's NaN).
 * One kernel launch, no workspace.
 * ------------------------------------------------------------------------- */
attn_status attn_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int Hq, int Hkv, int S, int D, float scale, float q_scale, float k_scale,
                         float v_scale, int causal, void* stream);

/* ---------------------------------------------------------------------------
 * Fused forward with a causal sliding window (bfloat16).
 *
 * As attn_fwd_bf16 with causal = 1, except that query i sees only keys
 * max(0, i - window + 1) .. i: its own position and the window - 1 before it.
 * Special masks like this one are what the ai-manual.ru tutorial gives as the
 * reason to write custom attention kernels (section 5's conclusions,
 * section 7).  Key tiles wholly before a query tile's window are skipped, as
 * the causal mask skips tiles after the diagonal.  window >= S gives exactly
 * the causal result.  window < 1 returns ATTN_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
attn_status attn_fwd_local_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int Hq, int Hkv, int S, int D, float scale, int window,
                                void* stream);

/* ---------------------------------------------------------------------------
 * Fused forward with a block mask (bfloat16): block-sparse attention.
 *
 * As attn_fwd_bf16, except that query i of (b, h) sees key j only if the
 * flag of its block pair is nonzero (and j <= i when causal = 1).  Blocks are
 * ATTN_MASK_BLOCK queries x ATTN_MASK_BLOCK keys; with nb = ceil(S / 64), the
 * flag of (b, h, query block qb, key block kb) is the byte
 *     block_mask[b * mask_stride_b + h * mask_stride_h + qb * nb + kb],
 * strides in bytes, >= 0 (0 broadcasts one mask over batches or heads).
 * Block-sparse masks are among the special masks the ai-manual.ru tutorial
 * gives as the reason to write custom attention kernels (section 5's
 * conclusions, section 7).  Key tiles no query of a 256-query tile may see
 * are neither loaded nor multiplied.  A query that sees no key gets out = 0
 * and lse = -inf (the "safe softmax" rule of the math backend described in
 * the SDPA section of the Hugging Face article).  block_mask is a device
 * pointer, read only; it must not overlap out or lse (ATTN_ERR_ALIAS).
 * S > ATTN_MASK_MAX_S returns ATTN_ERR_UNSUPPORTED.  One kernel launch, no
 * workspace.
 * ------------------------------------------------------------------------- */
#define ATTN_MASK_BLOCK 64
#define ATTN_MASK_MAX_S 131072
attn_status attn_fwd_blockmask_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                    const uint8_t* block_mask, int64_t mask_stride_b, int64_t mask_stride_h,
                                    int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * Split-KV forward for short query counts (bfloat16): a decode step.
 *
 * q, out: [B, Hq, Sq, D]; k, v: [B, Hkv, Skv, D] with 1 <= Sq <= Skv.  The
 * queries are the last Sq positions of the sequence whose keys and values are
 * given, so with causal = 1 query i sees keys 0 .. Skv - Sq + i (with Sq = 1,
 * every key, as with causal = 0).  Otherwise the same operation as
 * attn_fwd_bf16; lse [B, Hq, Sq] float32 or NULL.
 * The key axis is cut into nsplit ranges processed in parallel (the "split-k"
 * that the ai-manual.ru tutorial, section 4, lists as missing from its sketch
 * kernel), then merged with the ranges' log-sum-exps.  workspace: float32,
 * attn_splitkv_workspace_bytes(B, Hq, Sq, D, nsplit) bytes, 16-byte aligned,
 * caller-owned, overwritten.  nsplit in 1..4096 (ATTN_ERR_UNSUPPORTED
 * otherwise); attn_splitkv_default_splits suggests one.  Two kernel launches.
 * ------------------------------------------------------------------------- */
attn_status attn_fwd_splitkv_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                  float* workspace, int B, int Hq, int Hkv, int Sq, int Skv, int D,
                                  float scale, int causal, int nsplit, void* stream);
/* Workspace bytes for attn_fwd_splitkv_bf16: nsplit*B*Hq*Sq*(D+1)*4, or 0 on a
 * bad size. */
size_t attn_splitkv_workspace_bytes(int B, int Hq, int Sq, int D, int nsplit);
/* A split count that gives about two workgroups per compute unit, or 0 on a
 * bad size. */
int attn_splitkv_default_splits(int B, int Hq, int Hkv, int Sq, int Skv);

/* ---------------------------------------------------------------------------
 * Split-KV forward that allocates nothing (bfloat16).
 *
 * For callers that cannot allocate device memory at call time: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same operation, arguments, results and kernels as attn_fwd_splitkv_bf16,
 * without the workspace argument: the partial results live in a scratch
 * array of attn_splitkv_noalloc_max_bytes() bytes (16 MiB) that the library
 * holds on every GPU it runs on until the process ends.  A call whose
 * workspace (attn_splitkv_workspace_bytes) would exceed it returns
 * ATTN_ERR_TOO_LARGE and launches nothing.  No hipMalloc or hipFree; the
 * first call on a GPU looks up that GPU's scratch address once.  Calls that
 * overlap on one GPU (on different streams, or from several host threads)
 * share the scratch and race: serialise them.  Two kernel launches.
 * ------------------------------------------------------------------------- */
attn_status attn_fwd_splitkv_bf16_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                          int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                                          int causal, int nsplit, void* stream);
/* Bytes of the scratch behind attn_fwd_splitkv_bf16_noalloc (the largest
 * workspace it serves). */
size_t attn_splitkv_noalloc_max_bytes(void);

/* ---------------------------------------------------------------------------
 * Unfused trio, mirroring the naive pipeline one step per kernel.
 *
 * Step 1, attn_qk_gemm_*: scores[b,h,i,j] = q[b,h,i,:] . k[b,g,j,:] for every
 *   i and j (unscaled, unmasked), float32 [B,Hq,S,S] (attn_scores_bytes).
 * Steps 2-4, attn_masked_softmax_*: p[b,h,i,j] = exp(t_ij - lse_i) with
 *   t_ij = scale * scores[b,h,i,j], or -inf (so p = 0) for masked j; p is
 *   [B,H,S,S] in the call's dtype (attn_probs_bytes); lse [B,H,S] float32 or
 *   NULL.  H is the number of query heads.  The mask is applied on the fly:
 *   masked entries of scores are never read and need not hold data.
 * Step 5, attn_pv_gemm_*: out[b,h,i,:] = sum_j p[b,h,i,j] v[b,g,j,:], a plain
 *   product over every j (zeros in p are multiplied like any value); out is
 *   [B,Hq,S,D] in the call's dtype.
 * Each call is one kernel launch on stream.
 * ------------------------------------------------------------------------- */
attn_status attn_qk_gemm_bf16(const void* q, const void* k, float* scores,
                              int B, int Hq, int Hkv, int S, int D, void* stream);
attn_status attn_qk_gemm_f32(const float* q, const float* k, float* scores,
                             int B, int Hq, int Hkv, int S, int D, void* stream);
attn_status attn_masked_softmax_bf16(const float* scores, void* p, float* lse,
                                     int B, int H, int S, float scale, int causal, void* stream);
attn_status attn_masked_softmax_f32(const float* scores, float* p, float* lse,
                                    int B, int H, int S, float scale, int causal, void* stream);
attn_status attn_pv_gemm_bf16(const void* p, const void* v, void* out,
                              int B, int Hq, int Hkv, int S, int D, void* stream);
attn_status attn_pv_gemm_f32(const float* p, const float* v, float* out,
                             int B, int Hq, int Hkv, int S, int D, void* stream);

/* ---------------------------------------------------------------------------
 * Backward of the fused forward (bfloat16).
 *
 * Given dout = dL/dout for the forward above (no gradient reaches lse):
 *   delta_i = dout_i . out_i,  dp_ij = dout_i . v_j,
 *   ds_ij = p_ij (dp_ij - delta_i),  p_ij = exp(scale q_i . k_j - lse_i),
 *   dq_i = scale sum_j ds_ij k_j,   dk_j = scale sum_i ds_ij q_i,
 *   dv_j = sum_i p_ij dout_i,
 * the sums over i running over every query that sees key j, in every query
 * head of the key/value head's group.  This is the chain-rule derivative of
 * the forward; the pages only warn that the flash backward is the delicate
 * part (ai-manual.ru tutorial, section 6).
 *
 * q, k, v, causal, scale: as passed to attn_fwd_bf16.  out, lse: that call's
 * results (lse is required here).  dout: bfloat16 [B,Hq,S,D].
 * dq [B,Hq,S,D], dk and dv [B,Hkv,S,D]: bfloat16 outputs, fully written.
 * delta: float32 workspace of attn_bwd_workspace_bytes(B, Hq, S) bytes,
 * overwritten (it ends up holding delta_i).  Outputs and workspace must not
 * overlap the inputs or each other.  Three kernel launches on stream; the
 * probabilities are recomputed on chip, so no S x S buffer is involved.
 * ------------------------------------------------------------------------- */
attn_status attn_bwd_bf16(const void* q, const void* k, const void* v, const void* out, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, float* delta,
                          int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                          void* stream);
/* Bytes of attn_bwd_bf16's delta workspace: B*Hq*S*4, or 0 on a bad size. */
size_t attn_bwd_workspace_bytes(int B, int Hq, int S);

/* Bytes of the float32 score buffer: B*Hq*S*S*4, or 0 if a size is < 1 or
 * the product overflows size_t. */
size_t attn_scores_bytes(int B, int Hq, int S);
/* Bytes of the probability buffer: B*Hq*S*S*elem_bytes (2 for bf16, 4 for
 * float32), or 0 on a bad size. */
size_t attn_probs_bytes(int B, int Hq, int S, int elem_bytes);

/* Static, human-readable name of a status code. */
const char* attn_status_str(attn_status status);
/* The hipError_t of this host thread's last ATTN_ERR_HIP, or 0. */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
