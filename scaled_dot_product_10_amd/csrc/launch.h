// Internal launchers behind the C ABI (include/attn.h).  Arguments are
// already validated by the caller; each launcher enqueues exactly one kernel,
// except the backward's (three) and the split-KV forward's (two).
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;  // may be null
    int B, Hq, Hkv, S, D;
    float scale;  // > 0, finite
    int causal;   // 0 or 1
    int window;   // 0: none; >= 1 (bf16, causal only): sliding window of this many keys
    // bf16 only: block mask, one byte per 64 x 64 block at
    // bmask[b * bmask_stride_b + h * bmask_stride_h + qb * ceil(S/64) + kb]; null: none
    const uint8_t* bmask = nullptr;
    int64_t bmask_stride_b = 0, bmask_stride_h = 0;
    // bf16 only, optional: kStampWords 64-bit words per workgroup (stamped launch)
    unsigned long long* stamps = nullptr;
};

constexpr int kStampWords = 8;
// GPUs of one process with per-device cached state (for example CU counts)
constexpr int kMaxDevices = 64;
// Workgroups a bf16 forward launch may use (stamp records to provide).
int64_t fwd_bf16_max_workgroups(int B, int Hq, int S);

struct QkArgs {
    const void* q;
    const void* k;
    float* scores;
    int B, Hq, Hkv, S, D;
};

struct SoftmaxArgs {
    const float* scores;
    void* p;
    float* lse;  // may be null
    int B, H, S;
    float scale;
    int causal;
};

struct PvArgs {
    const void* p;
    const void* v;
    void* out;
    int B, Hq, Hkv, S, D;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* delta;  // workspace [B, Hq, S]
    int B, Hq, Hkv, S, D;
    float scale;
    int causal;
};

struct Fp8Args {
    const void* q;  // e4m3 codes [B, Hq, S, D]
    const void* k;  // e4m3 codes [B, Hkv, S, D]
    const void* v;
    void* out;      // bf16 [B, Hq, S, D]
    float* lse;     // may be null
    int B, Hq, Hkv, S, D;
    float scale, q_scale, k_scale, v_scale;
    int causal;
};

struct SplitKvArgs {
    const void* q;     // [B, Hq, Sq, D]
    const void* k;     // [B, Hkv, Skv, D]
    const void* v;
    void* out;         // [B, Hq, Sq, D]
    float* lse;        // [B, Hq, Sq] or null
    float* workspace;  // nsplit * B*Hq*Sq * (D + 1) floats
    int B, Hq, Hkv, Sq, Skv, D;
    float scale;
    int causal;
    int nsplit;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);
hipError_t launch_qk_gemm_bf16(const QkArgs& a, hipStream_t stream);
hipError_t launch_qk_gemm_f32(const QkArgs& a, hipStream_t stream);
hipError_t launch_masked_softmax_bf16(const SoftmaxArgs& a, hipStream_t stream);
hipError_t launch_masked_softmax_f32(const SoftmaxArgs& a, hipStream_t stream);
hipError_t launch_pv_gemm_bf16(const PvArgs& a, hipStream_t stream);
hipError_t launch_pv_gemm_f32(const PvArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);          // three kernels
hipError_t launch_splitkv_bf16(const SplitKvArgs& a, hipStream_t stream);  // two kernels
// Allocation-free split-KV: floats of the library's per-GPU scratch (16 MiB),
// and its device address on the stream's GPU (looked up on first use there).
constexpr int64_t kSplitkvScratchFloats = int64_t(4) << 20;
hipError_t splitkv_scratch(hipStream_t stream, float** ptr);
int splitkv_row_blocks(int Hq, int Hkv, int Sq);  // workgroups per (b, kv head) and split
int splitkv_chunk();                              // keys per workgroup step

}  // namespace attn
