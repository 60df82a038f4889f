// Internal host-side launchers, one per kernel family. The C entry points in
// rf_api.hip validate every argument first and then call these; each launcher
// only enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rf.h"

namespace rf {

// Size of the library-owned device scratch (one copy per GPU) and the lookup
// of its device address on the current device (noalloc.hip).
constexpr size_t kNoallocScratchBytes = RF_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** out);

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                               float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int d,
                               float scale, int causal, hipStream_t stream);

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
                                int causal, hipStream_t stream);

hipError_t launch_decode_split_bf16(const void* q, const void* k, const void* v, float* part_m,
                                    float* part_l, float* part_acc, int B, int Hq, int Hkv, int Lk,
                                    int d, int S, float scale, hipStream_t stream);

hipError_t launch_decode_split_f32(const float* q, const float* k, const float* v, float* part_m,
                                   float* part_l, float* part_acc, int B, int Hq, int Hkv, int Lk,
                                   int d, int S, float scale, hipStream_t stream);

hipError_t launch_merge_states(const float* part_m, const float* part_l, const float* part_acc,
                               int rows, int S, int d, int out_bf16, void* o, float* lse,
                               hipStream_t stream);

hipError_t launch_mla_decode_split(const void* q, const void* kv, float* part_m, float* part_l,
                                   float* part_acc, int B, int H, int Lk, int S, float scale,
                                   int* counters, void* o, float* lse, int out_bf16,
                                   hipStream_t stream);

hipError_t launch_softmax_topk(const float* logits, int T, int E, int k, int renormalize,
                               float* weights, int32_t* indices, hipStream_t stream);

hipError_t launch_softmax_rows(const float* x, int T, int E, int level, float* work, float* y,
                               hipStream_t stream);

hipError_t launch_row_variance(const float* x, int T, int E, int level, float* mean, float* var,
                               hipStream_t stream);

hipError_t launch_row_inertia(const float* x, const float* w, int T, int E, int level,
                              float* centre, float* inertia, hipStream_t stream);

hipError_t launch_absmax_quant_fp8(const void* x, int rows, int cols, uint8_t* q, float* scale,
                                   hipStream_t stream);

hipError_t launch_gemm_fp8_scaled(const uint8_t* a_q, const float* a_scale, const uint8_t* b_q,
                                  const float* b_scale, int M, int N, int K, void* c,
                                  hipStream_t stream);

hipError_t launch_gemm_fp8_running(const void* a, const uint8_t* b_q, const float* b_scale, int M,
                                   int N, int K, float* a_scale, void* c, hipStream_t stream);

hipError_t launch_peak_mfma(int kind, const void* src, int blocks, int iters, float* out,
                            unsigned long long* clk, hipStream_t stream);
hipError_t launch_peak_read(const void* src, long long bytes, int blocks, uint32_t* out,
                            hipStream_t stream);

}  // namespace rf
