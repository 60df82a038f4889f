// C entry points of the library: argument validation, then one or more launches
// on the caller's stream. Validation touches no HIP API, so every argument
// error is returned before anything is enqueued (and works on a machine
// without a GPU); only a launch the runtime refuses can leave earlier launches
// of the same call enqueued.
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>

#include "../../include/rf.h"
#include "rf_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

rf_status fail(rf_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

rf_status ok() {
  g_last_error[0] = '\0';
  return RF_OK;
}

rf_status from_launch(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(RF_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Product of non-negative sizes, saturated at 2^62 so that no argument values
// can overflow it; every "too large" bound below is far under 2^62.
long long prod(std::initializer_list<long long> xs) {
  constexpr long long kSat = 1LL << 62;
  long long p = 1;
  for (const long long x : xs) {
    if (x == 0) return 0;
    p = (p > kSat / x) ? kSat : p * x;
  }
  return p;
}

constexpr long long kMaxElems = 1LL << 40;  // elements in any one tensor
constexpr long long kMaxGrid = 1LL << 31;   // workgroups in one launch dimension

#define RF_REQUIRE(cond, status, ...)            \
  do {                                           \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

}  // namespace

extern "C" {

rf_status rf_attn_fwd(rf_dtype dt, const void* q, const void* k, const void* v, void* o,
                      float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
                      int causal, hipStream_t stream) {
  RF_REQUIRE(dt == RF_F32 || dt == RF_BF16, RF_ERR_INVALID_ARG, "rf_attn_fwd: unknown dtype %d", (int)dt);
  RF_REQUIRE(B >= 0 && Hq >= 0 && Hkv >= 0 && Lq >= 0 && Lk >= 0 && d >= 0, RF_ERR_INVALID_ARG,
             "rf_attn_fwd: negative size");
  if (prod({B, Hq, Lq}) == 0) return ok();
  RF_REQUIRE(Hkv >= 1 && Hq % Hkv == 0, RF_ERR_INVALID_ARG, "rf_attn_fwd: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  RF_REQUIRE(Lk >= 1, RF_ERR_INVALID_ARG, "rf_attn_fwd: Lk must be >= 1");
  RF_REQUIRE(!causal || Lq == Lk, RF_ERR_INVALID_ARG, "rf_attn_fwd: causal needs Lq == Lk (%d != %d)", Lq, Lk);
  RF_REQUIRE(q && k && v && o, RF_ERR_INVALID_ARG, "rf_attn_fwd: null tensor pointer");
  RF_REQUIRE(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(o, 16) && aligned(lse, 4),
             RF_ERR_INVALID_ARG, "rf_attn_fwd: pointers must be 16-byte aligned");
  RF_REQUIRE(__builtin_isfinite(scale), RF_ERR_INVALID_ARG, "rf_attn_fwd: scale is not finite");
  RF_REQUIRE(prod({B, Hq, Lq > Lk ? Lq : Lk, d}) < kMaxElems, RF_ERR_INVALID_ARG,
             "rf_attn_fwd: problem too large");
  if (dt == RF_F32) {
    RF_REQUIRE(d == 64 || d == 128, RF_ERR_UNSUPPORTED, "rf_attn_fwd: fp32 head size %d (need 64 or 128)", d);
    return from_launch(rf::launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                               static_cast<const float*>(v), static_cast<float*>(o), lse,
                                               B, Hq, Hkv, Lq, Lk, d, scale, causal, stream),
                       "rf_attn_fwd");
  }
  RF_REQUIRE(d == 64 || d == 128, RF_ERR_UNSUPPORTED, "rf_attn_fwd: bf16 head size %d (need 64 or 128)", d);
  RF_REQUIRE(prod({Lk, d, 2}) < (1LL << 31), RF_ERR_UNSUPPORTED,
             "rf_attn_fwd: one head's K/V must stay under 2 GiB (Lk=%d)", Lk);
  return from_launch(rf::launch_attn_fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, scale, causal, stream),
                     "rf_attn_fwd");
}

rf_status rf_attn_decode_split(rf_dtype dt, const void* q, const void* k, const void* v,
                               float* part_m, float* part_l, float* part_acc, int B, int Hq,
                               int Hkv, int Lk, int d, int S, float scale, hipStream_t stream) {
  RF_REQUIRE(dt == RF_F32 || dt == RF_BF16, RF_ERR_INVALID_ARG, "rf_attn_decode_split: unknown dtype %d", (int)dt);
  RF_REQUIRE(B >= 0 && Hq >= 0 && Hkv >= 0 && Lk >= 0 && d >= 0, RF_ERR_INVALID_ARG,
             "rf_attn_decode_split: negative size");
  RF_REQUIRE(S >= 1, RF_ERR_INVALID_ARG, "rf_attn_decode_split: S=%d must be >= 1", S);
  if (prod({B, Hq}) == 0) return ok();
  RF_REQUIRE(Hkv >= 1 && Hq % Hkv == 0, RF_ERR_INVALID_ARG,
             "rf_attn_decode_split: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  RF_REQUIRE(Lk >= 1, RF_ERR_INVALID_ARG, "rf_attn_decode_split: Lk must be >= 1");
  RF_REQUIRE(q && k && v && part_m && part_l && part_acc, RF_ERR_INVALID_ARG,
             "rf_attn_decode_split: null tensor pointer");
  RF_REQUIRE(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(part_acc, 16) &&
                 aligned(part_m, 4) && aligned(part_l, 4),
             RF_ERR_INVALID_ARG, "rf_attn_decode_split: pointers must be 16-byte aligned");
  RF_REQUIRE(__builtin_isfinite(scale), RF_ERR_INVALID_ARG, "rf_attn_decode_split: scale is not finite");
  RF_REQUIRE(prod({B, Hkv, Lk, d}) < kMaxElems && prod({B, Hq, S, d}) < kMaxElems && prod({B, Hkv, S}) < kMaxGrid,
             RF_ERR_INVALID_ARG, "rf_attn_decode_split: problem too large");
  RF_REQUIRE(d == 64 || d == 128, RF_ERR_UNSUPPORTED, "rf_attn_decode_split: head size %d (need 64 or 128)", d);
  const int esize = dt == RF_BF16 ? 2 : 4;
  RF_REQUIRE(prod({Lk, d, esize}) < (1LL << 31), RF_ERR_UNSUPPORTED,
             "rf_attn_decode_split: one head's K/V must stay under 2 GiB (Lk=%d)", Lk);
  RF_REQUIRE(Hq / Hkv <= 16, RF_ERR_UNSUPPORTED, "rf_attn_decode_split: GQA group %d > 16", Hq / Hkv);
  if (dt == RF_F32)
    return from_launch(rf::launch_decode_split_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                                   static_cast<const float*>(v), part_m, part_l, part_acc, B,
                                                   Hq, Hkv, Lk, d, S, scale, stream),
                       "rf_attn_decode_split");
  return from_launch(rf::launch_decode_split_bf16(q, k, v, part_m, part_l, part_acc, B, Hq, Hkv, Lk,
                                                  d, S, scale, stream),
                     "rf_attn_decode_split");
}

namespace {

// Arguments shared by rf_mla_decode_split and rf_mla_decode; `fn` names the
// caller in the error text.
rf_status check_mla(const char* fn, const void* q, const void* kv, float* part_m, float* part_l,
                    float* part_acc, int B, int H, int Lk, int Dqk, int Dv, int S, float scale) {
  RF_REQUIRE(Lk >= 1, RF_ERR_INVALID_ARG, "%s: Lk must be >= 1", fn);
  RF_REQUIRE(Dv >= 1 && Dv <= Dqk, RF_ERR_INVALID_ARG, "%s: value width %d must be in 1..%d", fn, Dv, Dqk);
  RF_REQUIRE(q && kv && part_m && part_l && part_acc, RF_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  RF_REQUIRE(aligned(q, 16) && aligned(kv, 16) && aligned(part_acc, 16) && aligned(part_m, 4) &&
                 aligned(part_l, 4),
             RF_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  RF_REQUIRE(__builtin_isfinite(scale), RF_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  RF_REQUIRE(Dqk == 576 && Dv == 512, RF_ERR_UNSUPPORTED,
             "%s: widths %d/%d (need 576 for keys, 512 for values)", fn, Dqk, Dv);
  RF_REQUIRE(H % 16 == 0 && H <= 128, RF_ERR_UNSUPPORTED,
             "%s: H=%d (need a multiple of 16, at most 128)", fn, H);
  RF_REQUIRE(prod({(long long)Lk + 96, Dqk, 2}) < (1LL << 31), RF_ERR_UNSUPPORTED,
             "%s: one sequence's cache reaches 2 GiB", fn);
  RF_REQUIRE(prod({B, S, H / 16}) < kMaxGrid && prod({B, H, S, Dv}) < kMaxElems,
             RF_ERR_INVALID_ARG, "%s: problem too large", fn);
  return ok();
}

}  // namespace

rf_status rf_mla_decode_split(const void* q, const void* kv, float* part_m, float* part_l,
                              float* part_acc, int B, int H, int Lk, int Dqk, int Dv, int S,
                              float scale, hipStream_t stream) {
  RF_REQUIRE(B >= 0 && H >= 0 && Lk >= 0 && Dqk >= 0 && Dv >= 0, RF_ERR_INVALID_ARG,
             "rf_mla_decode_split: negative size");
  RF_REQUIRE(S >= 1, RF_ERR_INVALID_ARG, "rf_mla_decode_split: S=%d must be >= 1", S);
  if (prod({B, H}) == 0) return ok();
  const rf_status st = check_mla("rf_mla_decode_split", q, kv, part_m, part_l, part_acc, B, H, Lk, Dqk,
                                 Dv, S, scale);
  if (st != RF_OK) return st;
  return from_launch(rf::launch_mla_decode_split(q, kv, part_m, part_l, part_acc, B, H, Lk, S, scale,
                                                 nullptr, nullptr, nullptr, 0, stream),
                     "rf_mla_decode_split");
}

rf_status rf_mla_decode(const void* q, const void* kv, float* part_m, float* part_l, float* part_acc,
                        int32_t* counters, rf_dtype out_dt, void* o, float* lse, int B, int H, int Lk,
                        int Dqk, int Dv, int S, float scale, hipStream_t stream) {
  RF_REQUIRE(out_dt == RF_F32 || out_dt == RF_BF16, RF_ERR_INVALID_ARG,
             "rf_mla_decode: unknown dtype %d", (int)out_dt);
  RF_REQUIRE(B >= 0 && H >= 0 && Lk >= 0 && Dqk >= 0 && Dv >= 0, RF_ERR_INVALID_ARG,
             "rf_mla_decode: negative size");
  RF_REQUIRE(S >= 1, RF_ERR_INVALID_ARG, "rf_mla_decode: S=%d must be >= 1", S);
  if (prod({B, H}) == 0) return ok();
  const rf_status st = check_mla("rf_mla_decode", q, kv, part_m, part_l, part_acc, B, H, Lk, Dqk, Dv,
                                 S, scale);
  if (st != RF_OK) return st;
  RF_REQUIRE(counters && o, RF_ERR_INVALID_ARG, "rf_mla_decode: null counters or output");
  RF_REQUIRE(aligned(counters, 4) && aligned(o, 16) && aligned(lse, 4), RF_ERR_INVALID_ARG,
             "rf_mla_decode: misaligned pointer");
  return from_launch(rf::launch_mla_decode_split(q, kv, part_m, part_l, part_acc, B, H, Lk, S, scale,
                                                 counters, o, lse, out_dt == RF_BF16 ? 1 : 0, stream),
                     "rf_mla_decode");
}

rf_status rf_merge_states(const float* part_m, const float* part_l, const float* part_acc,
                          int rows, int S, int d, rf_dtype out_dt, void* o, float* lse,
                          hipStream_t stream) {
  RF_REQUIRE(out_dt == RF_F32 || out_dt == RF_BF16, RF_ERR_INVALID_ARG,
             "rf_merge_states: unknown dtype %d", (int)out_dt);
  RF_REQUIRE(rows >= 0 && d >= 0, RF_ERR_INVALID_ARG, "rf_merge_states: negative size");
  RF_REQUIRE(S >= 1, RF_ERR_INVALID_ARG, "rf_merge_states: S=%d must be >= 1", S);
  if (rows == 0) return ok();
  RF_REQUIRE(d >= 1 && d <= 1024 && d % 4 == 0, RF_ERR_UNSUPPORTED,
             "rf_merge_states: d=%d (need 4 <= d <= 1024, d %% 4 == 0)", d);
  RF_REQUIRE(part_m && part_l && part_acc && o, RF_ERR_INVALID_ARG, "rf_merge_states: null tensor pointer");
  RF_REQUIRE(aligned(part_acc, 16) && aligned(o, out_dt == RF_BF16 ? 8 : 16) && aligned(part_m, 4) &&
                 aligned(part_l, 4) && aligned(lse, 4),
             RF_ERR_INVALID_ARG, "rf_merge_states: misaligned pointer");
  RF_REQUIRE(prod({rows, S, d}) < kMaxElems, RF_ERR_INVALID_ARG, "rf_merge_states: problem too large");
  return from_launch(rf::launch_merge_states(part_m, part_l, part_acc, rows, S, d, out_dt == RF_BF16, o,
                                             lse, stream),
                     "rf_merge_states");
}

rf_status rf_softmax_topk(const float* logits, int T, int E, int k, int renormalize,
                          float* weights, int32_t* indices, hipStream_t stream) {
  RF_REQUIRE(T >= 0 && E >= 0, RF_ERR_INVALID_ARG, "rf_softmax_topk: negative size");
  RF_REQUIRE(E >= 1 && k >= 1 && k <= E, RF_ERR_INVALID_ARG, "rf_softmax_topk: need 1 <= k <= E (k=%d, E=%d)", k, E);
  if (T == 0) return ok();
  RF_REQUIRE(E <= 1024 && E % 4 == 0, RF_ERR_UNSUPPORTED, "rf_softmax_topk: E=%d (need E <= 1024, E %% 4 == 0)", E);
  RF_REQUIRE(k <= 32, RF_ERR_UNSUPPORTED, "rf_softmax_topk: k=%d > 32", k);
  RF_REQUIRE(prod({T, E}) < kMaxElems, RF_ERR_INVALID_ARG, "rf_softmax_topk: problem too large");
  RF_REQUIRE(logits && weights && indices, RF_ERR_INVALID_ARG, "rf_softmax_topk: null tensor pointer");
  RF_REQUIRE(aligned(logits, 16) && aligned(weights, 4) && aligned(indices, 4), RF_ERR_INVALID_ARG,
             "rf_softmax_topk: misaligned pointer");
  return from_launch(rf::launch_softmax_topk(logits, T, E, k, renormalize != 0, weights, indices, stream),
                     "rf_softmax_topk");
}

rf_status rf_peak_mfma(int kind, const void* src, int blocks, int iters, float* out,
                       unsigned long long* clock, hipStream_t stream) {
  RF_REQUIRE(kind == RF_PEAK_BF16 || kind == RF_PEAK_FP8, RF_ERR_INVALID_ARG,
             "rf_peak_mfma: unknown kind %d", kind);
  RF_REQUIRE(blocks >= 1 && blocks <= 65536, RF_ERR_INVALID_ARG,
             "rf_peak_mfma: blocks=%d outside 1..65536", blocks);
  RF_REQUIRE(iters >= 1 && iters <= (1 << 20), RF_ERR_INVALID_ARG,
             "rf_peak_mfma: iters=%d outside 1..2^20", iters);
  RF_REQUIRE(src && out, RF_ERR_INVALID_ARG, "rf_peak_mfma: null pointer");
  RF_REQUIRE(aligned(src, 32) && aligned(out, 4) && aligned(clock, 8), RF_ERR_INVALID_ARG,
             "rf_peak_mfma: misaligned pointer");
  return from_launch(rf::launch_peak_mfma(kind, src, blocks, iters, out, clock, stream),
                     "rf_peak_mfma");
}

rf_status rf_peak_read(const void* src, long long bytes, int blocks, uint32_t* out,
                       hipStream_t stream) {
  RF_REQUIRE(bytes >= 0 && bytes % 16 == 0 && bytes < kMaxElems, RF_ERR_INVALID_ARG,
             "rf_peak_read: bytes=%lld must be a non-negative multiple of 16 below 2^40", bytes);
  RF_REQUIRE(blocks >= 1 && blocks <= 65536, RF_ERR_INVALID_ARG,
             "rf_peak_read: blocks=%d outside 1..65536", blocks);
  RF_REQUIRE(out && (src || bytes == 0), RF_ERR_INVALID_ARG, "rf_peak_read: null pointer");
  RF_REQUIRE(aligned(src, 16) && aligned(out, 4), RF_ERR_INVALID_ARG, "rf_peak_read: misaligned pointer");
  return from_launch(rf::launch_peak_read(src, bytes, blocks, out, stream), "rf_peak_read");
}

rf_status rf_wall_clock_khz(int* khz) {
  RF_REQUIRE(khz, RF_ERR_INVALID_ARG, "rf_wall_clock_khz: null pointer");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return from_launch(e, "rf_wall_clock_khz");
}

rf_status rf_softmax(const float* x, int T, int E, int level, float* work, float* y,
                     hipStream_t stream) {
  RF_REQUIRE(T >= 0 && E >= 0, RF_ERR_INVALID_ARG, "rf_softmax: negative size");
  RF_REQUIRE(level >= RF_FUSE_NONE && level <= RF_FUSE_BLOCK, RF_ERR_INVALID_ARG,
             "rf_softmax: unknown fusion level %d", level);
  if (T == 0) return ok();
  RF_REQUIRE(E >= 4 && E % 4 == 0, RF_ERR_INVALID_ARG, "rf_softmax: E=%d must be a positive multiple of 4", E);
  RF_REQUIRE(E <= 8192, RF_ERR_UNSUPPORTED, "rf_softmax: E=%d > 8192", E);
  RF_REQUIRE(x && y, RF_ERR_INVALID_ARG, "rf_softmax: null tensor pointer");
  RF_REQUIRE(level != RF_FUSE_NONE || work, RF_ERR_INVALID_ARG,
             "rf_softmax: the unfused cascade needs a workspace of 2*T floats");
  RF_REQUIRE(aligned(x, 16) && aligned(y, 16) && aligned(work, 4), RF_ERR_INVALID_ARG,
             "rf_softmax: misaligned pointer");
  RF_REQUIRE(prod({T, E}) < kMaxElems, RF_ERR_INVALID_ARG, "rf_softmax: problem too large");
  return from_launch(rf::launch_softmax_rows(x, T, E, level, work, y, stream), "rf_softmax");
}

rf_status rf_row_variance(const float* x, int T, int E, int level, float* mean, float* var,
                          hipStream_t stream) {
  RF_REQUIRE(T >= 0 && E >= 0, RF_ERR_INVALID_ARG, "rf_row_variance: negative size");
  RF_REQUIRE(level >= RF_FUSE_NONE && level <= RF_FUSE_BLOCK, RF_ERR_INVALID_ARG,
             "rf_row_variance: unknown fusion level %d", level);
  if (T == 0) return ok();
  RF_REQUIRE(E >= 4 && E % 4 == 0, RF_ERR_INVALID_ARG, "rf_row_variance: E=%d must be a positive multiple of 4", E);
  RF_REQUIRE(E <= 8192, RF_ERR_UNSUPPORTED, "rf_row_variance: E=%d > 8192", E);
  RF_REQUIRE(x && mean && var, RF_ERR_INVALID_ARG, "rf_row_variance: null tensor pointer");
  RF_REQUIRE(aligned(x, 16) && aligned(mean, 4) && aligned(var, 4), RF_ERR_INVALID_ARG,
             "rf_row_variance: misaligned pointer");
  RF_REQUIRE(prod({T, E}) < kMaxElems, RF_ERR_INVALID_ARG, "rf_row_variance: problem too large");
  return from_launch(rf::launch_row_variance(x, T, E, level, mean, var, stream), "rf_row_variance");
}

rf_status rf_row_inertia(const float* x, const float* w, int T, int E, int level, float* centre,
                         float* inertia, hipStream_t stream) {
  RF_REQUIRE(T >= 0 && E >= 0, RF_ERR_INVALID_ARG, "rf_row_inertia: negative size");
  RF_REQUIRE(level >= RF_FUSE_NONE && level <= RF_FUSE_BLOCK, RF_ERR_INVALID_ARG,
             "rf_row_inertia: unknown fusion level %d", level);
  if (T == 0) return ok();
  RF_REQUIRE(E >= 4 && E % 4 == 0, RF_ERR_INVALID_ARG, "rf_row_inertia: E=%d must be a positive multiple of 4", E);
  RF_REQUIRE(E <= 8192, RF_ERR_UNSUPPORTED, "rf_row_inertia: E=%d > 8192", E);
  RF_REQUIRE(x && w && centre && inertia, RF_ERR_INVALID_ARG, "rf_row_inertia: null tensor pointer");
  RF_REQUIRE(aligned(x, 16) && aligned(w, 16) && aligned(centre, 4) && aligned(inertia, 4),
             RF_ERR_INVALID_ARG, "rf_row_inertia: misaligned pointer");
  RF_REQUIRE(prod({T, E}) < kMaxElems, RF_ERR_INVALID_ARG, "rf_row_inertia: problem too large");
  return from_launch(rf::launch_row_inertia(x, w, T, E, level, centre, inertia, stream), "rf_row_inertia");
}

rf_status rf_absmax_quant_fp8(const void* x, int rows, int cols, uint8_t* q, float* scale,
                              hipStream_t stream) {
  RF_REQUIRE(rows >= 0 && cols >= 0, RF_ERR_INVALID_ARG, "rf_absmax_quant_fp8: negative size");
  if (rows == 0) return ok();
  RF_REQUIRE(cols >= 8 && cols % 8 == 0, RF_ERR_INVALID_ARG, "rf_absmax_quant_fp8: cols=%d must be a positive multiple of 8", cols);
  RF_REQUIRE(cols <= 8192, RF_ERR_UNSUPPORTED, "rf_absmax_quant_fp8: cols=%d > 8192", cols);
  RF_REQUIRE(prod({rows, cols}) < kMaxElems, RF_ERR_INVALID_ARG, "rf_absmax_quant_fp8: problem too large");
  RF_REQUIRE(x && q && scale, RF_ERR_INVALID_ARG, "rf_absmax_quant_fp8: null tensor pointer");
  RF_REQUIRE(aligned(x, 16) && aligned(q, 8) && aligned(scale, 4), RF_ERR_INVALID_ARG,
             "rf_absmax_quant_fp8: misaligned pointer");
  return from_launch(rf::launch_absmax_quant_fp8(x, rows, cols, q, scale, stream), "rf_absmax_quant_fp8");
}

rf_status rf_absmax_quant_gemm_fp8(const void* a, const uint8_t* b, const float* b_scale, int M,
                                   int N, int K, uint8_t* a_q, float* a_scale, void* c,
                                   hipStream_t stream) {
  RF_REQUIRE(M >= 0 && N >= 0 && K >= 0, RF_ERR_INVALID_ARG, "rf_absmax_quant_gemm_fp8: negative size");
  if (prod({M, N}) == 0) return ok();
  RF_REQUIRE(K >= 128 && K % 128 == 0, RF_ERR_INVALID_ARG,
             "rf_absmax_quant_gemm_fp8: K=%d must be a positive multiple of 128", K);
  RF_REQUIRE(K <= 8192, RF_ERR_UNSUPPORTED, "rf_absmax_quant_gemm_fp8: K=%d > 8192", K);
  RF_REQUIRE(prod({M, K}) < kMaxElems && prod({N, K}) < kMaxElems && prod({M, N}) < kMaxElems,
             RF_ERR_INVALID_ARG, "rf_absmax_quant_gemm_fp8: problem too large");
  RF_REQUIRE(a && b && b_scale && a_q && a_scale && c, RF_ERR_INVALID_ARG,
             "rf_absmax_quant_gemm_fp8: null tensor pointer");
  RF_REQUIRE(aligned(a, 16) && aligned(b, 16) && aligned(a_q, 16) && aligned(c, 4) &&
                 aligned(b_scale, 4) && aligned(a_scale, 4),
             RF_ERR_INVALID_ARG, "rf_absmax_quant_gemm_fp8: misaligned pointer");
  hipError_t e = rf::launch_absmax_quant_fp8(a, M, K, a_q, a_scale, stream);
  if (e != hipSuccess) return from_launch(e, "rf_absmax_quant_gemm_fp8 (quantise)");
  return from_launch(rf::launch_gemm_fp8_scaled(a_q, a_scale, b, b_scale, M, N, K, c, stream),
                     "rf_absmax_quant_gemm_fp8 (gemm)");
}

rf_status rf_absmax_quant_gemm_fp8_noalloc(const void* a, const uint8_t* b, const float* b_scale,
                                           int M, int N, int K, float* a_scale, void* c,
                                           hipStream_t stream) {
  RF_REQUIRE(M >= 0 && N >= 0 && K >= 0, RF_ERR_INVALID_ARG, "rf_absmax_quant_gemm_fp8_noalloc: negative size");
  if (prod({M, N}) == 0) return ok();
  RF_REQUIRE(K >= 128 && K % 128 == 0, RF_ERR_INVALID_ARG,
             "rf_absmax_quant_gemm_fp8_noalloc: K=%d must be a positive multiple of 128", K);
  RF_REQUIRE(K <= 8192, RF_ERR_UNSUPPORTED, "rf_absmax_quant_gemm_fp8_noalloc: K=%d > 8192", K);
  RF_REQUIRE(prod({M, K}) < kMaxElems && prod({N, K}) < kMaxElems && prod({M, N}) < kMaxElems,
             RF_ERR_INVALID_ARG, "rf_absmax_quant_gemm_fp8_noalloc: problem too large");
  RF_REQUIRE(prod({M, K}) <= (long long)rf::kNoallocScratchBytes, RF_ERR_UNSUPPORTED,
             "rf_absmax_quant_gemm_fp8_noalloc: M*K=%lld bytes of quantised A exceed the %lld-byte "
             "scratch (use rf_absmax_quant_gemm_fp8 with a workspace)",
             prod({M, K}), (long long)rf::kNoallocScratchBytes);
  RF_REQUIRE(a && b && b_scale && a_scale && c, RF_ERR_INVALID_ARG,
             "rf_absmax_quant_gemm_fp8_noalloc: null tensor pointer");
  RF_REQUIRE(aligned(a, 16) && aligned(b, 16) && aligned(c, 4) && aligned(b_scale, 4) &&
                 aligned(a_scale, 4),
             RF_ERR_INVALID_ARG, "rf_absmax_quant_gemm_fp8_noalloc: misaligned pointer");
  void* a_q = nullptr;
  hipError_t e = rf::noalloc_scratch(&a_q);
  if (e != hipSuccess) return from_launch(e, "rf_absmax_quant_gemm_fp8_noalloc (scratch address)");
  e = rf::launch_absmax_quant_fp8(a, M, K, static_cast<uint8_t*>(a_q), a_scale, stream);
  if (e != hipSuccess) return from_launch(e, "rf_absmax_quant_gemm_fp8_noalloc (quantise)");
  return from_launch(rf::launch_gemm_fp8_scaled(static_cast<const uint8_t*>(a_q), a_scale, b, b_scale, M,
                                                N, K, c, stream),
                     "rf_absmax_quant_gemm_fp8_noalloc (gemm)");
}

rf_status rf_absmax_quant_gemm_fp8_running(const void* a, const uint8_t* b, const float* b_scale,
                                           int M, int N, int K, float* a_scale, void* c,
                                           hipStream_t stream) {
  RF_REQUIRE(M >= 0 && N >= 0 && K >= 0, RF_ERR_INVALID_ARG,
             "rf_absmax_quant_gemm_fp8_running: negative size");
  if (prod({M, N}) == 0) return ok();
  RF_REQUIRE(K >= 128 && K % 128 == 0, RF_ERR_INVALID_ARG,
             "rf_absmax_quant_gemm_fp8_running: K=%d must be a positive multiple of 128", K);
  RF_REQUIRE(K <= 8192, RF_ERR_UNSUPPORTED, "rf_absmax_quant_gemm_fp8_running: K=%d > 8192", K);
  RF_REQUIRE(prod({M, K}) < kMaxElems && prod({N, K}) < kMaxElems && prod({M, N}) < kMaxElems,
             RF_ERR_INVALID_ARG, "rf_absmax_quant_gemm_fp8_running: problem too large");
  RF_REQUIRE(a && b && b_scale && a_scale && c, RF_ERR_INVALID_ARG,
             "rf_absmax_quant_gemm_fp8_running: null tensor pointer");
  RF_REQUIRE(aligned(a, 16) && aligned(b, 16) && aligned(c, 4) && aligned(b_scale, 4) &&
                 aligned(a_scale, 4),
             RF_ERR_INVALID_ARG, "rf_absmax_quant_gemm_fp8_running: misaligned pointer");
  return from_launch(rf::launch_gemm_fp8_running(a, b, b_scale, M, N, K, a_scale, c, stream),
                     "rf_absmax_quant_gemm_fp8_running");
}

const char* rf_status_string(rf_status s) {
  switch (s) {
    case RF_OK: return "RF_OK";
    case RF_ERR_INVALID_ARG: return "RF_ERR_INVALID_ARG";
    case RF_ERR_UNSUPPORTED: return "RF_ERR_UNSUPPORTED";
    case RF_ERR_LAUNCH: return "RF_ERR_LAUNCH";
    default: break;
  }
  return "unknown rf_status";
}

const char* rf_last_error(void) { return g_last_error; }

int rf_abi_version(void) { return RF_ABI_VERSION; }

#ifndef RF_BUILD_ID
#error "RF_BUILD_ID (the hash of the sources) is set by the build"
#endif
const char* rf_build_id(void) { return RF_BUILD_ID; }

}  // extern "C"
