// Calls every C entry point with invalid, extreme, empty and valid arguments
// and checks the status each returns and how many launches it made. Built
// with the launchers replaced by host-only stand-ins (stub_launchers.cpp) and
// run under AddressSanitizer and UndefinedBehaviorSanitizer: any overflow in
// the size arithmetic, out-of-range read of the error text or other undefined
// behaviour in the validation code stops the run.
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "../../include/rf.h"

extern int g_stub_calls;
extern hipError_t g_stub_status;

namespace {

int g_fails = 0;
void* const F = reinterpret_cast<void*>(0x10000);    // never dereferenced
void* const MIS = reinterpret_cast<void*>(0x10004);  // 4-byte aligned only
float* const FF = static_cast<float*>(F);
uint8_t* const FU = static_cast<uint8_t*>(F);
const int BIG = INT_MAX;

void check(int line, rf_status got, rf_status want, int launches_before, int launches_want) {
  const int launched = g_stub_calls - launches_before;
  if (got != want || launched != launches_want) {
    fprintf(stderr, "line %d: status %d (want %d), %d launches (want %d): %s\n", line, (int)got, (int)want,
            launched, launches_want, rf_last_error());
    ++g_fails;
  }
  if (got != RF_OK && strlen(rf_last_error()) == 0) {
    fprintf(stderr, "line %d: error without detail text\n", line);
    ++g_fails;
  }
}

#define EXPECT(call, want, launches)                 \
  do {                                               \
    const int before_ = g_stub_calls;                \
    const rf_status s_ = (call);                     \
    check(__LINE__, s_, (want), before_, (launches)); \
  } while (0)

rf_status attn(rf_dtype dt, void* q, void* o, int B, int Hq, int Hkv, int Lq, int Lk, int d, float scale,
               int causal) {
  return rf_attn_fwd(dt, q, F, F, o, FF, B, Hq, Hkv, Lq, Lk, d, scale, causal, nullptr);
}

rf_status dec(rf_dtype dt, void* k, int B, int Hq, int Hkv, int Lk, int d, int S) {
  return rf_attn_decode_split(dt, F, k, F, FF, FF, FF, B, Hq, Hkv, Lk, d, S, 0.1f, nullptr);
}

}  // namespace

int main() {
  const rf_status OK = RF_OK, INV = RF_ERR_INVALID_ARG, UNS = RF_ERR_UNSUPPORTED, LAUNCH = RF_ERR_LAUNCH;

  // ---- attention
  EXPECT(attn(RF_BF16, F, F, 1, 4, 2, 64, 64, 128, 0.1f, 0), OK, 1);
  EXPECT(attn(RF_BF16, F, F, 2, 8, 8, 300, 300, 64, 0.1f, 1), OK, 1);
  EXPECT(attn(RF_F32, F, F, 1, 4, 2, 64, 64, 64, 0.1f, 0), OK, 1);
  EXPECT(attn(RF_BF16, nullptr, nullptr, 0, 4, 2, 64, 64, 128, 0.1f, 0), OK, 0);
  EXPECT(attn((rf_dtype)7, F, F, 1, 4, 2, 64, 64, 128, 0.1f, 0), INV, 0);
  EXPECT(attn(RF_BF16, F, F, -1, 4, 2, 64, 64, 128, 0.1f, 0), INV, 0);
  EXPECT(attn(RF_BF16, F, F, 1, 4, 3, 64, 64, 128, 0.1f, 0), INV, 0);
  EXPECT(attn(RF_BF16, F, F, 1, 4, 0, 64, 64, 128, 0.1f, 0), INV, 0);
  EXPECT(attn(RF_BF16, F, F, 1, 4, 2, 64, 32, 128, 0.1f, 1), INV, 0);
  EXPECT(attn(RF_BF16, F, MIS, 1, 4, 2, 64, 64, 128, 0.1f, 0), INV, 0);
  EXPECT(attn(RF_BF16, F, F, 1, 4, 2, 64, 64, 128, NAN, 0), INV, 0);
  EXPECT(attn(RF_BF16, F, F, 1, 4, 2, 64, 64, 128, INFINITY, 0), INV, 0);
  EXPECT(attn(RF_BF16, F, F, 1, 4, 2, 64, 64, 128, 0.f, 0), OK, 1);
  EXPECT(attn(RF_BF16, F, F, 1, 4, 2, 64, 64, 128, -0.5f, 1), OK, 1);
  EXPECT(attn(RF_BF16, F, F, 1, 4, 2, 64, 64, 96, 0.1f, 0), UNS, 0);
  EXPECT(attn(RF_BF16, F, F, BIG, BIG, 1, BIG, BIG, 128, 0.1f, 0), INV, 0);    // too large
  EXPECT(attn(RF_BF16, F, F, 1, BIG, BIG, BIG, BIG, BIG, 0.1f, 0), INV, 0);
  EXPECT(attn(RF_BF16, F, F, 1, 1, 1, 1, BIG, 128, 0.1f, 0), UNS, 0);   // one head's K reaches 2 GiB

  // ---- split-KV decode
  EXPECT(dec(RF_BF16, F, 1, 8, 2, 100, 128, 4), OK, 1);
  EXPECT(dec(RF_F32, F, 2, 6, 2, 100, 64, 64), OK, 1);
  EXPECT(dec(RF_BF16, F, 0, 8, 2, 100, 128, 4), OK, 0);
  EXPECT(dec(RF_BF16, F, 1, 8, 2, 100, 128, 0), INV, 0);
  EXPECT(dec(RF_BF16, MIS, 1, 8, 2, 100, 128, 4), INV, 0);
  EXPECT(dec(RF_BF16, F, 1, 34, 2, 100, 128, 4), UNS, 0);
  EXPECT(dec(RF_F32, F, 1, 8, 2, 1 << 22, 128, 4), UNS, 0);
  EXPECT(dec(RF_BF16, F, BIG, BIG, 1, BIG, BIG, BIG), INV, 0);
  EXPECT(dec(RF_BF16, F, 1, 16, 1, BIG, 128, BIG), INV, 0);

  // ---- merge
  EXPECT(rf_merge_states(FF, FF, FF, 4, 2, 128, RF_BF16, F, FF, nullptr), OK, 1);
  EXPECT(rf_merge_states(FF, FF, FF, 4, 0, 128, RF_BF16, F, nullptr, nullptr), INV, 0);
  EXPECT(rf_merge_states(FF, FF, FF, BIG, BIG, 1024, RF_F32, F, nullptr, nullptr), INV, 0);
  EXPECT(rf_merge_states(nullptr, nullptr, nullptr, 0, 2, 128, RF_BF16, nullptr, nullptr, nullptr), OK, 0);

  // ---- multi-latent decode
  EXPECT(rf_mla_decode_split(F, F, FF, FF, FF, 2, 16, 100, 576, 512, 4, 0.1f, nullptr), OK, 1);
  EXPECT(rf_mla_decode_split(F, F, FF, FF, FF, BIG, 128, BIG, 576, 512, BIG, 0.1f, nullptr), UNS, 0);
  EXPECT(rf_mla_decode_split(F, F, FF, FF, FF, BIG, 128, 1000, 576, 512, BIG, 0.1f, nullptr), INV, 0);
  EXPECT(rf_mla_decode(F, F, FF, FF, FF, static_cast<int32_t*>(F), RF_BF16, F, FF, 2, 16, 100, 576, 512,
                       4, 0.1f, nullptr),
         OK, 1);
  EXPECT(rf_mla_decode(F, F, FF, FF, FF, nullptr, RF_BF16, F, FF, 2, 16, 100, 576, 512, 4, 0.1f, nullptr),
         INV, 0);

  // ---- routing and row reductions
  EXPECT(rf_softmax_topk(FF, 10, 256, 8, 1, FF, static_cast<int32_t*>(F), nullptr), OK, 1);
  EXPECT(rf_softmax_topk(FF, BIG, 1024, 32, 1, FF, static_cast<int32_t*>(F), nullptr), INV, 0);
  EXPECT(rf_softmax_topk(FF, 10, BIG, 8, 1, FF, static_cast<int32_t*>(F), nullptr), UNS, 0);
  EXPECT(rf_softmax(FF, 10, 1024, 0, FF, FF, nullptr), OK, 1);
  EXPECT(rf_softmax(FF, 10, 1024, 3, nullptr, FF, nullptr), OK, 1);
  EXPECT(rf_softmax(FF, BIG, 8192, 3, nullptr, FF, nullptr), INV, 0);
  EXPECT(rf_softmax(FF, 10, INT_MIN, 3, nullptr, FF, nullptr), INV, 0);
  EXPECT(rf_row_variance(FF, 10, 1024, 2, FF, FF, nullptr), OK, 1);
  EXPECT(rf_row_variance(FF, BIG, 8192, 2, FF, FF, nullptr), INV, 0);
  EXPECT(rf_row_inertia(FF, FF, 10, 1024, 1, FF, FF, nullptr), OK, 1);
  EXPECT(rf_row_inertia(FF, FF, BIG, 8192, 1, FF, FF, nullptr), INV, 0);

  // ---- FP8
  EXPECT(rf_absmax_quant_fp8(F, 4, 64, FU, FF, nullptr), OK, 1);
  EXPECT(rf_absmax_quant_fp8(F, BIG, 8192, FU, FF, nullptr), INV, 0);
  EXPECT(rf_absmax_quant_gemm_fp8(F, FU, FF, 64, 64, 256, FU, FF, F, nullptr), OK, 2);
  EXPECT(rf_absmax_quant_gemm_fp8(F, FU, FF, BIG, BIG, 8192, FU, FF, F, nullptr), INV, 0);
  EXPECT(rf_absmax_quant_gemm_fp8_running(F, FU, FF, 64, 64, 256, FF, F, nullptr), OK, 1);
  EXPECT(rf_absmax_quant_gemm_fp8_running(F, FU, FF, BIG, BIG, 8192, FF, F, nullptr), INV, 0);
  EXPECT(rf_absmax_quant_gemm_fp8_noalloc(F, FU, FF, 64, 64, 256, FF, F, nullptr), OK, 3);
  EXPECT(rf_absmax_quant_gemm_fp8_noalloc(F, FU, FF, BIG, BIG, 8192, FF, F, nullptr), INV, 0);
  EXPECT(rf_absmax_quant_gemm_fp8_noalloc(F, FU, FF, 4097, 64, 8192, FF, F, nullptr), UNS, 0);  // scratch
  EXPECT(rf_absmax_quant_gemm_fp8_noalloc(F, FU, FF, 4096, 64, 8192, FF, F, nullptr), OK, 3);

  // ---- measurement support
  EXPECT(rf_peak_mfma(0, F, 4, 8, FF, nullptr, nullptr), OK, 1);
  EXPECT(rf_peak_mfma(0, F, BIG, BIG, FF, nullptr, nullptr), INV, 0);
  EXPECT(rf_peak_read(F, 1024, 4, static_cast<uint32_t*>(F), nullptr), OK, 1);
  EXPECT(rf_peak_read(F, LLONG_MAX - 15, BIG, static_cast<uint32_t*>(F), nullptr), INV, 0);

  // ---- a launch the runtime refuses: the status names it, the first of two
  // launches stays made
  g_stub_status = hipErrorInvalidConfiguration;
  EXPECT(rf_softmax_topk(FF, 10, 256, 8, 1, FF, static_cast<int32_t*>(F), nullptr), LAUNCH, 1);
  EXPECT(rf_absmax_quant_gemm_fp8(F, FU, FF, 64, 64, 256, FU, FF, F, nullptr), LAUNCH, 1);
  g_stub_status = hipSuccess;

  for (int s = 0; s <= 4; ++s) {
    const char* name = rf_status_string((rf_status)s);
    if (!name || !*name) {
      fprintf(stderr, "no name for status %d\n", s);
      ++g_fails;
    }
  }
  if (rf_abi_version() != RF_ABI_VERSION || strlen(rf_build_id()) == 0) ++g_fails;

  printf("%s: %d failure(s)\n", g_fails ? "FAILED" : "passed", g_fails);
  return g_fails ? 1 : 0;
}
