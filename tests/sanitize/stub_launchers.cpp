// Host-only stand-ins for the kernel launchers behind the C entry points, so
// that the entry points' own host code (validation, dispatch, error text) can
// run under AddressSanitizer and UndefinedBehaviorSanitizer on a machine
// without a GPU. Each stand-in counts its calls and returns g_stub_status.
#include "../../online_softmax_attention_cascaded_amd/csrc/rf_launch.hpp"

int g_stub_calls = 0;
hipError_t g_stub_status = hipSuccess;

namespace {
hipError_t called() {
  ++g_stub_calls;
  return g_stub_status;
}
}  // namespace

namespace rf {

hipError_t noalloc_scratch(void** out) {
  static unsigned char fake[64];
  *out = fake;
  return called();
}
hipError_t launch_attn_fwd_f32(const float*, const float*, const float*, float*, float*, int, int,
                               int, int, int, int, float, int, hipStream_t) {
  return called();
}
hipError_t launch_attn_fwd_bf16(const void*, const void*, const void*, void*, float*, int, int, int,
                                int, int, int, float, int, hipStream_t) {
  return called();
}
hipError_t launch_decode_split_bf16(const void*, const void*, const void*, float*, float*, float*,
                                    int, int, int, int, int, int, float, hipStream_t) {
  return called();
}
hipError_t launch_decode_split_f32(const float*, const float*, const float*, float*, float*, float*,
                                   int, int, int, int, int, int, float, hipStream_t) {
  return called();
}
hipError_t launch_merge_states(const float*, const float*, const float*, int, int, int, int, void*,
                               float*, hipStream_t) {
  return called();
}
hipError_t launch_mla_decode_split(const void*, const void*, float*, float*, float*, int, int, int,
                                   int, float, int*, void*, float*, int, hipStream_t) {
  return called();
}
hipError_t launch_softmax_topk(const float*, int, int, int, int, float*, int32_t*, hipStream_t) {
  return called();
}
hipError_t launch_softmax_rows(const float*, int, int, int, float*, float*, hipStream_t) {
  return called();
}
hipError_t launch_row_variance(const float*, int, int, int, float*, float*, hipStream_t) {
  return called();
}
hipError_t launch_row_inertia(const float*, const float*, int, int, int, float*, float*, hipStream_t) {
  return called();
}
hipError_t launch_absmax_quant_fp8(const void*, int, int, uint8_t*, float*, hipStream_t) {
  return called();
}
hipError_t launch_gemm_fp8_scaled(const uint8_t*, const float*, const uint8_t*, const float*, int, int,
                                  int, void*, hipStream_t) {
  return called();
}
hipError_t launch_gemm_fp8_running(const void*, const uint8_t*, const float*, int, int, int, float*,
                                   void*, hipStream_t) {
  return called();
}
hipError_t launch_peak_mfma(int, const void*, int, int, float*, unsigned long long*, hipStream_t) {
  return called();
}
hipError_t launch_peak_read(const void*, long long, int, uint32_t*, hipStream_t) { return called(); }

}  // namespace rf
