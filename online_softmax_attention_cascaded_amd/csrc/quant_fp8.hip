// Per-token (per-row) abs-max, scale and e4m3 cast: the first reduction of the
// FP8 quantise-then-GEMM cascade ("RedFuser episode transcript", cue 33).
//
// One wave per row. A row of up to 8192 bf16 values (16 KB) stays in registers
// between the abs-max reduction and the cast, so HBM sees it exactly once. The
// abs-max is an integer max over the bf16 magnitude bits (for non-negative
// values the bit pattern orders like the value). The scale is
// s = fp32(absmax / 448) and every code is e4m3(fp32(x / s)) with the
// quotient correctly rounded: r = RN(1/s) once per row, then q = RN(x r),
// e = x - s q (by fma) and RN(q + e r), which is the correctly rounded x / s
// whenever r is the correctly rounded reciprocal and e is exact (Markstein's
// theorem for division by a reciprocal with one correction step). e is exact
// when s >= 2^-90 and |q| >= 2^-12: s q is then a multiple of 2^-148 and e,
// about 2^-23 |s q|, fits in 24 bits; smaller quotients encode to 0 whatever
// their last bits. |x / s| <= 448 (1 + 2^-23), so nothing overflows. Rows with
// 0 < s < 2^-90 (abs-max below about 3.6e-25) take plain division: there e can
// underflow, and one correction step gave wrong codes (2 of about 1100 bf16
// patterns at abs-max 2e-36, where s is subnormal). The e4m3 cast is the hardware
// round-to-nearest-even conversion (v_cvt_pk_fp8_f32); |x / s| stays below 464,
// so no value reaches the range where saturation would matter.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr float kMinFastScale = 0x1p-90f;  // smallest scale of the one-correction division

template <int NC>  // 16-byte chunks (8 values) per lane
__global__ __launch_bounds__(256) void absmax_quant_kernel(const uint16_t* __restrict__ x,
                                                           int rows, int cols,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wave
  const int nchunks = cols >> 3;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)row * cols);

  u32x4 ch[NC];
  uint32_t amax = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = lane + 64 * c;
    ch[c] = (idx < nchunks) ? __builtin_nontemporal_load(xr + idx) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = max(amax, ch[c][e] & 0x7fffu);
      amax = max(amax, (ch[c][e] >> 16) & 0x7fffu);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o, kWave));

  const float a = __uint_as_float(amax << 16);
  const float sc = a / 448.f;
  if (lane == 0) scale[row] = sc;
  const float rcp = (sc > 0.f) ? 1.f / sc : 0.f;

  u32x2* qr = reinterpret_cast<u32x2*>(q + (size_t)row * cols);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = lane + 64 * c;
    if (idx >= nchunks) continue;
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[2 * e] = bf16_lo(ch[c][e]);
      y[2 * e + 1] = bf16_hi(ch[c][e]);
    }
    if (!(sc > 0.f && sc < kMinFastScale)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float q0 = y[j] * rcp;
        const float r = fmaf(-sc, q0, y[j]);
        // The correction would turn -0 into +0; every other quotient already
        // has the sign of x.
        y[j] = __builtin_copysignf(fmaf(r, rcp, q0), y[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = y[j] / sc;
    }
    u32x2 w = {0u, 0u};
    if (sc > 0.f) {
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
      w = u32x2{(uint32_t)lo, (uint32_t)hi};
    }
    qr[idx] = w;
  }
}

}  // namespace

hipError_t launch_absmax_quant_fp8(const void* x, int rows, int cols, uint8_t* q, float* scale,
                                   hipStream_t stream) {
  const int nchunks = cols / 8;
  const int nc = (nchunks + 63) / 64;
  dim3 grid((rows + 3) / 4);
  auto xx = static_cast<const uint16_t*>(x);
  if (nc <= 1)
    hipLaunchKernelGGL(absmax_quant_kernel<1>, grid, dim3(256), 0, stream, xx, rows, cols, q, scale);
  else if (nc <= 2)
    hipLaunchKernelGGL(absmax_quant_kernel<2>, grid, dim3(256), 0, stream, xx, rows, cols, q, scale);
  else if (nc <= 4)
    hipLaunchKernelGGL(absmax_quant_kernel<4>, grid, dim3(256), 0, stream, xx, rows, cols, q, scale);
  else if (nc <= 8)
    hipLaunchKernelGGL(absmax_quant_kernel<8>, grid, dim3(256), 0, stream, xx, rows, cols, q, scale);
  else
    hipLaunchKernelGGL(absmax_quant_kernel<16>, grid, dim3(256), 0, stream, xx, rows, cols, q, scale);
  return hipGetLastError();
}

}  // namespace rf
