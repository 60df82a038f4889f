// Per-token (per-row) abs-max, scale and e4m3 cast: the first reduction of the
// FP8 quantise-then-GEMM cascade ("RedFuser episode transcript", cue 33).
//
// One wave per row. A row of up to 8192 bf16 values (16 KB) stays in registers
// between the abs-max reduction and the cast, so HBM sees it exactly once. The
// abs-max is an integer max over the bf16 magnitude bits (for non-negative
// values the bit pattern orders like the value). The scale is
// fp32(absmax / 448) and every code is e4m3(fp32(x / scale)), both with
// correctly rounded division, then round-to-nearest-even with saturation.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

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
  const float s = a / 448.f;
  if (lane == 0) scale[row] = s;

  u32x2* qr = reinterpret_cast<u32x2*>(q + (size_t)row * cols);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = lane + 64 * c;
    if (idx >= nchunks) continue;
    uint32_t code[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      code[2 * e] = (s > 0.f) ? e4m3_encode(bf16_lo(ch[c][e]) / s) : 0u;
      code[2 * e + 1] = (s > 0.f) ? e4m3_encode(bf16_hi(ch[c][e]) / s) : 0u;
    }
    u32x2 w = {code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24),
               code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24)};
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
