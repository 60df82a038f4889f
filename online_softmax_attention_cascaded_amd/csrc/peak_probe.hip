// Measurement support, not a step of the path: dense MFMA loops with no memory
// traffic inside the loop, for the matrix-core rate this GPU sustains on given
// operand data and the shader clock it runs at while doing so, and an HBM read
// stream for the bandwidth a read-dominated kernel can reach. The rate at
// which the chip can run its matrix cores depends on the operands: the board's
// power limit lowers the clock as more bits switch, so the loop multiplies
// data the caller supplies (random data for a realistic ceiling).
//
// Each workgroup has 4 waves; each lane loads 8 operand vectors, then every
// iteration issues 8 MFMAs (operands j and (j + 3) % 8) onto 4 independent
// accumulators, so consecutive MFMAs never wait for one another. Lane 0 of
// wave 0 records the shader-clock counter and the constant-rate counter at
// the workgroup's start and end.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

template <int KIND>  // 0: bf16 32x32x16, 1: e4m3 32x32x64
__global__ __launch_bounds__(256) void peak_mfma_kernel(const uint8_t* __restrict__ src, int iters,
                                                        float* __restrict__ out,
                                                        unsigned long long* __restrict__ clk) {
  unsigned long long c0 = 0, w0 = 0;
  if (threadIdx.x == 0) {
    c0 = clock64();
    w0 = wall_clock64();
  }
  // 256 bytes per lane: vector j at byte 32 j (bf16 uses its first 16 bytes)
  const uint8_t* p = src + ((size_t)blockIdx.x * 256 + threadIdx.x) * 256;
  f32x16 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x16{};
  if constexpr (KIND == 0) {
    bf16x8 op[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) op[j] = *reinterpret_cast<const bf16x8*>(p + 32 * j);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[j], op[(j + 3) & 7], acc[j & 3], 0, 0, 0);
    }
  } else {
    i32x8 op[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) op[j] = *reinterpret_cast<const i32x8*>(p + 32 * j);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op[j], op[(j + 3) & 7], acc[j & 3],
                                                                     0, 0, 0, 0, 0, 0);
    }
  }
  // Checksum: the sum of every accumulator element of the wave.
  float s = 0.f;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[n][e];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
  if (threadIdx.x == 0 && clk) {
    const unsigned long long c1 = clock64(), w1 = wall_clock64();
    clk[2 * blockIdx.x] = c1 - c0;
    clk[2 * blockIdx.x + 1] = w1 - w0;
  }
}

// HBM read stream: workgroup b reads its own contiguous share of the buffer,
// each thread keeping 8 independent 16-byte loads in flight (32 KB per
// workgroup), so every load instruction covers 1 KB of consecutive bytes and a
// wave walks its share in order; the XOR of every 32-bit word read is folded
// per workgroup, so the result does not depend on the order. (Grid-strided
// rounds, with a wave's successive loads far apart, ran 6.0-6.9 TB/s against
// 7.0-7.1 for this pattern.)
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ src, long long n16,
                                                        uint32_t* __restrict__ out) {
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long lo = min(n16, (long long)blockIdx.x * per), hi = min(n16, lo + per);
  u32x4 x = {0u, 0u, 0u, 0u};
  for (long long base = lo + threadIdx.x; base < hi; base += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const long long i = base + 256 * u;
      v[u] = i < hi ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u];
  }
  uint32_t w = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) w ^= (uint32_t)__shfl_xor((int)w, o, kWave);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_peak_read(const void* src, long long bytes, int blocks, uint32_t* out,
                            hipStream_t stream) {
  hipLaunchKernelGGL(peak_read_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(int kind, const void* src, int blocks, int iters, float* out,
                            unsigned long long* clk, hipStream_t stream) {
  const auto s = static_cast<const uint8_t*>(src);
  if (kind == 0)
    hipLaunchKernelGGL(peak_mfma_kernel<0>, dim3(blocks), dim3(256), 0, stream, s, iters, out, clk);
  else
    hipLaunchKernelGGL(peak_mfma_kernel<1>, dim3(blocks), dim3(256), 0, stream, s, iters, out, clk);
  return hipGetLastError();
}

}  // namespace rf
