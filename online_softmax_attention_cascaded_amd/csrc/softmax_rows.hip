// Safe softmax of rows of 4 .. 8192 fp32 values, with the max -> sum cascade
// fused at different levels of the reduction tree ("RedFuser episode
// transcript", cue 47: fusion levels on safe softmax; cue 17 for the running
// (m, l) state), against the unfused cascade of three kernels.
//
// One workgroup (256 threads) per row. In every fused form the row is read
// from HBM once and stays in registers (at most 32 values per thread) between
// the statistics and the normalisation; they differ only in where the running
// state (m, l) is updated:
//  * thread: each thread folds its own values one at a time into (m, l) —
//    two exponentials per value — and the threads' states are merged by the
//    rescale-and-add rule (across the wave, then across the four waves);
//  * wave: the wave walks its row segments 256 values at a time; per segment
//    a wave max, then l = l * exp(m_old - m_new) + wave sum of exp(x - m_new);
//    the four wave states are merged at the end;
//  * block: the workgroup walks the row 1024 values at a time with block-wide
//    max and sum per tile (the form FlashAttention uses, at the block level).
// The unfused form runs three kernels (row max, sum of exp(x - max), divide),
// reading the row three times.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// exp(x - m) for finite m (and 0 for x = -inf).
__device__ __forceinline__ float ex(float x, float m) { return fast_exp2((x - m) * kLog2e); }

// (m, l) merge of the four wave states through LDS, in a fixed order so every
// thread gets the same result.
__device__ __forceinline__ void block_merge(float& m, float& l, float* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm[2 * wave] = m;
    sm[2 * wave + 1] = l;
  }
  __syncthreads();
  m = sm[0];
  l = sm[1];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) merge_ml(m, l, sm[2 * w], sm[2 * w + 1]);
}

__device__ __forceinline__ float block_reduce_max(float v, float* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max(v);
  if (lane == 0) sm[wave] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_reduce_sum(float v, float* sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) sm[wave] = v;
  __syncthreads();
  const float r = (sm[0] + sm[1]) + (sm[2] + sm[3]);
  __syncthreads();
  return r;
}

// LEVEL 1 thread, 2 wave, 3 block. NJ = 16-byte chunks per thread; chunk j of
// thread t is chunk t + 256 j of the row (values 4 (t + 256 j) .. + 3), so the
// wave's lanes cover 256 consecutive values per j and the block 1024.
template <int NJ, int LEVEL>
__global__ __launch_bounds__(kThreads) void softmax_fused_kernel(const float* __restrict__ x,
                                                                 int E, float* __restrict__ y) {
  __shared__ float sm[2 * kWaves];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const int nch = E >> 2;
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * E);
  f32x4 v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int cidx = tid + kThreads * j;
    v[j] = (cidx < nch) ? __builtin_nontemporal_load(xr + cidx) : f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
  }

  float m = kNegInf, l = 0.f;
  if constexpr (LEVEL == 1) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xv = v[j][e];
        if (xv == kNegInf) continue;  // padding past E
        const float mn = fmaxf(m, xv);
        const float a = (m == kNegInf) ? 0.f : ex(m, mn);
        l = l * a + ex(xv, mn);
        m = mn;
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) merge_ml(m, l, __shfl_xor(m, o, kWave), __shfl_xor(l, o, kWave));
    block_merge(m, l, sm);
  } else if constexpr (LEVEL == 2) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float cm = wave_max(fmaxf(fmaxf(v[j][0], v[j][1]), fmaxf(v[j][2], v[j][3])));
      const float mn = fmaxf(m, cm);
      if (mn == kNegInf) continue;  // nothing seen yet in this wave
      const float a = (m == kNegInf) ? 0.f : ex(m, mn);
      const float s = (ex(v[j][0], mn) + ex(v[j][1], mn)) + (ex(v[j][2], mn) + ex(v[j][3], mn));
      l = l * a + wave_sum(s);
      m = mn;
    }
    block_merge(m, l, sm);
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (kThreads * j * 4 >= E) break;  // tile past the row (uniform)
      const float tm = block_reduce_max(fmaxf(fmaxf(v[j][0], v[j][1]), fmaxf(v[j][2], v[j][3])), sm);
      const float mn = fmaxf(m, tm);
      if (mn == kNegInf) continue;  // nothing finite seen yet (uniform)
      const float a = (m == kNegInf) ? 0.f : ex(m, mn);
      const float s = (ex(v[j][0], mn) + ex(v[j][1], mn)) + (ex(v[j][2], mn) + ex(v[j][3], mn));
      l = l * a + block_reduce_sum(s, sm);
      m = mn;
    }
  }

  const float inv = 1.f / l;
  f32x4* yr = reinterpret_cast<f32x4*>(y + row * E);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int cidx = tid + kThreads * j;
    if (cidx < nch)
      __builtin_nontemporal_store(f32x4{ex(v[j][0], m) * inv, ex(v[j][1], m) * inv,
                                        ex(v[j][2], m) * inv, ex(v[j][3], m) * inv},
                                  yr + cidx);
  }
}

// Unfused cascade: three kernels, each one pass over the row from HBM.
__global__ __launch_bounds__(kThreads) void row_max_kernel(const float* __restrict__ x, int E,
                                                           float* __restrict__ mout) {
  __shared__ float sm[kWaves];
  const size_t row = blockIdx.x;
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * E);
  float m = kNegInf;
  for (int c = threadIdx.x; c < (E >> 2); c += kThreads) {
    const f32x4 w = xr[c];
    m = fmaxf(m, fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3])));
  }
  m = block_reduce_max(m, sm);
  if (threadIdx.x == 0) mout[row] = m;
}
__global__ __launch_bounds__(kThreads) void row_sumexp_kernel(const float* __restrict__ x, int E,
                                                              const float* __restrict__ mrow,
                                                              float* __restrict__ lout) {
  __shared__ float sm[kWaves];
  const size_t row = blockIdx.x;
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * E);
  const float m = mrow[row];
  float s = 0.f;
  for (int c = threadIdx.x; c < (E >> 2); c += kThreads) {
    const f32x4 w = xr[c];
    s += (ex(w[0], m) + ex(w[1], m)) + (ex(w[2], m) + ex(w[3], m));
  }
  s = block_reduce_sum(s, sm);
  if (threadIdx.x == 0) lout[row] = s;
}
__global__ __launch_bounds__(kThreads) void row_normalise_kernel(const float* __restrict__ x, int E,
                                                                 const float* __restrict__ mrow,
                                                                 const float* __restrict__ lrow,
                                                                 float* __restrict__ y) {
  const size_t row = blockIdx.x;
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * E);
  f32x4* yr = reinterpret_cast<f32x4*>(y + row * E);
  const float m = mrow[row], inv = 1.f / lrow[row];
  for (int c = threadIdx.x; c < (E >> 2); c += kThreads) {
    const f32x4 w = xr[c];
    yr[c] = f32x4{ex(w[0], m) * inv, ex(w[1], m) * inv, ex(w[2], m) * inv, ex(w[3], m) * inv};
  }
}

template <int LEVEL>
hipError_t launch_level(const float* x, int T, int E, float* y, hipStream_t stream) {
  const dim3 grid(T), block(kThreads);
  if (E <= 1024)
    hipLaunchKernelGGL((softmax_fused_kernel<1, LEVEL>), grid, block, 0, stream, x, E, y);
  else if (E <= 2048)
    hipLaunchKernelGGL((softmax_fused_kernel<2, LEVEL>), grid, block, 0, stream, x, E, y);
  else if (E <= 4096)
    hipLaunchKernelGGL((softmax_fused_kernel<4, LEVEL>), grid, block, 0, stream, x, E, y);
  else
    hipLaunchKernelGGL((softmax_fused_kernel<8, LEVEL>), grid, block, 0, stream, x, E, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_rows(const float* x, int T, int E, int level, float* work, float* y,
                               hipStream_t stream) {
  switch (level) {
    case 1: return launch_level<1>(x, T, E, y, stream);
    case 2: return launch_level<2>(x, T, E, y, stream);
    case 3: return launch_level<3>(x, T, E, y, stream);
    default: break;
  }
  const dim3 grid(T), block(kThreads);
  hipLaunchKernelGGL(row_max_kernel, grid, block, 0, stream, x, E, work);
  hipLaunchKernelGGL(row_sumexp_kernel, grid, block, 0, stream, x, E, work, work + T);
  hipLaunchKernelGGL(row_normalise_kernel, grid, block, 0, stream, x, E, work, work + T, y);
  return hipGetLastError();
}

}  // namespace rf
