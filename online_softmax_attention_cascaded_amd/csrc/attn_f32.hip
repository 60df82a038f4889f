// fp32 attention forward: one pass over 64-key tiles with a running max,
// running denominator and running accumulator per query row, rescaled by
// exp(m_old - m_new) whenever a tile raises the max and divided by the
// denominator once at the end ("RedFuser episode transcript", cues 15-19).
//
// Plain FMA arithmetic (no MFMA): this path serves small fp32 problems where
// launch latency, not throughput, dominates. Workgroup = 4 waves; each wave owns
// 4 query rows. Lanes map to the 64 keys of a tile for the scores and to the
// head-size columns for the accumulator.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int kTileKeys = 64;
constexpr int kRowsPerWave = 4;
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(const float* __restrict__ q,
                                                           const float* __restrict__ k,
                                                           const float* __restrict__ v,
                                                           float* __restrict__ o,
                                                           float* __restrict__ lse, int Hq,
                                                           int Hkv, int Lq, int Lk, float scale,
                                                           int causal) {
  __shared__ float ks[kTileKeys][D + 1];  // odd row stride: lane j reads row j conflict-free
  __shared__ float vs[kTileKeys][D];
  __shared__ float qs[kRowsPerBlock][D];
  __shared__ float ps[kWaves][kRowsPerWave][kTileKeys];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (Hq / Hkv);
  const int q0 = blockIdx.x * kRowsPerBlock;
  const size_t qbase = ((size_t)b * Hq + h) * Lq;
  const size_t kbase = ((size_t)b * Hkv + hk) * Lk;

  for (int i = tid; i < kRowsPerBlock * D; i += 256) {
    const int r = i / D, c = i % D;
    qs[r][c] = (q0 + r < Lq) ? q[(qbase + q0 + r) * D + c] : 0.f;
  }

  float m[kRowsPerWave], l[kRowsPerWave], acc[kRowsPerWave][D / 64];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) acc[r][c] = 0.f;
  }

  int kend = Lk;
  if (causal) kend = min(Lk, q0 + kRowsPerBlock);  // keys past the last row are never visible

  for (int t0 = 0; t0 < kend; t0 += kTileKeys) {
    __syncthreads();
    for (int i = tid; i < kTileKeys * D; i += 256) {
      const int r = i / D, c = i % D;
      const int key = min(t0 + r, Lk - 1);  // rows past Lk are masked below
      ks[r][c] = k[(kbase + key) * D + c];
      vs[r][c] = v[(kbase + key) * D + c];
    }
    __syncthreads();

    const int key = t0 + lane;
    float alpha[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int row = q0 + wave * kRowsPerWave + r;
      const float* qr = qs[wave * kRowsPerWave + r];
      float dot = 0.f;
#pragma unroll 16
      for (int c = 0; c < D; ++c) dot = fmaf(qr[c], ks[lane][c], dot);
      float s = dot * scale;
      if (key >= Lk || (causal && key > row)) s = kNegInf;
      const float m_new = fmaxf(m[r], wave_max(s));
      // Correction for everything accumulated against the previous max; 1 while
      // nothing finite has been seen (the identity).
      alpha[r] = (m_new == kNegInf) ? 1.f : expf(m[r] - m_new);
      const float p = (s == kNegInf) ? 0.f : expf(s - m_new);
      l[r] = alpha[r] * l[r] + wave_sum(p);
      m[r] = m_new;
      ps[wave][r][lane] = p;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
#pragma unroll
      for (int c = 0; c < D / 64; ++c) {
        const int col = lane + 64 * c;
        float sum = 0.f;
#pragma unroll 8
        for (int j = 0; j < kTileKeys; ++j) sum = fmaf(ps[wave][r][j], vs[j][col], sum);
        acc[r][c] = alpha[r] * acc[r][c] + sum;
      }
    }
  }

#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int row = q0 + wave * kRowsPerWave + r;
    if (row >= Lq) continue;
    const float inv = 1.f / l[r];
#pragma unroll
    for (int c = 0; c < D / 64; ++c) o[(qbase + row) * D + lane + 64 * c] = acc[r][c] * inv;
    if (lse && lane == 0) lse[qbase + row] = m[r] + logf(l[r]);
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o,
                               float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int d,
                               float scale, int causal, hipStream_t stream) {
  dim3 grid((Lq + kRowsPerBlock - 1) / kRowsPerBlock, Hq, B);
  if (d == 64)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, dim3(256), 0, stream, q, k, v, o, lse, Hq,
                       Hkv, Lq, Lk, scale, causal);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, dim3(256), 0, stream, q, k, v, o, lse, Hq,
                       Hkv, Lq, Lk, scale, causal);
  return hipGetLastError();
}

}  // namespace rf
