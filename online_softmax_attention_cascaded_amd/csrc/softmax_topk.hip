// MoE routing: per row of logits, softmax then top-k, in one pass over the row
// ("RedFuser episode transcript", cue 11; "Online normalizer calculation for
// softmax", abstract: softmax and top-k fused).
//
// One wave per row; a 256-expert row is one 16-byte load per lane, so the row
// never leaves registers. Each lane first reduces its own values to an
// online-softmax state (m, l); the 64 lane states are then merged pairwise by
// rescaling to the larger max, exactly as partial states merge across blocks
// (cue 21). Top-k is k rounds of a wavefront argmax on (value, index) with ties
// to the lower index; ranking by the fp32 logit equals ranking by probability
// because softmax is strictly increasing. The top-1 logit is the row max, so
// the selected weights are exp(x_i - max) divided either by their own sum
// (renormalised) or by the merged denominator.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

template <int NC>  // 16-byte chunks (4 experts) per lane
__global__ __launch_bounds__(256) void softmax_topk_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int renorm,
                                                           float* __restrict__ weights,
                                                           int32_t* __restrict__ indices) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;  // uniform per wave
  const float* x = logits + (size_t)row * E;

  float val[4 * NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int chunk = lane + 64 * c;
    f32x4 w = {kNegInf, kNegInf, kNegInf, kNegInf};
    if (4 * chunk < E) w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x) + chunk);
#pragma unroll
    for (int e = 0; e < 4; ++e) val[4 * c + e] = w[e];
  }
  auto expert = [&](int j) { return 4 * (lane + 64 * (j >> 2)) + (j & 3); };

  // Denominator, only needed when the weights are not renormalised.
  float m = kNegInf, l = 0.f;
  if (!renorm) {
#pragma unroll
    for (int j = 0; j < 4 * NC; ++j) m = fmaxf(m, val[j]);
#pragma unroll
    for (int j = 0; j < 4 * NC; ++j) l += (val[j] == kNegInf) ? 0.f : fast_exp2((val[j] - m) * kLog2e);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(m, o, kWave), l2 = __shfl_xor(l, o, kWave);
      merge_ml(m, l, m2, l2);
    }
  }

  uint32_t taken = 0;
  float top = 0.f, esum = 0.f, my_e = 0.f;
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    float bv = kNegInf;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4 * NC; ++j) {
      const int id = expert(j);
      const bool better = val[j] > bv || (val[j] == bv && id < bi);
      if (!((taken >> j) & 1u) && id < E && better) {
        bv = val[j];
        bi = id;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // (bv, bi) is now the same in every lane; its owner marks it taken.
    const int chunk = bi >> 2;
    if ((chunk & 63) == lane) taken |= 1u << (4 * (chunk >> 6) + (bi & 3));
    if (r == 0) top = bv;
    const float e = expf(bv - top);
    esum += e;
    if (lane == r) {
      my_e = e;
      my_i = bi;
    }
  }
  if (lane < k) {
    const float w = renorm ? my_e / esum : my_e / l;
    weights[(size_t)row * k + lane] = w;
    indices[(size_t)row * k + lane] = my_i;
  }
}

}  // namespace

hipError_t launch_softmax_topk(const float* logits, int T, int E, int k, int renormalize,
                               float* weights, int32_t* indices, hipStream_t stream) {
  dim3 grid((T + 3) / 4);
  const int nc = (E + 255) / 256;
  if (nc <= 1)
    hipLaunchKernelGGL(softmax_topk_kernel<1>, grid, dim3(256), 0, stream, logits, T, E, k,
                       renormalize, weights, indices);
  else if (nc <= 2)
    hipLaunchKernelGGL(softmax_topk_kernel<2>, grid, dim3(256), 0, stream, logits, T, E, k,
                       renormalize, weights, indices);
  else
    hipLaunchKernelGGL(softmax_topk_kernel<4>, grid, dim3(256), 0, stream, logits, T, E, k,
                       renormalize, weights, indices);
  return hipGetLastError();
}

}  // namespace rf
