// MoE routing: per row of logits, softmax then top-k, in one pass over the row
// ("RedFuser episode transcript", cue 11; "Online normalizer calculation for
// softmax", abstract: softmax and top-k fused).
//
// One wave per row; a 256-expert row is one 16-byte load per lane, so the row
// never leaves registers (the non-incremental form, which the transcript notes
// is the faster one whenever the reduced axis fits on chip, cue 45). Logits are
// mapped to order-preserving unsigned keys, so ranking, ties and the wave
// reductions are integer operations. Top-k is k rounds of: each lane's best
// untaken key (lowest index among equals), a max over the lanes of the row by
// DPP, then the lowest expert index among the lanes holding that key. For 256
// experts and k <= 8 each lane sorts its candidates once, so a round only
// compares list heads; otherwise a lane rescans its keys every round. Ranking
// by the fp32 logit is the
// same as ranking by probability because softmax is strictly increasing. The
// top-1 logit is the row max, so the selected weights are exp(x_i - max),
// divided by their own sum (renormalised) or by the row's denominator.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

// Order-preserving map of a finite fp32 value to uint32 (-0 is folded onto +0
// first, so equal values have equal keys).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// DPP controls (gfx9): quad permutations, half-row and row mirrors.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// Max over the 64 lanes of the wave (result uniform).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<kDppXor1>(v));
  v = max(v, dpp<kDppXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  v = max(v, dpp<kDppMirror>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp<kDppXor1>(v));
  v = min(v, dpp<kDppXor2>(v));
  v = min(v, dpp<kDppHalfMirror>(v));
  v = min(v, dpp<kDppMirror>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return min(min(r0, r1), min(r2, r3));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __builtin_bit_cast(float, dpp<kDppXor1>(__builtin_bit_cast(uint32_t, v)));
  v += __builtin_bit_cast(float, dpp<kDppXor2>(__builtin_bit_cast(uint32_t, v)));
  v += __builtin_bit_cast(float, dpp<kDppHalfMirror>(__builtin_bit_cast(uint32_t, v)));
  v += __builtin_bit_cast(float, dpp<kDppMirror>(__builtin_bit_cast(uint32_t, v)));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

template <int NC>  // 16-byte chunks (4 experts) per lane
__global__ __launch_bounds__(256) void softmax_topk_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int renorm,
                                                           float* __restrict__ weights,
                                                           int32_t* __restrict__ indices) {
  constexpr int NV = 4 * NC;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;  // uniform per wave
  const float* x = logits + (size_t)row * E;

  // Value j of this lane is expert 4 (lane + 64 (j / 4)) + j % 4; padding keys are 0.
  uint32_t key[NV];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int chunk = lane + 64 * c;
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    const bool in = 4 * chunk < E;
    if (in) w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x) + chunk);
#pragma unroll
    for (int e = 0; e < 4; ++e) key[4 * c + e] = in ? order_key(w[e]) : 0u;
  }

  uint32_t taken = 0;
  uint32_t top = 0;        // key of the row max (rank 0)
  uint32_t my_key = 0;     // lane r keeps the key and index of rank r
  int my_idx = 0;
  for (int r = 0; r < k; ++r) {
    // This lane's best untaken key; the lowest index wins among equals because
    // values are scanned in index order and only a strictly larger key replaces.
    uint32_t bk = 0;
    int bj = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint32_t kj = ((taken >> j) & 1u) ? 0u : key[j];
      if (kj > bk) {
        bk = kj;
        bj = j;
      }
    }
    const uint32_t wk = wave_max_u32(bk);
    const uint64_t holders = __ballot(bk == wk);
    int widx;
    if (__popcll(holders) == 1) {
      const int wl = __ffsll((long long)holders) - 1;
      widx = __builtin_amdgcn_readlane(4 * (lane + 64 * (bj >> 2)) + (bj & 3), wl);
    } else {
      const uint32_t cand = (bk == wk) ? (uint32_t)(4 * (lane + 64 * (bj >> 2)) + (bj & 3)) : 0xffffffffu;
      widx = (int)wave_min_u32(cand);
    }
    // The owner of expert widx marks it taken.
    const int wchunk = widx >> 2;
    if ((wchunk & 63) == lane) taken |= 1u << (4 * (wchunk >> 6) + (widx & 3));
    if (r == 0) top = wk;
    if (lane == r) {
      my_key = wk;
      my_idx = widx;
    }
  }

  const float m = key_value(top);
  const float e = (lane < k) ? expf(key_value(my_key) - m) : 0.f;
  float denom;
  if (renorm) {
    denom = wave_sum_f32(e);
  } else {
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (key[j] != 0u) l += fast_exp2((key_value(key[j]) - m) * kLog2e);
    denom = wave_sum_f32(l);
  }
  if (lane < k) {
    weights[(size_t)row * k + lane] = e / denom;
    indices[(size_t)row * k + lane] = my_idx;
  }
}

// 16-lane reductions (DPP quad and row permutations only: every lane of a
// group of 16 ends with the same result).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, dpp<kDppXor1>(v));
  v = max(v, dpp<kDppXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  return max(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ uint32_t row16_min_u32(uint32_t v) {
  v = min(v, dpp<kDppXor1>(v));
  v = min(v, dpp<kDppXor2>(v));
  v = min(v, dpp<kDppHalfMirror>(v));
  return min(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ float row16_sum_f32(float v) {
  v += __builtin_bit_cast(float, dpp<kDppXor1>(__builtin_bit_cast(uint32_t, v)));
  v += __builtin_bit_cast(float, dpp<kDppXor2>(__builtin_bit_cast(uint32_t, v)));
  v += __builtin_bit_cast(float, dpp<kDppHalfMirror>(__builtin_bit_cast(uint32_t, v)));
  return v + __builtin_bit_cast(float, dpp<kDppMirror>(__builtin_bit_cast(uint32_t, v)));
}

// E = 256, k <= 16: four rows per wave, 16 lanes per row. Lane j of a row
// holds experts 64 c + 4 j + e (c, e = 0..3) in key[4 c + e], i.e. in
// increasing expert order, so "strictly larger replaces" keeps the lowest
// index among equal keys within the lane; across lanes the lowest index among
// the holders of the row max is a 16-lane min. Lane j records rank j.
__global__ __launch_bounds__(256) void softmax_topk_e256_kernel(const float* __restrict__ logits,
                                                                int T, int k, int renorm,
                                                                float* __restrict__ weights,
                                                                int32_t* __restrict__ indices) {
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  // A row past T reads the last row (valid memory) and writes nothing; all 64
  // lanes stay active for the DPP reductions.
  const float* x = logits + (size_t)min(row, T - 1) * 256;

  uint32_t key[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x) + 16 * c + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) key[4 * c + e] = order_key(w[e]);
  }

  uint32_t taken = 0, top = 0, my_key = 0;
  int my_idx = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t bk = 0;
    int bt = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t kt = ((taken >> t) & 1u) ? 0u : key[t];
      if (kt > bk) {
        bk = kt;
        bt = t;
      }
    }
    const uint32_t wk = row16_max_u32(bk);
    const uint32_t mine = 64 * (bt >> 2) + 4 * j + (bt & 3);
    const int widx = (int)row16_min_u32(bk == wk ? mine : 0xffffffffu);
    if (((widx >> 2) & 15) == j) taken |= 1u << (4 * (widx >> 6) + (widx & 3));
    if (r == 0) top = wk;
    if (j == r) {
      my_key = wk;
      my_idx = widx;
    }
  }

  const float m = key_value(top);
  const float e = (j < k) ? expf(key_value(my_key) - m) : 0.f;
  float denom;
  if (renorm) {
    denom = row16_sum_f32(e);
  } else {
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) l += fast_exp2((key_value(key[t]) - m) * kLog2e);
    denom = row16_sum_f32(l);
  }
  if (row < T && j < k) {
    weights[(size_t)row * k + j] = e / denom;
    indices[(size_t)row * k + j] = my_idx;
  }
}

// E = 256, k <= 8: the same mapping, but each lane first orders its 16
// candidates once, so a round costs one comparison of the row's 16 list heads
// instead of a rescan of 16 keys per lane. A candidate is the 64-bit value
// key << 32 | (15 - slot): equal keys order by the lower slot, which is the
// lower expert index within the lane. The two halves of a lane's 16 are sorted
// by an 8-input network (19 comparators); the elementwise max of one sorted
// half and the other reversed holds the lane's 8 best as a bitonic sequence,
// which three merge stages sort. A lane supplies at most k <= 8 winners, so 8
// entries suffice; the winning lane drops its head each round.
__device__ __forceinline__ void cx_desc(uint64_t& a, uint64_t& b) {
  const bool keep = a >= b;
  const uint64_t hi = keep ? a : b, lo = keep ? b : a;
  a = hi;
  b = lo;
}
template <int OFF>
__device__ __forceinline__ void sort8_desc(uint64_t (&v)[16]) {
  constexpr int net[19][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}, {0, 4}, {1, 5}, {2, 6},
                              {3, 7}, {0, 1}, {2, 3}, {4, 5}, {6, 7}, {2, 4}, {3, 5},
                              {1, 4}, {3, 6}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
  for (int c = 0; c < 19; ++c) cx_desc(v[OFF + net[c][0]], v[OFF + net[c][1]]);
}

__global__ __launch_bounds__(256) void softmax_topk_e256_k8_kernel(const float* __restrict__ logits,
                                                                   int T, int k, int renorm,
                                                                   float* __restrict__ weights,
                                                                   int32_t* __restrict__ indices) {
  const int lane = threadIdx.x & 63, j = lane & 15;
  const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  // A row past T reads the last row (valid memory) and writes nothing; all 64
  // lanes stay active for the DPP reductions.
  const float* x = logits + (size_t)min(row, T - 1) * 256;

  float xv[16];
  uint64_t v[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x) + 16 * c + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * c + e;
      xv[t] = w[e];
      v[t] = ((uint64_t)order_key(w[e]) << 32) | (uint64_t)(15 - t);
    }
  }
  sort8_desc<0>(v);
  sort8_desc<8>(v);
  uint64_t s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = v[i] >= v[15 - i] ? v[i] : v[15 - i];
#pragma unroll
  for (int d = 4; d > 0; d >>= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & d) == 0) cx_desc(s[i], s[i + d]);

  uint32_t top = 0, my_key = 0;
  int my_idx = 0;
  for (int r = 0; r < k; ++r) {
    const uint32_t hk = (uint32_t)(s[0] >> 32);
    const int slot = 15 - (int)(s[0] & 15u);
    const uint32_t wk = row16_max_u32(hk);
    const uint32_t mine = (hk == wk) ? (uint32_t)(64 * (slot >> 2) + 4 * j + (slot & 3)) : 0xffffffffu;
    const uint32_t widx = row16_min_u32(mine);
    const bool win = mine == widx;
#pragma unroll
    for (int i = 0; i < 7; ++i) s[i] = win ? s[i + 1] : s[i];
    s[7] = win ? 0ull : s[7];
    if (r == 0) top = wk;
    if (j == r) {
      my_key = wk;
      my_idx = (int)widx;
    }
  }

  const float m = key_value(top);
  const float e = (j < k) ? expf(key_value(my_key) - m) : 0.f;
  float denom;
  if (renorm) {
    denom = row16_sum_f32(e);
  } else {
    float l = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) l += fast_exp2((xv[t] - m) * kLog2e);
    denom = row16_sum_f32(l);
  }
  if (row < T && j < k) {
    weights[(size_t)row * k + j] = e / denom;
    indices[(size_t)row * k + j] = my_idx;
  }
}

}  // namespace

hipError_t launch_softmax_topk(const float* logits, int T, int E, int k, int renormalize,
                               float* weights, int32_t* indices, hipStream_t stream) {
#ifndef RF_TOPK_NO_SORTED
  if (E == 256 && k <= 8) {
    hipLaunchKernelGGL(softmax_topk_e256_k8_kernel, dim3((T + 15) / 16), dim3(256), 0, stream,
                       logits, T, k, renormalize, weights, indices);
    return hipGetLastError();
  }
#endif
  if (E == 256 && k <= 16) {
    hipLaunchKernelGGL(softmax_topk_e256_kernel, dim3((T + 15) / 16), dim3(256), 0, stream, logits,
                       T, k, renormalize, weights, indices);
    return hipGetLastError();
  }
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
