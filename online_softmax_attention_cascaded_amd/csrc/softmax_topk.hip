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
  // negative: all bits flipped; otherwise the sign bit set
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// DPP controls (gfx9): quad permutations, half-row and row mirrors.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// Every pattern used here reads a lane of the same row, and every caller runs
// with all 64 lanes active, so no source lane is out of range or disabled and
// the bound-control zero fill never applies; with it set and no old value to
// keep, the compiler folds the move into the max / min / add that consumes it.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
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

// E = 256, k <= 8: the same mapping, but each lane orders its 16 candidates
// once, so a round costs one comparison of the row's 16 list heads instead of
// a rescan of 16 keys per lane. A lane supplies at most k <= 8 winners, so its
// best 8 suffice; the winning lane drops its head each round.
//
// Fast form: a candidate is its key with the low 4 bits replaced by 15 - slot,
// sorted by a 63-comparator network of 32-bit max / min. Keys whose upper 28
// bits differ keep their order; keys that agree there (equal keys included)
// land next to each other, and if any lane of the wave has such a pair the
// wave takes the exact form instead: 64-bit candidates key << 32 | (15 - slot)
// (equal keys order by the lower slot, i.e. the lower expert index within the
// lane), both halves sorted by a 19-comparator 8-input network, the
// elementwise max of one half and the other reversed (the best 8 as a bitonic
// sequence) sorted by three merge stages. The fast form recovers a head's low
// key bits from a per-lane table before comparing across lanes, so the
// cross-lane comparison is always on the exact key.
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
// Batcher's odd-even merge sort of 16 (descending).
__device__ __forceinline__ void sort16_desc(uint32_t (&v)[16]) {
  constexpr int net[63][2] = {
      {0, 1},   {2, 3},   {0, 2},   {1, 3},   {1, 2},   {4, 5},   {6, 7},   {4, 6},   {5, 7},
      {5, 6},   {0, 4},   {2, 6},   {2, 4},   {1, 5},   {3, 7},   {3, 5},   {1, 2},   {3, 4},
      {5, 6},   {8, 9},   {10, 11}, {8, 10},  {9, 11},  {9, 10},  {12, 13}, {14, 15}, {12, 14},
      {13, 15}, {13, 14}, {8, 12},  {10, 14}, {10, 12}, {9, 13},  {11, 15}, {11, 13}, {9, 10},
      {11, 12}, {13, 14}, {0, 8},   {4, 12},  {4, 8},   {2, 10},  {6, 14},  {6, 10},  {2, 4},
      {6, 8},   {10, 12}, {1, 9},   {5, 13},  {5, 9},   {3, 11},  {7, 15},  {7, 11},  {3, 5},
      {7, 9},   {11, 13}, {1, 2},   {3, 4},   {5, 6},   {7, 8},   {9, 10},  {11, 12}, {13, 14}};
#pragma unroll
  for (int c = 0; c < 63; ++c) {
    const uint32_t a = v[net[c][0]], b = v[net[c][1]];
    v[net[c][0]] = max(a, b);
    v[net[c][1]] = min(a, b);
  }
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
  uint32_t key[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x) + 16 * c + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xv[4 * c + e] = w[e];
      key[4 * c + e] = order_key(w[e]);
    }
  }
  // expert index of slot t of this lane
  auto expert = [&](int t) { return (uint32_t)(64 * (t >> 2) + 4 * j + (t & 3)); };

  uint32_t top = 0, my_key = 0;
  int my_idx = 0;
  uint32_t cd[16], low_a = 0, low_b = 0;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    cd[t] = (key[t] & ~0xFu) | (uint32_t)(15 - t);
    if (t < 8)
      low_a |= (key[t] & 0xFu) << (4 * t);
    else
      low_b |= (key[t] & 0xFu) << (4 * (t - 8));
  }
  sort16_desc(cd);
  bool near = false;
#pragma unroll
  for (int i = 0; i < 15; ++i) near |= (cd[i] ^ cd[i + 1]) < 16u;

  if (!__any(near)) {
    for (int r = 0; r < k; ++r) {
      const uint32_t h = cd[0];
      const int slot = 15 - (int)(h & 15u);
      const uint32_t lw = slot < 8 ? low_a : low_b;
      const uint32_t hk = (h & ~0xFu) | ((lw >> (4 * (slot & 7))) & 0xFu);
      const uint32_t wk = row16_max_u32(hk);
      const uint32_t widx = row16_min_u32(hk == wk ? expert(slot) : 0xffffffffu);
      const bool win = hk == wk && expert(slot) == widx;
#pragma unroll
      for (int i = 0; i < 7; ++i) cd[i] = win ? cd[i + 1] : cd[i];
      if (r == 0) top = wk;
      if (j == r) {
        my_key = wk;
        my_idx = (int)widx;
      }
    }
  } else {
    uint64_t v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) v[t] = ((uint64_t)key[t] << 32) | (uint64_t)(15 - t);
    sort8_desc<0>(v);
    sort8_desc<8>(v);
    uint64_t s8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s8[i] = v[i] >= v[15 - i] ? v[i] : v[15 - i];
#pragma unroll
    for (int d = 4; d > 0; d >>= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((i & d) == 0) cx_desc(s8[i], s8[i + d]);
    for (int r = 0; r < k; ++r) {
      const uint32_t hk = (uint32_t)(s8[0] >> 32);
      const int slot = 15 - (int)(s8[0] & 15u);
      const uint32_t wk = row16_max_u32(hk);
      const uint32_t widx = row16_min_u32(hk == wk ? expert(slot) : 0xffffffffu);
      const bool win = hk == wk && expert(slot) == widx;
#pragma unroll
      for (int i = 0; i < 7; ++i) s8[i] = win ? s8[i + 1] : s8[i];
      if (r == 0) top = wk;
      if (j == r) {
        my_key = wk;
        my_idx = (int)widx;
      }
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
  if (E == 256 && k <= 8) {
    hipLaunchKernelGGL(softmax_topk_e256_k8_kernel, dim3((T + 15) / 16), dim3(256), 0, stream,
                       logits, T, k, renormalize, weights, indices);
    return hipGetLastError();
  }
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
