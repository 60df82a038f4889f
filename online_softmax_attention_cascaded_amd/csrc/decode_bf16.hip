// Split-KV decode (Multi-Segment) and the merge of partial states.
//
// First kernel: one workgroup per (batch, key/value head, segment). It streams
// the segment's K and V rows once for the whole GQA group of query heads and
// keeps, per query head, a running max m, a running denominator l and an
// unnormalised accumulator, rescaled by exp(m_old - m_new) when the max grows
// ("RedFuser episode transcript", cues 19 and 39). The four waves take
// interleaved 32-key steps of the segment and their states are merged at the
// end the same way partial states are merged across segments (cue 21); the
// merged, still unnormalised state (m, l, acc) is written to memory.
//
// Second kernel: per query row, rescale the S partial states to the common max,
// add, divide by l once (cue 21; "RedFuser episode visual explainer", widget
// "Merging partial states across blocks (FlashDecoding-style)").
//
// Decode is bound by HBM bandwidth: every K/V byte is read exactly once per
// GQA group. Both contractions use v_mfma_f32_16x16x32_bf16 with the group's
// query heads in the N (or M) dimension, so bf16 K/V never need a VALU widening.
// K rows go straight from global memory into the A operand (16-byte loads);
// V rows are transposed through a per-wave LDS buffer so the B operand of
// O = P V gets its 8 keys with one 16-byte read.
#include "rf_device.hpp"
#include "rf_launch.hpp"

namespace rf {
namespace {

constexpr int D = 128;
constexpr int STEP = 32;  // keys per wave step
constexpr int NW = 4;     // waves per workgroup
constexpr int kVtBytes = D * STEP * 2;  // one transposed V step, 8 KB

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed V step: row d holds the step's 32 keys (64 bytes, four 16-byte
// chunks, XOR-swizzled by d so 16 consecutive d rows hit distinct banks).
__device__ __forceinline__ int vt_off(int d, int key4) {
  return d * 64 + (((key4 >> 3) ^ ((d >> 1) & 3)) << 4) + ((key4 >> 2) & 1) * 8;
}

struct KRegs {
  u32x4 k[2][4];  // A operand of S^T = K Q^T: [key block][d step]
};
struct VRegs {
  u32x4 v[2][4];  // V rows: [key group half][key within group of 4]
};

__global__ __launch_bounds__(256, 2) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ part_m, float* __restrict__ part_l,
    float* __restrict__ part_acc, int Hq, int Hkv, int Lk, int S, int seg_len, float scale) {
  __shared__ __attribute__((aligned(16))) char smem[NW * kVtBytes + 512];

  const int s = blockIdx.x % S;
  const int bhk = blockIdx.x / S;  // b * Hkv + hk
  const int b = bhk / Hkv, hk = bhk - b * Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, lq = lane & 15;

  const int t0 = min(s * seg_len, Lk), t1 = min(t0 + seg_len, Lk);
  const int nsteps = (t1 - t0 + STEP - 1) / STEP;

  const uint16_t* kp = k + (size_t)bhk * Lk * D;
  const uint16_t* vp = v + (size_t)bhk * Lk * D;

  // Q^T as the B operand: lane holds query head hk*G + lq (zero if lq >= G), d = 32*ds + 8*g.
  bf16x8 qf[4];
  {
    const uint16_t* qrow = q + ((size_t)b * Hq + hk * G + lq) * D;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (lq < G) w = *reinterpret_cast<const u32x4*>(qrow + 32 * ds + 8 * g);
      qf[ds] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // K row loaded by this lane for key block kb: row i = lq of the block holds key
  // 8*(lq/4) + 4*kb + lq%4, so lane group g ends up with keys 8g..8g+7 of the step.
  const int krow0 = 8 * (lq >> 2) + (lq & 3);
  auto load_k = [&](int step, KRegs& r) {
    const int kbase = t0 + step * STEP;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(kbase + krow0 + 4 * kb, Lk - 1);
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        r.k[kb][ds] = *reinterpret_cast<const u32x4*>(kp + (size_t)key * D + 32 * ds + 8 * g);
    }
  };
  auto load_v = [&](int step, VRegs& r) {
    const int kbase = t0 + step * STEP;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kg = g + 4 * i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = min(kbase + 4 * kg + j, Lk - 1);
        r.v[i][j] = *reinterpret_cast<const u32x4*>(vp + (size_t)key * D + 8 * lq);
      }
    }
  };

  float m_run = kNegInf, l_run = 0.f;  // statistics of query head lq
  f32x4 oacc[8];                       // O[q = 4g + r][d = 16*nb + lq]
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = f32x4{};

  // K rows are loaded two steps ahead of their use and V rows one step ahead
  // (three K register sets and two V sets in rotation).
  KRegs kcur, knxt, knxt2;
  VRegs vcur, vnxt;
  // Each wave owns an 8 KB slice of LDS for its transposed V step and touches
  // no other wave's slice, so the loop needs no workgroup barrier: LDS
  // operations of one wave execute in issue order, and the fences below only
  // stop the compiler from moving the reads above the writes (or the next
  // step's writes above this step's reads).
  char* vt = smem + wave * kVtBytes;
  if (wave < nsteps) {
    load_k(wave, kcur);
    load_v(wave, vcur);
  }
  if (wave + NW < nsteps) load_k(wave + NW, knxt);
  for (int step = wave; step < nsteps; step += NW) {
    if (step + NW < nsteps) load_v(step + NW, vnxt);
    if (step + 2 * NW < nsteps) load_k(step + 2 * NW, knxt2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kg = g + 4 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t a0 = vcur.v[i][0][e], a1 = vcur.v[i][1][e];
        const uint32_t a2 = vcur.v[i][2][e], a3 = vcur.v[i][3][e];
        const int d = 8 * lq + 2 * e;
        u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        *reinterpret_cast<u32x2*>(vt + vt_off(d, 4 * kg)) = lo;
        *reinterpret_cast<u32x2*>(vt + vt_off(d + 1, 4 * kg)) = hi;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int kbase = t0 + step * STEP;
    // ---- S^T = K Q^T: sacc[kb][r] is the score of key kbase + 8g + 4kb + r, head lq.
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 a = f32x4{};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) a = mfma16(__builtin_bit_cast(bf16x8, kcur.k[kb][ds]), qf[ds], a);
      sacc[kb] = a;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float sc = sacc[kb][r] * scale;
        if (kbase + 8 * g + 4 * kb + r >= t1) sc = kNegInf;
        sacc[kb][r] = sc;
        mx = fmaxf(mx, sc);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float ms = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - ms) * kLog2e);
    // P enters the second product as a sum of two bf16 terms (p = hi + lo), so
    // the weights keep about 16 significant bits; the extra MFMAs are free in a
    // kernel bound by HBM.
    float rs = 0.f;
    bf16x8 pa, pa_lo;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2((sacc[kb][r] - ms) * kLog2e);
        rs += p;
        const __bf16 hi = (__bf16)p;
        pa[4 * kb + r] = hi;
        pa_lo[4 * kb + r] = (__bf16)(p - (float)hi);
      }
    rs += __shfl_xor(rs, 16, kWave);
    rs += __shfl_xor(rs, 32, kWave);
    l_run = alpha * l_run + rs;
    m_run = m_new;
    // ---- rescale O rows 4g + r by their head's alpha, then O += P V.
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r, kWave);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[nb][r] *= ar[r];
      const int d = 16 * nb + lq;
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(vt + vt_off(d, 8 * g));
      oacc[nb] = mfma16(pa, vb, oacc[nb]);
      oacc[nb] = mfma16(pa_lo, vb, oacc[nb]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    kcur = knxt;
    knxt = knxt2;
    vcur = vnxt;
  }

  // ---- merge the four waves' states (same rule as the merge across segments).
  __syncthreads();
  float* sm_m = reinterpret_cast<float*>(smem);      // [NW][16]
  float* sm_l = sm_m + NW * 16;                       // [NW][16]
  float* sm_acc = sm_l + NW * 16;                     // [NW][16][D]
  if (g == 0) {
    sm_m[wave * 16 + lq] = m_run;
    sm_l[wave * 16 + lq] = l_run;
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qh = 4 * g + r;
      if (qh < G) sm_acc[(wave * 16 + qh) * D + 16 * nb + lq] = oacc[nb][r];
    }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int qh = idx / D, d = idx - qh * D;
    float mw[NW], ms = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = sm_m[w * 16 + qh];
      ms = fmaxf(ms, mw[w]);
    }
    float l = 0.f, acc = 0.f;
    if (ms != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = (mw[w] == kNegInf) ? 0.f : fast_exp2((mw[w] - ms) * kLog2e);
        l += wt * sm_l[w * 16 + qh];
        acc += wt * sm_acc[(w * 16 + qh) * D + d];
      }
    }
    const size_t row = ((size_t)b * Hq + hk * G + qh) * S + s;
    part_acc[row * D + d] = acc;
    if (d == 0) {
      part_m[row] = ms;
      part_l[row] = l;
    }
  }
}

// One workgroup per row. Thread (slice, c) folds the states s = slice,
// slice + nslices, ... of its row into a running (m, l, acc[4 columns]) with the
// same rescale-and-add rule (cue 21), then slice 0 merges the slices' states
// from LDS and writes the row.
__global__ __launch_bounds__(256) void merge_states_kernel(const float* __restrict__ part_m,
                                                           const float* __restrict__ part_l,
                                                           const float* __restrict__ part_acc,
                                                           int rows, int S, int d, int out_bf16,
                                                           void* __restrict__ o,
                                                           float* __restrict__ lse) {
  __shared__ float sm_m[256], sm_l[256];
  __shared__ f32x4 sm_acc[256];
  const int row = blockIdx.x;
  const int nd4 = d >> 2;
  const int nslices = 256 / nd4;
  const int tid = threadIdx.x;
  const int slice = tid / nd4, c = tid - slice * nd4;
  const bool worker = slice < nslices;
  const float* mrow = part_m + (size_t)row * S;
  const float* lrow = part_l + (size_t)row * S;
  const float* arow = part_acc + (size_t)row * S * d + 4 * c;
  float m = kNegInf, l = 0.f;
  f32x4 acc = f32x4{};
  if (worker) {
    for (int s = slice; s < S; s += nslices) {
      const float ms = mrow[s];
      if (ms == kNegInf) continue;  // empty segment: the identity
      const float ls = lrow[s];
      const f32x4 as = *reinterpret_cast<const f32x4*>(arow + (size_t)s * d);
      const float mn = fmaxf(m, ms);
      const float a = (m == kNegInf) ? 0.f : fast_exp2((m - mn) * kLog2e);
      const float b = fast_exp2((ms - mn) * kLog2e);
      l = l * a + ls * b;
      acc = acc * a + as * b;
      m = mn;
    }
    sm_acc[tid] = acc;
    if (c == 0) {
      sm_m[slice] = m;
      sm_l[slice] = l;
    }
  }
  __syncthreads();
  if (slice != 0) return;
  float ms = kNegInf;
  for (int j = 0; j < nslices; ++j) ms = fmaxf(ms, sm_m[j]);
  float lt = 0.f;
  f32x4 at = f32x4{};
  if (ms != kNegInf) {
    for (int j = 0; j < nslices; ++j) {
      const float mj = sm_m[j];
      if (mj == kNegInf) continue;
      const float w = fast_exp2((mj - ms) * kLog2e);
      lt += w * sm_l[j];
      at += w * sm_acc[j * nd4 + c];
    }
  }
  const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
  at *= inv;
  if (out_bf16) {
    u32x2 w = {pack_bf16x2(at[0], at[1]), pack_bf16x2(at[2], at[3])};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + (size_t)row * d + 4 * c) = w;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(o) + (size_t)row * d + 4 * c) = at;
  }
  if (lse && c == 0) lse[row] = (ms == kNegInf) ? kNegInf : ms + logf(lt);
}

}  // namespace

hipError_t launch_decode_split_bf16(const void* q, const void* k, const void* v, float* part_m,
                                    float* part_l, float* part_acc, int B, int Hq, int Hkv, int Lk,
                                    int d, int S, float scale, hipStream_t stream) {
  (void)d;
  const int seg_len = (Lk + S - 1) / S;
  dim3 grid(B * Hkv * S);
  hipLaunchKernelGGL(decode_split_kernel, grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), part_m, part_l, part_acc, Hq, Hkv, Lk, S,
                     seg_len, scale);
  return hipGetLastError();
}

hipError_t launch_merge_states(const float* part_m, const float* part_l, const float* part_acc,
                               int rows, int S, int d, int out_bf16, void* o, float* lse,
                               hipStream_t stream) {
  hipLaunchKernelGGL(merge_states_kernel, dim3(rows), dim3(256), 0, stream, part_m, part_l,
                     part_acc, rows, S, d, out_bf16, o, lse);
  return hipGetLastError();
}

}  // namespace rf
